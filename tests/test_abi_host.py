"""The C-ABI library on the host, without a GPU: it loads, exports every
function the public headers declare, validates arguments by the documented
rules (host-only check entry points, no kernel launch), and its build keeps
the arithmetic it promises."""
import concurrent.futures
import glob
import os
import re
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "diffusion_transformer_elementwise_amd")


def _builder():
    import __graft_entry__
    return __graft_entry__.builder()


@pytest.fixture(scope="module")
def dte():
    b = _builder()
    if not os.path.exists(b.LIBRARY):
        b.build_library()
    import diffusion_transformer_elementwise_amd as m
    return m


def _declared_functions():
    names = []
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        src = re.sub(r"#[^\n]*", "", src)
        for m in re.finditer(r"\b([A-Za-z_]\w*)\s*\(([^;{]*?)\)\s*;", src):
            names.append(m.group(1))
    return names


def test_headers_declare_the_boundary():
    names = set(_declared_functions())
    assert {"rga_residual_gate_add", "rms_modulate", "rga_status_string",
            "rga_check_residual_gate_add", "rga_check_rms_modulate",
            "rga_copy", "rga_fill"} <= names


def test_library_exports_every_declared_symbol(dte):
    lib = dte.library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", dte.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in _declared_functions():
        assert name in exported, name


def test_status_strings(dte):
    for st in range(5):
        assert dte.status_string(st)
    assert dte.status_string(99) == "unknown status"


A = 0x7F0000000000  # aligned fake device addresses; nothing is dereferenced
MB = 1 << 20


def test_gate_add_validation_rules(dte):
    ck = dte.check_residual_gate_add
    FULL, BCAST = dte.GATE_FULL, dte.GATE_BCAST
    x, u, g, o = A, A + 64 * MB, A + 128 * MB, A + 192 * MB
    ok, bad, uns, ali = dte.RGA_OK, dte.RGA_ERR_INVALID_ARG, dte.RGA_ERR_UNSUPPORTED, dte.RGA_ERR_ALIAS
    assert ck(x, u, g, o, 1, 126, 2048, FULL) == ok
    assert ck(x, u, g, o, 2, 5, 4096, BCAST) == ok
    # invalid arguments
    assert ck(x, u, g, o, -1, 1, 8, FULL) == bad
    assert ck(x, u, g, o, 1, -1, 8, FULL) == bad
    assert ck(x, u, g, o, 1, 1, -8, FULL) == bad
    assert ck(x, u, g, o, 1, 1, 8, 2) == bad
    assert ck(x, u, g, o, 1, 1, 8, -1) == bad
    assert ck(x, u, g, o, 1 << 31, 1 << 31, 1 << 2, FULL) == bad  # bytes overflow int64
    assert ck(0, u, g, o, 1, 1, 8, FULL) == bad
    assert ck(x, u, g, 0, 1, 1, 8, FULL) == bad
    # empty is a no-op even with NULL pointers
    assert ck(0, 0, 0, 0, 0, 5, 8, FULL) == ok
    assert ck(0, 0, 0, 0, 3, 0, 8, BCAST) == ok
    assert ck(0, 0, 0, 0, 3, 5, 0, BCAST) == ok
    # unsupported
    assert ck(x, u, g, o, 1, 1, 12, FULL) == uns
    assert ck(x + 2, u, g, o, 1, 1, 8, FULL) == uns
    assert ck(x, u, g + 8, o, 1, 1, 8, BCAST) == uns
    # aliasing: exact in-place is allowed
    assert ck(x, u, g, x, 1, 4, 8, FULL) == ok
    assert ck(x, u, g, u, 1, 4, 8, BCAST) == ok
    assert ck(x, u, g, g, 1, 4, 8, FULL) == ok
    assert ck(x, u, g, g, 1, 4, 8, BCAST) == ali  # out over a broadcast row
    assert ck(x, u, g, x + 16, 1, 4, 8, FULL) == ali  # partial overlap
    assert ck(x, u, o + 32, o, 2, 4, 8, BCAST) == ali  # gate row inside out
    assert ck(x, x, x, o, 1, 4, 8, FULL) == ok  # inputs may alias each other
    # adjacent (touching) ranges do not overlap
    n = 1 * 4 * 8 * 2
    assert ck(x, u, g, x + n, 1, 4, 8, FULL) == ok


def test_rms_validation_rules(dte):
    ck = dte.check_rms_modulate
    x, s, t, o = A, A + 64 * MB, A + 65 * MB, A + 128 * MB
    ok, bad, uns, ali = dte.RGA_OK, dte.RGA_ERR_INVALID_ARG, dte.RGA_ERR_UNSUPPORTED, dte.RGA_ERR_ALIAS
    big = 1 << 30  # room for a [2, 32640, 4096] bf16 tensor per buffer
    assert ck(A, A + big, A + big + MB, 1e-6, A + 2 * big, 2, 32640, 4096) == ok
    assert ck(A, A + big, A + big + MB, 1e-6, A + MB, 2, 32640, 4096) == ali
    assert ck(x, s, t, 0.0, o, 1, 1, 8) == ok
    assert ck(x, s, t, -1e-6, o, 1, 1, 8) == bad
    assert ck(x, s, t, float("nan"), o, 1, 1, 8) == bad
    assert ck(x, s, t, float("inf"), o, 1, 1, 8) == bad
    assert ck(x, s, t, 1e-6, o, -1, 1, 8) == bad
    assert ck(x, 0, t, 1e-6, o, 1, 1, 8) == bad
    assert ck(0, 0, 0, 1e-6, 0, 0, 1, 8) == ok
    assert ck(x, s, t, 1e-6, o, 1, 1, 20) == uns
    assert ck(x, s, t, 1e-6, o, 1, 1, dte.RGA_RMS_MAX_D) == ok
    # longer rows are not an unsupported layout: they run the LDS-staged kernels
    assert ck(x, s, t, 1e-6, o, 1, 1, dte.RGA_RMS_MAX_D + 8) == ok
    assert ck(x, s, t, 1e-6, o, 1, 1, 16384) == ok
    assert ck(x, s, t, 1e-6, o, 1, 1, 16388) == uns
    assert ck(x, s + 4, t, 1e-6, o, 1, 1, 8) == uns
    assert ck(x, s, t, 1e-6, x, 1, 4, 8) == ok  # in place
    assert ck(x, s, t, 1e-6, x + 16, 1, 4, 8) == ali
    assert ck(x, o, t, 1e-6, o, 1, 4, 8) == ali  # out over scale row
    assert ck(x, s, o + 16, 1e-6, o, 1, 4, 8) == ali


def test_binding_rejects_host_tensors_before_the_abi(dte):
    import torch
    x = torch.zeros(1, 2, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dte.rga_residual_gate_add(x, x, x)
    with pytest.raises(TypeError):
        dte.rms_modulate(x.float(), x, x)


def test_product_never_imports_the_oracle():
    for path in glob.glob(os.path.join(PKG, "**", "*"), recursive=True):
        if path.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
            text = open(path, encoding="utf-8").read()
            assert not re.search(r"\boracle\b", text), path


def _device_asm(src_name):
    src = os.path.join(PKG, "csrc", src_name)
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        b = _builder()
        subprocess.run([b.HIPCC, *b.COMMON, *b.DEVICE, "-x", "hip", "--cuda-device-only",
                        "-S", src, "-o", out], check=True, capture_output=True)
        return open(out).read()


def _kernel_bodies(asm):
    bodies = {}
    for m in re.finditer(r"^(_Z\w+):.*?\n(.*?)^\.Lfunc_end", asm, flags=re.S | re.M):
        bodies[m.group(1)] = m.group(2)
    return bodies


def test_gate_add_isa_has_no_fused_multiply_add():
    # The product of two 2-byte values is exact in binary32, so a fused
    # multiply-add would change results only for subnormal products (and for
    # binary32 storage it would change many); the build must never contract.
    every = _kernel_bodies(_device_asm("gate_add.hip"))
    # measurement variants (rga_gate_add_variant): bf16 broadcast gate,
    # {1, 2, 4, 8} rows per wave x {nontemporal, plain, device-scope} stores
    variants = {n: b for n, b in every.items() if "rows_kernel" in n}
    bodies = {n: b for n, b in every.items() if "rows_kernel" not in n}
    assert len(variants) == 12, sorted(variants)
    for name, body in variants.items():
        assert not re.search(r"\bv_(pk_)?(fma|fmac|fmamk|fmaak|mad|mac)(_mix\w*)?_f(16|32|64)", body), name
        T = int(re.search(r"rows_kernelILi(\d)E", name).group(1))
        SP = int(re.search(r"rows_kernelILi\dELi(\d)E", name).group(1))
        # one gate load for the whole tile, x and u per row
        assert len(re.findall(r"global_load_dwordx4", body)) == 1 + 2 * T, name
        if SP == 2:   # device scope: buffer stores with the SC1 bit, no nt
            stores = re.findall(r"buffer_store_dwordx4[^\n]*", body)
            assert len(stores) == T and all("sc1" in s and "nt" not in s for s in stores), name
        else:
            stores = re.findall(r"global_store_dwordx4[^\n]*", body)
            assert len(stores) == T and all((" nt" in s) == (SP == 0) for s in stores), name
    # {full, bcast, generic full, generic bcast} x {bf16, f16, f32}
    assert len(bodies) == 12, sorted(bodies)
    fast = {n: b for n, b in bodies.items() if "generic" not in n}
    assert len(fast) == 6
    for name, body in bodies.items():
        # float multiply-adds of any form (integer v_mad_u64_u32 address
        # arithmetic is fine)
        assert not re.search(r"\bv_(pk_)?(fma|fmac|fmamk|fmaak|mad|mac)(_mix\w*)?_f(16|32|64)", body), name
        assert not re.search(r"\bv_pk_(add|mul|fma)_f32", body), name
    for name, body in fast.items():
        # 128-bit accesses on the pack path: every word of every pack is
        # loaded and stored (an f16 build once read only the first word of
        # each pack, through a bit_cast of a vector element)
        words = 2 if "ILi2E" in name else 1
        nload = len(re.findall(r"global_load_dwordx4", body))
        nstore = len(re.findall(r"global_store_dwordx4", body))
        assert nstore == words, name
        assert nload == 3 * words, name  # x, u and g
    # bf16 storage narrows with the hardware round-to-nearest-even convert
    bf16 = [b for n, b in bodies.items() if re.search(r"kernelILi0E", n)]
    assert len(bf16) == 4 and all("v_cvt_pk_bf16_f32" in b for b in bf16)


def test_device_code_keeps_subnormals_and_ieee_sqrt_div():
    srcs = ("rms_modulate.hip", "gate_add_rms_modulate.hip")
    # the two device compiles are the slowest step of the host suite: run them side by side
    with concurrent.futures.ThreadPoolExecutor(len(srcs)) as pool:
        asms = list(pool.map(_device_asm, srcs))
    for src, asm in zip(srcs, asms):
        assert ".amdhsa_float_denorm_mode_32 0" not in asm, src
        bodies = _kernel_bodies(asm)
        assert asm.count(".amdhsa_float_denorm_mode_32 3") == len(bodies), src
        for name, body in bodies.items():
            assert "v_div_fixup_f32" in body, name      # IEEE division sequence
            assert "v_rsq_f32" not in body, name        # no approximate rsqrt
            assert not re.search(r"\bv_pk_(add|mul|fma)_f32", body), name


def test_one_hip_runtime_per_process():
    # importing the package (even through a submodule first) must leave
    # exactly one HIP runtime mapped: torch's
    code = ("import diffusion_transformer_elementwise_amd.ops, torch, ctypes\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "libs = {l.split()[-1] for l in maps if 'libamdhip64' in l}\n"
            "print(len(libs)); print(sorted(libs))\n")
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True,
                       cwd=ROOT, check=True)
    lines = r.stdout.splitlines()
    assert lines[0] == "1", lines
    import torch
    assert os.path.dirname(torch.__file__) in lines[1], lines


def test_fused_validation_rules(dte):
    ck = dte.check_gate_add_rms_modulate
    FULL, BCAST = dte.GATE_FULL, dte.GATE_BCAST
    ok, bad, uns, ali = dte.RGA_OK, dte.RGA_ERR_INVALID_ARG, dte.RGA_ERR_UNSUPPORTED, dte.RGA_ERR_ALIAS
    x, u, g, s, t, xo, y = (A + k * 64 * MB for k in range(7))
    args = lambda **kw: {**dict(x=x, u=u, g=g, scale=s, shift=t, eps=1e-6, x_out=xo, y=y,
                                B=2, L=5, D=4096, gate_mode=BCAST), **kw}
    call = lambda **kw: ck(*args(**kw).values())
    assert call() == ok
    assert call(gate_mode=FULL) == ok
    assert call(gate_mode=3) == bad
    assert call(eps=-1.0) == bad
    assert call(eps=float("nan")) == bad
    assert call(B=-1) == bad
    assert call(y=0) == bad
    assert call(x=0, u=0, g=0, scale=0, shift=0, x_out=0, y=0, L=0) == ok
    assert call(D=4100) == uns
    assert call(D=8200) == ok      # above the register rows: staged in LDS
    assert call(D=8204) == uns
    assert call(shift=t + 8) == uns
    # in place: each output may be x or u (or g in full mode)
    assert call(x_out=x) == ok
    assert call(x_out=u, y=x) == ok
    assert call(y=u) == ok
    assert call(x_out=g, gate_mode=FULL) == ok
    assert call(x_out=g, gate_mode=BCAST) == ali
    assert call(x_out=x, y=x) == ali           # both outputs on one buffer
    assert call(y=xo + 16) == ali              # outputs overlap
    assert call(y=s) == ali                    # output over scale row
    assert call(x_out=x + 32) == ali           # partial overlap with x


def test_ex_validation_rules(dte):
    ok, bad, uns, ali = dte.RGA_OK, dte.RGA_ERR_INVALID_ARG, dte.RGA_ERR_UNSUPPORTED, dte.RGA_ERR_ALIAS
    BF, F16, F32 = dte.DTYPE_BF16, dte.DTYPE_F16, dte.DTYPE_F32
    ROW, TOK = dte.MOD_ROW, dte.MOD_TOKEN
    FULL, BCAST = dte.GATE_FULL, dte.GATE_BCAST
    x, u, g, o = A, A + 64 * MB, A + 128 * MB, A + 192 * MB
    ga = dte.check_residual_gate_add_ex
    # any D, element alignment only; the strict call still rejects them
    for D in (1, 7, 12, 4100):
        assert ga(x, u, g, o, 2, 3, D, FULL, BF) == ok
        assert dte.check_residual_gate_add(x, u, g, o, 2, 3, D, FULL) == (ok if D % 8 == 0 else uns)
    assert ga(x + 2, u, g, o, 1, 1, 8, FULL, BF) == ok
    assert ga(x + 2, u, g, o, 1, 1, 8, FULL, F16) == ok
    assert ga(x + 2, u, g, o, 1, 1, 8, FULL, F32) == uns
    assert ga(x + 4, u, g + 12, o, 1, 1, 8, BCAST, F32) == ok
    assert ga(x + 1, u, g, o, 1, 1, 8, FULL, BF) == uns
    assert ga(x, u, g, o, 1, 1, 8, FULL, 3) == bad
    assert ga(x, u, g, o, 1, 1, 8, FULL, -1) == bad
    assert ga(0, 0, 0, 0, 0, 1, 8, FULL, 7) == bad      # dtype checked before the no-op
    assert ga(0, 0, 0, 0, 0, 1, 8, FULL, F32) == ok
    # byte ranges scale with the element size
    n = 1 * 4 * 8
    assert ga(x, u, g, x + 2 * n, 1, 4, 8, FULL, BF) == ok
    assert ga(x, u, g, x + 2 * n, 1, 4, 8, FULL, F32) == ali
    assert ga(x, u, g, x + 4 * n, 1, 4, 8, FULL, F32) == ok
    assert ga(x, u, g, u, 1, 4, 8, FULL, F16) == ok
    assert ga(x, u, g, g, 1, 4, 8, BCAST, F32) == ali
    assert ga(1 << 20, 0, 0, 0, 1 << 30, 1 << 30, 1 << 2, FULL, F32) == bad  # overflow

    rm = dte.check_rms_modulate_ex
    s, t = A + 64 * MB, A + 96 * MB
    assert rm(x, s, t, 1e-6, o, 1, 3, dte.RGA_RMS_MAX_D + 8, ROW, BF) == ok
    assert dte.check_rms_modulate(x, s, t, 1e-6, o, 1, 3, dte.RGA_RMS_MAX_D + 8) == ok
    assert rm(x, s, t, 1e-6, o, 1, 3, 4097, TOK, F16) == ok
    assert rm(x, s, t, 1e-6, o, 1, 3, 8, 2, BF) == bad
    assert rm(x, s, t, -1.0, o, 1, 3, 8, ROW, BF) == bad
    assert rm(x, s + 2, t, 1e-6, o, 1, 3, 8, ROW, F32) == uns
    assert rm(x, s, t, 1e-6, x, 1, 3, 8, TOK, F32) == ok   # in place
    # per-token scale covers [B, L, D]; a row covers [B, 1, D]
    rowb, tokb = 1 * 8 * 2, 1 * 3 * 8 * 2
    assert rm(x, o - rowb, t, 1e-6, o, 1, 3, 8, ROW, BF) == ok
    assert rm(x, o - rowb + 2, t, 1e-6, o, 1, 3, 8, ROW, BF) == ali
    assert rm(x, o - rowb, t, 1e-6, o, 1, 3, 8, TOK, BF) == ali
    assert rm(x, o - tokb, t, 1e-6, o, 1, 3, 8, TOK, BF) == ok

    fu = dte.check_gate_add_rms_modulate_ex
    xo, y, s, t = A + 224 * MB, A + 256 * MB, A + 288 * MB, A + 320 * MB
    call = lambda **kw: fu(*{**dict(x=x, u=u, g=g, scale=s, shift=t, eps=1e-6, x_out=xo, y=y,
                                   B=2, L=5, D=4100, gate_mode=BCAST, mod_mode=ROW,
                                   dtype=BF), **kw}.values())
    assert call() == ok
    assert call(dtype=F32, mod_mode=TOK, gate_mode=FULL) == ok
    assert call(D=dte.RGA_RMS_MAX_D + 8) == ok
    assert call(mod_mode=5) == bad
    assert call(dtype=3) == bad
    assert call(y=y + 2, dtype=F32) == uns
    assert call(x_out=x, y=u) == ok
    assert call(x_out=x, y=x) == ali
    assert call(y=xo + 2 * 2 * 5 * 4100 - 2) == ali                 # tail overlap
    assert call(y=xo + 2 * 2 * 5 * 4100) == ok
    assert call(y=xo + 2 * 2 * 5 * 4100, dtype=F32) == ali
    assert call(scale=y + 2 * 5 * 4100 * 2 - 2 * 4100 * 2, mod_mode=ROW) == ali
    assert call(scale=y - 2 * 5 * 4100 * 2, mod_mode=TOK) == ok
    assert call(scale=y - 2 * 5 * 4100 * 2 + 2, mod_mode=TOK) == ali


def test_gelu_validation_rules(dte):
    ok, bad, uns, ali = dte.RGA_OK, dte.RGA_ERR_INVALID_ARG, dte.RGA_ERR_UNSUPPORTED, dte.RGA_ERR_ALIAS
    BF, F16, F32 = dte.DTYPE_BF16, dte.DTYPE_F16, dte.DTYPE_F32
    ck = dte.check_gelu_tanh
    GB = 1024 * MB
    assert ck(A, 0, A + 2 * GB, 32640, 16384, BF) == ok          # 1 GiB tensors
    assert ck(A, A + 4 * GB, A + 2 * GB, 32640, 16384, BF) == ok
    assert ck(A, 0, A + GB // 2, 32640, 16384, BF) == ali
    x, b, o = A, A + 64 * MB, A + 128 * MB
    assert ck(x, b, o, 3, 13, F16) == ok                 # element path
    assert ck(x + 2, 0, o, 3, 16, BF) == ok
    assert ck(x + 2, 0, o, 3, 16, F32) == uns
    assert ck(x, b + 2, o, 3, 16, F32) == uns
    assert ck(x, 0, o, -1, 16, BF) == bad
    assert ck(x, 0, o, 1, -16, BF) == bad
    assert ck(x, 0, o, 1, 16, 3) == bad
    assert ck(0, 0, o, 1, 16, BF) == bad
    assert ck(x, 0, 0, 1, 16, BF) == bad
    assert ck(0, 0, 0, 0, 16, BF) == ok                  # empty
    assert ck(0, 0, 0, 5, 0, F32) == ok
    assert ck(x, 0, x, 7, 16, BF) == ok                  # in place
    assert ck(x, 0, x + 2, 7, 16, BF) == ali
    assert ck(x, o + 16, o, 7, 16, BF) == ali            # bias inside out
    assert ck(x, o - 32, o, 7, 16, BF) == ok             # bias row just before out
    assert ck(x, o - 30, o, 7, 16, BF) == ali
    assert ck(x, 0, o, 1 << 40, 1 << 30, F32) == bad     # bytes overflow


def test_gelu_isa_keeps_subnormals_and_no_contraction():
    asm = _device_asm("gelu_tanh.hip")
    bodies = _kernel_bodies(asm)
    assert len(bodies) == 12, sorted(bodies)
    assert asm.count(".amdhsa_float_denorm_mode_32 3") == len(bodies)
    for name, body in bodies.items():
        assert not re.search(r"\bv_(pk_)?(fma|fmac|fmamk|fmaak|mad|mac)(_mix\w*)?_f(16|32|64)", body), name
        assert not re.search(r"\bv_pk_(add|mul|fma)_f32", body), name
        assert "v_exp_f32" in body and "v_rcp_f32" in body, name


def test_ln_modulate_validation_follows_the_ex_rules(dte):
    ck, ref = dte.check_ln_modulate, dte.check_rms_modulate_ex
    x, s, t, o = A, A + 64 * MB, A + 96 * MB, A + 128 * MB
    cases = [
        (x, s, t, 1e-6, o, 2, 3, 4096, 0, 0), (x, s, t, 1e-6, o, 1, 3, 4100, 1, 1),
        (x, s, t, 1e-6, o, 1, 3, 20000, 0, 2), (x, s, t, -1.0, o, 1, 3, 8, 0, 0),
        (x, s, t, 1e-6, o, 1, 3, 8, 2, 0), (x, s, t, 1e-6, o, 1, 3, 8, 0, 3),
        (x + 2, s, t, 1e-6, o, 1, 3, 8, 0, 2), (x, s, t, 1e-6, x, 1, 3, 8, 1, 0),
        (x, o - 16, t, 1e-6, o, 1, 3, 8, 0, 0), (x, o - 16, t, 1e-6, o, 1, 3, 8, 1, 0),
        (0, 0, 0, 1e-6, 0, 0, 3, 8, 0, 0), (0, s, t, 1e-6, o, 1, 3, 8, 0, 0),
    ]
    want = [dte.RGA_OK, dte.RGA_OK, dte.RGA_OK, dte.RGA_ERR_INVALID_ARG,
            dte.RGA_ERR_INVALID_ARG, dte.RGA_ERR_INVALID_ARG, dte.RGA_ERR_UNSUPPORTED,
            dte.RGA_OK, dte.RGA_OK, dte.RGA_ERR_ALIAS, dte.RGA_OK, dte.RGA_ERR_INVALID_ARG]
    for c, w in zip(cases, want):
        assert ck(*c) == w == ref(*c), c


def test_grid_limits(dte):
    # the broadcast add puts B on grid y (<= 65535); the full add is one flat
    # stream, so any B fits while the pack grid does
    ok, uns = dte.RGA_OK, dte.RGA_ERR_UNSUPPORTED
    GB = 1024 * MB
    x, u, g, o = A, A + 16 * GB, A + 32 * GB, A + 48 * GB
    assert dte.check_residual_gate_add(x, u, g, o, 65535, 1, 8, dte.GATE_BCAST) == ok
    assert dte.check_residual_gate_add(x, u, g, o, 65536, 1, 8, dte.GATE_BCAST) == uns
    assert dte.check_residual_gate_add(x, u, g, o, 65536, 1, 8, dte.GATE_FULL) == ok
    # element path of a full add (D % 8 != 0 on a misaligned pointer) keeps y = 1
    assert dte.check_residual_gate_add_ex(x + 2, u, g, o, 65536, 1, 7, dte.GATE_FULL,
                                          dte.DTYPE_BF16) == ok
    assert dte.check_rms_modulate_ex(x, u, g, 1e-6, o, 65536, 1, 8, dte.MOD_ROW,
                                     dte.DTYPE_BF16) == uns
    # pack grid of the full add: ceil((n/8 + 1) / 64) workgroups of 64 lanes
    # must stay below 2^32 work-items
    n_max = (((1 << 32) - 1) // 64) * 64 * 8      # elements at the limit, roughly
    x, u, g, o = (A + k * 256 * GB for k in range(4))  # room for 2 * n_max bf16 each
    assert dte.check_residual_gate_add(x, u, g, o, 1, 1, n_max // 2, dte.GATE_FULL) == ok
    assert dte.check_residual_gate_add(x, u, g, o, 1, 1, n_max * 2, dte.GATE_FULL) == uns


def test_grid_limit_of_the_lds_staged_rows(dte):
    # binary32 rows of the element path are staged in LDS by one workgroup
    # per row of about one wave per 4 KB of row (a power of two from 2 to
    # 8): 400-byte rows take 2 waves (128 work-items), 64000-byte rows 8
    # (512). L times the workgroup size must stay below 2^32, a tighter
    # limit than the 64-lane kernels' (rows of 2-byte elements in
    # registers); the fused call has the same limit
    ok, uns = dte.RGA_OK, dte.RGA_ERR_UNSUPPORTED
    GB = 1024 * MB
    for D, lanes in ((100, 128), (16000, 512)):
        L_max = ((1 << 32) - 1) // lanes
        gap = 1 << ((L_max * D * 4).bit_length() + 1)  # tensors far apart
        ts = [A + k * gap for k in range(8)]
        for L, want in ((L_max, ok), (L_max + 1, uns)):
            assert dte.check_rms_modulate_ex(ts[0], ts[1], ts[2], 1e-6, ts[3], 1, L, D,
                                             dte.MOD_ROW, dte.DTYPE_F32) == want, (D, L)
            assert dte.check_gate_add_rms_modulate_ex(ts[0], ts[1], ts[2], ts[3], ts[4], 1e-6,
                                                      ts[5], ts[6], 1, L, D, dte.GATE_FULL,
                                                      dte.MOD_TOKEN, dte.DTYPE_F32) == want, (D, L)
    # a length past the 128-lane limit with 2-byte rows runs the 64-lane
    # register kernels
    L = ((1 << 32) - 1) // 128 + 1
    ts = [A + k * 64 * GB for k in range(8)]
    assert dte.check_rms_modulate_ex(ts[0], ts[1], ts[2], 1e-6, ts[3], 1, L, 100,
                                     dte.MOD_ROW, dte.DTYPE_BF16) == ok
    # row modulation of 2-byte rows runs two rows per 128-lane workgroup:
    # ceil(L / 2) * 128 work-items, so the largest L is 2 * floor((2^32 - 1)
    # / 128), one below the 64-lane bound (2^32 work-items at that odd L)
    L_pair = 2 * (((1 << 32) - 1) // 128)
    assert L_pair + 1 == ((1 << 32) - 1) // 64
    for D in (100, 8):  # the element path's and the fast path's staged rows
        for L, want in ((L_pair, ok), (L_pair + 1, uns)):
            assert dte.check_rms_modulate_ex(ts[0], ts[1], ts[2], 1e-6, ts[3], 1, L, D,
                                             dte.MOD_ROW, dte.DTYPE_BF16) == want, (D, L)
            assert dte.check_gate_add_rms_modulate_ex(ts[0], ts[1], ts[2], ts[3], ts[4], 1e-6,
                                                      ts[5], ts[6], 1, L, D, dte.GATE_BCAST,
                                                      dte.MOD_ROW, dte.DTYPE_BF16) == want, (D, L)


def test_package_fails_loudly_without_the_library(tmp_path):
    # a copy of the Python package without librga.so must refuse to import
    # (no CPU fallback anywhere)
    dst = tmp_path / "diffusion_transformer_elementwise_amd"
    dst.mkdir()
    for name in os.listdir(PKG):
        if name.endswith(".py"):
            shutil.copy(os.path.join(PKG, name), dst / name)
    r = subprocess.run([sys.executable, "-c", "import diffusion_transformer_elementwise_amd"],
                       cwd=tmp_path, capture_output=True, text=True,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "no CPU fallback" in r.stderr, r.stderr[-2000:]


def test_measurement_validation_rules(dte):
    ok, bad, uns, ali = dte.RGA_OK, dte.RGA_ERR_INVALID_ARG, dte.RGA_ERR_UNSUPPORTED, dte.RGA_ERR_ALIAS
    st = dte.check_stream
    a, b, c, d, k = (A + i * 64 * MB for i in range(5))
    n = 16 * MB
    assert st([a, b, c], d, n, 1, 0) == ok          # 3 reads, 1 write
    assert st([a, b], a, n, 1, 0) == ok             # in place on the first source
    assert st([a, b], b, n, 1, 0) == ali            # only the first source may be dst
    assert st([a, b], a + 16, n, 1, 0) == ali
    assert st([a], None, n, 2, k) == ok             # read-only needs a sink
    assert st([a], None, n, 2, 0) == bad
    assert st([a], None, n, 2, a + 32) == ali       # sink inside a source
    assert st([], d, n, 4, 0) == ok                 # write-only
    assert st([], None, n, 1, k) == bad
    assert st([a, b, c, a], d, n, 1, 0) == bad      # at most 3 sources
    assert st([a], d, n, 3, 0) == bad               # 1, 2 or 4 words per lane
    assert st([a], d, -16, 1, 0) == bad
    assert st([a], d, 0, 1, 0) == ok                # empty: no-op
    assert st([a], d, n + 8, 1, 0) == uns
    assert st([a + 8], d, n, 1, 0) == uns
    assert st([0], d, n, 1, 0) == bad

    gv = dte.check_gate_add_variant
    x, u, g, o = (A + i * 512 * MB for i in range(4))
    for T in (1, 2, 4, 8):
        for sp in (dte.STORE_NT, dte.STORE_PLAIN, dte.STORE_DEVICE):
            assert gv(x, u, g, x, 1, 32640, 4096, T, sp) == ok
    assert gv(x, u, g, o, 2, 32640, 4096, 3, 0) == bad
    assert gv(x, u, g, o, 2, 32640, 4096, 1, 3) == bad
    assert gv(x, u, g, o, 2, 33, 4100, 1, 0) == uns   # D % 8 != 0
    assert gv(x, u, g + 2, o, 2, 33, 4096, 1, 0) == uns
    assert gv(x, u, g, g, 2, 33, 4096, 1, 0) == ali   # out over the broadcast row
    assert gv(0, 0, 0, 0, 0, 33, 4096, 1, 0) == ok


def test_schedule_variants_take_the_workload_rows_only(dte):
    ok, bad, uns = dte.RGA_OK, dte.RGA_ERR_INVALID_ARG, dte.RGA_ERR_UNSUPPORTED
    x, s, t, o, u, g, y = (A + i * 512 * MB for i in range(7))
    mv, fv = dte.check_modulate_variant, dte.check_fused_variant
    for sched in range(5):
        assert mv(x, s, t, 1e-6, o, 2, 32640, 4096, sched) == ok
        assert fv(x, u, g, s, t, 1e-6, x, y, 2, 32640, 4096, sched) == ok
    for sched in (-1, 5):
        assert mv(x, s, t, 1e-6, o, 2, 32640, 4096, sched) == bad
        assert fv(x, u, g, s, t, 1e-6, x, y, 2, 32640, 4096, sched) == bad
    # only 4096-element rows; layout rules of the strict calls; empty is a no-op
    for D in (4104, 2048, 8192):
        assert mv(x, s, t, 1e-6, o, 2, 31, D, 0) == uns
        assert fv(x, u, g, s, t, 1e-6, x, y, 2, 31, D, 0) == uns
    assert mv(x + 2, s, t, 1e-6, o, 2, 31, 4096, 0) == uns
    assert fv(x, u, g + 8, s, t, 1e-6, x, y, 2, 31, 4096, 0) == uns
    assert mv(x, s, t, 1e-6, o, 0, 31, 4100, 0) == ok
    assert mv(x, s, t, -1.0, o, 2, 31, 4096, 0) == bad
    assert fv(x, u, g, s, t, 1e-6, x, x, 2, 31, 4096, 0) == dte.RGA_ERR_ALIAS
    assert mv(x, s, t, 1e-6, s, 2, 31, 4096, 0) == dte.RGA_ERR_ALIAS


def test_occupancy_helpers_follow_the_ex_rules(dte):
    ok, bad, uns = dte.RGA_OK, dte.RGA_ERR_INVALID_ARG, dte.RGA_ERR_UNSUPPORTED
    x, s, t, o, u, g, y = (A + i * 512 * MB for i in range(7))
    mo, ref = dte.check_modulate_occupancy, dte.check_rms_modulate_ex
    for D, dt in ((4096, 0), (4100, 0), (4096, 2), (8200, 1)):
        for w in (-1, 0, 4, 16):
            assert mo(x, s, t, 1e-6, o, 2, 32640, D, dt, w) == ok == ref(
                x, s, t, 1e-6, o, 2, 32640, D, dte.MOD_ROW, dt)
    assert mo(x, s, t, 1e-6, o, 2, 32640, 4096, 0, 17) == bad
    assert mo(x, s, t, 1e-6, o, 2, 32640, 4096, 0, -2) == bad
    assert mo(x + 1, s, t, 1e-6, o, 2, 3, 4096, 0, 4) == uns
    assert mo(x, s, t, -1.0, o, 2, 3, 4096, 0, 4) == bad
    fo = dte.check_fused_occupancy
    for gm in (dte.GATE_BCAST, dte.GATE_FULL):
        assert fo(x, u, g, s, t, 1e-6, x, y, 2, 32640, 4096, gm, 0, 4) == ok
    assert fo(x, u, g, s, t, 1e-6, x, y, 2, 32640, 4096, 1, 0, 99) == bad
    assert fo(x, u, g, s, t, 1e-6, x, x, 2, 32640, 4096, 1, 0, 4) == dte.RGA_ERR_ALIAS
