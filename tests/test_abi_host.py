"""The C-ABI library on the host, without a GPU: it loads, exports every
function the public headers declare, validates arguments by the documented
rules (host-only check entry points, no kernel launch), and its build keeps
the arithmetic it promises."""
import glob
import os
import re
import subprocess
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
    assert ck(x, s, t, 1e-6, o, 1, 1, dte.RGA_RMS_MAX_D + 8) == uns
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
    # The product of two bf16 values is exact in binary32, so a fused
    # multiply-add would change results only for subnormal products; the
    # build must still not contract. Also check 128-bit accesses.
    bodies = _kernel_bodies(_device_asm("gate_add.hip"))
    assert len(bodies) == 2
    for name, body in bodies.items():
        # float multiply-adds of any form (integer v_mad_u64_u32 address
        # arithmetic is fine)
        assert not re.search(r"\bv_(pk_)?(fma|fmac|fmamk|fmaak|mad|mac)(_mix\w*)?_f(16|32|64)", body), name
        assert "global_load_dwordx4" in body and "global_store_dwordx4" in body, name
        assert "v_cvt_pk_bf16_f32" in body, name
        assert not re.search(r"\bv_pk_(add|mul|fma)_f32", body), name


def test_device_code_keeps_subnormals_and_ieee_sqrt_div():
    asm = _device_asm("rms_modulate.hip")
    assert ".amdhsa_float_denorm_mode_32 3" in asm
    body = next(iter(_kernel_bodies(asm).values()))
    assert "v_div_fixup_f32" in body          # IEEE division sequence
    assert "v_rsq_f32" not in body            # no approximate reciprocal sqrt
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32", body)


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
    assert call(D=8200) == uns
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
