"""Parity of the extended entry points (the _ex calls) with the oracle's
extended functions: every storage type (bf16, binary16, binary32), D of any
size (ragged last group, rows beyond the register-resident limit), tensors
that start at any element offset, per-token modulation, and the ideogram4
shape from the residual-gate page's benchmark table.

Bars, as for the bf16 calls: the gated residual add is bit-exact for every
storage type; the modulation is within one ULP of its storage type and, since
the library and the oracle fix the same binary32 order, in fact identical.
"""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import (BF16, EXTRA_CASES, F16, F32, GATE_BCAST, GATE_FULL, N001, N01, N02,
                          U11, make_inputs, random_typed)
from tests.test_gpu_gelu import _check as gelu_check, _values as gelu_inputs
from tests.gpu_util import (first_mismatch_typed, same_bits_typed, say, to_dev, to_dev_typed,
                            to_host, to_host_typed, ulp_diff_typed)

pytestmark = pytest.mark.gpu

MOD_ROW, MOD_TOKEN = oracle.MOD_ROW, oracle.MOD_TOKEN
DTYPES = [BF16, F16, F32]
NAMES = {BF16: "bf16", F16: "f16", F32: "f32"}


@pytest.fixture(scope="module")
def dte():
    import diffusion_transformer_elementwise_amd as m
    return m


def _bit_exact(got, want, dtype, label):
    assert same_bits_typed(got, want, dtype), f"{label}: " + first_mismatch_typed(got, want, dtype)


def _zero_ulp(got, want, dtype, label):
    d = ulp_diff_typed(got, want, dtype)
    hist = np.bincount(np.minimum(d.ravel(), 3), minlength=4)
    say(f"[{label}] ULP histogram 0:{hist[0]} 1:{hist[1]} 2:{hist[2]} >2:{hist[3]}")
    assert d.max() <= 1, f"{label}: max {d.max()} ULP"
    assert d.max() == 0, f"{label}: pinned order, expected identical results"


# (B, L, D): multiples of 8 (pack path), ragged D (element path), one-element
# rows, rows longer than the register-resident limit
SHAPES = [
    (1, 1, 8), (2, 5, 24), (3, 7, 520), (2, 33, 1032), (1, 333, 3072),
    (1, 3, 1), (2, 5, 7), (3, 7, 13), (1, 1, 515), (2, 9, 1001), (1, 17, 4100), (2, 3, 8200),
]


def _gate_inputs(seed, B, L, D, mode, dtype):
    x = random_typed(seed, (B, L, D), N02, dtype)
    u = random_typed(seed + 1, (B, L, D), N01, dtype)
    g = random_typed(seed + 2, (B, L, D) if mode == GATE_FULL else (B, 1, D), U11, dtype)
    return x, u, g


def _mod_inputs(seed, B, L, D, mod, dtype):
    shape = (B, L, D) if mod == MOD_TOKEN else (B, 1, D)
    return random_typed(seed, shape, N001, dtype), random_typed(seed + 1, shape, N001, dtype)


@pytest.mark.parametrize("dtype", DTYPES, ids=NAMES.get)
@pytest.mark.parametrize("mode", [GATE_FULL, GATE_BCAST])
@pytest.mark.parametrize("B,L,D", SHAPES)
def test_gate_add_ex(dte, B, L, D, mode, dtype):
    say(f"[gate-add ex] {NAMES[dtype]} B={B} L={L} D={D} mode={mode}")
    x, u, g = _gate_inputs(1000 + 7 * B + L + D, B, L, D, mode, dtype)
    want = oracle.gate_add_ex(x, u, g, mode, dtype)
    out = dte.rga_residual_gate_add_ex(to_dev_typed(x, dtype), to_dev_typed(u, dtype),
                                       to_dev_typed(g, dtype), gate_mode=mode)
    _bit_exact(to_host_typed(out), want, dtype, "gate-add ex")


@pytest.mark.parametrize("dtype", DTYPES, ids=NAMES.get)
@pytest.mark.parametrize("mod", [MOD_ROW, MOD_TOKEN])
@pytest.mark.parametrize("B,L,D", SHAPES)
def test_rms_modulate_ex(dte, B, L, D, mod, dtype):
    say(f"[rms ex] {NAMES[dtype]} B={B} L={L} D={D} mod={mod}")
    seed = 2000 + 5 * B + L + D
    x = random_typed(seed, (B, L, D), N02, dtype)
    s, t = _mod_inputs(seed + 1, B, L, D, mod, dtype)
    want = oracle.rms_modulate_ex(x, s, t, 1e-6, mod, dtype)
    out = dte.rga_rms_modulate_ex(to_dev_typed(x, dtype), to_dev_typed(s, dtype),
                                  to_dev_typed(t, dtype), 1e-6, mod_mode=mod)
    _zero_ulp(to_host_typed(out), want, dtype, f"rms ex {NAMES[dtype]} {B}x{L}x{D} mod={mod}")


@pytest.mark.parametrize("dtype", DTYPES, ids=NAMES.get)
@pytest.mark.parametrize("mode,mod", [(GATE_FULL, MOD_ROW), (GATE_BCAST, MOD_ROW),
                                      (GATE_BCAST, MOD_TOKEN), (GATE_FULL, MOD_TOKEN)])
@pytest.mark.parametrize("B,L,D", SHAPES)
def test_fused_ex(dte, B, L, D, mode, mod, dtype):
    say(f"[fused ex] {NAMES[dtype]} B={B} L={L} D={D} mode={mode} mod={mod}")
    seed = 3000 + 3 * B + L + D
    x, u, g = _gate_inputs(seed, B, L, D, mode, dtype)
    s, t = _mod_inputs(seed + 3, B, L, D, mod, dtype)
    want_x, want_y = oracle.gate_add_rms_modulate_ex(x, u, g, s, t, 1e-6, mode, mod, dtype)
    xo, y = dte.rga_gate_add_rms_modulate_ex(
        to_dev_typed(x, dtype), to_dev_typed(u, dtype), to_dev_typed(g, dtype),
        to_dev_typed(s, dtype), to_dev_typed(t, dtype), 1e-6, gate_mode=mode, mod_mode=mod)
    _bit_exact(to_host_typed(xo), want_x, dtype, "fused ex x_out")
    _zero_ulp(to_host_typed(y), want_y, dtype, f"fused ex y {NAMES[dtype]} {B}x{L}x{D}")


@pytest.mark.parametrize("dtype", DTYPES, ids=NAMES.get)
@pytest.mark.parametrize("D", [64, 4096, 13])
def test_element_offsets(dte, D, dtype):
    # every tensor one element into its allocation: 2- or 4-byte aligned
    # addresses take the element-wise kernels, with the same results
    B, L = 2, 37
    say(f"[offsets] {NAMES[dtype]} B={B} L={L} D={D}")
    x, u, g = _gate_inputs(4000 + D, B, L, D, GATE_BCAST, dtype)
    s, t = _mod_inputs(4100 + D, B, L, D, MOD_ROW, dtype)
    dx, du, dg = (to_dev_typed(a, dtype, offset=1) for a in (x, u, g))
    ds, dt = (to_dev_typed(a, dtype, offset=1) for a in (s, t))
    assert dx.data_ptr() % 16 != 0
    want = oracle.gate_add_ex(x, u, g, GATE_BCAST, dtype)
    _bit_exact(to_host_typed(dte.rga_residual_gate_add_ex(dx, du, dg)), want, dtype, "gate")
    want_y = oracle.rms_modulate_ex(x, s, t, 1e-6, MOD_ROW, dtype)
    _zero_ulp(to_host_typed(dte.rga_rms_modulate_ex(dx, ds, dt, 1e-6)), want_y, dtype, "rms")
    wx, wy = oracle.gate_add_rms_modulate_ex(x, u, g, s, t, 1e-6, GATE_BCAST, MOD_ROW, dtype)
    xo = torch.empty(B * L * D + 1, dtype=dx.dtype, device=dx.device)[1:].view(B, L, D)
    yo = torch.empty(B * L * D + 1, dtype=dx.dtype, device=dx.device)[1:].view(B, L, D)
    dte.rga_gate_add_rms_modulate_ex(dx, du, dg, ds, dt, 1e-6, x_out=xo, y=yo)
    _bit_exact(to_host_typed(xo), wx, dtype, "fused x_out")
    _zero_ulp(to_host_typed(yo), wy, dtype, "fused y")


def _empty_at(shape, like, offset):
    n = int(np.prod(shape))
    return torch.empty(n + offset, dtype=like.dtype, device=like.device)[offset:].view(shape)


# each entry of the element path's slot ladder (ceil(ceil(D / 8) / 64) slots
# of 8-element groups per lane: 1, 2, 4, 6, 8, 9, 12, 16), rows past it
# (staged in LDS: binary32 rows and 2-byte rows up to 64 KB) and rows past
# the LDS limit (two passes)
MIXED_D = [1, 100, 1000, 1500, 2500, 4000, 4500, 6000, 8191, 8193, 16370, 33001]


@pytest.mark.parametrize("dtype", DTYPES, ids=NAMES.get)
@pytest.mark.parametrize("D", MIXED_D)
def test_mixed_offsets(dte, D, dtype):
    # every operand at its own element offset (so the realignment into and
    # out of registers differs per operand), outputs too
    B, L = 2, 6
    say(f"[mixed offsets] {NAMES[dtype]} B={B} L={L} D={D}")
    x, u, g = _gate_inputs(5000 + D, B, L, D, GATE_BCAST, dtype)
    s, t = _mod_inputs(5100 + D, B, L, D, MOD_ROW, dtype)
    ts, tt = _mod_inputs(5200 + D, B, L, D, MOD_TOKEN, dtype)
    dx, du, dg = to_dev_typed(x, dtype, 1), to_dev_typed(u, dtype, 2), to_dev_typed(g, dtype, 3)
    ds, dt = to_dev_typed(s, dtype, 5), to_dev_typed(t, dtype, 6)
    dts, dtt = to_dev_typed(ts, dtype, 7), to_dev_typed(tt, dtype, 3)
    for off in (0, 5):
        out = _empty_at((B, L, D), dx, off)
        dte.rga_residual_gate_add_ex(dx, du, dg, out=out)
        _bit_exact(to_host_typed(out), oracle.gate_add_ex(x, u, g, GATE_BCAST, dtype), dtype,
                   f"gate bcast out+{off}")
        gf = random_typed(5300 + D, (B, L, D), U11, dtype)
        dte.rga_residual_gate_add_ex(dx, du, to_dev_typed(gf, dtype, 4), out=out,
                                     gate_mode=GATE_FULL)
        _bit_exact(to_host_typed(out), oracle.gate_add_ex(x, u, gf, GATE_FULL, dtype), dtype,
                   f"gate full out+{off}")
        dte.rga_rms_modulate_ex(dx, ds, dt, 1e-6, out=out)
        _zero_ulp(to_host_typed(out), oracle.rms_modulate_ex(x, s, t, 1e-6, MOD_ROW, dtype),
                  dtype, f"rms row out+{off}")
        dte.rga_rms_modulate_ex(dx, dts, dtt, 1e-6, out=out, mod_mode=MOD_TOKEN)
        _zero_ulp(to_host_typed(out), oracle.rms_modulate_ex(x, ts, tt, 1e-6, MOD_TOKEN, dtype),
                  dtype, f"rms token out+{off}")
        dte.rga_ln_modulate(dx, ds, dt, 1e-6, out=out)
        _zero_ulp(to_host_typed(out), oracle.ln_modulate(x, s, t, 1e-6, MOD_ROW, dtype),
                  dtype, f"ln row out+{off}")
        yo = _empty_at((B, L, D), dx, off + 2)
        dte.rga_gate_add_rms_modulate_ex(dx, du, dg, ds, dt, 1e-6, x_out=out, y=yo)
        wx, wy = oracle.gate_add_rms_modulate_ex(x, u, g, s, t, 1e-6, GATE_BCAST, MOD_ROW, dtype)
        _bit_exact(to_host_typed(out), wx, dtype, f"fused x_out+{off}")
        _zero_ulp(to_host_typed(yo), wy, dtype, f"fused y+{off + 2}")
        dte.gelu_tanh(dx, out=out)
        gelu_check(to_host_typed(out), oracle.gelu_tanh(x, dtype), gelu_inputs(x, dtype), dtype,
                   f"gelu out+{off}")


@pytest.mark.parametrize("dtype", [BF16, F16], ids=NAMES.get)
@pytest.mark.parametrize("D", [1000, 4100])
def test_every_offset_of_every_operand(dte, D, dtype):
    # the register-resident rows realign each operand with code for its byte
    # offset inside a 16-byte word (8 even offsets for a 2-byte type): each
    # operand is moved through all 8 element offsets, every operand at a
    # different one. D = 1000 keeps an operand's rows at one offset, D = 4100
    # alternates two.
    B, L = 2, 3
    x, u, g = _gate_inputs(5400 + D, B, L, D, GATE_BCAST, dtype)
    gf = random_typed(5401 + D, (B, L, D), U11, dtype)
    s, t = _mod_inputs(5402 + D, B, L, D, MOD_ROW, dtype)
    ts, tt = _mod_inputs(5403 + D, B, L, D, MOD_TOKEN, dtype)
    want_gate = oracle.gate_add_ex(x, u, g, GATE_BCAST, dtype)
    want_rms = oracle.rms_modulate_ex(x, s, t, 1e-6, MOD_ROW, dtype)
    want_rms_tok = oracle.rms_modulate_ex(x, ts, tt, 1e-6, MOD_TOKEN, dtype)
    want_ln = oracle.ln_modulate(x, s, t, 1e-6, MOD_ROW, dtype)
    want_ln_tok = oracle.ln_modulate(x, ts, tt, 1e-6, MOD_TOKEN, dtype)
    wbx, wby = oracle.gate_add_rms_modulate_ex(x, u, g, s, t, 1e-6, GATE_BCAST, MOD_ROW, dtype)
    wfx, wfy = oracle.gate_add_rms_modulate_ex(x, u, gf, ts, tt, 1e-6, GATE_FULL, MOD_TOKEN,
                                               dtype)
    for o in range(8):
        say(f"[every offset] {NAMES[dtype]} D={D} rotation {o}")
        dx, du, dg, dgf, ds, dt, dts, dtt = (
            to_dev_typed(a, dtype, (o + k) % 8) for k, a in enumerate((x, u, g, gf, s, t, ts, tt)))
        out = _empty_at((B, L, D), dx, (o + 3) % 8)
        yo = _empty_at((B, L, D), dx, (o + 6) % 8)
        dte.rga_residual_gate_add_ex(dx, du, dg, out=out)
        _bit_exact(to_host_typed(out), want_gate, dtype, f"gate, rotation {o}")
        dte.rga_rms_modulate_ex(dx, ds, dt, 1e-6, out=out)
        _zero_ulp(to_host_typed(out), want_rms, dtype, f"rms row, rotation {o}")
        dte.rga_rms_modulate_ex(dx, dts, dtt, 1e-6, out=out, mod_mode=MOD_TOKEN)
        _zero_ulp(to_host_typed(out), want_rms_tok, dtype, f"rms token, rotation {o}")
        dte.rga_ln_modulate(dx, ds, dt, 1e-6, out=out)
        _zero_ulp(to_host_typed(out), want_ln, dtype, f"ln row, rotation {o}")
        dte.rga_ln_modulate(dx, dts, dtt, 1e-6, out=out, mod_mode=MOD_TOKEN)
        _zero_ulp(to_host_typed(out), want_ln_tok, dtype, f"ln token, rotation {o}")
        dte.rga_gate_add_rms_modulate_ex(dx, du, dg, ds, dt, 1e-6, x_out=out, y=yo)
        _bit_exact(to_host_typed(out), wbx, dtype, f"fused bcast x_out, rotation {o}")
        _zero_ulp(to_host_typed(yo), wby, dtype, f"fused bcast y, rotation {o}")
        dte.rga_gate_add_rms_modulate_ex(dx, du, dgf, dts, dtt, 1e-6, x_out=out, y=yo,
                                         gate_mode=GATE_FULL, mod_mode=MOD_TOKEN)
        _bit_exact(to_host_typed(out), wfx, dtype, f"fused full x_out, rotation {o}")
        _zero_ulp(to_host_typed(yo), wfy, dtype, f"fused full y, rotation {o}")


# register-resident rows run with K slots from the ladder 1, 2, 4, 6, 8, 9,
# 12, 16; an instance sums the slots below the previous entry without
# masks, so each K is checked on the shortest row it serves (512 times the
# previous entry, plus one) and the longest (512 K)
LADDER_D = [1, 512, 513, 1024, 1025, 2048, 2049, 3072, 3073, 4096, 4097, 4608, 4609, 6144,
            6145, 8192]


@pytest.mark.parametrize("D", LADDER_D)
def test_register_rows_across_the_slot_ladder(dte, D):
    B, L = 2, 3
    dtype = BF16
    say(f"[slot ladder] bf16 B={B} L={L} D={D}")
    x, u, g = _gate_inputs(5700 + D, B, L, D, GATE_BCAST, dtype)
    s, t = _mod_inputs(5701 + D, B, L, D, MOD_ROW, dtype)
    dx, du, dg = to_dev_typed(x, dtype, 1), to_dev_typed(u, dtype), to_dev_typed(g, dtype, 2)
    ds, dt = to_dev_typed(s, dtype, 3), to_dev_typed(t, dtype)
    _zero_ulp(to_host_typed(dte.rga_rms_modulate_ex(dx, ds, dt, 1e-6)),
              oracle.rms_modulate_ex(x, s, t, 1e-6, MOD_ROW, dtype), dtype, "rms")
    _zero_ulp(to_host_typed(dte.rga_ln_modulate(dx, ds, dt, 1e-6)),
              oracle.ln_modulate(x, s, t, 1e-6, MOD_ROW, dtype), dtype, "ln")
    wx, wy = oracle.gate_add_rms_modulate_ex(x, u, g, s, t, 1e-6, GATE_BCAST, MOD_ROW, dtype)
    xo, yo = dte.rga_gate_add_rms_modulate_ex(dx, du, dg, ds, dt, 1e-6)
    _bit_exact(to_host_typed(xo), wx, dtype, "fused x_out")
    _zero_ulp(to_host_typed(yo), wy, dtype, "fused y")


# rows staged in LDS run with 2, 4 or 8 waves per row, switching at 12288
# and 24576 bytes of row: binary32 rows on both sides of each switch, 2-byte
# rows (staged from 8193 elements on) on both sides of the second
LDS_SIZES = [(F32, 3072), (F32, 3073), (F32, 6144), (F32, 6145), (BF16, 8193),
             (BF16, 12288), (BF16, 12289)]


@pytest.mark.parametrize("dtype,D", LDS_SIZES, ids=[f"{NAMES[t]}-{d}" for t, d in LDS_SIZES])
def test_lds_rows_at_the_wave_count_switches(dte, dtype, D):
    B, L = 2, 5
    say(f"[lds row sizes] {NAMES[dtype]} B={B} L={L} D={D}")
    x, u, g = _gate_inputs(5600 + D, B, L, D, GATE_BCAST, dtype)
    s, t = _mod_inputs(5601 + D, B, L, D, MOD_ROW, dtype)
    dx, du, dg = to_dev_typed(x, dtype, 1), to_dev_typed(u, dtype), to_dev_typed(g, dtype)
    ds, dt = to_dev_typed(s, dtype), to_dev_typed(t, dtype, 3)
    _zero_ulp(to_host_typed(dte.rga_rms_modulate_ex(dx, ds, dt, 1e-6)),
              oracle.rms_modulate_ex(x, s, t, 1e-6, MOD_ROW, dtype), dtype, "rms")
    _zero_ulp(to_host_typed(dte.rga_ln_modulate(dx, ds, dt, 1e-6)),
              oracle.ln_modulate(x, s, t, 1e-6, MOD_ROW, dtype), dtype, "ln")
    wx, wy = oracle.gate_add_rms_modulate_ex(x, u, g, s, t, 1e-6, GATE_BCAST, MOD_ROW, dtype)
    xo, yo = dte.rga_gate_add_rms_modulate_ex(dx, du, dg, ds, dt, 1e-6)
    _bit_exact(to_host_typed(xo), wx, dtype, "fused x_out")
    _zero_ulp(to_host_typed(yo), wy, dtype, "fused y")


def test_bf16_ex_runs_the_same_kernels_as_the_bf16_calls(dte):
    # with bf16, row modulation, D % 8 == 0 and aligned tensors the _ex calls
    # take the pack path: identical results to the original calls
    B, L, D = 2, 129, 4096
    say(f"[ex == original] B={B} L={L} D={D}")
    x, u, g = _gate_inputs(5000, B, L, D, GATE_BCAST, BF16)
    s, t = _mod_inputs(5003, B, L, D, MOD_ROW, BF16)
    dx, du, dg, ds, dt = (to_dev(a) for a in (x, u, g, s, t))
    a = to_host(dte.rga_residual_gate_add_ex(dx, du, dg))
    b = to_host(dte.rga_residual_gate_add(dx, du, dg))
    assert np.array_equal(a, b)
    a = to_host(dte.rga_rms_modulate_ex(dx, ds, dt, 1e-6))
    b = to_host(dte.rms_modulate(dx, ds, dt, 1e-6))
    assert np.array_equal(a, b)
    a = [to_host(v) for v in dte.rga_gate_add_rms_modulate_ex(dx, du, dg, ds, dt, 1e-6)]
    b = [to_host(v) for v in dte.rga_gate_add_rms_modulate(dx, du, dg, ds, dt, 1e-6)]
    assert all(np.array_equal(p, q) for p, q in zip(a, b))


@pytest.mark.parametrize("dtype", [F16, F32], ids=NAMES.get)
def test_gate_add_every_pattern(dtype, dte):
    # x over bit patterns (every binary16 pattern; 2**16 spread binary32
    # patterns incl. NaN, inf, subnormals), u and g random patterns: special
    # values, overflow to inf and subnormal results go through both sides
    say(f"[patterns] {NAMES[dtype]}")
    rng = np.random.default_rng(6000 + dtype)
    n = 1 << 16
    if dtype == F16:
        x = np.arange(n, dtype=np.uint16).reshape(1, 64, 1024)
        u = rng.integers(0, 1 << 16, size=n, dtype=np.uint16).reshape(x.shape)
        g = rng.integers(0, 1 << 16, size=n, dtype=np.uint16).reshape(x.shape)
    else:
        w = lambda: rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
        x = w().view(np.float32).reshape(1, 64, 1024)
        u = w().view(np.float32).reshape(x.shape)
        g = w().view(np.float32).reshape(x.shape)
        # exponents near the bottom and the top of the range
        u[0, :8] = (np.arange(8 * 1024, dtype=np.uint32) | 0x00700000).view(np.float32).reshape(8, 1024)
        g[0, 8:16] = np.float32(2.0 ** 100)
    want = oracle.gate_add_ex(x, u, g, GATE_FULL, dtype)
    got = to_host_typed(dte.rga_residual_gate_add_ex(
        to_dev_typed(x, dtype), to_dev_typed(u, dtype), to_dev_typed(g, dtype)))
    _bit_exact(got, want, dtype, f"patterns {NAMES[dtype]}")


def test_ideogram4_bcast_full_size(dte):
    case = EXTRA_CASES["ideogram4"]
    say(f"[gate-add] {case.name} B={case.B} L={case.L} D={case.D}")
    inp = make_inputs(case)
    want = oracle.gate_add(inp["x"], inp["u"], inp["g"], case.gate)
    out = dte.rga_residual_gate_add(to_dev(inp["x"]), to_dev(inp["u"]), to_dev(inp["g"]),
                                    gate_mode=case.gate)
    _bit_exact(to_host(out), want, BF16, case.name)


@pytest.mark.parametrize("dtype", [F16, F32], ids=NAMES.get)
def test_token_modulation_at_video_scale(dte, dtype):
    # per-token scale/shift at a DiT shape, through the pack path
    B, L, D = 1, 4096, 3072
    say(f"[token mod] {NAMES[dtype]} B={B} L={L} D={D}")
    x, u, g = _gate_inputs(7000 + dtype, B, L, D, GATE_BCAST, dtype)
    s, t = _mod_inputs(7003 + dtype, B, L, D, MOD_TOKEN, dtype)
    want_y = oracle.rms_modulate_ex(x, s, t, 1e-6, MOD_TOKEN, dtype)
    dx, ds, dt = (to_dev_typed(a, dtype) for a in (x, s, t))
    _zero_ulp(to_host_typed(dte.rga_rms_modulate_ex(dx, ds, dt, 1e-6)), want_y, dtype, "token rms")
    wx, wy = oracle.gate_add_rms_modulate_ex(x, u, g, s, t, 1e-6, GATE_BCAST, MOD_TOKEN, dtype)
    xo, y = dte.rga_gate_add_rms_modulate_ex(dx, to_dev_typed(u, dtype), to_dev_typed(g, dtype),
                                             ds, dt, 1e-6)
    _bit_exact(to_host_typed(xo), wx, dtype, "token fused x_out")
    _zero_ulp(to_host_typed(y), wy, dtype, "token fused y")


@pytest.mark.parametrize("dtype,D", [(F16, 1003), (F32, 1003), (BF16, 16390), (BF16, 33001)],
                         ids=["regs", "lds-f32", "lds-wide", "two-pass"])
def test_in_place_ex(dte, dtype, D):
    # element paths in place: out == x for the gate-add and the modulation,
    # x_out == x and y == u for the fused call (D % 8 != 0); rows held in
    # registers, staged in LDS (binary32, long rows) and over 64 KB
    B, L = 2, 11
    say(f"[in place ex] {NAMES[dtype]} B={B} L={L} D={D}")
    x, u, g = _gate_inputs(8000, B, L, D, GATE_FULL, dtype)
    s, t = _mod_inputs(8003, B, L, D, MOD_TOKEN, dtype)
    dx = to_dev_typed(x, dtype)
    dte.rga_residual_gate_add_ex(dx, to_dev_typed(u, dtype), to_dev_typed(g, dtype), out=dx)
    _bit_exact(to_host_typed(dx), oracle.gate_add_ex(x, u, g, GATE_FULL, dtype), dtype, "gate")
    dx = to_dev_typed(x, dtype)
    dte.rga_rms_modulate_ex(dx, to_dev_typed(s, dtype), to_dev_typed(t, dtype), 1e-6, out=dx)
    _zero_ulp(to_host_typed(dx), oracle.rms_modulate_ex(x, s, t, 1e-6, MOD_TOKEN, dtype),
              dtype, "rms in place")
    dx, du = to_dev_typed(x, dtype), to_dev_typed(u, dtype)
    dte.rga_gate_add_rms_modulate_ex(dx, du, to_dev_typed(g, dtype), to_dev_typed(s, dtype),
                                     to_dev_typed(t, dtype), 1e-6, x_out=dx, y=du)
    wx, wy = oracle.gate_add_rms_modulate_ex(x, u, g, s, t, 1e-6, GATE_FULL, MOD_TOKEN, dtype)
    _bit_exact(to_host_typed(dx), wx, dtype, "fused x_out in place")
    _zero_ulp(to_host_typed(du), wy, dtype, "fused y over u")


@pytest.mark.parametrize("mode", [GATE_BCAST, GATE_FULL])
@pytest.mark.parametrize("dtype,B,L,D", [(BF16, 2, 33, 4100), (F16, 1, 17, 1003),
                                         (BF16, 2, 9, 8191), (BF16, 1, 21, 4096)],
                         ids=["k9", "k2-f16", "k16", "k8-offset"])
def test_in_place_row_modulation_element_path(dte, dtype, B, L, D, mode):
    # the element path's staged rows (row modulation: scale, shift and a
    # broadcast gate staged per workgroup) in place: out == x for the
    # modulation, x_out == x and y == u for the fused call. Rows of ragged D
    # share a 16-byte word with their neighbours, each writing only its own
    # bytes of it; "k8-offset" runs D = 4096 one element off a 16-byte
    # boundary (the element path at every row)
    off = 1 if D == 4096 else 0
    say(f"[in place rows] {NAMES[dtype]} B={B} L={L} D={D} mode={mode} offset={off}")
    x, u, g = _gate_inputs(8100 + D, B, L, D, mode, dtype)
    s, t = _mod_inputs(8103 + D, B, L, D, MOD_ROW, dtype)
    dx = to_dev_typed(x, dtype, offset=off)
    dte.rga_rms_modulate_ex(dx, to_dev_typed(s, dtype, offset=off),
                            to_dev_typed(t, dtype, offset=off), 1e-6, out=dx)
    _zero_ulp(to_host_typed(dx), oracle.rms_modulate_ex(x, s, t, 1e-6, MOD_ROW, dtype),
              dtype, "rms rows in place")
    dx, du = to_dev_typed(x, dtype, offset=off), to_dev_typed(u, dtype, offset=off)
    dte.rga_gate_add_rms_modulate_ex(dx, du, to_dev_typed(g, dtype, offset=off),
                                     to_dev_typed(s, dtype, offset=off),
                                     to_dev_typed(t, dtype, offset=off), 1e-6, x_out=dx, y=du,
                                     gate_mode=mode)
    wx, wy = oracle.gate_add_rms_modulate_ex(x, u, g, s, t, 1e-6, mode, MOD_ROW, dtype)
    _bit_exact(to_host_typed(dx), wx, dtype, "fused rows x_out in place")
    _zero_ulp(to_host_typed(du), wy, dtype, "fused rows y over u")


def test_ex_rejections(dte):
    x = torch.zeros(1, 2, 8, dtype=torch.float64, device="cuda")
    with pytest.raises(TypeError):
        dte.rga_residual_gate_add_ex(x, x, x)
    a = torch.zeros(1, 2, 8, dtype=torch.float16, device="cuda")
    b = torch.zeros(1, 2, 8, dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        dte.rga_residual_gate_add_ex(a, b, a)        # mixed storage types
    with pytest.raises(TypeError):
        dte.rga_residual_gate_add(a, a, a)           # original call is bf16 only
    odd = torch.zeros(1, 2, 9, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dte.RGAError) as e:
        dte.rga_residual_gate_add(odd, odd, odd)
    assert e.value.status == dte.RGA_ERR_UNSUPPORTED
    dte.rga_residual_gate_add_ex(odd, odd, odd)      # the _ex call takes it
    torch.cuda.synchronize()
