"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Gate-add: bit-exact (NaN compared by class). Modulation: at most one bf16
ULP (the bound of the RMSNorm+modulate page, "风险与影响" item 1); the
library and the oracle fix the same binary32 order, so the tests also
check that the results are in fact identical.

Every workload configuration is compared over all of its elements, at its
full size and in the launch configuration the bench uses.
"""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import (BF16, CASES, GATE_BCAST, GATE_FULL, N001, N01, N02, U11, make_inputs,
                          random_bits)
from tests.exact_round import f32_to_bf16_bits
from tests.gpu_util import first_mismatch, same_bits, say, to_dev, to_host, ulp_diff

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dte():
    import diffusion_transformer_elementwise_amd as m
    return m


def _gate_case(dte, key):
    case = CASES[key]
    say(f"[gate-add] {key} {case.name} B={case.B} L={case.L} D={case.D} "
        f"mode={case.gate} inplace={case.inplace}")
    inp = make_inputs(case)
    want = oracle.gate_add(inp["x"], inp["u"], inp["g"], case.gate)
    x, u, g = to_dev(inp["x"]), to_dev(inp["u"]), to_dev(inp["g"])
    out = x if case.inplace else torch.empty_like(x)
    dte.rga_residual_gate_add(x, u, g, out=out, gate_mode=case.gate)
    got = to_host(out)
    assert same_bits(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("key", ["c1", "c2a", "c2b", "c2c", "c3", "c4"])
def test_gate_add_configs_bit_exact(dte, key):
    _gate_case(dte, key)


def _rms_check(got, want, label):
    d = ulp_diff(got, want)
    hist = np.bincount(np.minimum(d.ravel(), 3), minlength=4)
    say(f"[rms] {label}: ULP histogram 0:{hist[0]} 1:{hist[1]} 2:{hist[2]} >2:{hist[3]}")
    assert d.max() <= 1, f"{label}: max {d.max()} ULP"
    return d


def test_rms_modulate_c1(dte):
    case = CASES["c1"]
    say(f"[rms] c1 {case.name}")
    inp = make_inputs(case)
    want = oracle.rms_modulate(inp["x"], inp["scale"], inp["shift"], case.eps)
    y = dte.rms_modulate(to_dev(inp["x"]), to_dev(inp["scale"]), to_dev(inp["shift"]), case.eps)
    got = to_host(y)
    d = _rms_check(got, want, "c1")
    assert d.max() == 0, "pinned order: expected identical results"


def test_c5_modulate_then_gated_residual(dte):
    # y = rms_modulate(x) into its own buffer, then x += u * g in place (the
    # DiT residual reading), both on the same stream, as the bench runs them
    case = CASES["c5"]
    say(f"[c5] {case.name}: generating inputs")
    inp = make_inputs(case)
    x, u, g = to_dev(inp["x"]), to_dev(inp["u"]), to_dev(inp["g"])
    sc, sh = to_dev(inp["scale"]), to_dev(inp["shift"])
    y = torch.empty_like(x)
    say("[c5] launching rms_modulate then in-place bcast gate-add")
    dte.rms_modulate(x, sc, sh, case.eps, out=y)
    dte.rga_residual_gate_add(x, u, g, out=x, gate_mode=GATE_BCAST)
    got_y, got_x = to_host(y), to_host(x)
    del x, u, g, y
    say("[c5] oracle")
    want_y = oracle.rms_modulate(inp["x"], inp["scale"], inp["shift"], case.eps)
    d = _rms_check(got_y, want_y, "c5")
    assert d.max() == 0, "pinned order: expected identical results"
    want_x = oracle.gate_add(inp["x"], inp["u"], inp["g"], GATE_BCAST)
    assert same_bits(got_x, want_x), first_mismatch(got_x, want_x)


RAGGED = [
    (1, 1, 8), (1, 3, 8), (2, 5, 24), (3, 7, 520), (1, 126, 2048),
    (2, 33, 1032), (1, 1000, 3080), (2, 4099, 4096), (1, 8191, 264),
    (5, 999, 2056), (1, 65, 8192),
]


@pytest.mark.parametrize("B,L,D", RAGGED)
@pytest.mark.parametrize("mode", [GATE_FULL, GATE_BCAST])
def test_gate_add_ragged_shapes(dte, B, L, D, mode):
    say(f"[gate-add ragged] B={B} L={L} D={D} mode={mode}")
    seed = 7 * B + 11 * L + D + mode
    x = random_bits(seed, (B, L, D))
    u = random_bits(seed + 1, (B, L, D))
    g = random_bits(seed + 2, (B, L, D) if mode == GATE_FULL else (B, 1, D), U11)
    want = oracle.gate_add(x, u, g, mode)
    got = to_host(dte.rga_residual_gate_add(to_dev(x), to_dev(u), to_dev(g), gate_mode=mode))
    assert same_bits(got, want), first_mismatch(got, want)


# 4608: nine packs per lane, whole rows; 4104: nine packs per lane, rows at
# every line phase
@pytest.mark.parametrize("B,L,D", RAGGED + [(1, 17, 6144), (2, 3, 7680), (1, 19, 4608),
                                            (2, 9, 4104)])
def test_rms_ragged_shapes(dte, B, L, D):
    say(f"[rms ragged] B={B} L={L} D={D}")
    seed = 5 * B + 3 * L + D
    x = random_bits(seed, (B, L, D), N02)
    s = random_bits(seed + 1, (B, 1, D), N001)
    t = random_bits(seed + 2, (B, 1, D), N001)
    want = oracle.rms_modulate(x, s, t, 1e-6)
    got = to_host(dte.rms_modulate(to_dev(x), to_dev(s), to_dev(t), 1e-6))
    d = _rms_check(got, want, f"{B}x{L}x{D}")
    assert d.max() == 0


# Element-path rows that (nearly) fill their slots: the line phase is cut
# to the room the slots leave (64 K - ceil(D / 8) groups: 0 or 1 here), so
# rows whose line position asks for more run at a smaller phase.
@pytest.mark.parametrize("D", [1009, 1023, 3057, 3071, 4600, 4607])
def test_element_rows_near_slot_capacity(dte, D):
    B, L = 2, 19
    say(f"[element rows near capacity] B={B} L={L} D={D}")
    seed = 9000 + D
    x = random_bits(seed, (B, L, D), N02)
    s = random_bits(seed + 1, (B, 1, D), N001)
    t = random_bits(seed + 2, (B, 1, D), N001)
    got = to_host(dte.rga_rms_modulate_ex(to_dev(x), to_dev(s), to_dev(t), 1e-6))
    want = oracle.rms_modulate_ex(x, s, t, 1e-6, oracle.MOD_ROW, BF16)
    d = _rms_check(got, want, f"rms {B}x{L}x{D}")
    assert d.max() == 0
    u = random_bits(seed + 3, (B, L, D), N01)
    for mode in (GATE_BCAST, GATE_FULL):
        g = random_bits(seed + 4 + mode, (B, L, D) if mode == GATE_FULL else (B, 1, D), N001)
        want_x, want_y = oracle.gate_add_rms_modulate_ex(x, u, g, s, t, 1e-6, mode,
                                                         oracle.MOD_ROW, BF16)
        got_x, got_y = dte.rga_gate_add_rms_modulate_ex(to_dev(x), to_dev(u), to_dev(g),
                                                        to_dev(s), to_dev(t), 1e-6,
                                                        gate_mode=mode)
        hx, hy = to_host(got_x), to_host(got_y)
        assert same_bits(hx, want_x), first_mismatch(hx, want_x)
        assert _rms_check(hy, want_y, f"fused {B}x{L}x{D} mode {mode}").max() == 0


def test_gate_add_every_x_pattern_and_special_products(dte):
    # all 65536 bf16 x patterns against normal, subnormal, overflowing, zero,
    # infinite and NaN products
    pairs = [(1.5, 0.75), (1.0078125 * 2.0 ** -70, 1.9921875 * 2.0 ** -62),
             (2.0 ** -100, 2.0 ** -60), (1.5 * 2.0 ** 100, 1.75 * 2.0 ** 30),
             (0.0, 5.0), (-0.0, 5.0), (float("inf"), 0.5), (float("inf"), 0.0),
             (float("nan"), 1.0), (-3.0e-3, 2.5e2)]
    xs = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    n = xs.size
    x = np.tile(xs, len(pairs)).reshape(1, len(pairs), n)
    uv = f32_to_bf16_bits(np.array([p[0] for p in pairs], dtype=np.float32))
    gv = f32_to_bf16_bits(np.array([p[1] for p in pairs], dtype=np.float32))
    u = np.repeat(uv, n).reshape(1, len(pairs), n)
    g = np.repeat(gv, n).reshape(1, len(pairs), n)
    say("[gate-add] 65536 x patterns x special products")
    want = oracle.gate_add(x, u, g, GATE_FULL)
    got = to_host(dte.rga_residual_gate_add(to_dev(x), to_dev(u), to_dev(g), gate_mode=GATE_FULL))
    assert same_bits(got, want), first_mismatch(got, want)


def test_gate_add_subnormal_products_are_rounded_before_the_add(dte):
    # sums near bf16 ties whose binary32 product is subnormal and inexact:
    # a fused multiply-add could round differently from multiply-then-add
    rng = np.random.default_rng(3)
    n = 1 << 16
    ue = rng.integers(-80, -60, n)
    ge = -126 - 8 - ue + rng.integers(-2, 3, n)
    um = 1 + rng.integers(0, 128, n) / 128
    gm = 1 + rng.integers(0, 128, n) / 128
    uf = (um * np.exp2(ue.astype(np.float64))).astype(np.float32)
    gf = (gm * np.exp2(ge.astype(np.float64))).astype(np.float32)
    xf = (rng.integers(1, 256, n) * np.exp2(-133.0)).astype(np.float32)
    x = f32_to_bf16_bits(xf).reshape(1, 1, n)
    u = f32_to_bf16_bits(uf).reshape(1, 1, n)
    g = f32_to_bf16_bits(gf * np.where(rng.integers(0, 2, n) == 0, 1, -1).astype(np.float32)).reshape(1, 1, n)
    say("[gate-add] subnormal products")
    want = oracle.gate_add(x, u, g, GATE_FULL)
    got = to_host(dte.rga_residual_gate_add(to_dev(x), to_dev(u), to_dev(g), gate_mode=GATE_FULL))
    assert same_bits(got, want), first_mismatch(got, want)


def test_rms_special_rows(dte):
    # zero rows -> shift; rows with inf/NaN -> NaN where the product is
    # undefined; huge rows whose squares overflow; subnormal rows; eps = 0
    D = 1024
    rows = []
    rows.append(np.zeros(D, np.float32))
    r = np.ones(D, np.float32); r[5] = np.inf; rows.append(r)
    r = np.ones(D, np.float32); r[7] = np.nan; rows.append(r)
    rows.append(np.full(D, 3.0e38, np.float32))
    rows.append(np.full(D, 1.0e-39, np.float32))
    rows.append(np.full(D, -2.0 ** -10, np.float32))
    r = np.zeros(D, np.float32); r[0] = 1.0; rows.append(r)
    x = f32_to_bf16_bits(np.stack(rows)).reshape(1, len(rows), D)
    s = random_bits(1, (1, 1, D), N001)
    t = random_bits(2, (1, 1, D), N001)
    for eps in (1e-6, 0.0):
        say(f"[rms] special rows eps={eps}")
        want = oracle.rms_modulate(x, s, t, eps)
        got = to_host(dte.rms_modulate(to_dev(x), to_dev(s), to_dev(t), eps))
        assert same_bits(got, want), first_mismatch(got, want)


def test_in_place_aliases(dte):
    B, L, D = 2, 300, 1536
    x = random_bits(41, (B, L, D))
    u = random_bits(42, (B, L, D))
    gf = random_bits(43, (B, L, D), U11)
    gb = random_bits(44, (B, 1, D), U11)
    say("[alias] gate-add out=x/u/g, rms out=x")
    for mode, g in ((GATE_FULL, gf), (GATE_BCAST, gb)):
        want = oracle.gate_add(x, u, g, mode)
        for target in ("x", "u", "g"):
            if target == "g" and mode == GATE_BCAST:
                continue
            t = {"x": to_dev(x), "u": to_dev(u), "g": to_dev(g)}
            dte.rga_residual_gate_add(t["x"], t["u"], t["g"], out=t[target], gate_mode=mode)
            got = to_host(t[target])
            assert same_bits(got, want), (mode, target, first_mismatch(got, want))
    s = random_bits(45, (B, 1, D), N001)
    sh = random_bits(46, (B, 1, D), N001)
    want = oracle.rms_modulate(x, s, sh, 1e-6)
    xd = to_dev(x)
    dte.rms_modulate(xd, to_dev(s), to_dev(sh), 1e-6, out=xd)
    assert same_bits(to_host(xd), want)


def test_rejections_through_the_binding(dte):
    x = to_dev(random_bits(1, (1, 4, 16)))
    with pytest.raises(dte.RGAError) as e:
        dte.rga_residual_gate_add(x, x, x, gate_mode=7)
    assert e.value.status == dte.RGA_ERR_INVALID_ARG
    big = torch.zeros(1, 4, 24, dtype=torch.bfloat16, device=x.device)
    odd = big.view(-1)[4:4 + 4 * 20].view(1, 4, 20)  # D % 8 != 0
    with pytest.raises(dte.RGAError) as e:
        dte.rga_residual_gate_add(odd, odd, odd)
    assert e.value.status == dte.RGA_ERR_UNSUPPORTED
    mis = big.view(-1)[1:1 + 16].view(1, 2, 8)  # 2-byte offset: misaligned
    with pytest.raises(dte.RGAError) as e:
        dte.rga_residual_gate_add(mis, mis, mis)
    assert e.value.status == dte.RGA_ERR_UNSUPPORTED
    buf = torch.zeros(1, 3, 16, dtype=torch.bfloat16, device=x.device)
    a = buf.view(-1)[:32].view(1, 2, 16)
    b = buf.view(-1)[8:40].view(1, 2, 16)  # overlaps a, not identical
    with pytest.raises(dte.RGAError) as e:
        dte.rga_residual_gate_add(a, a, a, out=b)
    assert e.value.status == dte.RGA_ERR_ALIAS
    # the modulation rejects only the layout (D % 8, alignment); rows longer
    # than the register-held ones run (their parity: tests/test_gpu_measure.py)
    ragged = torch.zeros(1, 2, 8204, dtype=torch.bfloat16, device=x.device)
    rrow = torch.zeros(1, 1, 8204, dtype=torch.bfloat16, device=x.device)
    with pytest.raises(dte.RGAError) as e:
        dte.rms_modulate(ragged, rrow, rrow)
    assert e.value.status == dte.RGA_ERR_UNSUPPORTED
    wide = torch.zeros(1, 2, 8200, dtype=torch.bfloat16, device=x.device)
    row = torch.zeros(1, 1, 8200, dtype=torch.bfloat16, device=x.device)
    y = dte.rms_modulate(wide, row, row)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0   # zero rows: y = shift = 0


def test_empty_inputs_are_no_ops(dte):
    for shape in ((0, 4, 8), (2, 0, 8), (2, 4, 0)):
        x = torch.empty(shape, dtype=torch.bfloat16, device="cuda:0")
        out = dte.rga_residual_gate_add(x, x, x, gate_mode=GATE_FULL)
        assert out.shape == x.shape
        row = torch.empty((shape[0], 1, shape[2]), dtype=torch.bfloat16, device="cuda:0")
        assert dte.rms_modulate(x, row, row).shape == x.shape


def test_side_stream_and_determinism(dte):
    x = random_bits(51, (2, 2000, 4096), N02)
    s = random_bits(52, (2, 1, 4096), N001)
    t = random_bits(53, (2, 1, 4096), N001)
    xd, sd, td = to_dev(x), to_dev(s), to_dev(t)
    side = torch.cuda.Stream()
    say("[stream] rms_modulate on a side stream, twice")
    with torch.cuda.stream(side):
        a = dte.rms_modulate(xd, sd, td)
        b = dte.rms_modulate(xd, sd, td)
    side.synchronize()
    ha, hb = to_host(a), to_host(b)
    assert np.array_equal(ha, hb)
    assert np.array_equal(ha, oracle.rms_modulate(x, s, t, 1e-6))


def test_copy_and_fill_helpers(dte):
    src = torch.arange(1 << 20, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    dte.copy_(dst, src)
    assert torch.equal(dst, src)
    dte.fill_(dst, 0x12345678)
    torch.cuda.synchronize()
    assert bool((dst == 0x12345678).all())


@pytest.mark.parametrize("words", [1 << 16, 5 * 256 * 1024 + 12345])
def test_read_helper_folds_every_word(dte, words):
    # one grid pass, and five passes of the 256 x 1024-lane grid plus a
    # ragged remainder (the four-load loop, then the one-load tail)
    src = torch.arange(4 * words, dtype=torch.int32, device="cuda:0")
    src = src * 2654435761 % (1 << 31)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    dte.read_(src, sink)
    want = np.bitwise_xor.reduce(src.cpu().numpy().reshape(-1, 4), axis=0)
    assert np.array_equal(sink.cpu().numpy(), want)


def _fused_case(dte, B, L, D, mode, seed, inplace=None):
    x = random_bits(seed, (B, L, D), N02)
    u = random_bits(seed + 1, (B, L, D), N01)
    g = random_bits(seed + 2, (B, L, D) if mode == GATE_FULL else (B, 1, D), N001)
    s = random_bits(seed + 3, (B, 1, D), N001)
    t = random_bits(seed + 4, (B, 1, D), N001)
    want_x, want_y = oracle.gate_add_rms_modulate(x, u, g, s, t, 1e-6, mode)
    xd, ud, gd = to_dev(x), to_dev(u), to_dev(g)
    xo = {"x": xd, "u": ud}.get(inplace[0]) if inplace else None
    yo = {"x": xd, "u": ud}.get(inplace[1]) if inplace else None
    got_x, got_y = dte.rga_gate_add_rms_modulate(xd, ud, gd, to_dev(s), to_dev(t), 1e-6,
                                                 x_out=xo, y=yo, gate_mode=mode)
    hx, hy = to_host(got_x), to_host(got_y)
    assert same_bits(hx, want_x), first_mismatch(hx, want_x)
    d = _rms_check(hy, want_y, f"fused {B}x{L}x{D} mode {mode}")
    assert d.max() == 0


@pytest.mark.parametrize("mode", [GATE_FULL, GATE_BCAST])
def test_fused_residual_then_modulation_at_video_scale(dte, mode):
    say(f"[fused] [2,32640,4096] mode={mode}")
    _fused_case(dte, 2, 32640, 4096, mode, 1200 + mode)


@pytest.mark.parametrize("B,L,D", RAGGED + [(1, 17, 6144), (1, 19, 4608), (2, 9, 4104)])
@pytest.mark.parametrize("mode", [GATE_FULL, GATE_BCAST])
def test_fused_ragged_shapes(dte, B, L, D, mode):
    say(f"[fused ragged] B={B} L={L} D={D} mode={mode}")
    _fused_case(dte, B, L, D, mode, 1300 + 3 * B + L + D + mode)


@pytest.mark.parametrize("inplace", [("x", None), ("u", "x"), (None, "u"), ("x", "u")])
def test_fused_in_place(dte, inplace):
    say(f"[fused in place] x_out={inplace[0]} y={inplace[1]}")
    _fused_case(dte, 2, 301, 2048, GATE_BCAST, 1400, inplace=inplace)
