"""GPU tests of the calls the bench leans on beyond the path itself, and of
the strict calls on rows longer than the register-held ones.

- rms_modulate and rga_gate_add_rms_modulate (the calls without a dtype)
  take D % 8 == 0 rows of any length: above RGA_RMS_MAX_D they run the
  LDS-staged kernels, with the same fixed summation order, so they must
  match the oracle exactly (0 ULP) like the register-held rows.
- rga_gate_add_variant (the broadcast-gate add in other kernel shapes: rows
  per wave, store cache policy) must give exactly the library's result.
- rga_stream (the read:write mix ceilings) must write the XOR of its
  sources, in place too, and leave everything alone when read-only.
"""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import GATE_BCAST, GATE_FULL, N001, N02, U11, random_bits
from tests.gpu_util import first_mismatch, same_bits, say, to_dev, to_host, ulp_diff

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dte():
    import diffusion_transformer_elementwise_amd as m
    return m


@pytest.mark.parametrize("B,L,D", [(2, 37, 8200), (1, 19, 16384), (2, 5, 32768)])
def test_strict_modulation_of_long_rows(dte, B, L, D):
    say(f"[strict long rows] rms_modulate B={B} L={L} D={D}")
    seed = 3 * B + L + D
    x = random_bits(seed, (B, L, D), N02)
    s = random_bits(seed + 1, (B, 1, D), N001)
    t = random_bits(seed + 2, (B, 1, D), N001)
    want = oracle.rms_modulate(x, s, t, 1e-6)
    got = to_host(dte.rms_modulate(to_dev(x), to_dev(s), to_dev(t), 1e-6))
    d = ulp_diff(got, want)
    assert d.max() == 0, f"max {d.max()} ULP"


@pytest.mark.parametrize("mode", [GATE_BCAST, GATE_FULL])
@pytest.mark.parametrize("B,L,D", [(2, 23, 8200), (1, 11, 16384)])
def test_strict_fused_call_on_long_rows(dte, B, L, D, mode):
    say(f"[strict long rows] fused B={B} L={L} D={D} mode={mode}")
    seed = 5 * B + L + D + mode
    x = random_bits(seed, (B, L, D), N02)
    u = random_bits(seed + 1, (B, L, D))
    g = random_bits(seed + 2, (B, L, D) if mode == GATE_FULL else (B, 1, D), U11)
    s = random_bits(seed + 3, (B, 1, D), N001)
    t = random_bits(seed + 4, (B, 1, D), N001)
    want_x, want_y = oracle.gate_add_rms_modulate(x, u, g, s, t, 1e-6, mode)
    dx = to_dev(x)
    y = torch.empty_like(dx)
    dte.rga_gate_add_rms_modulate(dx, to_dev(u), to_dev(g), to_dev(s), to_dev(t), 1e-6,
                                  x_out=dx, y=y, gate_mode=mode)
    got_x, got_y = to_host(dx), to_host(y)
    assert same_bits(got_x, want_x), first_mismatch(got_x, want_x)
    d = ulp_diff(got_y, want_y)
    assert d.max() == 0, f"max {d.max()} ULP"


@pytest.mark.parametrize("B,L,D", [(2, 37, 4096), (1, 13, 520), (3, 9, 8)])
def test_gate_add_variants_equal_the_library(dte, B, L, D):
    seed = 11 * B + L + D
    x = to_dev(random_bits(seed, (B, L, D)))
    u = to_dev(random_bits(seed + 1, (B, L, D)))
    g = to_dev(random_bits(seed + 2, (B, 1, D), U11))
    want = to_host(dte.rga_residual_gate_add(x, u, g, gate_mode=GATE_BCAST))
    for T in (1, 2, 4, 8):
        for sp in (dte.STORE_NT, dte.STORE_PLAIN, dte.STORE_DEVICE):
            say(f"[gate-add variant] B={B} L={L} D={D} rows/wave={T} store={sp}")
            got = to_host(dte.gate_add_variant(x, u, g, rows_per_wave=T, store_policy=sp))
            assert same_bits(got, want), first_mismatch(got, want)
            # in place, as the bench runs it
            xi = x.clone()
            dte.gate_add_variant(xi, u, g, out=xi, rows_per_wave=T, store_policy=sp)
            got = to_host(xi)
            assert same_bits(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("wpl", [1, 2, 4])
def test_stream_writes_the_xor_of_its_sources(dte, wpl):
    say(f"[stream] words per lane {wpl}")
    n = 64 * 64 * 4 * 3 + 16 * 5  # ragged against every workgroup's span
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(97 + wpl)
    src = [torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device="cuda:0",
                         generator=gen) for _ in range(3)]
    want = (src[0] ^ src[1] ^ src[2]).cpu()
    dst = torch.full_like(src[0], 7)
    dte.stream_(src, dst, words_per_lane=wpl)
    assert torch.equal(dst.cpu(), want)
    two = (src[0] ^ src[1]).cpu()
    a = src[0].clone()
    dte.stream_([a, src[1]], a, words_per_lane=wpl)          # in place
    assert torch.equal(a.cpu(), two)
    one = src[2].clone()
    dte.stream_([src[1]], one, words_per_lane=wpl)          # copy
    assert torch.equal(one.cpu(), src[1].cpu())
    before = [s.cpu() for s in src]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    dte.stream_(src, None, words_per_lane=wpl, sink=sink)    # read-only
    torch.cuda.synchronize()
    assert all(torch.equal(s.cpu(), b) for s, b in zip(src, before))
    assert torch.count_nonzero(sink).item() == 0
    w = torch.zeros_like(src[0])
    dte.stream_([], w, words_per_lane=wpl)                   # write-only: a pattern
    torch.cuda.synchronize()
    assert torch.count_nonzero(w).item() > 0


@pytest.mark.parametrize("D,dt", [(4096, 0), (2048, 1), (4100, 0), (520, 1)])
def test_occupancy_helpers_equal_the_library(dte, D, dt):
    from tests.gpu_util import to_dev_typed, to_host_typed
    from synth_inputs import random_typed
    B, L = 2, 37
    seed = D + dt
    x = to_dev_typed(random_typed(seed, (B, L, D), N02, dt), dt)
    u = to_dev_typed(random_typed(seed + 1, (B, L, D), dtype=dt), dt)
    g = to_dev_typed(random_typed(seed + 2, (B, 1, D), U11, dt), dt)
    s = to_dev_typed(random_typed(seed + 3, (B, 1, D), N001, dt), dt)
    t = to_dev_typed(random_typed(seed + 4, (B, 1, D), N001, dt), dt)
    want_y = to_host_typed(dte.rga_rms_modulate_ex(x, s, t, 1e-6))
    want_xo, want_fy = (to_host_typed(a) for a in dte.rga_gate_add_rms_modulate_ex(x, u, g, s, t, 1e-6))
    for w in (-1, 0, 3, 5, 12):
        say(f"[occupancy] D={D} dtype={dt} wg_per_cu={w}")
        got = to_host_typed(dte.modulate_occupancy(x, s, t, 1e-6, wg_per_cu=w))
        assert np.array_equal(got, want_y)
        xo, fy = dte.fused_occupancy(x, u, g, s, t, 1e-6, wg_per_cu=w)
        assert np.array_equal(to_host_typed(xo), want_xo)
        assert np.array_equal(to_host_typed(fy), want_fy)


# odd L (a wave past the last row), L = 1, L = 2 (a two-row wave's second
# row absent for half the workgroups), and a larger grid
@pytest.mark.parametrize("B,L", [(2, 37), (1, 1), (2, 2), (1, 515)])
def test_schedule_variants_equal_the_oracle(dte, B, L):
    D = 4096
    seed = 13 * B + L
    x = random_bits(seed, (B, L, D), N02)
    u = random_bits(seed + 1, (B, L, D))
    g = random_bits(seed + 2, (B, 1, D), U11)
    s = random_bits(seed + 3, (B, 1, D), N001)
    t = random_bits(seed + 4, (B, 1, D), N001)
    want_y = oracle.rms_modulate(x, s, t, 1e-6)
    want_x, want_fy = oracle.gate_add_rms_modulate(x, u, g, s, t, 1e-6, GATE_BCAST)
    dx, du, dg, ds, dt = (to_dev(a) for a in (x, u, g, s, t))
    for sched in (dte.SCHED_LIBRARY, dte.SCHED_LOADS_FIRST, dte.SCHED_ONE_PLUS,
                  dte.SCHED_TWO_ROWS, dte.SCHED_PREFETCH):
        say(f"[schedule variant] B={B} L={L} schedule={sched}")
        got = to_host(dte.modulate_variant(dx, ds, dt, 1e-6, schedule=sched))
        d = ulp_diff(got, want_y)
        assert d.max() == 0, f"modulation, schedule {sched}: max {d.max()} ULP"
        xo, fy = dte.fused_variant(dx, du, dg, ds, dt, 1e-6, schedule=sched)
        got_x, got_y = to_host(xo), to_host(fy)
        assert same_bits(got_x, want_x), first_mismatch(got_x, want_x)
        d = ulp_diff(got_y, want_fy)
        assert d.max() == 0, f"fused call, schedule {sched}: max {d.max()} ULP"
        # in place, as the bench runs it
        xi = dx.clone()
        y = torch.empty_like(xi)
        dte.fused_variant(xi, du, dg, ds, dt, 1e-6, x_out=xi, y=y, schedule=sched)
        assert same_bits(to_host(xi), want_x)
        assert ulp_diff(to_host(y), want_fy).max() == 0
