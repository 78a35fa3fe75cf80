"""Tensors past 2^31 elements: 64-bit indexing in every kernel family.

Each input repeats a small seeded pattern (elements, or whole rows, with a
period that does not divide the word or row structure), built on the device
by repetition, so the expected output repeats too and the oracle evaluates
one period. Outputs are compared at positions around element 2^31 (and row
2^31 / D), at the start and at the end, where a 32-bit index or offset
anywhere in a kernel would land on the wrong element.
"""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import BF16, GATE_BCAST, GATE_FULL, N001, N01, N02, U11, random_typed
from tests.gpu_util import say, to_dev_typed, to_host_typed, ulp_diff_typed

pytestmark = pytest.mark.gpu

TWO31 = 1 << 31


@pytest.fixture(scope="module")
def dte():
    import diffusion_transformer_elementwise_amd as m
    yield m
    torch.cuda.empty_cache()


def _tile(pat_dev, n):
    """The pattern repeated to n elements along dim 0 (device)."""
    reps = -(-n // pat_dev.shape[0])
    return pat_dev.repeat((reps,) + (1,) * (pat_dev.dim() - 1))[:n].contiguous()


def _positions(n, span=2048, seed=0):
    rng = np.random.default_rng(seed)
    around = np.arange(TWO31 - span, min(TWO31 + span, n))
    ends = np.concatenate([np.arange(0, span), np.arange(n - span, n)])
    return np.unique(np.concatenate([around, ends, rng.integers(0, n, 4096)]))


def _gather(t_flat, idx):
    out = t_flat[torch.from_numpy(idx).to(t_flat.device)]
    return to_host_typed(out)


def _at_offset(t, offset):
    """t moved `offset` elements into a fresh allocation (offset 0: t)."""
    if offset == 0:
        return t
    flat = torch.empty(t.numel() + offset, dtype=t.dtype, device=t.device)
    view = flat[offset:].view(t.shape)
    view.copy_(t)
    return view


@pytest.mark.parametrize("offset", [0, 1])
def test_full_gate_add(dte, offset):
    # a flat run of B*L*D > 2^31 elements: the pack kernel with its trailing
    # partial pack (n % 8 == 4), and at a one-element offset the element
    # path's chunks (a run of more than 2^32 bytes)
    D = 4100
    L = TWO31 // D + 3
    n = L * D
    assert n > TWO31 and n % 8 == 4
    P = 4099 * 8 + 3
    say(f"[large full gate] L={L} D={D} n={n} offset={offset}")
    xp, up, gp = (random_typed(9000 + k, (P,), d) for k, d in enumerate((N02, N01, U11)))
    dev = [to_dev_typed(a, BF16) for a in (xp, up, gp)]
    x, u, g = (_at_offset(_tile(a, n).view(1, L, D), offset) for a in dev)
    torch.cuda.empty_cache()
    out = _at_offset(torch.empty_like(x), offset)
    dte.rga_residual_gate_add_ex(x, u, g, out=out, gate_mode=GATE_FULL)
    want_p = oracle.gate_add_ex(xp.reshape(1, 1, P), up.reshape(1, 1, P), gp.reshape(1, 1, P),
                                GATE_FULL, BF16).ravel()
    idx = _positions(n)
    got = _gather(out.view(-1), idx)
    want = want_p[idx % P]
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} mismatches, first at element {int(idx[bad[0]])}"
    del x, u, g, out
    torch.cuda.empty_cache()


def _row_tile(rows_dev, L):
    return _tile(rows_dev, L)


@pytest.mark.parametrize("D", [4096, 4100])
def test_bcast_gate_add_and_rms(dte, D):
    # one batch of L rows with L * D > 2^31: the broadcast gate-add and the
    # modulation (pack kernels at D = 4096, element kernels at D = 4100)
    L = TWO31 // D + 5
    R = 7  # row period
    say(f"[large rows] L={L} D={D} n={L * D}")
    xp = random_typed(9100, (R, D), N02)
    up = random_typed(9101, (R, D), N01)
    g = random_typed(9102, (1, 1, D), U11)
    s = random_typed(9103, (1, 1, D), N001)
    t = random_typed(9104, (1, 1, D), N001)
    x = _row_tile(to_dev_typed(xp, BF16), L).view(1, L, D)
    u = _row_tile(to_dev_typed(up, BF16), L).view(1, L, D)
    dg, ds, dt = (to_dev_typed(a, BF16) for a in (g, s, t))
    rows = np.unique(np.concatenate([
        np.arange(0, 3), np.arange(TWO31 // D - 3, TWO31 // D + 4), np.arange(L - 3, L)]))
    ridx = torch.from_numpy(rows).to(x.device)

    y = dte.rga_rms_modulate_ex(x, ds, dt, 1e-6)
    got_y = to_host_typed(y[0][ridx])
    del y
    want_yp = oracle.rms_modulate_ex(xp.reshape(1, R, D), s, t, 1e-6, oracle.MOD_ROW, BF16)[0]
    d = ulp_diff_typed(got_y, want_yp[rows % R], BF16)
    say(f"[large rms] D={D} max ULP {int(d.max())} over rows {rows.tolist()}")
    assert d.max() == 0

    out = dte.rga_residual_gate_add_ex(x, u, dg, out=x)  # in place, as the bench runs it
    got = to_host_typed(out[0][ridx])
    want_p = oracle.gate_add_ex(xp.reshape(1, R, D), up.reshape(1, R, D), g, GATE_BCAST, BF16)[0]
    assert np.array_equal(got, want_p[rows % R]), f"bcast gate D={D}"
    del x, u, out
    torch.cuda.empty_cache()


def test_gelu_flat(dte):
    rows, F = TWO31 // 16384 + 2, 16384
    n = rows * F
    P = 16381
    say(f"[large gelu] rows={rows} F={F} n={n}")
    xp = random_typed(9200, (P,), N02)
    x = _tile(to_dev_typed(xp, BF16), n).view(rows, F)
    out = dte.gelu_tanh(x)
    want_p = oracle.gelu_tanh(xp.reshape(1, P), BF16).ravel()
    idx = _positions(n, seed=1)
    got = _gather(out.view(-1), idx)
    d = ulp_diff_typed(got, want_p[idx % P], BF16)
    assert d.max() <= 1
    del x, out
    torch.cuda.empty_cache()
