"""The element-wise paths at the bench's full sizes, against the oracle.

Ragged D (rows start at alternating offsets inside their 16-byte words) and
tensors one element into their allocations take the element-wise kernels;
these run them at the shapes the bench times and compare a sample of rows
(rows are independent; the first and last rows are always in the sample)
with the oracle: bit for bit for the gated add and the fused call's x_out,
identical for the modulations (pinned order), within one ULP for the GELU.
"""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import BF16, F32, GATE_BCAST, N001, N01, N02, U11, random_typed
from tests.gpu_util import say, to_dev_typed, to_host_typed, ulp_diff_typed

pytestmark = pytest.mark.gpu

MOD_ROW = oracle.MOD_ROW


@pytest.fixture(scope="module")
def dte():
    import diffusion_transformer_elementwise_amd as m
    return m


def _rows(L, n=600, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, L - 2, L - 1], rng.integers(0, L, n)]))


def _sample(a, rows):
    return np.ascontiguousarray(a[:, rows, :])


def _same(got, want, label):
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), label


def _zero_ulp(got, want, label):
    d = ulp_diff_typed(got, want, BF16)
    say(f"[{label}] max ULP {int(d.max())} over {d.size} elements")
    assert d.max() == 0, label


@pytest.mark.parametrize("L,D,offset", [(32640, 4100, 0), (32640, 4096, 1)])
def test_bcast_gate_add(dte, L, D, offset):
    B = 1
    say(f"[element gate] B={B} L={L} D={D} offset={offset}: inputs")
    x = random_typed(7001, (B, L, D), N02)
    u = random_typed(7002, (B, L, D), N01)
    g = random_typed(7003, (B, 1, D), U11)
    dx, du, dg = (to_dev_typed(a, BF16, offset) for a in (x, u, g))
    out = torch.empty(B * L * D + offset, dtype=dx.dtype, device=dx.device)[offset:].view(B, L, D)
    dte.rga_residual_gate_add_ex(dx, du, dg, out=out)
    rows = _rows(L)
    got = _sample(to_host_typed(out), rows)
    want = oracle.gate_add_ex(_sample(x, rows), _sample(u, rows), g, GATE_BCAST, BF16)
    _same(got, want, f"gate D={D} offset={offset}")


@pytest.mark.parametrize("norm", ["rms", "ln"])
@pytest.mark.parametrize("L,D,offset", [(32640, 4100, 0), (32640, 4096, 1)])
def test_modulations(dte, norm, L, D, offset):
    B = 2
    say(f"[element {norm}] B={B} L={L} D={D} offset={offset}: inputs")
    x = random_typed(7101, (B, L, D), N02)
    s = random_typed(7102, (B, 1, D), N001)
    t = random_typed(7103, (B, 1, D), N001)
    dx, ds, dt = (to_dev_typed(a, BF16, offset) for a in (x, s, t))
    call = dte.rga_rms_modulate_ex if norm == "rms" else dte.rga_ln_modulate
    got = to_host_typed(call(dx, ds, dt, 1e-6))
    del dx
    rows = _rows(L, seed=1)
    if norm == "rms":
        want = oracle.rms_modulate_ex(_sample(x, rows), s, t, 1e-6, MOD_ROW, BF16)
    else:
        want = oracle.ln_modulate(_sample(x, rows), s, t, 1e-6, MOD_ROW, BF16)
    _zero_ulp(_sample(got, rows), want, f"{norm} D={D} offset={offset}")


@pytest.mark.parametrize("dtype,L,D", [(BF16, 8160, 16384), (F32, 32640, 4100)])
def test_modulation_staged_in_lds(dte, dtype, L, D):
    # rows past the register-resident limit and binary32 rows: the row staged
    # in LDS once
    B = 1
    say(f"[element rms lds] dtype={dtype} B={B} L={L} D={D}: inputs")
    x = random_typed(7401, (B, L, D), N02, dtype)
    s = random_typed(7402, (B, 1, D), N001, dtype)
    t = random_typed(7403, (B, 1, D), N001, dtype)
    got = to_host_typed(dte.rga_rms_modulate_ex(*(to_dev_typed(a, dtype) for a in (x, s, t)), 1e-6))
    rows = _rows(L, seed=4)
    want = oracle.rms_modulate_ex(_sample(x, rows), s, t, 1e-6, MOD_ROW, dtype)
    d = ulp_diff_typed(_sample(got, rows), want, dtype)
    say(f"[element rms lds] max ULP {int(d.max())} over {d.size} elements")
    assert d.max() == 0


def test_fused_ragged(dte):
    B, L, D = 2, 32640, 4100
    say(f"[element fused] B={B} L={L} D={D}: inputs")
    x = random_typed(7201, (B, L, D), N02)
    u = random_typed(7202, (B, L, D), N01)
    g = random_typed(7203, (B, 1, D), U11)
    s = random_typed(7204, (B, 1, D), N001)
    t = random_typed(7205, (B, 1, D), N001)
    dx, du, dg, ds, dt = (to_dev_typed(a, BF16) for a in (x, u, g, s, t))
    xo, y = dte.rga_gate_add_rms_modulate_ex(dx, du, dg, ds, dt, 1e-6)
    got_x, got_y = to_host_typed(xo), to_host_typed(y)
    del dx, du, xo, y
    rows = _rows(L, seed=2)
    wx, wy = oracle.gate_add_rms_modulate_ex(_sample(x, rows), _sample(u, rows), g, s, t, 1e-6,
                                             GATE_BCAST, MOD_ROW, BF16)
    _same(_sample(got_x, rows), wx, "fused x_out")
    _zero_ulp(_sample(got_y, rows), wy, "fused y")


def test_gelu_bias_ragged(dte):
    rows_n, F = 32640, 16380
    say(f"[element gelu] rows={rows_n} F={F}: inputs")
    x = random_typed(7301, (rows_n, F), N02)
    b = random_typed(7302, (F,), N01)
    got = to_host_typed(dte.gelu_tanh(to_dev_typed(x, BF16), to_dev_typed(b, BF16)))
    rows = _rows(rows_n, seed=3)
    want = oracle.gelu_tanh(np.ascontiguousarray(x[rows]), BF16, bias=b)
    d = ulp_diff_typed(got[rows], want, BF16)
    say(f"[element gelu] max ULP {int(d.max())} over {d.size} elements")
    assert d.max() <= 1
