"""torch integration: custom ops with fake implementations (traced opaquely
by torch.compile) and the caller-side first-use check."""
import warnings

import numpy as np
import pytest
import torch

import diffusion_transformer_elementwise_amd as dte
from diffusion_transformer_elementwise_amd import integration as I


# ---- CPU: guard logic -----------------------------------------------------

class _Calls:
    def __init__(self, fn):
        self.fn, self.n = fn, 0

    def __call__(self, *a, **k):
        self.n += 1
        return self.fn(*a, **k)


def test_guard_checks_each_key_once():
    fn = _Calls(lambda x: x * 2)
    ref = _Calls(lambda x: x + x)
    guard = I.FirstUseGuard(fn, ref)
    a = torch.arange(6.0).reshape(2, 3)
    b = torch.arange(8.0).reshape(2, 4)
    for _ in range(3):
        assert torch.equal(guard(a), a * 2)
    assert ref.n == 1 and fn.n == 3 and guard.state(a) is True
    guard(b)
    assert ref.n == 2 and guard.state(b) is True


def test_guard_raises_on_mismatch_by_default():
    guard = I.FirstUseGuard(lambda x: x * 2, lambda x: x * 3)
    with pytest.raises(I.GuardMismatch):
        guard(torch.ones(4))
    assert guard.state(torch.ones(4)) is None


def test_guard_fallback_serves_the_reference():
    fn = _Calls(lambda x: x * 2)
    guard = I.FirstUseGuard(fn, lambda x: x * 3, fallback=True)
    x = torch.ones(4)
    with warnings.catch_warnings(record=True):
        warnings.simplefilter("always")
        assert torch.equal(guard(x), x * 3)
    assert torch.equal(guard(x), x * 3)
    assert fn.n == 1 and guard.state(x) is False


def test_guard_launch_error_handling():
    def boom(x):
        raise dte.RGAError(dte.RGA_ERR_UNSUPPORTED, "test")
    with pytest.raises(dte.RGAError):
        I.FirstUseGuard(boom, lambda x: x)(torch.ones(2))
    guard = I.FirstUseGuard(boom, lambda x: x + 1, fallback=True)
    with warnings.catch_warnings(record=True):
        warnings.simplefilter("always")
        assert torch.equal(guard(torch.ones(2)), torch.full((2,), 2.0))


def test_checks():
    a = torch.tensor([1.0, 2.0], dtype=torch.bfloat16)
    b = torch.tensor([1.0, 2.015625], dtype=torch.bfloat16)  # one bf16 ulp above 2
    assert I.bitwise_equal(a, a) and not I.bitwise_equal(a, b)
    assert I.allclose(3e-2, 1e-2)(a, b)
    # +0 and -0 differ bit for bit
    assert not I.bitwise_equal(torch.tensor([0.0]).bfloat16(), torch.tensor([-0.0]).bfloat16())


# ---- CPU: tracing through the fake implementations -------------------------

def test_ops_are_opaque_to_tracing():
    from torch.fx.experimental.proxy_tensor import make_fx
    from torch._subclasses.fake_tensor import FakeTensorMode

    def block(x, u, g, s, t):
        x1 = torch.ops.rga.residual_gate_add(x, u, g)
        y = torch.ops.rga.rms_modulate(x1, s, t, 1e-6)
        x2, y2 = torch.ops.rga.gate_add_rms_modulate(x1, y, g, s, t, 1e-6)
        return x2, y2

    with FakeTensorMode():
        mk = lambda *shape: torch.empty(*shape, dtype=torch.bfloat16, device="cuda")
        args = (mk(2, 5, 64), mk(2, 5, 64), mk(2, 1, 64), mk(2, 1, 64), mk(2, 1, 64))
        gm = make_fx(block, tracing_mode="fake")(*args)
    targets = [str(n.target) for n in gm.graph.nodes if n.op == "call_function"]
    assert "rga.residual_gate_add.default" in targets
    assert "rga.rms_modulate.default" in targets
    assert "rga.gate_add_rms_modulate.default" in targets
    assert not any("ctypes" in t for t in targets)


def test_extended_ops_are_opaque_to_tracing():
    from torch.fx.experimental.proxy_tensor import make_fx
    from torch._subclasses.fake_tensor import FakeTensorMode

    def block(x, u, g, s, t, b):
        x1 = torch.ops.rga.residual_gate_add_ex(x, u, g)
        y = torch.ops.rga.ln_modulate(x1, s, t, 1e-6)
        x2, y2 = torch.ops.rga.gate_add_rms_modulate_ex(x1, y, g, s, t, 1e-6)
        y3 = torch.ops.rga.rms_modulate_ex(x2, s, t, 1e-6)
        h = torch.ops.rga.gelu_tanh(y3, b)
        return h, y2

    with FakeTensorMode():
        mk = lambda *shape: torch.empty(*shape, dtype=torch.float16, device="cuda")
        args = (mk(2, 5, 24), mk(2, 5, 24), mk(2, 1, 24), mk(2, 5, 24), mk(2, 5, 24), mk(24))
        gm = make_fx(block, tracing_mode="fake")(*args)
    targets = {str(n.target) for n in gm.graph.nodes if n.op == "call_function"}
    for name in ("residual_gate_add_ex", "ln_modulate", "gate_add_rms_modulate_ex",
                 "rms_modulate_ex", "gelu_tanh"):
        assert f"rga.{name}.default" in targets, (name, targets)


# ---- GPU -------------------------------------------------------------------

def _dev_inputs(seed, B=2, L=333, D=2048):
    from synth_inputs import N001, N01, N02, U11, random_bits
    from tests.gpu_util import to_dev
    x = to_dev(random_bits(seed, (B, L, D), N02))
    u = to_dev(random_bits(seed + 1, (B, L, D), N01))
    g = to_dev(random_bits(seed + 2, (B, 1, D), U11))
    s = to_dev(random_bits(seed + 3, (B, 1, D), N001))
    t = to_dev(random_bits(seed + 4, (B, 1, D), N001))
    return x, u, g, s, t


@pytest.mark.gpu
def test_compiled_block_matches_eager_and_oracle():
    import oracle
    from tests.gpu_util import say, to_host

    def block(x, u, g, s, t):
        x1 = torch.ops.rga.residual_gate_add(x, u, g)
        y = torch.ops.rga.rms_modulate(x1, s, t, 1e-6)
        x2, y2 = torch.ops.rga.gate_add_rms_modulate(x1, y, g, s, t, 1e-6)
        return x1, y, x2, y2

    args = _dev_inputs(2000)
    say("[compile] torch.compile(fullgraph=True, backend=aot_eager) over rga custom ops")
    compiled = torch.compile(block, fullgraph=True, backend="aot_eager")
    got = compiled(*args)
    eager = block(*args)
    for a, b in zip(got, eager):
        assert I.bitwise_equal(a, b)
    h = [to_host(a) for a in args]
    x1 = oracle.gate_add(h[0], h[1], h[2], oracle.GATE_BCAST)
    y = oracle.rms_modulate(x1, h[3], h[4], 1e-6)
    x2, y2 = oracle.gate_add_rms_modulate(x1, y, h[2], h[3], h[4], 1e-6, oracle.GATE_BCAST)
    for a, w in zip(got, (x1, y, x2, y2)):
        assert np.array_equal(to_host(a), w)


@pytest.mark.gpu
def test_compiled_extended_block_matches_eager():
    from tests.gpu_util import say

    def block(x, u, g, s, t, b):
        x1 = torch.ops.rga.residual_gate_add_ex(x, u, g)
        y = torch.ops.rga.ln_modulate(x1, s, t, 1e-6)
        x2, y2 = torch.ops.rga.gate_add_rms_modulate_ex(x1, y, g, s, t, 1e-6)
        h = torch.ops.rga.gelu_tanh(torch.ops.rga.rms_modulate_ex(x2, s, t, 1e-6), b)
        return x1, y, x2, y2, h

    gen = torch.Generator(device="cuda").manual_seed(5)
    mk = lambda *shape: torch.randn(*shape, generator=gen, device="cuda").to(torch.float16)
    args = (mk(2, 77, 1000), mk(2, 77, 1000), mk(2, 1, 1000), mk(2, 77, 1000) * 0.1,
            mk(2, 77, 1000) * 0.1, mk(1000))
    say("[compile] extended ops, float16, per-token modulation, D = 1000")
    got = torch.compile(block, fullgraph=True, backend="aot_eager")(*args)
    for a, b in zip(got, block(*args)):
        assert I.bitwise_equal(a, b)


@pytest.mark.gpu
def test_guard_with_model_math_references():
    from tests.gpu_util import say
    x, u, g, s, t = _dev_inputs(2100)
    # gate-add: the fp32 expression of the model math is the same arithmetic
    # (exact product, one binary32 add, one bf16 rounding): bit for bit
    gate_ref = lambda x, u, g: (x.float() + u.float() * g.float()).bfloat16()
    guard = I.FirstUseGuard(I.residual_gate_add, gate_ref)
    say("[guard] gate-add first use against the fp32 expression")
    out = guard(x, u, g)
    assert guard.state(x, u, g) is True
    assert I.bitwise_equal(out, gate_ref(x, u, g))
    # modulation: eager fp32 rms_norm has another summation order; the pages'
    # own tolerance decides
    D = x.shape[-1]
    rms_ref = lambda x, s, t, eps: (torch.nn.functional.rms_norm(x.float(), [D], eps=eps)
                                    * (1 + s.float()) + t.float()).bfloat16()
    guard2 = I.FirstUseGuard(I.rms_modulate, rms_ref, check=I.allclose(3e-2, 1e-2))
    say("[guard] rms_modulate first use against eager fp32 within the pages' tolerance")
    guard2(x, s, t, 1e-6)
    assert guard2.state(x, s, t, 1e-6) is True
    # a reference that disagrees is caught on first use
    bad = I.FirstUseGuard(I.residual_gate_add, lambda x, u, g: gate_ref(x, u, g) * 2)
    with pytest.raises(I.GuardMismatch):
        bad(x, u, g)
