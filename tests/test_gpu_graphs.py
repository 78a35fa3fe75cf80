"""The library under HIP graph capture.

Every call enqueues kernels on the caller's stream and does nothing else
(no allocation, no memset, no synchronisation), so a block of calls can be
captured once and replayed; at launch-bound sizes that removes the per-call
launch cost. The test captures a DiT-block-shaped sequence at the small
c1 shape, replays the graph several times with the program's own eager work
and synchronisations in between, and checks every replay bit for bit against
the eager results.
"""
import numpy as np
import pytest
import torch

from synth_inputs import CASES, GATE_FULL, make_inputs
from tests.gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dte():
    import diffusion_transformer_elementwise_amd as m
    return m


def _block(dte, x, u, g, s, t, outs):
    # residual update, next modulation (fused), LayerNorm modulation and the
    # GELU, each into a preallocated output (a graph replays fixed addresses)
    x1, y1, y2, h = outs
    dte.rga_residual_gate_add(x, u, g, out=x1, gate_mode=GATE_FULL)
    dte.rga_gate_add_rms_modulate(x1, u, g, s, t, 1e-6, x_out=x1, y=y1, gate_mode=GATE_FULL)
    dte.rga_ln_modulate(x1, s, t, 1e-6, out=y2)
    dte.gelu_tanh(y2, out=h)


def test_captured_block_replays_match_eager(dte):
    case = CASES["c1"]
    inp = make_inputs(case)
    x, u, g = to_dev(inp["x"]), to_dev(inp["u"]), to_dev(inp["g"])
    s, t = to_dev(inp["scale"]), to_dev(inp["shift"])
    outs = [torch.empty_like(x) for _ in range(4)]
    say(f"[graph] eager reference at {tuple(x.shape)}")
    _block(dte, x, u, g, s, t, outs)
    want = [to_host(o) for o in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up off the default stream
        _block(dte, x, u, g, s, t, outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    for o in outs:
        o.zero_()
    say("[graph] capture")
    with torch.cuda.graph(graph):
        _block(dte, x, u, g, s, t, outs)
    torch.cuda.synchronize()

    for rep in range(5):
        for o in outs:                     # eager work between replays
            o.fill_(float(rep + 1))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (o, w) in enumerate(zip(outs, want)):
            assert np.array_equal(to_host(o), w), f"replay {rep}, output {k}"
    say("[graph] 5 replays bit-identical to eager")


def test_graph_replay_amortizes_launches(dte):
    # 50 launch-bound calls captured once: replay time per call against eager
    case = CASES["c1"]
    inp = make_inputs(case)
    x, u, g = to_dev(inp["x"]), to_dev(inp["u"]), to_dev(inp["g"])
    out = torch.empty_like(x)
    n = 50
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            dte.rga_residual_gate_add(x, u, g, out=out, gate_mode=GATE_FULL)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for _ in range(n):
            dte.rga_residual_gate_add(x, u, g, out=out, gate_mode=GATE_FULL)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        dte.rga_residual_gate_add(x, u, g, out=out, gate_mode=GATE_FULL)
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / n
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / n
    say(f"[graph] c1 gate-add per call: eager {eager_us:.2f} us, graph replay {graph_us:.2f} us")
    want = to_host(dte.rga_residual_gate_add(x, u, g, gate_mode=GATE_FULL))
    assert np.array_equal(to_host(out), want)


def test_captured_element_paths_replay(dte):
    # ragged rows (element-wise kernels: chunked gated add and GELU, rows in
    # registers for the modulations and the fused call), captured and
    # replayed like the block above
    from synth_inputs import N001, N01, N02, U11, random_bits
    B, L, D = 2, 37, 1003
    x = to_dev(random_bits(61, (B, L, D), N02))
    u = to_dev(random_bits(62, (B, L, D), N01))
    g = to_dev(random_bits(63, (B, 1, D), U11))
    s = to_dev(random_bits(64, (B, 1, D), N001))
    t = to_dev(random_bits(65, (B, 1, D), N001))
    outs = [torch.empty_like(x) for _ in range(5)]

    def block():
        o1, o2, o3, o4, o5 = outs
        dte.rga_residual_gate_add_ex(x, u, g, out=o1)
        dte.rga_rms_modulate_ex(o1, s, t, 1e-6, out=o2)
        dte.rga_gate_add_rms_modulate_ex(o1, u, g, s, t, 1e-6, x_out=o3, y=o4)
        dte.gelu_tanh(o4, out=o5)

    say(f"[graph] element paths, eager reference at {(B, L, D)}")
    block()
    want = [to_host(o) for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        block()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        block()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float(-rep - 1))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (o, w) in enumerate(zip(outs, want)):
            assert np.array_equal(to_host(o), w), f"replay {rep}, output {k}"
    say("[graph] element paths: 4 replays bit-identical to eager")

