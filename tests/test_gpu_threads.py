"""Calls from several host threads at once, each on its own stream.

The library keeps no state between calls (it validates on the host and
enqueues one kernel), so concurrent callers on different streams must get
exactly the results a single caller gets. Four threads each run a mix of
the calls (fast and element-wise paths) many times on their own stream;
every result is compared with the oracle.
"""
import threading

import numpy as np
import pytest
import torch

import oracle
from synth_inputs import BF16, GATE_BCAST, N001, N01, N02, U11, random_typed
from tests.gpu_util import say, to_dev_typed, to_host_typed

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dte():
    import diffusion_transformer_elementwise_amd as m
    return m


def test_threads_on_their_own_streams(dte):
    cases = []
    for k, (L, D) in enumerate([(64, 4096), (33, 4100), (96, 3072), (17, 1001)]):
        x = random_typed(8000 + k, (2, L, D), N02)
        u = random_typed(8100 + k, (2, L, D), N01)
        g = random_typed(8200 + k, (2, 1, D), U11)
        s = random_typed(8300 + k, (2, 1, D), N001)
        t = random_typed(8400 + k, (2, 1, D), N001)
        want_gate = oracle.gate_add_ex(x, u, g, GATE_BCAST, BF16)
        want_rms = oracle.rms_modulate_ex(x, s, t, 1e-6, oracle.MOD_ROW, BF16)
        cases.append(((x, u, g, s, t), want_gate, want_rms))
    reps = 25
    errors = []

    def worker(i):
        try:
            (x, u, g, s, t), want_gate, want_rms = cases[i]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                dx, du, dg, ds, dt = (to_dev_typed(a, BF16) for a in (x, u, g, s, t))
                outs = []
                for _ in range(reps):
                    outs.append((dte.rga_residual_gate_add_ex(dx, du, dg),
                                 dte.rga_rms_modulate_ex(dx, ds, dt, 1e-6)))
            stream.synchronize()
            for og, orms in outs:
                if not np.array_equal(to_host_typed(og), want_gate):
                    errors.append(f"thread {i}: gate-add differs")
                    return
                if not np.array_equal(to_host_typed(orms), want_rms):
                    errors.append(f"thread {i}: rms_modulate differs")
                    return
        except Exception as e:  # reported by the main thread
            errors.append(f"thread {i}: {e!r}")

    say(f"[threads] 4 threads x {reps} rounds of gate-add + rms_modulate")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
