"""The seeded input recipe and the byte accounting, checked against the
numbers the pages print (tests/golden/pages_facts.json)."""
import json
import os
import re

import numpy as np

from synth_inputs import CASES, GATE_BCAST, GATE_FULL, N01, U11, Case, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def _facts():
    with open(GOLDEN) as f:
        return json.load(f)


def _shape_of(name):
    m = re.search(r"_s(\d+)_c(\d+)$", name)
    return 1, int(m.group(1)), int(m.group(2))


def test_gate_add_cases_are_pages_workloads():
    pages = {}
    for row in _facts()["residual_gate_workloads"]["rows"]:
        kind = GATE_FULL if row["gate"] == "full" else GATE_BCAST
        pages[_shape_of(row["name"])] = kind
    for key, case in CASES.items():
        if key == "c5":
            continue  # B = 2 sequence case built on the video hidden size
        assert pages.get((case.B, case.L, case.D)) == case.gate, key


def test_rms_hidden_sizes_and_eps_follow_pages():
    f = _facts()["rms_modulate_test"]
    for key in ("c1", "c5"):
        assert CASES[key].rms and CASES[key].D in f["hidden"]
        assert CASES[key].eps == f["eps"]


def test_ncu_counts_fix_element_width_and_load_width():
    f = _facts()["ncu_large_broadcast"]
    B, L, D = f["shape"]
    n = B * L * D
    # the flat candidate read x, u and g once per element: 3*n elements in
    # 32-byte L1 sectors means 2-byte (bf16) elements
    assert f["flat_candidate"]["l1tex_load_sectors"] * 32 == 3 * n * 2
    # ... with 32-lane warps moving 16 bytes per lane (256 elements per load)
    assert f["flat_candidate"]["global_load_inst"] * 256 == 3 * n
    # the row-tiled path reads the gate row once per 4 rows: 2n + n/4 elements
    rt = f["row_tile_4x"]
    assert rt["global_load_inst"] * 256 == 2 * n + n // rt["rows_per_gate_load"]


def test_algorithmic_bytes_per_config():
    # each input element read once, each output element written once,
    # 2 bytes per element; a broadcast row counts once per call
    def gate_bytes(c):
        n = c.elems
        return (4 * n if c.gate == GATE_FULL else 3 * n + c.B * c.D) * 2
    assert gate_bytes(CASES["c3"]) == 267_386_880
    assert gate_bytes(CASES["c4"]) == 802_168_832
    c5 = CASES["c5"]
    assert gate_bytes(c5) == 1_604_337_664
    assert (2 * c5.elems + 2 * c5.B * c5.D) * 2 == 1_069_580_288


def test_generator_is_seeded_and_chunk_invariant():
    c = Case("t", 1, 3000, 16, 5, GATE_FULL)
    a = make_inputs(c)
    b = make_inputs(c)
    for k in a:
        assert np.array_equal(a[k], b[k])
    # one draw of the whole tensor gives the same stream as the row chunks
    rng = np.random.default_rng(5)
    from synth_inputs import to_bf16_bits
    x = to_bf16_bits(N01.draw(rng, (3000 * 16,))).reshape(1, 3000, 16)
    u = to_bf16_bits(N01.draw(rng, (3000 * 16,))).reshape(1, 3000, 16)
    g = to_bf16_bits(U11.draw(rng, (3000 * 16,))).reshape(1, 3000, 16)
    assert np.array_equal(a["x"], x) and np.array_equal(a["u"], u) and np.array_equal(a["g"], g)


def test_distributions_have_the_stated_moments():
    from tests.exact_round import bf16_bits_to_f32
    c5 = make_inputs(Case("m", 1, 512, 1024, 7, GATE_BCAST,
                          x=CASES["c5"].x, g=CASES["c5"].g, rms=True))
    x = bf16_bits_to_f32(c5["x"])
    assert abs(x.std() - 2.0) < 0.02 and abs(x.mean()) < 0.02
    g = bf16_bits_to_f32(c5["g"])
    assert abs(g.std() - 0.1) < 0.01
    c3 = make_inputs(Case("m", 1, 512, 1024, 8, GATE_FULL))
    gu = bf16_bits_to_f32(c3["g"])
    assert gu.min() >= -1 and gu.max() <= 1 and abs(gu.std() - 1 / np.sqrt(3)) < 0.01


def test_typed_ulp_metric():
    # neighbours, signed zeros, NaN classes and infinities for each layout
    from tests.exact_round import is_nan_typed, ulp_diff_typed
    h = lambda *v: np.array(v, dtype=np.uint16)
    assert list(ulp_diff_typed(h(0x3C00, 0x8000, 0x7E00, 0x7C00),
                               h(0x3C01, 0x0000, 0x7C01, 0x7BFF), 1)) == [1, 0, 0, 1]
    assert list(is_nan_typed(h(0x7C00, 0x7C01, 0xFE00, 0x7F80), 1)) == [False, True, True, True]
    f = np.array([1.0, -0.0, np.inf, np.nan], dtype=np.float32)
    g = np.array([np.nextafter(np.float32(1), np.float32(2)), 0.0,
                  np.finfo(np.float32).max, np.nan], dtype=np.float32)
    assert list(ulp_diff_typed(f, g, 2)) == [1, 0, 1, 0]
    assert ulp_diff_typed(np.float32([np.nan]), np.float32([1.0]), 2)[0] > 1 << 30
    # one step across zero: the smallest subnormals of either sign are 2 apart
    assert ulp_diff_typed(h(0x0001), h(0x8001), 1)[0] == 2
    assert ulp_diff_typed(h(0x0001), h(0x8001), 0)[0] == 2


def test_typed_generator_matches_library_conversions():
    from synth_inputs import BF16, F16, F32, N01, random_bits, random_typed
    a32 = random_typed(9, (2, 3, 40), N01, F32)
    assert a32.dtype == np.float32 and a32.shape == (2, 3, 40)
    a16 = random_typed(9, (2, 3, 40), N01, F16)
    assert np.array_equal(a16.view(np.float16), a32.astype(np.float16))
    assert np.array_equal(random_typed(9, (2, 3, 40), N01, BF16), random_bits(9, (2, 3, 40), N01))
