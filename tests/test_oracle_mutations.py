"""The oracle's pins catch plausible mistakes planted in the oracle.

Each case copies ``oracle/oracle.c``, plants one mistake of the kind a
careful reader could still make (a dropped term, a wrong sign, index or
constant, a sum in another order, a rounding done twice), builds the copy
with the oracle's own compiler flags (warnings not fatal), points the ``oracle`` module at the
copy and runs the fast pins of the matching test module: at least one of
them must fail. A control case builds the unchanged source the same way and
requires every pin to pass, so a failure is the planted mistake's and not
the harness's. CPU only; the product library plays no part.

Each mistake is planted at the first occurrence of a text after an anchor
(the function it belongs to), so a change to the oracle that moves or
rewords that text makes the case fail to plant, loudly, instead of going
quiet.
"""
from __future__ import annotations

import concurrent.futures
import importlib
import inspect
import os
import subprocess

import pytest

import oracle
from oracle import build as oracle_build

# name, pin module, anchor, text, replacement. Left out as equivalent
# (no input tells them apart): a fused multiply-add in the bf16 gated add
# (a product of two bf16 values has at most 16 significant bits, so it is
# exact in binary32 unless subnormal, and there the bf16 rounding of the sum
# cannot see the lost bits), and binary16's overflow threshold moved to
# 65536 (values in [65520, 65536) round up to infinity through the carry).
MUTANTS = [
    # bf16 rounding and the gated residual add
    ("rne_ties_away", "test_oracle_gate_add", "static uint16_t narrow_rne",
     "w += 0x7FFFu + ((w >> 16) & 1u);", "w += 0x8000u;"),
    ("rne_truncates", "test_oracle_gate_add", "static uint16_t narrow_rne",
     "w += 0x7FFFu + ((w >> 16) & 1u);", "w += 0u;"),
    ("nan_takes_rounding_route", "test_oracle_gate_add", "static uint16_t narrow_rne",
     "if ((w & 0x7FFFFFFFu) > 0x7F800000u)\n        return", "if (0)\n        return"),
    ("nan_not_quieted", "test_oracle_gate_add", "static uint16_t narrow_rne",
     "| 0x0040u", "| 0x0000u"),
    ("bcast_gate_ignores_batch", "test_oracle_gate_add", "void oracle_gate_add(",
     "g[b * D + d]", "g[d]"),
    ("gate_product_flushed_to_zero", "test_oracle_gate_add", "void oracle_gate_add(",
     "const float p = widen(u[i]) * widen(gi);",
     "float p = widen(u[i]) * widen(gi);\n"
     "                if (fabsf(p) < 0x1p-126f) p = 0.0f;"),
    ("gate_subtracts", "test_oracle_gate_add", "void oracle_gate_add(",
     "const float s = widen(x[i]) + p;", "const float s = widen(x[i]) - p;"),
    ("gate_on_the_sum", "test_oracle_gate_add", "void oracle_gate_add(",
     "const float p = widen(u[i]) * widen(gi);\n"
     "                const float s = widen(x[i]) + p;",
     "const float p = widen(u[i]) + widen(x[i]);\n"
     "                const float s = p * widen(gi);"),
    # weightless RMSNorm modulation
    ("rms_eps_outside_sqrt", "test_oracle_rms", "static float rms_factor_pinned",
     "const float t = ms + eps;\n    const float q = sqrtf(t);",
     "const float t = ms;\n    const float q = sqrtf(t) + eps;"),
    ("rms_no_mean", "test_oracle_rms", "static float rms_factor_pinned",
     "const float ms = ss / (float)D;", "const float ms = ss;"),
    ("rms_wrong_partial", "test_oracle_rms", "static float rms_factor_pinned",
     "const float ss = part[0];", "const float ss = part[1];"),
    ("rms_tree_skips_a_level", "test_oracle_rms", "static float rms_factor_pinned",
     "for (int m = 1; m < P; m <<= 1)", "for (int m = 2; m < P; m <<= 1)"),
    ("rms_groups_reassigned", "test_oracle_rms", "static float rms_factor_pinned",
     "const int j = (int)(k % P);", "const int j = (int)((k / 2) % P);"),
    ("rms_abs_not_square", "test_oracle_rms", "static float rms_factor_pinned",
     "const float sq = v * v;", "const float sq = fabsf(v);"),
    ("rms_drops_one_plus", "test_oracle_rms", "int oracle_rms_modulate(",
     "const float a = 1.0f + widen(sc[d]);", "const float a = widen(sc[d]);"),
    ("rms_scale_shift_swapped", "test_oracle_rms", "int oracle_rms_modulate(",
     "const float a = 1.0f + widen(sc[d]);\n"
     "                const float m = n * a;\n"
     "                const float y = m + widen(sh[d]);",
     "const float a = 1.0f + widen(sh[d]);\n"
     "                const float m = n * a;\n"
     "                const float y = m + widen(sc[d]);"),
    ("rms_scale_row_of_batch_0", "test_oracle_rms", "int oracle_rms_modulate(",
     "const uint16_t* sc = scale + b * D;", "const uint16_t* sc = scale;"),
    ("rms_shift_row_of_batch_0", "test_oracle_rms", "int oracle_rms_modulate(",
     "const uint16_t* sh = shift + b * D;", "const uint16_t* sh = shift;"),
    ("sequential_sum_unbiased", "test_oracle_rms", "static float rms_factor_sequential",
     "const float ms = ss / (float)D;", "const float ms = ss / (float)(D - 1);"),
    ("fused_normalizes_the_input", "test_oracle_rms", "int oracle_gate_add_rms_modulate(",
     "return oracle_rms_modulate(x_out,", "return oracle_rms_modulate(x,"),
    # binary16 / binary32 storage, per-token modulation, any D
    ("f16_ties_away", "test_oracle_variants", "static uint16_t narrow_f16",
     "((m + 0xFFFu + ((m >> 13) & 1u)) >> 13)", "((m + 0x1000u) >> 13)"),
    ("f16_overflow_threshold_low", "test_oracle_variants", "static uint16_t narrow_f16",
     "if (a >= 0x477FF000u)", "if (a >= 0x477FE000u)"),
    ("f16_subnormal_truncates", "test_oracle_variants", "static uint16_t narrow_f16",
     "rintf(mag * 0x1p24f)", "truncf(mag * 0x1p24f)"),
    ("f16_nan_becomes_inf", "test_oracle_variants", "static uint16_t narrow_f16",
     "sign | 0x7E00u |", "sign | 0x7C00u |"),
    ("f16_widen_bias_off_by_one", "test_oracle_variants", "static float widen_f16",
     "((e + 112u) << 23)", "((e + 111u) << 23)"),
    ("f16_widen_subnormal_scale", "test_oracle_variants", "static float widen_f16",
     "(float)m * 0x1p-24f", "(float)m * 0x1p-23f"),
    ("f16_stored_as_bf16", "test_oracle_variants", "static void store_elem",
     "else if (dtype == ORACLE_F16)", "else if (0)"),
    ("ex_bcast_gate_ignores_batch", "test_oracle_variants", "int oracle_gate_add_ex(",
     "? i : b * D + d;", "? i : d;"),
    ("ex_gate_add_fused", "test_oracle_variants", "int oracle_gate_add_ex(",
     "const float s = load_elem(x, i, dtype) + p;",
     "const float s = fmaf(load_elem(u, i, dtype), load_elem(g, gi, dtype), "
     "load_elem(x, i, dtype)); (void)p;"),
    ("ex_token_rows_ignored", "test_oracle_variants", "int oracle_rms_modulate_ex(",
     "const int64_t mrow = (mod_mode == ORACLE_MOD_TOKEN) ? row : b * D;",
     "const int64_t mrow = b * D;"),
    ("ex_drops_the_short_group", "test_oracle_variants", "static float rms_factor_ex",
     "const int64_t groups = (D + 7) / 8;", "const int64_t groups = D / 8;"),
    ("ex_fused_normalizes_the_input", "test_oracle_variants",
     "int oracle_gate_add_rms_modulate_ex(",
     "return oracle_rms_modulate_ex(x_out,", "return oracle_rms_modulate_ex(x,"),
    # tanh-GELU
    ("gelu_cubic_coefficient", "test_oracle_gelu", "double oracle_gelu_tanh_f64",
     "0.044715 * (h * h * h)", "0.04471 * (h * h * h)"),
    ("gelu_square_not_cube", "test_oracle_gelu", "double oracle_gelu_tanh_f64",
     "0.044715 * (h * h * h)", "0.044715 * (h * h)"),
    ("gelu_drops_the_2", "test_oracle_gelu", "double oracle_gelu_tanh_f64",
     "h / (1.0 + exp(-2.0 * a))", "h / (1.0 + exp(-a))"),
    ("gelu_exponent_sign", "test_oracle_gelu", "double oracle_gelu_tanh_f64",
     "h / (1.0 + exp(-2.0 * a))", "h / (1.0 + exp(2.0 * a))"),
    ("gelu_sqrt_1_over_pi", "test_oracle_gelu", "double oracle_gelu_tanh_f64",
     "sqrt(2.0 / acos(-1.0))", "sqrt(1.0 / acos(-1.0))"),
    ("gelu_minus_inf_to_plus_zero", "test_oracle_gelu", "double oracle_gelu_tanh_f64",
     "return h > 0 ? h : -0.0;", "return h > 0 ? h : 0.0;"),
    ("gelu_round_to_odd_misses_the_bit", "test_oracle_gelu", "static float round_to_odd_f32",
     "w |= 1u;", "w |= 0u;"),
    ("gelu_round_to_odd_keeps_the_away_neighbour", "test_oracle_gelu",
     "static float round_to_odd_f32",
     "f = nextafterf(f, 0.0f);", "(void)0;"),
    ("gelu_rounds_twice_to_nearest", "test_oracle_gelu", "int oracle_gelu_tanh(",
     "store_elem(out, i, round_to_odd_f32(y), dtype);", "store_elem(out, i, (float)y, dtype);"),
    ("gelu_ignores_bias", "test_oracle_gelu", "int oracle_gelu_tanh(",
     "h = h + load_elem(bias, f, dtype);", "(void)bias;"),
    ("gelu_bias_added_in_binary64", "test_oracle_gelu", "int oracle_gelu_tanh(",
     "h = h + load_elem(bias, f, dtype);\n"
     "            const double y = oracle_gelu_tanh_f64((double)h);",
     "(void)0;\n"
     "            const double y = oracle_gelu_tanh_f64((double)h + (bias ? "
     "(double)load_elem(bias, f, dtype) : 0.0));"),
    # weightless LayerNorm modulation
    ("ln_variance_not_centred", "test_oracle_ln", "static float pinned_sum",
     "const float dev = v - mean;", "const float dev = v + 0.0f * mean;"),
    ("ln_sum_groups_shifted", "test_oracle_ln", "static float pinned_sum",
     "const int j = (int)(k % P);", "const int j = (int)((k + 1) % P);"),
    ("ln_mean_over_d_minus_1", "test_oracle_ln", "static void ln_row_factors",
     "const float mu = s1 / (float)D;", "const float mu = s1 / (float)(D - 1);"),
    ("ln_unbiased_variance", "test_oracle_ln", "static void ln_row_factors",
     "const float var = s2 / (float)D;", "const float var = s2 / (float)(D - 1);"),
    ("ln_eps_outside_sqrt", "test_oracle_ln", "static void ln_row_factors",
     "const float t = var + eps;\n    const float q = sqrtf(t);",
     "const float t = var;\n    const float q = sqrtf(t) + eps;"),
    ("ln_output_not_centred", "test_oracle_ln", "int oracle_ln_modulate_ex(",
     "const float dev = load_elem(x, row + d, dtype) - mu;",
     "const float dev = load_elem(x, row + d, dtype) - 0.0f * mu;"),
    ("ln_token_rows_ignored", "test_oracle_ln", "int oracle_ln_modulate_ex(",
     "const int64_t mrow = (mod_mode == ORACLE_MOD_TOKEN) ? row : b * D;",
     "const int64_t mrow = b * D;"),
    ("ln_scale_sign", "test_oracle_ln", "int oracle_ln_modulate_ex(",
     "const float a = 1.0f + load_elem(scale, mrow + d, dtype);",
     "const float a = 1.0f - load_elem(scale, mrow + d, dtype);"),
    ("ln_drops_the_shift", "test_oracle_ln", "int oracle_ln_modulate_ex(",
     "const float y = m + load_elem(shift, mrow + d, dtype);", "const float y = m;"),
]

PIN_MODULES = ["test_oracle_gate_add", "test_oracle_rms", "test_oracle_variants",
               "test_oracle_gelu", "test_oracle_ln"]

# exhaustive sweeps that take seconds each; the planted mistakes are caught
# without them
SLOW = {"test_all_x_patterns_against_exact_arithmetic",
        "test_every_2_byte_pattern_is_correctly_rounded"}


def _plant(src: str, anchor: str, old: str, new: str) -> str:
    assert src.count(anchor) == 1, f"anchor {anchor!r} not unique in oracle.c"
    start = src.index(anchor)
    at = src.find(old, start)
    assert at >= 0, f"text {old!r} not found after {anchor!r}"
    return src[:at] + new + src[at + len(old):]


def _build(src: str, path: str) -> None:
    c_path = path[:-3] + ".c"
    with open(c_path, "w") as f:
        f.write(src)
    # the oracle's flags, less -Werror: a planted mistake may leave a
    # parameter or variable unused
    flags = [f for f in oracle_build.CFLAGS if f != "-Werror"]
    r = subprocess.run(["gcc", *flags, c_path, "-o", path, "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, f"build of {c_path} failed:\n{r.stderr}"


def _pins(module):
    """(name, function, kwargs) for every case of the module's fast pins,
    parametrize marks expanded in declaration order."""
    for name, fn in list(vars(module).items()):
        if not name.startswith("test_") or not callable(fn) or name in SLOW:
            continue
        combos = [{}]
        for mark in getattr(fn, "pytestmark", []):
            if mark.name != "parametrize":
                continue
            names = mark.args[0]
            names = [s.strip() for s in names.split(",")] if isinstance(names, str) else list(names)
            expanded = []
            for c in combos:
                for v in mark.args[1]:
                    v = getattr(v, "values", v)
                    v = (v,) if len(names) == 1 else tuple(v)
                    expanded.append({**c, **dict(zip(names, v))})
            combos = expanded
        wanted = set(inspect.signature(fn).parameters)
        for kw in combos:
            assert wanted == set(kw), f"{name} needs fixtures {wanted - set(kw)}"
            yield name, fn, kw


@pytest.fixture(scope="module")
def libraries(tmp_path_factory):
    root = tmp_path_factory.mktemp("oracle_mutants")
    with open(oracle_build.SOURCE) as f:
        src = f.read()
    jobs = {"control": src}
    for name, _, anchor, old, new in MUTANTS:
        jobs[name] = _plant(src, anchor, old, new)
    paths = {name: str(root / f"lib{name}.so") for name in jobs}
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as pool:
        for fut in [pool.submit(_build, jobs[n], paths[n]) for n in jobs]:
            fut.result()
    return paths


def _use(monkeypatch, path):
    monkeypatch.setattr(oracle, "LIBRARY", path)
    monkeypatch.setattr(oracle, "_LIB", None)


def test_mutant_names_are_unique():
    names = [m[0] for m in MUTANTS]
    assert len(names) == len(set(names))
    assert {m[1] for m in MUTANTS} == set(PIN_MODULES)


@pytest.mark.parametrize("module_name", PIN_MODULES)
def test_control_build_passes_every_fast_pin(module_name, libraries, monkeypatch):
    _use(monkeypatch, libraries["control"])
    module = importlib.import_module(f"tests.{module_name}")
    count = 0
    for _, fn, kw in _pins(module):
        fn(**kw)
        count += 1
    assert count > 5


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(mutant, libraries, monkeypatch):
    name, module_name = mutant[0], mutant[1]
    _use(monkeypatch, libraries[name])
    module = importlib.import_module(f"tests.{module_name}")
    for pin, fn, kw in _pins(module):
        try:
            fn(**kw)
        except AssertionError:
            return
    pytest.fail(f"mistake {name!r} passes every fast pin of {module_name}")
