"""The pins are strong enough: each plausible mistake, planted in a copy of the
oracle's C source and compiled on the CPU, makes at least one pin fail."""
import inspect
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "drops_last_term": ("for (int64_t k = 0; k < K; ++k) {\n        double p",
                        "for (int64_t k = 0; k + 1 < K; ++k) {\n        double p"),
    "ignores_k_block_of_scale": ("(n / 128) * kblocks + (k / 128)", "(n / 128) * kblocks"),
    "ignores_n_block_of_scale": ("(n / 128) * kblocks + (k / 128)", "(k / 128)"),
    "e4m3_loses_sign": ("return sign ? -mag : mag;", "return mag;"),
    "e4m3_wrong_bias": ("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    "e4m3_wrong_subnormal_scale": ("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    "bf16_wrong_shift": ("(uint32_t)code << 16", "(uint32_t)code << 15"),
    "absum_without_abs": ("mag += fabs(p);", "mag += p;"),
    "x_row_stride_wrong": ("const double* xr = j->xv + m * K;", "const double* xr = j->xv;"),
    "accumulates_in_fp32": ("double acc = 0.0, mag = 0.0;", "float acc = 0.0f; double mag = 0.0;"),
}


def _pin_functions():
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if name.startswith("test_") and not inspect.signature(fn).parameters:
            yield name, fn


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_some_pin_catches_mutant(mutant, tmp_path):
    old, new = MUTANTS[mutant]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site moved; update the mutant"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", str(so), str(path),
                    "-lpthread", "-lm"], check=True)
    saved = oracle._lib
    oracle._lib = oracle._bind(str(so))
    caught = []
    try:
        for name, fn in _pin_functions():
            try:
                fn()
            except AssertionError:
                caught.append(name)
    finally:
        oracle._lib = saved
    assert caught, f"no pin catches the mutant {mutant}"


# Mistakes in the Python-level routing of the mixture-of-experts linear: each
# planted in a copy of oracle.moe_linear must make one of the MoE pins fail.
MOE_MUTANTS = {
    "token_row_for_shared_x": ("x[rs] if x_per_route else x[rs // topk]", "x[rs]"),
    "route_row_for_per_route_x": ("x[rs] if x_per_route else x[rs // topk]", "x[rs // topk]"),
    "first_expert_scales": ("scales[e], threads", "scales[0], threads"),
    "wraps_negative_ids": ("rs = np.nonzero(flat == e)[0]", "rs = np.nonzero(flat % E == e)[0]"),
    "swiglu_gate_up_swapped": ("bf16_encode(silu(g) * u)", "bf16_encode(silu(u) * g)"),
    "first_choice_only": ("flat = ids.reshape(-1)", "flat = np.repeat(ids[:, 0], topk)"),
}


@pytest.mark.parametrize("mutant", sorted(MOE_MUTANTS))
def test_some_moe_pin_catches_mutant(mutant, monkeypatch):
    old, new = MOE_MUTANTS[mutant]
    src = inspect.getsource(oracle.moe_linear)
    assert src.count(old) == 1, "mutation site moved; update the mutant"
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), "<moe_mutant>", "exec"), ns)
    monkeypatch.setattr(oracle, "moe_linear", ns["moe_linear"])
    caught = []
    calls = [(n, fn, {}) for n, fn in _pin_functions() if "moe" in n]
    calls += [("test_moe_linear_vs_exact_rationals_bf16", pins.test_moe_linear_vs_exact_rationals_bf16,
               {"x_per_route": v}) for v in (False, True)]
    for name, fn, params in calls:
        try:
            fn(**params)
        except (AssertionError, ValueError, IndexError):
            caught.append(name)
    assert caught, f"no pin catches the mutant {mutant}"


# Mistakes in the oracle's Python helpers and the gated MLP chain: each planted
# in a copy of the one function must make some pin fail (pins reach the
# function through the module, so the copy replaces it for all of them).
HELPER_MUTANTS = {
    "silu_wrong_sign": ("silu", "np.exp(-v)", "np.exp(v)"),
    "silu_is_sigmoid": ("silu", "return v / (1.0 + np.exp(-v))", "return 1.0 / (1.0 + np.exp(-v))"),
    "bf16_truncates": ("bf16_encode", "sig = np.rint(f * 256.0)", "sig = np.floor(f * 256.0)"),
    "bf16_rounds_half_up": ("bf16_encode", "sig = np.rint(f * 256.0)", "sig = np.floor(f * 256.0 + 0.5)"),
    "bf16_nan_as_infinity": ("bf16_encode", "np.uint16(0x7FC0)", "np.uint16(0x7F80)"),
    "mlp_gate_up_swapped": ("mlp_swiglu", "h = bf16_encode(silu(g) * u)", "h = bf16_encode(silu(u) * g)"),
    "mlp_gate_not_rounded": ("mlp_swiglu", "g = bf16_decode(bf16_encode(gu[:, :I]))", "g = gu[:, :I]"),
    "mlp_wrong_half_for_gate": ("mlp_swiglu", "g = bf16_decode(bf16_encode(gu[:, :I]))",
                                "g = bf16_decode(bf16_encode(gu[:, I:]))"),
    "argmax_last_of_ties": ("argmax_first", "if best_i is None or x > v[m, best_i]:",
                            "if best_i is None or x >= v[m, best_i]:"),
    # The reading before NaN ranked below -inf: a leading NaN held index 0.
    "argmax_nan_first_kept": ("argmax_first", "best_i = None                              # no number seen yet",
                              "best_i = 0"),
    "argmax_nan_not_skipped": ("argmax_first", "if np.isnan(x):\n                continue",
                               "if np.isnan(x):\n                pass"),
    "greedy_bound_sign": ("greedy_valid", "hi[rows, idx] >= np.max(lo, axis=1)",
                          "lo[rows, idx] >= np.max(lo, axis=1)"),
    "greedy_without_output_rounding": ("greedy_valid", "lo, hi = accepted(y_ref, a)",
                                       "lo, hi = y_ref - bound(a), y_ref + bound(a)"),
    "greedy_max_over_rows": ("greedy_valid", "np.max(lo, axis=1)", "np.max(lo)"),
    "bound_without_absolute_term": ("bound", "REL_TOL * np.asarray(a, np.float64) + ABS_TOL",
                                    "REL_TOL * np.asarray(a, np.float64)"),
    "accepted_without_bracket": ("accepted", "return np.minimum(y_ref - b, lo_b), np.maximum(y_ref + b, hi_b)",
                                 "return y_ref - b, y_ref + b"),
    "accepted_rounded_not_bracketed": ("accepted", "lo_b, hi_b = bf16_bracket(y_ref)",
                                       "lo_b = hi_b = bf16_decode(bf16_encode(y_ref))"),
    "bracket_a_step_wide": ("bf16_bracket", "np.maximum(c - 1, 0)", "np.maximum(c - 2, 0)"),
    "bracket_sign_not_mirrored": ("bf16_bracket",
                                  "return np.where(v < 0, -above, below), np.where(v < 0, -below, above)",
                                  "return np.where(v < 0, -below, below), np.where(v < 0, -above, above)"),
    "check_signed_error": ("check", "err = np.abs(y - y_ref)", "err = y - y_ref"),
    "check_wrong_side": ("check", "np.where(y >= y_ref, hi - y_ref, y_ref - lo)",
                         "np.where(y >= y_ref, y_ref - lo, hi - y_ref)"),
    "check_rejects_at_bound": ("check", "np.all(ratio <= 1.0)", "np.all(ratio < 1.0)"),
    "bf16_decode_wrong_shift": ("bf16_decode", "astype(np.uint32) << 16", "astype(np.uint32) << 15"),
}


@pytest.mark.parametrize("mutant", sorted(HELPER_MUTANTS))
def test_some_pin_catches_helper_mutant(mutant, monkeypatch):
    fname, old, new = HELPER_MUTANTS[mutant]
    src = inspect.getsource(getattr(oracle, fname))
    assert src.count(old) == 1, "mutation site moved; update the mutant"
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), "<helper_mutant>", "exec"), ns)
    monkeypatch.setattr(oracle, fname, ns[fname])
    caught = []
    for name, fn in _pin_functions():
        try:
            fn()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(name)
    assert caught, f"no pin catches the mutant {mutant}"
