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
    "argmax_last_of_ties": ("argmax_first", "if not np.isnan(x) and x > best_v:",
                            "if not np.isnan(x) and x >= best_v:"),
    "argmax_nan_first_kept": ("argmax_first", "best_v = -np.inf if np.isnan(v[m, 0]) else v[m, 0]",
                              "best_v = v[m, 0]"),
    "greedy_bound_sign": ("greedy_valid", "(y_ref[rows, idx] + b[rows, idx]) >= lo",
                          "(y_ref[rows, idx] - b[rows, idx]) >= lo"),
    "greedy_without_output_rounding": ("greedy_valid", "b = bound(a, y_ref)", "b = bound(a)"),
    "greedy_max_over_rows": ("greedy_valid", "np.max(y_ref - b, axis=1)", "np.max(y_ref - b)"),
    "bound_without_absolute_term": ("bound", "REL_TOL * np.asarray(a, np.float64) + ABS_TOL",
                                    "REL_TOL * np.asarray(a, np.float64)"),
    "bound_without_half_ulp": ("bound", "b = b + bf16_half_ulp(y_ref)", "b = b"),
    "half_ulp_a_bit_wide": ("bf16_half_ulp", "np.ldexp(1.0, e - 9)", "np.ldexp(1.0, e - 8)"),
    "half_ulp_a_bit_narrow": ("bf16_half_ulp", "np.ldexp(1.0, e - 9)", "np.ldexp(1.0, e - 10)"),
    "check_signed_error": ("check", "err = np.abs(np.asarray(y_gpu, np.float64) - y_ref)",
                           "err = np.asarray(y_gpu, np.float64) - y_ref"),
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
