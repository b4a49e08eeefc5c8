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
