"""Seeded random shapes against the fp64 oracle, to reach the planner's paths
in combinations the hand-picked cases do not: dtype, M = 1..16, ragged N and
K (up to tens of thousands), automatic and forced variants and grid sizes
(so K-chunk splits of 2^k and 3 x 2^k, window walks, both tile workgroup
shapes and the row kernel), and MoE launches with random routing (ids
outside [0, E) included), both x modes and the SwiGLU input."""
import numpy as np
import pytest

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import synth
from tests.gpu_util import assert_matches_oracle, need_gpu, run_bf16, run_fp8
from tests.test_moe_gpu import experts_bf16, experts_fp8, run_moe

pytestmark = pytest.mark.gpu

MAX_MACS = 60_000_000


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _dense_cases(n=160, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        fp8 = bool(rng.integers(2))
        M = int(rng.integers(1, 17))
        step = 16 if fp8 else 8
        K = int(np.exp(rng.uniform(np.log(step), np.log(40000)))) // step * step or step
        N = max(1, int(np.exp(rng.uniform(0, np.log(4000)))))
        N = max(1, min(N, MAX_MACS // (M * K)))
        variants = [sg.VARIANT_AUTO, sg.VARIANT_MFMA]
        if M <= 8 and not (fp8 and K > 32768):
            variants.append(sg.VARIANT_VECTOR)
        var = variants[int(rng.integers(len(variants)))]
        waves = [0, 0, 4, 8, 64, 300, 2048][int(rng.integers(7))]
        cases.append((i, fp8, M, N, K, var, waves))
    return cases


@pytest.mark.parametrize("case", _dense_cases(), ids=lambda c: "d%d" % c[0])
def test_random_dense(case):
    i, fp8, M, N, K, var, waves = case
    x = synth.tensor_bf16(0, synth.stream_id("rnd-x", i, M, K), M, K, 1.0)
    what = f"case {i}: {'fp8' if fp8 else 'bf16'} M={M} N={N} K={K} variant={var} waves={waves}"
    if fp8:
        q, s, _ = synth.fp8_weight_bs128(0, synth.stream_id("rnd-q", i, N, K), N, K)
        y_ref, a, _ = oracle.linear_fp8_bs128(x, q, s)
        y = run_fp8(x, q, s, M, N, variant=var, waves=waves)
    else:
        w = synth.tensor_bf16(0, synth.stream_id("rnd-w", i, N, K), N, K, 0.02)
        y_ref, a, _ = oracle.linear_bf16(x, w)
        y = run_bf16(x, w, M, N, variant=var, waves=waves)
    assert_matches_oracle(y, y_ref, a, what)


def _moe_cases(n=40, seed=77):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        fp8 = bool(rng.integers(2))
        E = int(rng.integers(1, 13))
        T = int(rng.integers(1, 17))
        topk = int(rng.integers(1, 5))
        step = 16 if fp8 else 8
        K = int(np.exp(rng.uniform(np.log(64), np.log(9000)))) // step * step
        N = int(rng.integers(16, 700))
        per_route = bool(rng.integers(2))
        swiglu = per_route and bool(rng.integers(2))
        cases.append((i, fp8, E, T, topk, N, K, per_route, swiglu))
    return cases


def _moe_cases_swiglu_shared(n=10, seed=78):
    """The SwiGLU input read from a shared row per token ([T][2K], not per
    route), which the cases above never draw."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        fp8 = bool(rng.integers(2))
        E = int(rng.integers(1, 13))
        T = int(rng.integers(1, 17))
        topk = int(rng.integers(1, 5))
        step = 16 if fp8 else 8
        K = int(np.exp(rng.uniform(np.log(64), np.log(9000)))) // step * step
        N = int(rng.integers(16, 700))
        cases.append((100 + i, fp8, E, T, topk, N, K, False, True))
    return cases


@pytest.mark.parametrize("case", _moe_cases() + _moe_cases_swiglu_shared(),
                         ids=lambda c: "m%d" % c[0])
def test_random_moe(case):
    i, fp8, E, T, topk, N, K, per_route, swiglu = case
    rng = np.random.default_rng(1000 + i)
    ids = rng.integers(-1, E + 1, (T, topk)).astype(np.int32)     # -1 and E: no expert
    tag = f"rnd-moe{i}"
    if fp8:
        w, s = experts_fp8(tag, E, N, K)
    else:
        w, s = experts_bf16(tag, E, N, K), None
    x = synth.tensor_bf16(0, synth.stream_id(tag, "x"), T * topk if per_route else T,
                          2 * K if swiglu else K, 1.0)
    y_ref, a = oracle.moe_linear(x, ids, w, scales=s, x_per_route=per_route, swiglu=swiglu)
    y = run_moe(x, ids, w, s, x_per_route=per_route, swiglu=swiglu)
    ok, worst, idx = oracle.check(y.float().cpu().double().numpy(), y_ref, a)
    assert ok, (f"case {i}: {'fp8' if fp8 else 'bf16'} E={E} T={T} topk={topk} N={N} K={K} "
                f"per_route={per_route} swiglu={swiglu}: worst err/bound {worst:.3g} at {idx}")
