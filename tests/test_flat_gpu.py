"""The flat row kernel (skinny_rows_flat) at every token count it takes, against
the fp64 oracle: launches under 0.4 GB of weights run it for up to 4 tokens
(bf16) or 2 (FP8).  The automatic plan is asserted to pick it, so these cases
exercise it and no other kernel.  Forced grids of one or a few workgroups
make each workgroup hold more outputs than its LDS buffer (4096 bf16 values
per token row group), switch linears mid-stream and end on a ragged unit."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import synth
from tests.gpu_util import (assert_matches_oracle, dev_bf16, dev_f32, dev_u8, need_gpu, out,
                            run_bf16, run_fp8)

pytestmark = pytest.mark.gpu

FLAT = next(k for k, v in sg.KERNEL_NAMES.items() if v == "skinny_rows_flat")
MAX_M = {sg.BF16: 4, sg.FP8_BS128: 2}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _kernel(descs, M):
    return sg.plan_query(descs, M).kernel


def _plan_is_flat(dtype, shapes, M):
    scale = None if dtype == sg.BF16 else 0x300000
    lins = [sg.Linear(dtype, N, K, 0, 0x100000, scale, 0x2000000, 0x4000000) for N, K in shapes]
    return _kernel(lins, M) == FLAT


# K = 8: one chunk; 264 / 1000 / 3696: ragged row ends; 8192: whole segments.
BF16_SHAPES = [(1, 8), (17, 264), (100, 1000), (257, 3696), (1280, 8192)]
FP8_SHAPES = [(1, 16), (130, 272), (300, 1024), (257, 3696), (1280, 8192)]


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("N,K", BF16_SHAPES)
def test_flat_bf16_vs_oracle(M, N, K):
    assert _plan_is_flat(sg.BF16, [(N, K)], M)
    x = synth.tensor_bf16(0, synth.stream_id("flat-bf16", M, N, K, "x"), M, K, 1.0)
    w = synth.tensor_bf16(0, synth.stream_id("flat-bf16", N, K, "w"), N, K, 0.02)
    y_ref, a, _ = oracle.linear_bf16(x, w)
    for waves in (0, 8, 40):
        y = run_bf16(x, w, M, N, waves=waves)
        assert_matches_oracle(y, y_ref, a, f"bf16 M={M} N={N} K={K} waves={waves}")


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("N,K", FP8_SHAPES)
def test_flat_fp8_vs_oracle(M, N, K):
    assert _plan_is_flat(sg.FP8_BS128, [(N, K)], M)
    x = synth.tensor_bf16(0, synth.stream_id("flat-fp8", M, N, K, "x"), M, K, 1.0)
    q, s, _ = synth.fp8_weight_bs128(0, synth.stream_id("flat-fp8", N, K, "w"), N, K)
    y_ref, a, _ = oracle.linear_fp8_bs128(x, q, s)
    for waves in (0, 8, 40):
        y = run_fp8(x, q, s, M, N, waves=waves)
        assert_matches_oracle(y, y_ref, a, f"fp8 M={M} N={N} K={K} waves={waves}")


@pytest.mark.parametrize("dtype", [sg.BF16, sg.FP8_BS128])
def test_flat_output_buffer_refills(dtype):
    """N = 8203 rows on one workgroup (1026 units of 8 rows): more than the
    1024 / 512 / 341 / 256 units whose outputs the LDS buffer holds at M = 1 /
    2 / 3 / 4, and a ragged last unit; also on three workgroups."""
    N, K = 8203, 80
    for M in range(1, MAX_M[dtype] + 1):
        assert _plan_is_flat(dtype, [(N, K)], M)
        x = synth.tensor_bf16(0, synth.stream_id("flat-refill", M, dtype, "x"), M, K, 1.0)
        for waves in (8, 24):
            if dtype == sg.BF16:
                w = synth.tensor_bf16(0, synth.stream_id("flat-refill", "w"), N, K, 0.02)
                y_ref, a, _ = oracle.linear_bf16(x, w)
                y = run_bf16(x, w, M, N, waves=waves)
            else:
                q, s, _ = synth.fp8_weight_bs128(0, synth.stream_id("flat-refill", "q"), N, K)
                y_ref, a, _ = oracle.linear_fp8_bs128(x, q, s)
                y = run_fp8(x, q, s, M, N, waves=waves)
            assert_matches_oracle(y, y_ref, a, f"dtype={dtype} M={M} waves={waves}")


@pytest.mark.parametrize("dtype", [sg.BF16, sg.FP8_BS128])
def test_flat_stack_switches_linears(dtype):
    """Five linears of different K and ragged N in one launch, each with its
    own x: a workgroup's units cross from one linear to the next (its outputs
    written, the next x staged).  Rows of N not a multiple of 8 are written
    value by value, the others 8 at a time.  The last linear is large enough
    (about 0.1 GB) for the automatic plan to take the flat kernel with five
    linears in the launch."""
    N5 = 12000 if dtype == sg.BF16 else 24000
    shapes = [(9, 272), (1000, 3696), (3, 16), (523, 1024), (N5, 4096)]
    weights = []                                           # host weights and device copies
    for i, (N, K) in enumerate(shapes):
        if dtype == sg.BF16:
            w = synth.tensor_bf16(0, synth.stream_id("flat-stack", i, "w"), N, K, 0.02)
            weights.append(((w,), dev_bf16(w), None))
        else:
            q, s, _ = synth.fp8_weight_bs128(0, synth.stream_id("flat-stack", i, "q"), N, K)
            weights.append(((q, s), dev_u8(q), dev_f32(s)))
    for M in range(1, MAX_M[dtype] + 1):
        assert _plan_is_flat(dtype, shapes, M)
        descs, refs, ys, keep = [], [], [], []
        for i, (N, K) in enumerate(shapes):
            x = synth.tensor_bf16(0, synth.stream_id("flat-stack", M, i, "x"), M, K, 1.0)
            host, wd, sd = weights[i]
            refs.append(oracle.linear_bf16(x, *host) if dtype == sg.BF16
                        else oracle.linear_fp8_bs128(x, *host))
            xd, yd = dev_bf16(x), out(M, N)
            keep.append(xd)
            ys.append(yd)
            descs.append(sg.make_linear(xd, wd, yd, w_scale=sd))
        assert _kernel(descs, M) == FLAT
        ws = torch.empty(sg.stack_workspace_bytes(descs, M), dtype=torch.uint8, device="cuda")
        for waves in (0, 8, 16):
            for yd in ys:
                yd.fill_(float("nan"))
            sg.linear_run(descs, M, ws, waves=waves)
            torch.cuda.synchronize()
            for i, (yd, (y_ref, a, _)) in enumerate(zip(ys, refs)):
                assert_matches_oracle(yd, y_ref, a, f"dtype={dtype} M={M} waves={waves} linear {i}")


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_flat_greedy_tokens(M):
    """Vocabulary projection of 30011 rows through the flat kernel's greedy
    epilogue (one pair per workgroup and token): W row n is one-hot at column
    perm[n], so the logits are x[:, perm] exactly and the token is decided
    exactly, the smallest index winning ties."""
    N, K = 30011, 1024
    rng = np.random.default_rng(90 + M)
    perm = rng.integers(0, K, N)
    vals = torch.tensor(rng.normal(size=7), dtype=torch.float64).to(torch.bfloat16)
    x = vals.view(torch.int16).numpy().view(np.uint16)[rng.integers(0, 7, (M, K))]
    w = np.zeros((N, K), np.uint16)
    w[np.arange(N), perm] = 0x3F80                        # 1.0
    assert _plan_is_flat(sg.BF16, [(N, K)], M)
    xd, wd, yd = dev_bf16(x), dev_bf16(w), out(M, N)
    tok = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    lin = sg.make_linear(xd, wd, yd)
    ws = torch.empty(sg.lm_head_workspace_bytes(lin, M), dtype=torch.uint8, device="cuda")
    sg.lm_head_argmax(lin, M, tok, ws)
    torch.cuda.synchronize()
    logits = torch.from_numpy(x[:, perm].view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(yd.double().cpu().numpy(), logits)
    assert tok.cpu().numpy().tolist() == oracle.argmax_first(logits).tolist()
