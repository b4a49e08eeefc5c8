"""The 8-wave tile workgroup in its exact-fit LDS layout (FP8 launches of at
least eight 128-row groups per CU, plain x): swizzled W tiles and x rows, no
pad chunk and no zero row, absent tokens reading token 0.  Checked against the
oracle on every output of a launch of that size, with ragged N and K (rows
ending inside a 512-byte segment, x windows ending inside a swizzle group),
at token counts around the layout's limits: M = 5 and 6 fit K = 8192 whole,
7 and 8 split it, 9 and 16 walk their windows and repeat the x swizzle
(tokens m and m + 8)."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import synth
from tests.gpu_util import assert_matches_oracle, dev_bf16, need_gpu, out

pytestmark = pytest.mark.gpu

# (N, K): 1094 + 1016 row groups of 128 rows, enough for the 8-wave shape on a
# 256-CU GPU; K = 1040 and 2064 are 2.03 and 4.03 segments of 512 bytes.
SHAPES = ((140_000, 1040), (130_000, 2064))
WIDE = 5        # enum skinny_kernel: skinny_tiles (8-wave)


@pytest.fixture(scope="module")
def weights():
    need_gpu()
    from gemv_skinny_gemm_amd.synth import gpu as sgpu
    out_ = []
    for i, (N, K) in enumerate(SHAPES):
        q, s = sgpu.fp8_weight_bs128(0, synth.stream_id("fit-w", i, N, K), N, K)
        out_.append((q, s, q.cpu().numpy(), s.cpu().numpy()))
    torch.cuda.synchronize()
    yield out_
    del out_
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [2, 5, 6, 7, 9, 16])
def test_fp8_large_launch_every_output(weights, M):
    xs, xds, ys, lins = [], [], [], []      # device tensors kept alive for the call
    for i, ((N, K), (q, s, _, _)) in enumerate(zip(SHAPES, weights)):
        x = synth.tensor_bf16(0, synth.stream_id("fit-x", i, M, K), M, K, 1.0)
        xd, yd = dev_bf16(x), out(M, N)
        xs.append(x)
        xds.append(xd)
        ys.append(yd)
        lins.append(sg.make_linear(xd, q, yd, w_scale=s))
    plan = sg.plan_query(lins, M)
    assert plan.kernel == WIDE, f"M={M}: expected the 8-wave tile kernel, plan {plan.kernel}"
    ws = torch.empty(sg.stack_workspace_bytes(lins, M), dtype=torch.uint8, device="cuda")
    sg.decode_linear_stack(lins, M, ws)
    torch.cuda.synchronize()
    for i, ((N, K), (_, _, qh, sh)) in enumerate(zip(SHAPES, weights)):
        y_ref, a, _ = oracle.linear_fp8_bs128(xs[i], qh, sh)
        assert_matches_oracle(ys[i], y_ref, a, f"M={M} linear {i} (N={N}, K={K})")
