"""The workspace the library asks for is enough: each call that writes
partial sums (split K in either tile workgroup shape, the gated MLP's
intermediate and slots, a split MoE launch) runs with exactly the
*_workspace_bytes it reports, followed by a guard region that must come back
untouched, and its outputs are checked against the oracle."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import synth, workloads as wl
from gemv_skinny_gemm_amd.synth import gpu as sgpu
from tests.gpu_util import dev_bf16, need_gpu

pytestmark = pytest.mark.gpu

GUARD = 1 << 16


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def guarded(nbytes):
    """A workspace of exactly nbytes (16-byte aligned) followed by a guard."""
    full = torch.empty(nbytes + GUARD, dtype=torch.uint8, device="cuda")
    full[nbytes:].fill_(0xA5)
    return full[:nbytes], full[nbytes:]


def assert_guard(guard):
    torch.cuda.synchronize()
    assert bool(torch.all(guard == 0xA5)), "a kernel wrote past the workspace it asked for"


@pytest.mark.parametrize("M", [2, 8, 16])
def test_tp8_layer_split(M):
    sets, tensors = sgpu.materialise(wl.tp8_layer(wl.BF16), M)
    ws, guard = guarded(sg.stack_workspace_bytes(sets[0], M))
    sg.decode_linear_stack(sets[0], M, ws)
    assert_guard(guard)


@pytest.mark.parametrize("M", [6, 16])
def test_fp8_large_workgroup_split(M):
    """2048 row groups of 128 rows: the 8-wave shape, K split at M = 16."""
    spec = wl.LinearSpec("guard-fp8", 262144, 8192, wl.FP8_BS128,
                         synth.stream_id("guard-fp8", "w"), synth.stream_id("guard-fp8", M, "x"))
    sets, tensors = sgpu.materialise([spec], M)
    ws, guard = guarded(sg.stack_workspace_bytes(sets[0], M))
    sg.decode_linear_stack(sets[0], M, ws)
    assert_guard(guard)
    x_dev, q_dev, s_dev, y_dev = tensors[0][0]
    x = synth.tensor_bf16(0, spec.x_stream, M, spec.K, wl.X_SIGMA)
    q, sc, r0 = synth.fp8_weight_bs128(0, spec.w_stream, spec.N, spec.K, wl.W_SIGMA, 1000, 1)
    y_ref, a, _ = oracle.linear_fp8_bs128(x, q, sc)
    ok, worst, idx = oracle.check(y_dev[:, r0:r0 + 128].float().cpu().double().numpy(), y_ref, a)
    assert ok, f"worst err/bound {worst:.3g} at {idx}"


@pytest.mark.parametrize("M", [1, 6])
def test_mlp(M):
    sets, tensors = sgpu.materialise(wl.mlp(8, wl.FP8_BS128), M)
    t = tensors[0]
    mlp = sg.make_mlp(t[0][0], t[0][1], t[1][1], t[1][3], t[0][2], t[1][2])
    ws, guard = guarded(sg.mlp_workspace_bytes(mlp, M))
    sg.mlp_swiglu(mlp, M, ws)
    assert_guard(guard)


def test_moe_split():
    E, N, K, T, topk = 3, 64, 16384, 3, 2
    w = synth.tensor_bf16(0, 911, E * N, K, 0.02).reshape(E, N, K)
    ids = np.array([[0, 2], [2, 1], [1, 0]], np.int32)
    x = synth.tensor_bf16(0, 912, T, K, 1.0)
    wd = dev_bf16(w.reshape(E * N, K)).view(E, N, K)
    ex = sg.make_experts(wd)
    ws, guard = guarded(sg.moe_workspace_bytes(ex, T, topk))
    y = torch.empty((T * topk, N), dtype=torch.bfloat16, device="cuda")
    sg.moe_linear(ex, dev_bf16(x), torch.from_numpy(ids).cuda(), y, ws)
    assert_guard(guard)
    y_ref, a = oracle.moe_linear(x, ids, w)
    ok, worst, idx = oracle.check(y.float().cpu().double().numpy(), y_ref, a)
    assert ok, f"worst err/bound {worst:.3g} at {idx}"
