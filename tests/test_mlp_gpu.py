"""The gated MLP (gate_up, silu(g) * u fused into down's input staging, down)
through skinny_mlp_swiglu, against the fp64 oracle's chain with the same bf16
roundings of g, u and h: outputs within the stated bound of the down linear,
at the TP=8 and TP=1 Qwen2.5-72B MLP shapes and small ragged ones."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import synth, workloads as wl
from tests.gpu_util import dev_bf16, dev_f32, dev_u8, host_codes, need_gpu, out

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run_mlp(x, wg, wd, M, sg_=None, sd=None):
    dev = [dev_bf16(x)]
    if sg_ is None:
        dev += [dev_bf16(wg), dev_bf16(wd)]
        scales = (None, None)
    else:
        dev += [dev_u8(wg), dev_u8(wd)]
        scales = (dev_f32(sg_), dev_f32(sd))
    y = out(M, wd.shape[0])
    mlp = sg.make_mlp(dev[0], dev[1], dev[2], y, *scales)
    ws = torch.empty(sg.mlp_workspace_bytes(mlp, M), dtype=torch.uint8, device="cuda")
    sg.mlp_swiglu(mlp, M, ws)
    torch.cuda.synchronize()
    return y


def check(y, y_ref, a, what):
    ok, worst, idx = oracle.check(y.float().cpu().double().numpy(), y_ref, a)
    assert ok, f"{what}: worst err/bound {worst:.3g} at {idx}"
    return worst


@pytest.mark.parametrize("M", [1, 3, 16])
@pytest.mark.parametrize("H,I", [(64, 64), (1000, 264), (256, 3696)])
def test_small_mlp_bf16(M, H, I):
    x = synth.tensor_bf16(0, synth.stream_id("mlp", M, H, I, "x"), M, H, 1.0)
    wg = synth.tensor_bf16(0, synth.stream_id("mlp", H, I, "wg"), 2 * I, H, 0.05)
    wd = synth.tensor_bf16(0, synth.stream_id("mlp", H, I, "wd"), H, I, 0.05)
    y_ref, a, _ = oracle.mlp_swiglu(x, wg, wd)
    check(run_mlp(x, wg, wd, M), y_ref, a, f"bf16 M={M} H={H} I={I}")


@pytest.mark.parametrize("M", [1, 6])
def test_small_mlp_fp8(M):
    H, I = 512, 1024
    x = synth.tensor_bf16(0, synth.stream_id("mlp8", M, "x"), M, H, 1.0)
    qg, sg8, _ = synth.fp8_weight_bs128(0, synth.stream_id("mlp8", "wg"), 2 * I, H, 0.05)
    qd, sd8, _ = synth.fp8_weight_bs128(0, synth.stream_id("mlp8", "wd"), H, I, 0.05)
    y_ref, a, _ = oracle.mlp_swiglu(x, qg, qd, scales=(sg8, sd8))
    check(run_mlp(x, qg, qd, M, sg8, sd8), y_ref, a, f"fp8 M={M}")


@pytest.mark.parametrize("tp,dtype,M", [(8, wl.BF16, 1), (8, wl.BF16, 2), (8, wl.BF16, 6),
                                        (8, wl.BF16, 16), (8, wl.FP8_BS128, 1),
                                        (8, wl.FP8_BS128, 6), (1, wl.BF16, 1), (1, wl.BF16, 6),
                                        (1, wl.FP8_BS128, 6)])
def test_qwen_mlp(tp, dtype, M):
    """W ~ N(0, 0.02), x ~ N(0, 1), seed 0.  Weights made on the GPU by the
    input generator; x and sampled rows (FP8: whole scale bands) regenerated
    on the host and checked to be identical first."""
    from gemv_skinny_gemm_amd.synth import gpu as sgpu
    specs = wl.mlp(tp, dtype)
    sets, tensors = sgpu.materialise(specs, M)
    (x_dev, wg_dev, sg_dev, _), (_, wd_dev, sd_dev, _) = tensors[0]
    gate_up, down = specs
    x = synth.tensor_bf16(0, gate_up.x_stream, M, gate_up.K, wl.X_SIGMA)
    assert np.array_equal(host_codes(x_dev), x)
    for spec, w_dev, s_dev in ((gate_up, wg_dev, sg_dev), (down, wd_dev, sd_dev)):
        rows = [0, spec.N // 3, spec.N - 1]
        if dtype == wl.BF16:
            w = synth.tensor_rows_bf16(0, spec.w_stream, rows, spec.K, wl.W_SIGMA)
            assert np.array_equal(host_codes(w_dev[rows]), w)
        else:
            for band in sorted(set(r // 128 for r in rows)):
                q, sc, r0 = synth.fp8_weight_bs128(0, spec.w_stream, spec.N, spec.K,
                                                   wl.W_SIGMA, band, 1)
                assert np.array_equal(w_dev[r0:r0 + q.shape[0]].cpu().numpy(), q)
                assert np.array_equal(s_dev[band:band + 1].cpu().numpy(), sc)
    y = out(M, down.N)
    if dtype == wl.BF16:
        mlp = sg.make_mlp(x_dev, wg_dev, wd_dev, y)
        y_ref, a, _ = oracle.mlp_swiglu(x, host_codes(wg_dev), host_codes(wd_dev))
    else:
        mlp = sg.make_mlp(x_dev, wg_dev, wd_dev, y, sg_dev, sd_dev)
        y_ref, a, _ = oracle.mlp_swiglu(x, wg_dev.cpu().numpy(), wd_dev.cpu().numpy(),
                                        scales=(sg_dev.cpu().numpy(), sd_dev.cpu().numpy()))
    ws = torch.empty(sg.mlp_workspace_bytes(mlp, M), dtype=torch.uint8, device="cuda")
    sg.mlp_swiglu(mlp, M, ws)
    torch.cuda.synchronize()
    worst = check(y, y_ref, a, f"tp{tp} dtype={dtype} M={M}")
    assert worst < 0.5
    del tensors, sets
