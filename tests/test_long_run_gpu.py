"""Long run: 1000 back-to-back calls of the TP=8 layer (bf16 at M = 1 on the
row kernel, bf16 at M = 8 on the tile kernel with its second pass, FP8 at
M = 6) stay bitwise identical to the first call, and the time per call does
not drift over the run (10 batches of 100 calls, timed with events)."""
import pytest
import torch

import gemv_skinny_gemm_amd as sg
from gemv_skinny_gemm_amd import workloads as wl
from gemv_skinny_gemm_amd.synth import gpu as sgpu
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu

CALLS = 1000
BATCH = 100


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("dtype,M", [(wl.BF16, 1), (wl.BF16, 8), (wl.FP8_BS128, 6)])
def test_thousand_calls_bitwise_and_no_drift(dtype, M):
    specs = wl.tp8_layer(dtype)
    sets, tensors = sgpu.materialise(specs, M)
    descs = sets[0]
    ys = [t[3] for t in tensors[0]]
    ws = torch.empty(sg.stack_workspace_bytes(descs, M), dtype=torch.uint8, device="cuda")
    sg.decode_linear_stack(descs, M, ws)
    torch.cuda.synchronize()
    refs = [y.clone().view(torch.int16) for y in ys]
    # Bitwise: every call's outputs compared on the GPU with the first call's.
    mismatches = torch.zeros((), dtype=torch.int64, device="cuda")
    for _ in range(CALLS):
        sg.decode_linear_stack(descs, M, ws)
        for y, r in zip(ys, refs):
            mismatches += torch.ne(y.view(torch.int16), r).sum()
    torch.cuda.synchronize()
    assert int(mismatches) == 0, f"{int(mismatches)} outputs changed over {CALLS} calls"
    # Drift: the same calls alone, in event-timed batches.
    times = []
    for _ in range(CALLS // BATCH):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(BATCH):
            sg.decode_linear_stack(descs, M, ws)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / BATCH)
    med = sorted(times)[len(times) // 2]
    print(f"us per call by batch: {[round(t, 1) for t in times]}")
    assert max(times) < 1.25 * med and times[-1] < 1.1 * min(times[:3]) + 2.0, times
