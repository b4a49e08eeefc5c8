"""Calls made from several host threads at once, each on its own stream with
its own workspace and outputs (the contract for concurrent calls): every
result is bitwise equal to the same call made alone.  The threads run the row
kernel (M = 1 and 2) and the tile kernel with its second pass (M = 8 and 16)
side by side, so the library's per-device caches are read and filled from
several threads while kernels of every kind share the GPU."""
import threading

import pytest
import torch

import gemv_skinny_gemm_amd as sg
from gemv_skinny_gemm_amd import workloads as wl
from gemv_skinny_gemm_amd.synth import gpu as sgpu
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def test_threads_on_separate_streams():
    specs = wl.tp8_layer(wl.BF16)
    Ms = [1, 2, 8, 16]
    iters = 25
    _, tensors = sgpu.materialise(specs, max(Ms))
    jobs = []
    for M in Ms:
        ys = [torch.empty((M, s.N), dtype=torch.bfloat16, device="cuda") for s in specs]
        descs = [sg.make_linear(t[0][:M], t[1], y, w_scale=t[2]) for t, y in zip(tensors[0], ys)]
        ws = torch.empty(sg.stack_workspace_bytes(descs, M), dtype=torch.uint8, device="cuda")
        jobs.append((M, descs, ys, ws, torch.cuda.Stream()))
    torch.cuda.synchronize()
    errors = []

    def worker(M, descs, ys, ws, stream):
        try:
            for _ in range(iters):
                sg.decode_linear_stack(descs, M, ws, stream=stream)
        except Exception as e:                       # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=j) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    got = [[y.clone() for y in j[2]] for j in jobs]
    for (M, descs, ys, ws, _), g in zip(jobs, got):
        for y in ys:
            y.fill_(float("nan"))
        sg.decode_linear_stack(descs, M, ws)         # alone, on the current stream
        torch.cuda.synchronize()
        for a, b in zip(g, ys):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"M = {M} differs"
