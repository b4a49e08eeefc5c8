"""decode_linear_stack_noalloc, whose split-K partial sums live in the
library's static device buffer, against decode_linear_stack with a caller's
workspace.  Both run the same launches, so the outputs must be bitwise equal,
and both are checked against the oracle.  Two calls in a row, the second on
a smaller input, so the second runs over what the first left in the buffer.
Cases: one TP=8 decoder layer, bf16 at M = 8 then 4 (the tile kernel with its
K split and second pass), and FP8 at M = 6 then 1."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import workloads as wl
from gemv_skinny_gemm_amd.synth import gpu as sgpu
from tests.gpu_util import host_codes, need_gpu

pytestmark = pytest.mark.gpu


def _oracle_check(specs, tensors, M, what):
    worst = 0.0
    for s, (x, w, sc, y) in zip(specs, tensors):
        if s.dtype == wl.BF16:
            y_ref, a, _ = oracle.linear_bf16(host_codes(x), host_codes(w))
        else:
            y_ref, a, _ = oracle.linear_fp8_bs128(host_codes(x), w.cpu().numpy(), sc.cpu().numpy())
        ok, wr, idx = oracle.check(y.float().cpu().double().numpy(), y_ref, a)
        assert ok, f"{what} {s.name} M={M}: worst err/bound {wr:.3g} at {idx}"
        worst = max(worst, wr)
    return worst


@pytest.mark.parametrize("dtype,Ms", [(wl.BF16, (8, 4)), (wl.FP8_BS128, (6, 1))])
def test_noalloc_stack_matches_workspace_stack(dtype, Ms):
    need_gpu()
    specs = wl.tp8_layer(dtype)
    runs = []
    for M in Ms:
        sets, tensors = sgpu.materialise(specs, M)
        assert sg.stack_workspace_bytes(sets[0], M) <= sg.STATIC_SCRATCH_BYTES
        runs.append((M, sets[0], tensors[0]))
    # Both calls in a row on the static buffer, the second on the smaller input.
    for M, descs, tensors in runs:
        sg.decode_linear_stack_noalloc(descs, M)
    torch.cuda.synchronize()
    got = [[t[3].clone() for t in tensors] for _, _, tensors in runs]
    for (M, descs, tensors), outs in zip(runs, got):
        for t in tensors:
            t[3].fill_(float("nan"))
        ws = torch.full((sg.stack_workspace_bytes(descs, M),), 0xFF, dtype=torch.uint8,
                        device="cuda")
        sg.decode_linear_stack(descs, M, ws)
        torch.cuda.synchronize()
        for s, t, o in zip(specs, tensors, outs):
            assert torch.equal(o.view(torch.int16), t[3].view(torch.int16)), f"{s.name} M={M}"
        worst = _oracle_check(specs, tensors, M, "noalloc")
        assert worst < 0.5
