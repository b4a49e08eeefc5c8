"""The library's calls captured in a HIP graph (through torch.cuda.CUDAGraph)
and replayed: every replay, with the inputs changed in place by ordinary
eager work between replays, gives the same bytes as the eager call on the
same inputs.  The path records no memset and allocates nothing, so a caller
can capture a decode step once and replay it."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
from gemv_skinny_gemm_amd import synth, workloads as wl
from gemv_skinny_gemm_amd.synth import gpu as sgpu
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _check_replays(call, xs, outs, replays=3):
    """call() enqueues the work on the current stream; xs are its input
    tensors (changed in place between replays), outs its outputs."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(5)
    for r in range(replays):
        for x in xs:                                # eager work between replays
            x.copy_((torch.randn(x.shape, generator=gen, device="cuda")).to(x.dtype))
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        for o in outs:
            o.fill_(float("nan"))
        call()                                      # eager on the same inputs
        torch.cuda.synchronize()
        for a, b in zip(got, outs):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {r} differs"


@pytest.mark.parametrize("M", [1, 8])
def test_tp8_layer_graph(M):
    """Row kernel (M = 1) and tile kernel with its second pass (M = 8)."""
    specs = wl.tp8_layer(wl.BF16)
    sets, tensors = sgpu.materialise(specs, M)
    ws = torch.empty(sg.stack_workspace_bytes(sets[0], M), dtype=torch.uint8, device="cuda")
    _check_replays(lambda: sg.decode_linear_stack(sets[0], M, ws),
                   [t[0] for t in tensors[0]], [t[3] for t in tensors[0]])


def test_mlp_graph():
    specs = wl.mlp(8, wl.FP8_BS128)
    M = 6
    sets, tensors = sgpu.materialise(specs, M)
    t = tensors[0]
    mlp = sg.make_mlp(t[0][0], t[0][1], t[1][1], t[1][3], t[0][2], t[1][2])
    ws = torch.empty(sg.mlp_workspace_bytes(mlp, M), dtype=torch.uint8, device="cuda")
    _check_replays(lambda: sg.mlp_swiglu(mlp, M, ws), [t[0][0]], [t[1][3]])


@pytest.mark.parametrize("T", [1, 6])
def test_moe_graph(T):
    """MoE (one token: the row kernel's form; six: the tile kernel's): the
    routing is read on the device, so new router choices written between
    replays are honoured by the captured launch."""
    E, N, K, topk = 8, 512, 2048, 2
    w = synth.tensor_bf16(0, 901, E * N, K, 0.02)
    wd = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda().view(E, N, K)
    ex = sg.make_experts(wd)
    want = sg.VARIANT_VECTOR if T == 1 else sg.VARIANT_MFMA
    assert sg.moe_plan_query(ex, T, topk).variant == want
    x = torch.zeros((T, K), dtype=torch.bfloat16, device="cuda")
    ids = torch.from_numpy(synth.route_topk(0, 902, T, E, topk)).cuda()
    y = torch.empty((T * topk, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(sg.moe_workspace_bytes(ex, T, topk), dtype=torch.uint8, device="cuda")
    routes = [torch.from_numpy(synth.route_topk(0, 903 + r, T, E, topk)).cuda() for r in range(3)]

    def call():
        sg.moe_linear(ex, x, ids, y, ws)

    _check_replays(call, [x], [y])
    # New routes between replays: replay against eager with each routing.
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        call()
    for r in routes:
        ids.copy_(r)
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        call()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), y.view(torch.int16))
