"""Launches of more linears than the kernel arguments hold: their descriptors
go in a table copied into the workspace ahead of the launch, and every
linear of one dtype runs in one launch.  Against the fp64 oracle: ragged
shapes in both dtypes, automatic and forced variants and grids (K split with
its second pass reading the table too), bf16 and FP8 linears interleaved (one
launch per dtype), the allocation-free entry point on the same linears (its
launches keep to the kernel arguments), repeated calls bitwise equal, and a
stream under graph capture (launches of kernel-argument size, replayed)."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import synth
from tests.gpu_util import assert_matches_oracle, dev_bf16, dev_f32, dev_u8, need_gpu, out

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _shapes(n, dtype, seed):
    rng = np.random.default_rng(seed)
    step = 16 if dtype == sg.FP8_BS128 else 8
    Ns = rng.integers(1, 700, n)
    Ks = (rng.integers(1, 2600 // step, n) * step).astype(int)
    return [(int(N), int(K)) for N, K in zip(Ns, Ks)]


def _build(shapes, dtypes, M, tag):
    """Device tensors, descriptors and oracle references of one stack."""
    descs, outs, refs = [], [], []
    keep = []
    for i, ((N, K), dt) in enumerate(zip(shapes, dtypes)):
        x = synth.tensor_bf16(0, synth.stream_id(tag, "x", i), M, K, 1.0)
        if dt == sg.BF16:
            w = synth.tensor_bf16(0, synth.stream_id(tag, "w", i), N, K, 0.02)
            refs.append(oracle.linear_bf16(x, w))
            xd, wd, yd = dev_bf16(x), dev_bf16(w), out(M, N)
            descs.append(sg.make_linear(xd, wd, yd))
            keep.append((xd, wd))
        else:
            q, s, _ = synth.fp8_weight_bs128(0, synth.stream_id(tag, "q", i), N, K)
            refs.append(oracle.linear_fp8_bs128(x, q, s))
            xd, qd, sd, yd = dev_bf16(x), dev_u8(q), dev_f32(s), out(M, N)
            descs.append(sg.make_linear(xd, qd, yd, w_scale=sd))
            keep.append((xd, qd, sd))
        outs.append(yd)
    return descs, outs, refs, keep


def _check(outs, refs, what):
    worst = 0.0
    for i, (yd, (y_ref, a, _)) in enumerate(zip(outs, refs)):
        worst = max(worst, assert_matches_oracle(yd, y_ref, a, f"{what} linear {i}"))
    return worst


@pytest.mark.parametrize("dtype", [sg.BF16, sg.FP8_BS128])
@pytest.mark.parametrize("M", [1, 3, 6, 16])
def test_table_stack_vs_oracle(dtype, M):
    n = 48
    shapes = _shapes(n, dtype, 100 + M)
    descs, outs, refs, keep = _build(shapes, [dtype] * n, M, f"tbl-{dtype}-{M}")
    assert sg.launch_count(descs) == 1
    ws = torch.empty(sg.stack_workspace_bytes(descs, M), dtype=torch.uint8, device="cuda")
    sg.decode_linear_stack(descs, M, ws)
    torch.cuda.synchronize()
    _check(outs, refs, f"auto M={M}")
    first = [y.clone() for y in outs]
    sg.decode_linear_stack(descs, M, ws)
    torch.cuda.synchronize()
    for y0, y1 in zip(first, outs):
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    variants = [sg.VARIANT_MFMA] + ([sg.VARIANT_VECTOR] if M <= 8 else [])
    for var in variants:
        for waves in (0, 64, 2048):              # small grids split K: partial sums, second pass
            for y in outs:
                y.fill_(float("nan"))
            sg.linear_run(descs, M, ws, variant=var, waves=waves)
            torch.cuda.synchronize()
            _check(outs, refs, f"variant={var} waves={waves} M={M}")


@pytest.mark.parametrize("M", [1, 6])
def test_table_stack_mixed_dtypes_and_noalloc(M):
    n = 70
    rng = np.random.default_rng(7 + M)
    dtypes = [sg.BF16 if b else sg.FP8_BS128 for b in rng.integers(0, 2, n)]
    shapes = [_shapes(1, dt, 1000 + i)[0] for i, dt in enumerate(dtypes)]
    descs, outs, refs, keep = _build(shapes, dtypes, M, f"tblmix-{M}")
    assert sg.launch_count(descs) == 2
    ws = torch.empty(sg.stack_workspace_bytes(descs, M), dtype=torch.uint8, device="cuda")
    sg.decode_linear_stack(descs, M, ws)
    torch.cuda.synchronize()
    _check(outs, refs, f"mixed M={M}")
    for y in outs:
        y.fill_(float("nan"))
    sg.decode_linear_stack_noalloc(descs, M)
    torch.cuda.synchronize()
    _check(outs, refs, f"noalloc M={M}")


@pytest.mark.parametrize("M,variant", [(1, sg.VARIANT_VECTOR), (8, sg.VARIANT_MFMA)])
def test_table_stack_under_graph_capture(M, variant):
    """Under capture the call keeps to launches of kernel-argument size (a
    table copy in a graph would read this call's host memory at every
    replay); every replay, with new inputs written in place between replays,
    matches the oracle on those inputs."""
    n = 40
    shapes = _shapes(n, sg.BF16, 300 + M)
    descs, outs, refs, keep = _build(shapes, [sg.BF16] * n, M, f"tblg-{M}")
    ws = torch.empty(sg.stack_workspace_bytes(descs, M), dtype=torch.uint8, device="cuda")
    call = lambda: sg.linear_run(descs, M, ws, variant=variant)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        new_refs = []
        for i, (N, K) in enumerate(shapes):
            x = synth.tensor_bf16(r + 1, synth.stream_id("tblg-x", M, i), M, K, 1.0)
            keep[i][0].copy_(dev_bf16(x))
            w = keep[i][1].cpu().view(torch.int16).numpy().view(np.uint16)
            new_refs.append(oracle.linear_bf16(x, w))
        for y in outs:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check(outs, new_refs, f"replay {r} M={M}")
