"""Mixture-of-experts linear through skinny_moe_linear against the fp64
oracle's route-by-route definition: routing found on the device from ids
(duplicates, unused experts, ids outside [0, E), experts with more routes than
tokens), shared and per-route x, the SwiGLU input, the split-K second pass,
and the synthetic verify-step workload at full size (8 experts, top 2,
hidden 4096, 6 tokens; bf16 and FP8)."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import synth, workloads as wl
from tests.gpu_util import dev_bf16, dev_f32, dev_u8, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def experts_bf16(tag, E, N, K, sigma=0.05):
    return synth.tensor_bf16(0, synth.stream_id("moe", tag, E, N, K), E * N, K, sigma).reshape(E, N, K)


def experts_fp8(tag, E, N, K, sigma=0.05):
    """Each expert quantized on its own (its own 128 x 128 blocks)."""
    qs, ss = [], []
    for e in range(E):
        q, s, _ = synth.fp8_weight_bs128(0, synth.stream_id("moe8", tag, e, N, K), N, K, sigma)
        qs.append(q)
        ss.append(s)
    return np.stack(qs), np.stack(ss)


def run_moe(x, ids, w, scales=None, x_per_route=False, swiglu=False, reps=1):
    xd = dev_bf16(x)
    idd = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    if scales is None:
        keep = (dev_bf16(w.reshape(-1, w.shape[2])).view(w.shape),)
        ex = sg.make_experts(keep[0])
    else:
        keep = (dev_u8(w), dev_f32(scales))
        ex = sg.make_experts(*keep)
    T, topk = ids.shape
    ws = torch.empty(sg.moe_workspace_bytes(ex, T, topk, x_per_route, swiglu), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for _ in range(reps):
        # NaN-filled: a route the kernels never write cannot pass.
        y = torch.full((T * topk, w.shape[1]), float("nan"), dtype=torch.bfloat16, device="cuda")
        sg.moe_linear(ex, xd, idd, y, ws, x_per_route=x_per_route, swiglu=swiglu)
        outs.append(y)
    torch.cuda.synchronize()
    del keep
    return outs if reps > 1 else outs[0]


def check(y, y_ref, a, what):
    ok, worst, idx = oracle.check(y.float().cpu().double().numpy(), y_ref, a)
    assert ok, f"{what}: worst err/bound {worst:.3g} at {idx}"
    return worst


def x_for(tag, rows, K):
    return synth.tensor_bf16(0, synth.stream_id("moe-x", tag, rows, K), rows, K, 1.0)


IRREGULAR_IDS = np.array([[2, 0, 2], [-1, 1, 0], [0, 5, 1], [3, 3, 3]], np.int32)  # E = 5: 4 unused


@pytest.mark.parametrize("x_per_route", [False, True])
def test_small_bf16_irregular_routing(x_per_route):
    E, N, K = 5, 200, 520
    T, topk = IRREGULAR_IDS.shape
    w = experts_bf16("small", E, N, K)
    x = x_for("small", T * topk if x_per_route else T, K)
    y_ref, a = oracle.moe_linear(x, IRREGULAR_IDS, w, x_per_route=x_per_route)
    y = run_moe(x, IRREGULAR_IDS, w, x_per_route=x_per_route)
    check(y, y_ref, a, f"bf16 per_route={x_per_route}")
    dead = [3, 7]                                                      # ids -1 and 5
    assert torch.all(y[dead].float() == 0)


def test_small_fp8_ragged_blocks():
    E, N, K = 4, 300, 1040
    ids = synth.route_topk(0, 401, 6, E, 2)
    q, s = experts_fp8("small", E, N, K)
    x = x_for("small8", 6, K)
    y_ref, a = oracle.moe_linear(x, ids, q, scales=s)
    check(run_moe(x, ids, q, s), y_ref, a, "fp8 ragged")


@pytest.mark.parametrize("dtype", [sg.BF16, sg.FP8_BS128])
def test_swiglu_input_per_route(dtype):
    E, N, I = 4, 256, 1024
    ids = synth.route_topk(0, 402, 5, E, 2)
    gu = x_for("gu", 10, 2 * I)
    if dtype == sg.BF16:
        w, s = experts_bf16("down", E, N, I), None
    else:
        w, s = experts_fp8("down", E, N, I)
    y_ref, a = oracle.moe_linear(gu, ids, w, scales=s, x_per_route=True, swiglu=True)
    check(run_moe(gu, ids, w, s, x_per_route=True, swiglu=True), y_ref, a, f"swiglu {dtype}")


# One- and two-token slices (one token: the row kernel's MoE form, two: the
# tile kernel's): E = 5, so ids 5 and -1 have no expert; N = 200 and
# K = 4112 end inside a row group, a 128 x 128 scale block and a row segment.
ROW_IDS = {1: np.array([[3, 5, 0]], np.int32),
           2: np.array([[2, -1, 4], [4, 2, 2]], np.int32)}


@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("x_per_route", [False, True])
@pytest.mark.parametrize("T", [1, 2])
@pytest.mark.parametrize("dtype", [sg.BF16, sg.FP8_BS128])
def test_one_and_two_token_slices(dtype, T, x_per_route, swiglu):
    E, N, K = 5, 200, 4112
    ids = ROW_IDS[T]
    tag = f"rows{T}{int(x_per_route)}{int(swiglu)}"
    if dtype == sg.BF16:
        w, s = experts_bf16(tag, E, N, K), None
    else:
        w, s = experts_fp8(tag, E, N, K)
    x = x_for(tag, ids.size if x_per_route else T, 2 * K if swiglu else K)
    y_ref, a = oracle.moe_linear(x, ids, w, scales=s, x_per_route=x_per_route, swiglu=swiglu)
    y1, y2 = run_moe(x, ids, w, s, x_per_route=x_per_route, swiglu=swiglu, reps=2)
    check(y1, y_ref, a, f"{dtype} T={T} per_route={x_per_route} swiglu={swiglu}")
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    dead = np.flatnonzero((ids.reshape(-1) < 0) | (ids.reshape(-1) >= E))
    assert torch.all(y1[torch.from_numpy(dead).cuda()].float() == 0)


@pytest.mark.parametrize("dtype", [sg.BF16, sg.FP8_BS128])
def test_one_token_short_and_long_rows(dtype):
    """One token with rows too short for the row kernel (K = 1536, the verify
    step's down shape) and an x row too long for its x window (K = 33024:
    66 KB of bf16): the tile kernel takes both."""
    E, N = 3, 96
    ids = np.array([[2, 0]], np.int32)
    for K in (1536, 33024):
        if dtype == sg.BF16:
            w, s = experts_bf16(f"k{K}", E, N, K, 0.02), None
        else:
            w, s = experts_fp8(f"k{K}", E, N, K, 0.02)
        x = x_for(f"k{K}", 1, K)
        y_ref, a = oracle.moe_linear(x, ids, w, scales=s)
        check(run_moe(x, ids, w, s), y_ref, a, f"K={K} {dtype}")


@pytest.mark.parametrize("swiglu,x_per_route", [(False, False), (False, True), (True, False),
                                                  (True, True)])
@pytest.mark.parametrize("dtype,K", [(sg.BF16, 520), (sg.BF16, 1024), (sg.FP8_BS128, 1040),
                                     (sg.FP8_BS128, 2048)])
def test_one_token_k_split_tiles(dtype, K, swiglu, x_per_route):
    """One token with rows of 2-4 segments of 512 bytes: the tile kernel's
    K-split form, where the workgroup's four waves share each 16-row tile's
    segments (some waves get none) and add their partial tiles in LDS.  N =
    200 ends inside a tile; id 4 names no expert."""
    E, N = 4, 200
    ids = np.array([[3, 4, 1]], np.int32)
    tag = f"ks{K}{int(swiglu)}{int(x_per_route)}"
    if dtype == sg.BF16:
        w, s = experts_bf16(tag, E, N, K), None
    else:
        w, s = experts_fp8(tag, E, N, K)
    x = x_for(tag, ids.size if x_per_route else 1, 2 * K if swiglu else K)
    y_ref, a = oracle.moe_linear(x, ids, w, scales=s, x_per_route=x_per_route, swiglu=swiglu)
    y1, y2 = run_moe(x, ids, w, s, x_per_route=x_per_route, swiglu=swiglu, reps=2)
    check(y1, y_ref, a, f"{dtype} K={K} swiglu={swiglu} per_route={x_per_route}")
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.all(y1[1].float() == 0)


def test_one_expert_takes_more_routes_than_tokens():
    """Duplicates: 8 routes of 2 tokens to expert 1 make 4 slices of it."""
    E, N, K = 3, 128, 512
    ids = np.array([[1, 1, 1, 1], [1, 1, 1, 1]], np.int32)
    w = experts_bf16("dup", E, N, K)
    x = x_for("dup", 8, K)
    y_ref, a = oracle.moe_linear(x, ids, w, x_per_route=True)
    check(run_moe(x, ids, w, x_per_route=True), y_ref, a, "duplicates")


def test_every_route_without_an_expert_gives_zeros():
    E, N, K = 2, 96, 256
    ids = np.array([[-1, 2], [7, -5]], np.int32)
    w = experts_bf16("none", E, N, K)
    y = run_moe(x_for("none", 2, K), ids, w)
    assert torch.all(y.float() == 0)


@pytest.mark.parametrize("dtype", [sg.BF16, sg.FP8_BS128])
def test_split_k_second_pass(dtype):
    """Three row groups and a long K: too few units to occupy the workers,
    so the planner splits K and the slices go through the MoE second pass."""
    E, N, K = 3, 64, 16384
    ids = np.array([[0, 2], [2, 1], [1, 0]], np.int32)
    if dtype == sg.BF16:
        w, s = experts_bf16("split", E, N, K, 0.02), None
    else:
        w, s = experts_fp8("split", E, N, K, 0.02)
    x = x_for("split", 3, K)
    y_ref, a = oracle.moe_linear(x, ids, w, scales=s)
    y1, y2 = run_moe(x, ids, w, s, reps=2)
    check(y1, y_ref, a, f"split {dtype}")
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))    # deterministic


def test_most_routes_many_experts():
    """16 tokens x top 16 = 256 routes over 300 experts (FP8)."""
    E, N, K = 300, 128, 256
    ids = synth.route_topk(0, 403, 16, E, 16, hot=8, hot_bias=1.5)
    q, s = experts_fp8("many", E, N, K)
    x = x_for("many", 16, K)
    y_ref, a = oracle.moe_linear(x, ids, q, scales=s)
    check(run_moe(x, ids, q, s), y_ref, a, "256 routes")


@pytest.mark.parametrize("T", [1, 6, 16])
@pytest.mark.parametrize("dtype", [sg.BF16, sg.FP8_BS128])
def test_verify_step_experts_full_size(dtype, T):
    """The synthetic verify-step MoE at full size: gate_up then down (the
    down reading gate_up's bf16 outputs through the SwiGLU), every route
    against the oracle, against the stated bound.  At 6 and 16 tokens the
    gate_up's x window does not fit the LDS budget in one piece, so each unit
    walks its windows in turn (no K split, no second pass)."""
    (gu_spec, dn_spec) = wl.moe_experts(dtype)
    ids = synth.route_topk(0, synth.stream_id("moe-full", T), T, wl.MOE_EXPERTS, wl.MOE_TOPK)
    E = wl.MOE_EXPERTS
    if dtype == sg.BF16:
        wg, sgu = experts_bf16("full-gu", E, gu_spec.N // E, gu_spec.K, 0.02), None
        wd, sdn = experts_bf16("full-dn", E, dn_spec.N // E, dn_spec.K, 0.02), None
    else:
        wg, sgu = experts_fp8("full-gu", E, gu_spec.N // E, gu_spec.K, 0.02)
        wd, sdn = experts_fp8("full-dn", E, dn_spec.N // E, dn_spec.K, 0.02)
    x = x_for("full", T, gu_spec.K)
    g_ref, ga = oracle.moe_linear(x, ids, wg, scales=sgu)
    g = run_moe(x, ids, wg, sgu)
    worst = check(g, g_ref, ga, f"gate_up {dtype} T={T}")
    assert worst < 0.5
    # down reads the GPU's own gate_up output, as the chained layer does.
    h = g.cpu().view(torch.int16).numpy().view(np.uint16)
    d_ref, da = oracle.moe_linear(h, ids, wd, scales=sdn, x_per_route=True, swiglu=True)
    d = run_moe(h, ids, wd, sdn, x_per_route=True, swiglu=True)
    worst = check(d, d_ref, da, f"down {dtype} T={T}")
    assert worst < 0.5
