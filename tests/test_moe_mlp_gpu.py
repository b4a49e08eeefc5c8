"""The experts' gated MLP through skinny_moe_mlp_swiglu against the fp64
oracle's chain (gate_up per route, then down reading the GPU's own bf16
gate_up outputs through the SiLU-gated product, as the chained layer does):
the one-token launch (verify-step shape, random shapes with dead and
duplicate routes, repeated calls, graph replay, a wait that gives up) and the
two-launch form (several tokens, mixed dtypes)."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import synth, workloads as wl
from tests.gpu_util import dev_bf16, dev_f32, dev_u8, need_gpu
from tests.test_moe_gpu import check, experts_bf16, experts_fp8, x_for

pytestmark = pytest.mark.gpu

CTR_BYTES = sg.MOE_MLP_COUNTER_BYTES
DEFAULT_SPIN = 1 << 22


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    sg.moe_mlp_set_spin_limit(DEFAULT_SPIN)


def experts(tag, dtype, E, N, K, sigma=0.05):
    if dtype == sg.BF16:
        w = experts_bf16(tag, E, N, K, sigma)
        dev = (dev_bf16(w.reshape(-1, K)).view(E, N, K),)
        return w, None, dev, sg.make_experts(dev[0])
    q, s = experts_fp8(tag, E, N, K, sigma)
    dev = (dev_u8(q), dev_f32(s))
    return q, s, dev, sg.make_experts(*dev)


def gate_up_outputs(ws, exg, exd, T, topk, N1):
    """The gate_up outputs the call left in its workspace: bf16 rows (two
    launches) or 64-bit words of a call number above two bf16 (one launch)."""
    body = ws[CTR_BYTES:]
    if sg.moe_mlp_plan_query(exg, exd, T, topk).kernel == 7:
        words = body[:T * topk * N1 * 4].view(torch.int32).view(T * topk, N1 // 2, 2)
        return words[:, :, 0].contiguous().view(torch.bfloat16).view(T * topk, N1).clone()
    return body[:T * topk * N1 * 2].view(torch.bfloat16).view(T * topk, N1).clone()


class Mlp:
    """Host and device copies of one MoE MLP's experts."""

    def __init__(self, tag, dt_gu, dt_dn, E, I, H, sigma=0.05):
        self.g = experts(tag + "-gu", dt_gu, E, 2 * I, H, sigma)
        self.d = experts(tag + "-dn", dt_dn, E, H, I, sigma)
        self.E, self.I, self.H = E, I, H

    def run(self, x, ids, reps=1, ws=None):
        T, topk = ids.shape
        xd = dev_bf16(x)
        idd = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
        exg, exd = self.g[3], self.d[3]
        if ws is None:
            ws = torch.zeros(sg.moe_mlp_workspace_bytes(exg, exd, T, topk), dtype=torch.uint8,
                             device="cuda")
        ys = []
        for _ in range(reps):
            y = torch.full((T * topk, self.H), float("nan"), dtype=torch.bfloat16, device="cuda")
            sg.moe_mlp_swiglu(exg, exd, xd, idd, y, ws)
            ys.append(y)
        torch.cuda.synchronize()
        return ys, gate_up_outputs(ws, exg, exd, T, topk, 2 * self.I), ws

    def check(self, x, ids, y, gu, what):
        """gate_up of the valid routes against the oracle, then down from the
        GPU's own gate_up outputs; every output row."""
        valid = (ids.ravel() >= 0) & (ids.ravel() < self.E)
        g_ref, ga = oracle.moe_linear(x, ids, self.g[0], scales=self.g[1])
        worst = 0.0
        if valid.any():
            worst = check(gu[torch.from_numpy(valid).cuda()], g_ref[valid], ga[valid],
                          f"{what} gate_up")
        h = gu.cpu().view(torch.int16).numpy().view(np.uint16)
        d_ref, da = oracle.moe_linear(h, ids, self.d[0], scales=self.d[1], x_per_route=True,
                                      swiglu=True)
        return max(worst, check(y, d_ref, da, f"{what} down"))


@pytest.mark.parametrize("dtype", [sg.BF16, sg.FP8_BS128])
def test_verify_step_one_launch(dtype):
    """The synthetic verify step at one token (8 experts, top 2, hidden 4096,
    expert width 1536) in one launch: every output against the stated bound,
    three calls on one workspace bitwise equal, the workgroup count grown by
    exactly the grid per call and no wait given up."""
    gu_spec, dn_spec = wl.moe_experts(dtype)
    E, H, I = wl.MOE_EXPERTS, gu_spec.K, dn_spec.K
    mlp = Mlp("v1", dtype, dtype, E, I, H, 0.02)
    ids = synth.route_topk(0, synth.stream_id("moe-mlp", 1), 1, E, wl.MOE_TOPK)
    x = x_for("mlp-v1", 1, H)
    plan = sg.moe_mlp_plan_query(mlp.g[3], mlp.d[3], 1, wl.MOE_TOPK)
    assert sg.KERNEL_NAMES[plan.kernel] == "skinny_moe_mlp1"
    ys, gu, ws = mlp.run(x, ids, reps=3)
    worst = mlp.check(x, ids, ys[0], gu, f"verify {dtype}")
    assert worst < 0.5
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    assert int(ws[:8].view(torch.int64)[0]) == 3 * (plan.waves // 8)
    assert not sg.moe_mlp_gave_up(ws)


def _random_cases(n=24, seed=91):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = [sg.BF16, sg.FP8_BS128][int(rng.integers(2))]
        E = int(rng.integers(1, 13))
        topk = int(rng.integers(1, 9)) if i % 6 else 16
        I = int(rng.integers(4, 97)) * 16
        H = int(rng.integers(4, 257)) * 16
        out.append((i, dtype, E, topk, I, H))
    return out


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: "r%d" % c[0])
def test_random_one_token(case):
    """One token, random shapes (ragged rows, segments and scale blocks),
    ids outside [0, E) and duplicates."""
    i, dtype, E, topk, I, H = case
    mlp = Mlp(f"r{i}", dtype, dtype, E, I, H)
    rng = np.random.default_rng(500 + i)
    ids = rng.integers(-1, E + 1, (1, topk)).astype(np.int32)
    x = x_for(f"mlp-r{i}", 1, H)
    ys, gu, _ = mlp.run(x, ids)
    mlp.check(x, ids, ys[0], gu, f"case {i}: {dtype} E={E} topk={topk} I={I} H={H}")


@pytest.mark.parametrize("T", [2, 6])
@pytest.mark.parametrize("dtype", [sg.BF16, sg.FP8_BS128])
def test_several_tokens_two_launches(dtype, T):
    E, I, H = 6, 384, 1040
    mlp = Mlp(f"t{T}", dtype, dtype, E, I, H)
    ids = synth.route_topk(0, synth.stream_id("moe-mlp", T), T, E, 2)
    ids[0, 1] = E                                          # a dead route
    assert sg.moe_mlp_plan_query(mlp.g[3], mlp.d[3], T, 2).kernel != 7
    x = x_for(f"mlp-t{T}", T, H)
    ys, gu, _ = mlp.run(x, ids)
    mlp.check(x, ids, ys[0], gu, f"{dtype} T={T}")


def test_mixed_dtypes_two_launches():
    E, I, H = 4, 256, 768
    mlp = Mlp("mixed", sg.FP8_BS128, sg.BF16, E, I, H)
    ids = np.array([[3, 0, 1]], np.int32)
    assert sg.moe_mlp_plan_query(mlp.g[3], mlp.d[3], 1, 3).kernel != 7
    x = x_for("mlp-mixed", 1, H)
    ys, gu, _ = mlp.run(x, ids)
    mlp.check(x, ids, ys[0], gu, "fp8 gate_up, bf16 down")


def test_graph_replay():
    """The one-token launch captured once and replayed with new inputs (and
    eager work in between): every replay matches an eager call."""
    E, I, H = 8, 512, 2048
    mlp = Mlp("graph", sg.FP8_BS128, sg.FP8_BS128, E, I, H)
    exg, exd = mlp.g[3], mlp.d[3]
    ids = torch.tensor([[5, 2]], dtype=torch.int32, device="cuda")
    xs = [dev_bf16(x_for(f"mlp-g{k}", 1, H)) for k in range(3)]
    x = xs[0].clone()
    y = torch.empty(2, H, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(sg.moe_mlp_workspace_bytes(exg, exd, 1, 2), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        sg.moe_mlp_swiglu(exg, exd, x, ids, y, ws)            # warm-up outside the graph
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        sg.moe_mlp_swiglu(exg, exd, x, ids, y, ws)
    ref_ws = torch.zeros_like(ws)
    for k in range(3):
        x.copy_(xs[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = torch.empty_like(y)
        sg.moe_mlp_swiglu(exg, exd, xs[k], ids, ref, ref_ws)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"replay {k}"
    assert not sg.moe_mlp_gave_up(ws)


def test_wait_that_gives_up_returns():
    """A wait forced to give up (spin limit < 0, set from the host) ends the
    launch with counter word 2 set instead of hanging; with the limit back,
    the next call on that workspace (word 2 cleared) is correct again."""
    E, I, H = 4, 256, 1024
    mlp = Mlp("giveup", sg.BF16, sg.BF16, E, I, H)
    ids = np.array([[1, 3]], np.int32)
    plan = sg.moe_mlp_plan_query(mlp.g[3], mlp.d[3], 1, 2)
    assert plan.kernel == 7
    x = x_for("mlp-giveup", 1, H)
    sg.moe_mlp_set_spin_limit(-1)
    _, _, ws = mlp.run(x, ids)
    assert sg.moe_mlp_gave_up(ws)
    assert int(ws[:8].view(torch.int64)[0]) == plan.waves // 8
    sg.moe_mlp_set_spin_limit(DEFAULT_SPIN)
    ws[8:12].zero_()
    ys, gu, ws = mlp.run(x, ids, ws=ws)
    assert not sg.moe_mlp_gave_up(ws)
    mlp.check(x, ids, ys[0], gu, "after a wait gave up")
