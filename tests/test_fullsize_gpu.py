"""The 80-layer Qwen2.5-72B TP=1 decode linear stacks at their real size
(140 GB bf16, 70 GB FP8), in the launch configuration bench.py times, checked
on sampled outputs.

Weights are made on the GPU by the input generator.  For every sampled output
row, the row (and, for FP8, its whole 128-row band with the block scales) is
regenerated on the host from the same counter-based stream and first checked
to be byte-identical to what the GPU holds; the oracle then computes the
sampled outputs one by one and the GPU's outputs must be within the stated
bound 2e-3 * sum|x w| + 1e-6."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import synth, workloads as wl
from tests.gpu_util import host_codes, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.empty_cache()


def _sample(specs, n_lin, rows_per_lin, rng):
    """Linears spread over the stack (every projection type, first and last
    layer) and rows within each (first, last and random)."""
    idx = sorted(set([0, 1, 2, 3, len(specs) - 4, len(specs) - 3, len(specs) - 2,
                      len(specs) - 1] + list(rng.choice(len(specs), n_lin, replace=False))))
    out = []
    for i in idx:
        N = specs[i].N
        rows = sorted(set([0, N - 1] + list(rng.choice(N, rows_per_lin, replace=False))))
        out.append((i, rows))
    return out


def _run_stack(specs, M):
    from gemv_skinny_gemm_amd.synth import gpu as sgpu
    sets, tensors = sgpu.materialise(specs, M)
    descs = sets[0]
    ws = torch.empty(sg.stack_workspace_bytes(descs, M), dtype=torch.uint8, device="cuda")
    sg.decode_linear_stack(descs, M, ws)
    torch.cuda.synchronize()
    return tensors[0]


@pytest.mark.parametrize("M", [1])
def test_tp1_stack_bf16_sampled(M):
    specs = wl.tp1_stack(wl.BF16)
    tensors = _run_stack(specs, M)
    rng = np.random.default_rng(0)
    worst = 0.0
    for i, rows in _sample(specs, 8, 24, rng):
        s = specs[i]
        x_dev, w_dev, _, y_dev = tensors[i]
        x = synth.tensor_bf16(0, s.x_stream, M, s.K, wl.X_SIGMA)
        assert np.array_equal(host_codes(x_dev), x), f"{s.name}: x differs"
        w = synth.tensor_rows_bf16(0, s.w_stream, rows, s.K, wl.W_SIGMA)
        assert np.array_equal(host_codes(w_dev[rows]), w), f"{s.name}: W rows differ"
        y_ref, a, _ = oracle.linear_bf16(x, w)
        y = y_dev[:, rows].float().cpu().double().numpy()
        ok, wr, idx = oracle.check(y, y_ref, a)
        assert ok, f"{s.name}: worst err/bound {wr:.3g} at {idx}"
        worst = max(worst, wr)
    assert worst < 0.5
    del tensors


@pytest.mark.parametrize("M", [1, 6])
def test_tp1_stack_fp8_sampled(M):
    specs = wl.tp1_stack(wl.FP8_BS128)
    tensors = _run_stack(specs, M)
    rng = np.random.default_rng(1)
    worst = 0.0
    for i, rows in _sample(specs, 4, 3, rng):
        s = specs[i]
        x_dev, q_dev, s_dev, y_dev = tensors[i]
        x = synth.tensor_bf16(0, s.x_stream, M, s.K, wl.X_SIGMA)
        assert np.array_equal(host_codes(x_dev), x), f"{s.name}: x differs"
        for band in sorted(set(r // 128 for r in rows)):
            q, sc, r0 = synth.fp8_weight_bs128(0, s.w_stream, s.N, s.K, wl.W_SIGMA, band, 1)
            assert np.array_equal(q_dev[r0:r0 + q.shape[0]].cpu().numpy(), q), f"{s.name}: codes"
            assert np.array_equal(s_dev[band:band + 1].cpu().numpy(), sc), f"{s.name}: scales"
            sel = [r - r0 for r in rows if r // 128 == band]
            # Rows of one band share its scale row, so the selected rows form a
            # valid (shorter) FP8 matrix with the same [1][ceil(K/128)] scales.
            y_ref, a, _ = oracle.linear_fp8_bs128(x, np.ascontiguousarray(q[sel]), sc)
            y = y_dev[:, [r0 + r for r in sel]].float().cpu().double().numpy()
            ok, wr, idx = oracle.check(y, y_ref, a)
            assert ok, f"{s.name} band {band}: worst err/bound {wr:.3g} at {idx}"
            worst = max(worst, wr)
    assert worst < 0.5
    del tensors



@pytest.mark.parametrize("M", [2, 16])
def test_fp8_large_workgroup_sampled(M):
    """One FP8 linear of 262144 x 8192 (2 GB): enough 128-row groups per CU for
    the 8-wave tile workgroup, K-chunks from parallelism (M = 2) and from the
    x window (M = 16, with the second pass); sampled rows as above."""
    spec = wl.LinearSpec("wide-fp8", 262144, 8192, wl.FP8_BS128,
                         synth.stream_id("wide-fp8", "w"), synth.stream_id("wide-fp8", M, "x"))
    tensors = _run_stack([spec], M)
    x_dev, q_dev, s_dev, y_dev = tensors[0]
    x = synth.tensor_bf16(0, spec.x_stream, M, spec.K, wl.X_SIGMA)
    assert np.array_equal(host_codes(x_dev), x)
    rng = np.random.default_rng(M)
    worst = 0.0
    for band in sorted(set([0, 2047] + list(rng.choice(2048, 6, replace=False)))):
        q, sc, r0 = synth.fp8_weight_bs128(0, spec.w_stream, spec.N, spec.K, wl.W_SIGMA, band, 1)
        assert np.array_equal(q_dev[r0:r0 + 128].cpu().numpy(), q)
        assert np.array_equal(s_dev[band:band + 1].cpu().numpy(), sc)
        y_ref, a, _ = oracle.linear_fp8_bs128(x, q, sc)
        ok, wr, idx = oracle.check(y_dev[:, r0:r0 + 128].float().cpu().double().numpy(), y_ref, a)
        assert ok, f"band {band}: worst err/bound {wr:.3g} at {idx}"
        worst = max(worst, wr)
    assert worst < 0.5
    del tensors


@pytest.mark.parametrize("dtype,M,K", [(wl.BF16, 6, 4096), (wl.BF16, 16, 2048),
                                       (wl.FP8_BS128, 16, 4096)])
def test_window_walk_sampled(dtype, M, K):
    """One linear of 524288 rows: its row groups alone give every tile
    workgroup 16 units (no K split for parallelism), and the x window of
    M + 1 token rows holds half of K, so from M = 5 (bf16) or 9 (FP8) tokens
    on each unit walks its two x windows with the sums in registers (no
    partial sums, no second pass); FP8 on the 8-wave workgroup.  Sampled rows
    against the oracle as above."""
    N = 524288
    tag = f"walk-{dtype}-{M}-{K}"
    spec = wl.LinearSpec(tag, N, K, dtype, synth.stream_id(tag, "w"), synth.stream_id(tag, "x"))
    tensors = _run_stack([spec], M)
    x_dev, w_dev, s_dev, y_dev = tensors[0]
    x = synth.tensor_bf16(0, spec.x_stream, M, K, wl.X_SIGMA)
    assert np.array_equal(host_codes(x_dev), x)
    rng = np.random.default_rng(M)
    worst = 0.0
    if dtype == wl.BF16:
        rows = sorted(set([0, 63, 64, N - 1] + list(rng.choice(N, 60, replace=False))))
        w = synth.tensor_rows_bf16(0, spec.w_stream, rows, K, wl.W_SIGMA)
        assert np.array_equal(host_codes(w_dev[rows]), w)
        y_ref, a, _ = oracle.linear_bf16(x, w)
        ok, worst, idx = oracle.check(y_dev[:, rows].float().cpu().double().numpy(), y_ref, a)
        assert ok, f"worst err/bound {worst:.3g} at {idx}"
    else:
        for band in sorted(set([0, N // 128 - 1] + list(rng.choice(N // 128, 4, replace=False)))):
            q, sc, r0 = synth.fp8_weight_bs128(0, spec.w_stream, N, K, wl.W_SIGMA, band, 1)
            assert np.array_equal(w_dev[r0:r0 + 128].cpu().numpy(), q)
            assert np.array_equal(s_dev[band:band + 1].cpu().numpy(), sc)
            y_ref, a, _ = oracle.linear_fp8_bs128(x, q, sc)
            ok, wr, idx = oracle.check(y_dev[:, r0:r0 + 128].float().cpu().double().numpy(), y_ref, a)
            assert ok, f"band {band}: worst err/bound {wr:.3g} at {idx}"
            worst = max(worst, wr)
    assert worst < 0.5
    del tensors
