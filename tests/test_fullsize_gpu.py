"""The 80-layer Qwen2.5-72B TP=1 decode linear stacks at their real size
(140 GB bf16, 70 GB FP8), in the launch configuration bench.py times.

Weights are made on the GPU by the input generator.  For sampled rows of every
checked linear (FP8: whole 128-row bands with their block scales) the host
regenerates the data from the same counter-based stream and first checks it
is byte-identical to what the GPU holds; the linear's weights are then copied
back from the device and the oracle computes its outputs.  Checked against the
oracle: every output of the first and the last eight layers (32 linears each,
layers 0-7 and 72-79), and in every other block of eight layers one whole
layer plus one full 128-row band of each of its other linears.  The whole
stack of each dtype runs as one launch."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import synth, workloads as wl
from tests.gpu_util import host_codes, need_gpu

pytestmark = pytest.mark.gpu

BLOCK = 32                  # linears of eight layers


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.empty_cache()


def _run_stack(specs, M):
    from gemv_skinny_gemm_amd.synth import gpu as sgpu
    sets, tensors = sgpu.materialise(specs, M)
    descs = sets[0]
    ws = torch.empty(sg.stack_workspace_bytes(descs, M), dtype=torch.uint8, device="cuda")
    sg.decode_linear_stack(descs, M, ws)
    torch.cuda.synchronize()
    return tensors[0]


def _plan(n_linears, rng):
    """(linear, rows) to check: None = every row, else the start of a 128-row
    band.  All of the first and last block of eight layers; in each other
    block one whole layer (4 linears) and one band of each of its other
    linears."""
    blocks = (n_linears + BLOCK - 1) // BLOCK
    out = []
    for g in range(blocks):
        lins = range(g * BLOCK, min((g + 1) * BLOCK, n_linears))
        if g in (0, blocks - 1):
            out += [(i, None) for i in lins]
            continue
        layer = int(rng.choice(len(lins) // 4))
        whole = set(lins[4 * layer:4 * layer + 4])
        out += [(i, None if i in whole else -1) for i in lins]
    return out


def _generator_check_bf16(s, x_dev, w_dev, M, rng):
    x = synth.tensor_bf16(0, s.x_stream, M, s.K, wl.X_SIGMA)
    assert np.array_equal(host_codes(x_dev), x), f"{s.name}: x differs"
    rows = sorted(set([0, s.N - 1] + list(rng.choice(s.N, 6, replace=False))))
    w = synth.tensor_rows_bf16(0, s.w_stream, rows, s.K, wl.W_SIGMA)
    assert np.array_equal(host_codes(w_dev[rows]), w), f"{s.name}: W rows differ"
    return x


def _generator_check_fp8(s, x_dev, q_dev, s_dev, M, bands):
    x = synth.tensor_bf16(0, s.x_stream, M, s.K, wl.X_SIGMA)
    assert np.array_equal(host_codes(x_dev), x), f"{s.name}: x differs"
    for band in bands:
        q, sc, r0 = synth.fp8_weight_bs128(0, s.w_stream, s.N, s.K, wl.W_SIGMA, band, 1)
        assert np.array_equal(q_dev[r0:r0 + q.shape[0]].cpu().numpy(), q), f"{s.name}: codes"
        assert np.array_equal(s_dev[band:band + 1].cpu().numpy(), sc), f"{s.name}: scales"
    return x


@pytest.mark.parametrize("M", [1])
def test_tp1_stack_bf16(M):
    specs = wl.tp1_stack(wl.BF16)
    tensors = _run_stack(specs, M)
    rng = np.random.default_rng(0)
    worst, outputs = 0.0, 0
    for i, band in _plan(len(specs), rng):
        s = specs[i]
        x_dev, w_dev, _, y_dev = tensors[i]
        x = _generator_check_bf16(s, x_dev, w_dev, M, rng)
        if band is None:
            r0, r1 = 0, s.N
        else:
            r0 = 128 * int(rng.integers(0, (s.N + 127) // 128))
            r1 = min(r0 + 128, s.N)
        w = host_codes(w_dev[r0:r1])
        y_ref, a, _ = oracle.linear_bf16(x, w)
        ok, wr, idx = oracle.check(y_dev[:, r0:r1].float().cpu().double().numpy(), y_ref, a)
        assert ok, f"{s.name} rows {r0}-{r1}: worst err/bound {wr:.3g} at {idx}"
        worst = max(worst, wr)
        outputs += M * (r1 - r0)
    print(f"bf16 M={M}: {outputs} outputs checked, worst err/bound {worst:.4f}", flush=True)
    assert worst < 0.5
    del tensors


@pytest.mark.parametrize("M", [1, 6])
def test_tp1_stack_fp8(M):
    specs = wl.tp1_stack(wl.FP8_BS128)
    tensors = _run_stack(specs, M)
    rng = np.random.default_rng(1)
    worst, outputs = 0.0, 0
    for i, band in _plan(len(specs), rng):
        s = specs[i]
        x_dev, q_dev, s_dev, y_dev = tensors[i]
        nb = (s.N + 127) // 128
        # Regenerating an FP8 band on the host takes ~0.2 s: one band of each
        # linear checked whole, x of every linear.
        if band is None:
            b0, b1 = 0, nb
            check_bands = [int(rng.integers(0, nb))]
        else:
            b0 = int(rng.integers(0, nb))
            b1 = b0 + 1
            check_bands = []
        x = _generator_check_fp8(s, x_dev, q_dev, s_dev, M, check_bands)
        r0, r1 = 128 * b0, min(128 * b1, s.N)
        q = q_dev[r0:r1].cpu().numpy()
        sc = s_dev[b0:b1].cpu().numpy()
        y_ref, a, _ = oracle.linear_fp8_bs128(x, q, sc)
        ok, wr, idx = oracle.check(y_dev[:, r0:r1].float().cpu().double().numpy(), y_ref, a)
        assert ok, f"{s.name} rows {r0}-{r1}: worst err/bound {wr:.3g} at {idx}"
        worst = max(worst, wr)
        outputs += M * (r1 - r0)
    print(f"fp8 M={M}: {outputs} outputs checked, worst err/bound {worst:.4f}", flush=True)
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
    M + 1 token rows holds half of K, so from M = 5 (bf16) or 4 (FP8, on the
    8-wave workgroup) tokens on each unit walks its two x windows with the
    sums in registers (no partial sums, no second pass).  Sampled rows
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
