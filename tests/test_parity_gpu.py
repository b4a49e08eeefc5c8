"""GPU path vs the fp64 oracle: element by element on seeded inputs, both
compute variants, forced wave counts (split-K), pins through the GPU, and the
small full-size configurations."""
import json
import os

import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import synth
from tests.gpu_util import (assert_matches_oracle, dev_bf16, host_codes,
                            host_values, need_gpu, out, run_bf16, run_fp8, variants_for,
                            workspace)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BF16_ONE = 0x3F80


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


# --- random inputs: several tiles, ragged tails, every M ------------------------

# K = 20480: an odd number of whole row-kernel batches; K = 3696: ragged row ends.
SHAPES = [(1, 8), (17, 264), (100, 1000), (257, 3696), (1280, 8192), (300, 20480)]


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 8, 16])
@pytest.mark.parametrize("N,K", SHAPES)
def test_bf16_random_vs_oracle(M, N, K):
    x = synth.tensor_bf16(0, synth.stream_id("t-bf16", M, N, K, "x"), M, K, 1.0)
    w = synth.tensor_bf16(0, synth.stream_id("t-bf16", N, K, "w"), N, K, 0.02)
    y_ref, a, _ = oracle.linear_bf16(x, w)
    for var in variants_for(M):
        for waves in (0, 4, 28):           # forced grids: whole workgroups, at least one
            y = run_bf16(x, w, M, N, variant=var, waves=waves)
            assert_matches_oracle(y, y_ref, a, f"bf16 M={M} N={N} K={K} var={var} waves={waves}")


FP8_SHAPES = [(1, 16), (130, 272), (300, 1024), (257, 3696)]


@pytest.mark.parametrize("M", [1, 2, 4, 6, 8, 16])
@pytest.mark.parametrize("N,K", FP8_SHAPES)
def test_fp8_random_vs_oracle(M, N, K):
    x = synth.tensor_bf16(0, synth.stream_id("t-fp8", M, N, K, "x"), M, K, 1.0)
    q, s, _ = synth.fp8_weight_bs128(0, synth.stream_id("t-fp8", N, K, "w"), N, K)
    y_ref, a, _ = oracle.linear_fp8_bs128(x, q, s)
    for var in variants_for(M):
        for waves in (0, 4, 20):
            y = run_fp8(x, q, s, M, N, variant=var, waves=waves)
            assert_matches_oracle(y, y_ref, a, f"fp8 M={M} N={N} K={K} var={var} waves={waves}")


# --- pins through the GPU: exact results --------------------------------------

@pytest.mark.parametrize("M", [1, 4, 16])
def test_identity_is_exact(M):
    K = 256
    x = synth.tensor_bf16(0, 7, M, K, 1.0)
    w = np.zeros((K, K), np.uint16)
    w[np.arange(K), np.arange(K)] = BF16_ONE
    q = np.zeros((K, K), np.uint8)
    q[np.arange(K), np.arange(K)] = 0x38
    s = np.ones((2, 2), np.float32)
    for var in variants_for(M):
        assert np.array_equal(host_codes(run_bf16(x, w, M, K, variant=var)), x)
        assert np.array_equal(host_codes(run_fp8(x, q, s, M, K, variant=var)), x)


def test_permutation_is_exact():
    K, N, M = 512, 300, 3
    perm = np.random.default_rng(5).permutation(K)[:N]
    x = synth.tensor_bf16(0, 8, M, K, 1.0)
    w = np.zeros((N, K), np.uint16)
    w[np.arange(N), perm] = BF16_ONE
    for var in variants_for(M):
        for waves in (0, 12):
            assert np.array_equal(host_codes(run_bf16(x, w, M, N, variant=var, waves=waves)),
                                  x[:, perm])


def test_constant_closed_form():
    K, N, M = 8192, 40, 2
    x = np.full((M, K), 0x3F00, np.uint16)                   # 0.5
    w = np.full((N, K), 0x3E00, np.uint16)                   # 0.125
    q = np.full((N, K), 0x30, np.uint8)                      # 0.5 ...
    s = np.full((1, K // 128), 0.25, np.float32)             # ... x 0.25 = 0.125
    for var in variants_for(M):
        for waves in (0, 4, 52):
            assert np.all(host_values(run_bf16(x, w, M, N, variant=var, waves=waves)) == 512.0)
            assert np.all(host_values(run_fp8(x, q, s, M, N, variant=var, waves=waves)) == 512.0)


def _ex2():
    d = json.load(open(os.path.join(GOLDEN, "p2_ex2_column_split.json")))
    x = np.array(d["x"], np.float64)
    w = np.array(d["w_kn"], np.float64).T
    return d, x, w


def codes_of(v):
    return torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def e4m3_of(v):
    return torch.tensor(v, dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_page_example_column_split():
    d, x, w = _ex2()
    # K = 4 is padded with zeros to the 16-element granularity of the kernels.
    xp = np.zeros((2, 16)); xp[:, :4] = x
    wp = np.zeros((6, 16)); wp[:, :4] = w
    for var in variants_for(2):
        assert host_values(run_bf16(codes_of(xp), codes_of(wp), 2, 6, variant=var)).tolist() \
            == d["y_printed"]
        assert host_values(run_fp8(codes_of(xp), e4m3_of(wp), np.ones((1, 1), np.float32), 2, 6,
                                   variant=var)).tolist() == d["y_printed"]
        y0 = run_bf16(codes_of(xp), codes_of(wp[:3]), 2, 3, variant=var)
        assert host_values(y0).tolist() == d["device0_printed"]


def test_page_example_split_k_partials_in_workspace():
    """The page's MLP example split over K into two halves that land in two
    different K-chunks of the split-K pass: each chunk's partial slot holds the
    printed partial and the second pass writes the printed sum."""
    d = json.load(open(os.path.join(GOLDEN, "p2_ex3_mlp_split.json")))
    x = np.array(d["x"], np.float64)
    a_m = np.array([[((8 * i + j) % 7) - 3 for j in range(8)] for i in range(4)], np.float64)
    b_m = np.array([[((4 * i + j) % 5) - 2 for j in range(4)] for i in range(8)], np.float64)
    h = np.maximum(x @ a_m, 0.0)                 # inputs of the second product (integers)
    # x of two tokens over K = 32768 is larger than either kernel's LDS window,
    # so both cut K into chunks and the halves, K / 2 apart, land in different ones.
    K = 32768
    hp = np.zeros((2, K)); hp[:, 0:4] = h[:, 0:4]; hp[:, K // 2:K // 2 + 4] = h[:, 4:8]
    wp = np.zeros((4, K)); wp[:, 0:4] = b_m[0:4].T; wp[:, K // 2:K // 2 + 4] = b_m[4:8].T
    for var in variants_for(2):
        ws = workspace(2, 4, K)
        ws.zero_()
        y = run_bf16(codes_of(hp), codes_of(wp), 2, 4, variant=var, ws=ws)
        assert host_values(y).tolist() == d["sum_printed"]
        slots = ws.view(torch.float32).cpu().numpy()
        # Slots [slot][M][band rows]; only the two slots whose K range holds
        # k = 0..3 or k = 4096..4099 are nonzero, in K order.
        R = sg.band_rows(sg.BF16, var, 2)
        n = min(slots.size // (2 * R), 4096)
        per = slots[:n * 2 * R].reshape(n, 2, R)
        nz = [c for c in range(n) if np.any(per[c] != 0)]
        assert len(nz) == 2, nz
        p0, p1 = per[nz[0]][:, :4], per[nz[1]][:, :4]
        assert p0.tolist() == d["partial0_printed"]
        assert p1.tolist() == d["partial1_printed"]


@pytest.mark.parametrize("M", [1, 6, 16])
def test_linearity_power_of_two(M):
    N, K = 300, 2048
    x = synth.tensor_bf16(0, 31, M, K, 1.0)
    w = synth.tensor_bf16(0, 32, N, K, 0.02)
    x4 = codes_of(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy() * 4)
    for var in variants_for(M):
        y1 = host_values(run_bf16(x, w, M, N, variant=var))
        y4 = host_values(run_bf16(x4, w, M, N, variant=var))
        assert np.array_equal(y4, 4 * y1)


# --- determinism and split agreement -----------------------------------------

@pytest.mark.parametrize("M", [1, 8])
def test_bitwise_repeatable_and_splits_agree(M):
    N, K = 1280, 8192
    x = synth.tensor_bf16(0, 41, M, K, 1.0)
    w = synth.tensor_bf16(0, 42, N, K, 0.02)
    y_ref, a, _ = oracle.linear_bf16(x, w)
    for var in variants_for(M):
        first = host_codes(run_bf16(x, w, M, N, variant=var))
        for _ in range(3):
            assert np.array_equal(host_codes(run_bf16(x, w, M, N, variant=var)), first)
        for waves in (4, 8, 80, 1000, 8192):
            y = run_bf16(x, w, M, N, variant=var, waves=waves)
            assert_matches_oracle(y, y_ref, a, f"waves={waves}")


@pytest.mark.parametrize("K,waves", [(8192, 4), (8192, 12), (29568, 4), (29568, 48)])
def test_fp8_window_set_chunk_counts(K, waves):
    """M = 6: the x window sets 3 K-chunks at K = 8192 and 12 at K = 29568 (3 x
    2^k counts) once a small forced grid asks for little parallelism; grids of
    1, 3 and 12 workgroups, the first not divisible by the count (its units
    then change K-chunk, and x window, every time)."""
    M, N = 6, 200
    x = synth.tensor_bf16(0, synth.stream_id("w3", K, "x"), M, K, 1.0)
    w = synth.tensor_bf16(0, synth.stream_id("w3", K, "w"), N, K, 0.02)
    q, s = synth.quantize_bs128(w)
    y_ref, a, _ = oracle.linear_fp8_bs128(x, q, s)
    y = run_fp8(x, q, s, M, N, variant=sg.VARIANT_MFMA, waves=waves)
    assert_matches_oracle(y, y_ref, a, f"fp8 M={M} K={K} waves={waves}")


# --- configurations at their real sizes ----------------------------------------

def test_qkv_tp8_gemv_seed0():
    """y[1 x 1280] = x[1 x 8192] . W^T, W ~ N(0, 0.02), x ~ N(0, 1), seed 0."""
    from gemv_skinny_gemm_amd import workloads
    lin = workloads.qkv_tp8_gemv()[0]
    x = synth.tensor_bf16(0, lin.x_stream, 1, lin.K, 1.0)
    w = synth.tensor_bf16(0, lin.w_stream, lin.N, lin.K, 0.02)
    y_ref, a, _ = oracle.linear_bf16(x, w)
    xd, wd, yd = dev_bf16(x), dev_bf16(w), out(1, lin.N)
    sg.skinny_gemm_bf16(xd, wd, yd, workspace(1, lin.N, lin.K))
    torch.cuda.synchronize()
    worst = assert_matches_oracle(yd, y_ref, a, "qkv gemv")
    assert worst < 0.5          # margin: the error is the bf16 output rounding


@pytest.mark.parametrize("M", [1, 2, 4, 6, 8, 16])
def test_tp8_layer_stack(M):
    """One decoder layer's TP=8-shard linears through decode_linear_stack."""
    from gemv_skinny_gemm_amd import workloads
    lins = workloads.tp8_layer()
    host, dev, refs = [], [], []
    for L in lins:
        x = synth.tensor_bf16(0, L.x_stream, M, L.K, 1.0)
        w = synth.tensor_bf16(0, L.w_stream, L.N, L.K, 0.02)
        refs.append(oracle.linear_bf16(x, w))
        xd, wd, yd = dev_bf16(x), dev_bf16(w), out(M, L.N)
        dev.append((xd, wd, yd))
    descs = [sg.make_linear(xd, wd, yd) for xd, wd, yd in dev]
    ws = torch.empty(sg.stack_workspace_bytes(descs, M), dtype=torch.uint8, device="cuda")
    for var in variants_for(M):
        sg.linear_run(descs, M, ws, variant=var)
        torch.cuda.synchronize()
        for L, (xd, wd, yd), (y_ref, a, _) in zip(lins, dev, refs):
            assert_matches_oracle(yd, y_ref, a, f"{L.name} M={M} var={var}")


def test_automatic_variant():
    """bf16 takes the row kernel at M <= 2, and at M = 3-4 for launches of at
    least 2.5 GB of weights (two TP=1 layers); the tile kernel otherwise.  FP8
    takes the tile kernel but for one-token launches of at least 1 GB of
    weights.  Launches under 0.4 GB of up to 4 tokens (bf16) or 2 (FP8), and
    one-token FP8 ones of at least 1 GB, run the flat row kernel.  A call makes
    one launch per dtype."""
    V, T = sg.VARIANT_VECTOR, sg.VARIANT_MFMA

    def variant(shapes, M, dt=sg.BF16):
        scale = None if dt == sg.BF16 else 0x300000
        lins = [sg.Linear(dt, N, K, 0, 0x100000, scale, 0x2000000, 0x4000000) for N, K in shapes]
        return sg.plan_query(lins, M).variant
    tp8 = [(1280, 8192), (8192, 1024), (7392, 8192), (8192, 3696)]
    tp1 = [(10240, 8192), (8192, 8192), (59136, 8192), (8192, 29568)]
    assert [variant(tp8, M) for M in (1, 2, 3, 4, 5, 8, 16)] == [V, V, V, V, T, T, T]
    assert [variant(tp1, M) for M in (1, 2, 3, 4)] == [V, V, T, T]                  # 1.76 GB
    assert [variant(tp1 * 2, M) for M in (1, 2, 3, 4, 5, 6, 8)] == [V, V, V, V, T, T, T]
    assert [variant(tp1 * 2, M, sg.FP8_BS128) for M in (1, 2, 4)] == [V, T, T]   # 1.76 GB
    assert variant(tp1, 1, sg.FP8_BS128) == T                                     # 0.88 GB
    assert variant([(152064, 8192)], 1, sg.FP8_BS128) == V                       # 1.25 GB
    assert [variant(tp8, M, sg.FP8_BS128) for M in (1, 2, 3)] == [V, V, T]       # 0.11 GB

    def kernel(shapes, M, dt=sg.BF16):
        scale = None if dt == sg.BF16 else 0x300000
        lins = [sg.Linear(dt, N, K, 0, 0x100000, scale, 0x2000000, 0x4000000) for N, K in shapes]
        return sg.KERNEL_NAMES[sg.plan_query(lins, M).kernel]
    assert kernel(tp1 * 2, 1, sg.FP8_BS128) == "skinny_rows_flat"
    assert kernel(tp1 * 2, 1) == "skinny_rows (lean)"
    assert kernel(tp8, 1) == "skinny_rows_flat"                                 # 0.22 GB
    assert kernel(tp8, 4) == "skinny_rows_flat"
    assert kernel(tp8, 2, sg.FP8_BS128) == "skinny_rows_flat"
    assert kernel(tp8, 3, sg.FP8_BS128) == "skinny_tiles"
    assert kernel(tp8, 8) == "skinny_tiles"
