"""Edge cases of y = x . W^T through the GPU against the fp64 oracle: FP8
blocks at the ends of the format (scale 0 over zero and non-zero codes, every
code +-448, scales from 2^-24 to 2^16), token rows of x that are exactly zero,
and rows far longer than any benchmark shape (many K-chunks; FP8 past the row
kernel's 256 scale blocks)."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import synth
from tests.gpu_util import assert_matches_oracle, need_gpu, run_bf16, run_fp8, variants_for

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _x(tag, M, K):
    return synth.tensor_bf16(0, synth.stream_id("edge-x", tag, M, K), M, K, 1.0)


def _extreme_fp8(N, K, seed):
    """Random E4M3FN codes (no NaN codes) with blocks set to the extremes."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, (N, K)).astype(np.uint8)
    q[q == 0x7F] = 0x7E                                   # 0x7F / 0xFF are NaN: +-448 instead
    q[q == 0xFF] = 0xFE
    nb, kb = (N + 127) // 128, (K + 127) // 128
    s = (2.0 ** rng.integers(-10, 5, (nb, kb))).astype(np.float32)
    q[0:128, 0:128] = 0                                   # an all-zero block, scale 0
    s[0, 0] = 0.0
    q[0:128, 128:256] = np.where(rng.random((128, 128)) < 0.5, 0x7E, 0xFE)   # every code +-448
    s[0, 1] = 2.0 ** -24
    s[0, 2] = 2.0 ** 16                                   # |w| up to 448 * 65536
    s[1, 0] = 0.0                                         # scale 0 over non-zero codes
    s[2, 3] = 1.0 / 448.0
    return q, s


@pytest.mark.parametrize("M", [1, 6, 16])
def test_fp8_extreme_blocks(M):
    N, K = 259, 400                                       # ragged in both block dimensions
    q, s = _extreme_fp8(N, K, 11)
    x = _x("fp8x", M, K)
    y_ref, a, _ = oracle.linear_fp8_bs128(x, q, s)
    for var in variants_for(M):
        for waves in (0, 4):
            y = run_fp8(x, q, s, M, N, variant=var, waves=waves)
            # Small K: half a bf16 ulp of y_ref is allowed on top of the bound.
            assert_matches_oracle(y, y_ref, a, f"M={M} var={var} waves={waves}")


@pytest.mark.parametrize("dtype", [sg.BF16, sg.FP8_BS128])
def test_zero_token_rows_give_zero(dtype):
    M, N, K = 6, 300, 1024
    x = _x("zero", M, K)
    x[1] = 0
    x[4] = 0x8000                                         # -0.0
    if dtype == sg.BF16:
        w = synth.tensor_bf16(0, synth.stream_id("edge-zero-w"), N, K, 0.02)
        y_ref, a, _ = oracle.linear_bf16(x, w)
        runs = [run_bf16(x, w, M, N, variant=v) for v in variants_for(M)]
    else:
        q, s, _ = synth.fp8_weight_bs128(0, synth.stream_id("edge-zero-q"), N, K)
        y_ref, a, _ = oracle.linear_fp8_bs128(x, q, s)
        runs = [run_fp8(x, q, s, M, N, variant=v) for v in variants_for(M)]
    for y in runs:
        assert torch.all(y[1].float() == 0) and torch.all(y[4].float() == 0)
        assert_matches_oracle(y, y_ref, a, f"dtype={dtype}")


@pytest.mark.parametrize("M", [1, 16])
def test_bf16_very_long_rows(M):
    N, K = 40, 1 << 20                                    # 2 MB rows: many K-chunks
    x = _x("longbf16", M, K)
    w = synth.tensor_bf16(0, synth.stream_id("edge-long-w", K), N, K, 0.02)
    y_ref, a, _ = oracle.linear_bf16(x, w)
    for var in variants_for(M):
        for waves in (0, 8):
            y = run_bf16(x, w, M, N, variant=var, waves=waves)
            assert_matches_oracle(y, y_ref, a, f"M={M} var={var} waves={waves}")


@pytest.mark.parametrize("M", [1, 6])
def test_fp8_very_long_rows(M):
    """K = 131072: 1024 scale blocks per row, past the row kernel's limit of
    256, so the automatic plan and the matrix-core kernel take it and the
    vector kernel refuses it on the host."""
    N, K = 130, 1 << 17
    x = _x("longfp8", M, K)
    q, s, _ = synth.fp8_weight_bs128(0, synth.stream_id("edge-long-q", K), N, K)
    y_ref, a, _ = oracle.linear_fp8_bs128(x, q, s)
    for var in (sg.VARIANT_AUTO, sg.VARIANT_MFMA):
        for waves in (0, 8):
            y = run_fp8(x, q, s, M, N, variant=var, waves=waves)
            assert_matches_oracle(y, y_ref, a, f"M={M} var={var} waves={waves}")
    with pytest.raises(sg.SkinnyError):
        run_fp8(x, q, s, M, N, variant=sg.VARIANT_VECTOR)
