"""The seeded input generator: Philox known answers, the bf16 normal sampler,
row regeneration, and the FP8 block quantizer's invariants."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from gemv_skinny_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    d = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for v in d["vectors"]:
        c = [np.array([int(h, 16)], np.uint32) for h in v["ctr"]]
        k = [int(h, 16) for h in v["key"]]
        out = synth.philox4x32_10(*c, *k)
        assert ["%08x" % int(o[0]) for o in out] == v["out"]


def test_words_are_counter_addressed():
    full = synth.random_words(0, 77, 0, 1001)
    assert np.array_equal(synth.random_words(0, 77, 333, 100), full[333:433])
    assert np.array_equal(synth.random_words(0, 77, 1, 3), full[1:4])
    assert not np.array_equal(synth.random_words(1, 77, 0, 64), full[:64])
    assert not np.array_equal(synth.random_words(0, 78, 0, 64), full[:64])


@pytest.mark.parametrize("sigma", [1.0, 0.02])
def test_normal_bf16_distribution(sigma):
    n = 1 << 21
    codes = synth.normal_bf16(0, synth.stream_id("dist", sigma), 0, n, sigma)
    v = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert abs(v.mean()) < 5 * sigma / math.sqrt(n)
    assert abs(v.std() / sigma - 1.0) < 4e-3
    # Kolmogorov-Smirnov distance to N(0, sigma^2), allowing for bf16 rounding.
    xs = np.sort(v)
    cdf = 0.5 * (1 + np.vectorize(math.erf)(xs[:: 64] / (sigma * math.sqrt(2))))
    emp = (np.arange(n)[:: 64] + 0.5) / n
    assert np.max(np.abs(cdf - emp)) < 5e-3
    # Roughly symmetric and no specials.
    assert np.all(np.isfinite(v))
    assert abs(np.mean(v > 0) - 0.5) < 2e-3


def test_rows_regenerate_bitwise():
    full = synth.tensor_bf16(3, 99, 40, 300, 0.02)
    part = synth.tensor_bf16(3, 99, 7, 300, 0.02, row_begin=11)
    assert np.array_equal(part, full[11:18])
    picked = synth.tensor_rows_bf16(3, 99, [39, 0, 17], 300, 0.02)
    assert np.array_equal(picked, full[[39, 0, 17]])


def _finite_e4m3():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = np.array([oracle.e4m3_value(int(c)) for c in codes])
    return codes, vals


def test_encode_e4m3_round_trips_every_finite_code():
    codes, vals = _finite_e4m3()
    enc = synth.encode_e4m3(vals)
    # -0 encodes as +0; every other code maps back to itself.
    exp = np.where(codes == 0x80, 0, codes)
    assert np.array_equal(enc, exp)


def test_encode_e4m3_is_nearest_ties_to_even_and_saturates():
    codes, vals = _finite_e4m3()
    order = np.argsort(vals, kind="stable")
    pos_codes = [c for c in codes if c < 0x80]
    pos_vals = np.array([oracle.e4m3_value(int(c)) for c in pos_codes])
    rng = np.random.default_rng(0)
    probes = np.concatenate([
        rng.uniform(-500, 500, 4000),
        rng.uniform(-1, 1, 4000) * 2.0 ** rng.integers(-12, 9, 4000),
        (pos_vals[:-1] + pos_vals[1:]) / 2,                     # exact midpoints (ties)
        -(pos_vals[:-1] + pos_vals[1:]) / 2,
        [448.0, 449.0, 463.9, 464.0, 1e9, -1e9, 2.0 ** -10, 2.0 ** -10 * 3],
    ])
    got = np.array([oracle.e4m3_value(int(c)) for c in synth.encode_e4m3(probes)])
    for p, g in zip(probes, got):
        a = min(abs(p), 448.0)
        d = np.abs(pos_vals - a)
        best = np.flatnonzero(d == d.min())
        if len(best) == 1:
            want = pos_vals[best[0]]
        else:                                   # tie: the code with an even mantissa
            even = [b for b in best if (pos_codes[b] & 1) == 0]
            assert len(even) == 1
            want = pos_vals[even[0]]
        want = math.copysign(want, p) if want != 0 else 0.0
        assert g == want or (g == 0 and want == 0), (p, g, want)


def test_quantizer_invariants():
    N, K = 300, 260                                        # ragged 128-blocks on both axes
    w = synth.tensor_bf16(0, 21, N, K, 0.02)
    w[128:256, 128:256] = 0                                # one all-zero block
    q, s = synth.quantize_bs128(w)
    wv = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert s.shape == (3, 3) and q.shape == (N, K)
    for i in range(3):
        for j in range(3):
            blk = wv[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            qb = q[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            amax = np.abs(blk).max()
            assert s[i, j] == np.float32(amax / 448.0)
            if amax == 0:
                assert np.all(qb == 0)
                continue
            # The block's largest magnitude maps to +-448.
            r, c = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert qb[r, c] == (0xFE if blk[r, c] < 0 else 0x7E)
            # Dequantised weights are within half an e4m3 step of the originals.
            deq = np.vectorize(oracle.e4m3_value)(qb) * float(s[i, j])
            step = np.where(np.abs(blk) / s[i, j] < 2.0 ** -6, 2.0 ** -9,
                            2.0 ** (np.floor(np.log2(np.maximum(np.abs(blk) / s[i, j], 2.0 ** -6))) - 3))
            assert np.all(np.abs(deq - blk) <= 0.5 * step * s[i, j] * (1 + 1e-12))
    assert not np.any((q & 0x7F) == 0x7F)                  # never NaN


def test_fp8_bands_regenerate_bitwise():
    N, K = 300, 256
    q, s, r0 = synth.fp8_weight_bs128(4, 5, N, K)
    qb, sb, rb = synth.fp8_weight_bs128(4, 5, N, K, band_begin=2, bands=1)
    assert r0 == 0 and rb == 256
    assert np.array_equal(qb, q[256:]) and np.array_equal(sb, s[2:3])
