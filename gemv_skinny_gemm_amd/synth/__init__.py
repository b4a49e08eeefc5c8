"""Seeded synthetic inputs for the skinny GEMM: weights, activations, FP8 codes.

This module holds input generation only.  It contains none of the linear
layer's arithmetic (no dot products, no dequantization, no output rounding);
both the GPU library's tests and the fp64 oracle consume the bytes it makes.

Generator (identical on the host and, in ``synth_gpu.hip``, on the GPU):

* Random bits come from Philox4x32-10, the counter-based generator of
  Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
  1, 2, 3" (SC'11).  Element ``i`` of a tensor takes 32-bit word ``i % 4``
  of the block ``philox(counter=(i // 4) as (lo, hi, 0, 0), key=(seed, stream))``.
  Any element, row or block of rows can therefore be regenerated on its own.
* A normal variate rounded to bf16 is drawn by exact inverse-CDF sampling in
  integers: bit 31 of the word is the sign, bits 0..30 are a uniform
  ``u`` in [0, 2^31) and the magnitude's bf16 code is the first code whose
  threshold exceeds ``u``.  Thresholds are ``round(2^31 * P(|Z| < edge))``
  for each bf16 code's upper rounding edge, with ``Z ~ N(0, sigma^2)``.
  Sampling is then integer-only, so host and GPU agree bit for bit.
* FP8 weights: W ~ N(0, 0.02) (as bf16 values) is cut into 128 x 128 blocks;
  each block's scale is ``fp32(amax / 448)`` and each code is the OCP E4M3FN
  value nearest to ``w / scale`` (computed in fp64), ties to even, saturated
  to +-448.  An all-zero block gets scale 0 and codes 0.
"""
from __future__ import annotations

import math
import zlib
from concurrent.futures import ThreadPoolExecutor
from functools import lru_cache

import numpy as np

PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = np.uint32(0x9E3779B9)
PHILOX_W1 = np.uint32(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)

E4M3_MAX = 448.0
BLOCK = 128


def stream_id(*parts) -> int:
    """32-bit stream id of a named tensor, e.g. stream_id("stack", 17, "gate_up", "w")."""
    return zlib.crc32("/".join(str(p) for p in parts).encode()) & 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds on uint32 arrays (vectorised).

    Each round multiplies words 0 and 2 by the two round constants, keeps the
    high and low halves, and mixes them with words 1 and 3 and the key; the
    key is bumped by the two Weyl constants between rounds."""
    c0 = np.asarray(c0, np.uint32)
    c1 = np.asarray(c1, np.uint32)
    c2 = np.asarray(c2, np.uint32)
    c3 = np.asarray(c3, np.uint32)
    k0 = np.uint32(k0 & 0xFFFFFFFF)
    k1 = np.uint32(k1 & 0xFFFFFFFF)
    for r in range(10):
        if r:
            k0 = np.uint32((int(k0) + int(PHILOX_W0)) & 0xFFFFFFFF)
            k1 = np.uint32((int(k1) + int(PHILOX_W1)) & 0xFFFFFFFF)
        p0 = c0.astype(np.uint64) * PHILOX_M0
        p1 = c2.astype(np.uint64) * PHILOX_M1
        hi0 = (p0 >> np.uint64(32)).astype(np.uint32)
        lo0 = (p0 & _MASK32).astype(np.uint32)
        hi1 = (p1 >> np.uint64(32)).astype(np.uint32)
        lo1 = (p1 & _MASK32).astype(np.uint32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def random_words(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Words start .. start+count-1 of the (seed, stream) sequence, uint32."""
    if count <= 0:
        return np.zeros(0, np.uint32)
    b0 = start // 4
    b1 = (start + count - 1) // 4 + 1
    blk = np.arange(b0, b1, dtype=np.uint64)
    lo = (blk & _MASK32).astype(np.uint32)
    hi = (blk >> np.uint64(32)).astype(np.uint32)
    z = np.zeros_like(lo)
    r0, r1, r2, r3 = philox4x32_10(lo, hi, z, z, seed, stream)
    words = np.stack([r0, r1, r2, r3], axis=1).reshape(-1)
    off = start - b0 * 4
    return words[off:off + count]


def _bf16_code_values(codes: np.ndarray) -> np.ndarray:
    """Value of bf16 codes (format plumbing: a bf16 code is the top half of a binary32)."""
    return (codes.astype(np.uint32) << np.uint32(16)).view(np.float32)


@lru_cache(maxsize=16)
def normal_table(sigma: float):
    """(thresholds uint32, codes uint16) for |Z| ~ |N(0, sigma^2)| rounded to bf16.

    Code ``codes[j]`` is drawn when ``thresholds[j-1] <= u < thresholds[j]``
    for a uniform 31-bit ``u``; the last threshold is 2^31."""
    pos = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)      # +0 .. largest finite
    vals = _bf16_code_values(pos).astype(np.float64)
    edges = np.empty_like(vals)
    edges[:-1] = 0.5 * (vals[:-1] + vals[1:])
    edges[-1] = math.inf
    scale = 1.0 / (sigma * math.sqrt(2.0))
    cdf = np.array([1.0 if math.isinf(e) else math.erf(e * scale) for e in edges])
    thr = np.minimum(np.rint(cdf * 2.0 ** 31), 2.0 ** 31).astype(np.int64)
    keep = np.empty(thr.shape, bool)
    keep[0] = thr[0] > 0
    keep[1:] = thr[1:] > thr[:-1]
    thr, codes = thr[keep], pos[keep]
    thr[-1] = 2 ** 31
    return thr.astype(np.uint32), codes.astype(np.uint16)


def words_to_bf16(words: np.ndarray, sigma: float) -> np.ndarray:
    thr, codes = normal_table(float(sigma))
    mag = words & np.uint32(0x7FFFFFFF)
    j = np.searchsorted(thr, mag, side="right")
    c = codes[j]
    sign = ((words >> np.uint32(31)).astype(np.uint16) << np.uint16(15))
    sign[c == 0] = 0
    return (c | sign).astype(np.uint16)


def _chunks(start: int, count: int, size: int):
    return [(s, min(size, start + count - s)) for s in range(start, start + count, size)]


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import os
        try:
            n = len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            n = os.cpu_count() or 1
        _POOL = ThreadPoolExecutor(max_workers=max(1, min(16, n)))
    return _POOL


def normal_bf16(seed: int, stream: int, start: int, count: int, sigma: float) -> np.ndarray:
    """Elements start .. start+count-1 of N(0, sigma^2) rounded to bf16, as uint16 codes."""
    normal_table(float(sigma))  # build once before threads start
    out = np.empty(count, np.uint16)
    parts = _chunks(start, count, 1 << 20)

    def work(p):
        s, n = p
        out[s - start:s - start + n] = words_to_bf16(random_words(seed, stream, s, n), sigma)

    if len(parts) <= 1:
        for p in parts:
            work(p)
    else:
        list(_pool().map(work, parts))
    return out


def tensor_bf16(seed: int, stream: int, rows: int, cols: int, sigma: float,
                row_begin: int = 0) -> np.ndarray:
    """Rows row_begin .. row_begin+rows-1 of a [*][cols] N(0, sigma^2) bf16 tensor."""
    flat = normal_bf16(seed, stream, row_begin * cols, rows * cols, sigma)
    return flat.reshape(rows, cols)


def tensor_rows_bf16(seed: int, stream: int, row_ids, cols: int, sigma: float) -> np.ndarray:
    """Selected rows (any order) of a [*][cols] N(0, sigma^2) bf16 tensor."""
    row_ids = [int(r) for r in row_ids]
    out = np.empty((len(row_ids), cols), np.uint16)
    for i, r in enumerate(row_ids):
        out[i] = normal_bf16(seed, stream, r * cols, cols, sigma)
    return out


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3FN) block quantizer: produces the weight-only FP8 checkpoint
# format the FP8 path consumes.


def encode_e4m3(r: np.ndarray) -> np.ndarray:
    """Nearest OCP E4M3FN code to each fp64 value, ties to even, saturating at +-448."""
    r = np.asarray(r, np.float64)
    a = np.minimum(np.abs(r), E4M3_MAX)
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    e = np.clip(ex - 1, -6, 8)                # binade; below 2^-6 the spacing stays 2^-9
    quantum = np.ldexp(1.0, e - 3)
    val = np.rint(a / quantum) * quantum      # exact scaling; rint rounds ties to even
    f, ex2 = np.frexp(val)
    ebias = ex2 - 1 + 7
    normal = (val > 0) & (ebias >= 1)
    mant_n = np.where(normal, np.rint((2.0 * f - 1.0) * 8.0), 0.0)
    mant_s = np.rint(val / 2.0 ** -9)
    code = np.where(normal, (ebias.astype(np.int64) << 3) | mant_n.astype(np.int64),
                    mant_s.astype(np.int64))
    code = np.where(val == 0, 0, code)
    sign = (r < 0) & (val != 0)
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def quantize_bs128(w_codes: np.ndarray):
    """bf16 weights [N][K] -> (e4m3 codes [N][K] uint8, scales [ceil(N/128)][ceil(K/128)] fp32)."""
    w = _bf16_code_values(np.ascontiguousarray(w_codes, np.uint16)).astype(np.float64)
    N, K = w.shape
    nb, kb = (N + BLOCK - 1) // BLOCK, (K + BLOCK - 1) // BLOCK
    q = np.empty((N, K), np.uint8)
    scale = np.empty((nb, kb), np.float32)

    def band(i):
        r0, r1 = i * BLOCK, min(N, (i + 1) * BLOCK)
        blk = w[r0:r1]
        for j in range(kb):
            c0, c1 = j * BLOCK, min(K, (j + 1) * BLOCK)
            t = blk[:, c0:c1]
            amax = float(np.max(np.abs(t))) if t.size else 0.0
            s = np.float32(amax / E4M3_MAX)
            scale[i, j] = s
            if s == 0:
                q[r0:r1, c0:c1] = 0
            else:
                q[r0:r1, c0:c1] = encode_e4m3(t / float(s))

    if nb > 1:
        list(_pool().map(band, range(nb)))
    else:
        for i in range(nb):
            band(i)
    return q, scale


def fp8_weight_bs128(seed: int, stream: int, N: int, K: int, sigma: float = 0.02,
                     band_begin: int = 0, bands: int | None = None):
    """FP8 weights of an [N][K] N(0, sigma^2) tensor, for 128-row bands
    band_begin .. band_begin+bands-1 (all bands by default).

    Returns (codes [rows][K] uint8, scales [bands][ceil(K/128)] fp32, first row)."""
    nb = (N + BLOCK - 1) // BLOCK
    if bands is None:
        bands = nb - band_begin
    r0 = band_begin * BLOCK
    r1 = min(N, (band_begin + bands) * BLOCK)
    w = tensor_bf16(seed, stream, r1 - r0, K, sigma, row_begin=r0)
    q, s = quantize_bs128(w)
    return q, s, r0


def route_topk(seed: int, stream: int, T: int, E: int, topk: int, hot: int = 2,
               hot_bias: float = 1.0) -> np.ndarray:
    """Synthetic router choices for T tokens over E experts: ids [T][topk] int32.

    Token t scores expert e with a N(0, 1) draw (rounded to bf16, element
    t * E + e of the stream) plus ``hot_bias`` for the first ``hot`` experts,
    so a few experts are busier than the rest, as real routers are
    ("Multi-GPU Inference and Serving at Scale", Example 8, which routes to
    the top 2 of 8 experts with experts 0 and 1 favoured by +1.0).  Each
    token takes its topk best experts, best first, ties to the lower index:
    the experts of one token are distinct."""
    if topk > E:
        raise ValueError("topk must not exceed E")
    s = _bf16_code_values(normal_bf16(seed, stream, 0, T * E, 1.0)).astype(np.float64)
    s = s.reshape(T, E) + np.where(np.arange(E) < hot, hot_bias, 0.0)
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -s), axis=1)
    return np.ascontiguousarray(order[:, :topk], np.int32)
