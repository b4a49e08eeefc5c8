"""fp64 CPU oracle for the decode-phase linear layer y = x . W^T.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
loads it, and it loads nothing of the GPU library.

The arithmetic lives in ``oracle.c`` (plain C, fp64, threaded over output
rows).  This module builds it with gcc when needed and marshals numpy arrays.

Greedy next token (``argmax_first``): the smallest index of the largest logit
of each token row, NaN below every number (-inf included); ``greedy_valid``
decides whether a GPU's choice is one the accepted error allows.

Gated MLP (``mlp_swiglu``): the two linears above with the activation h =
silu(g) * u between them, g and u and h rounded to bf16 as the method's
16-bit activations are (``bf16_encode``: round to nearest, ties to even).

Mixture-of-experts linear (``moe_linear``): each route (token, choice) of a
batch goes through its own expert's linear; a route to no expert gives zeros.

Definition followed (see oracle.c for the citations):
    y_ref[m][n] = sum_k x[m][k] * w[n][k]            in fp64
    w[n][k]     = bf16 value                         (bf16 weights)
                = e4m3(q[n][k]) * S[n//128][k//128]  (FP8 weights)
    A[m][n]     = sum_k |x[m][k] * w[n][k]|
A GPU result passes when, for every output, |y - y_ref| <= 2e-3 * A + 1e-6
or y is one of the two bf16 values around y_ref (``accepted``: the output is
bf16, and where the terms barely cancel half a bf16 step can exceed the
stated bound).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

REL_TOL = 2e-3
ABS_TOL = 1e-6

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (host only, no HIP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                        "-o", tmp, _SRC, "-lpthread", "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    """Load a compiled oracle and declare its C signatures."""
    lib = ctypes.CDLL(path)
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_linear_bf16.restype = ctypes.c_int
    lib.oracle_linear_bf16.argtypes = [p, p, i64, i64, i64, p, p, ctypes.c_int]
    lib.oracle_linear_fp8_bs128.restype = ctypes.c_int
    lib.oracle_linear_fp8_bs128.argtypes = [p, p, p, i64, i64, i64, p, p, ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = _bind(_LIB)
    return _lib


def host_threads() -> int:
    """Cores this process may run on (the oracle's default thread count)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def bf16_value(code: int) -> float:
    return _load().oracle_bf16_value(int(code) & 0xFFFF)


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(int(code) & 0xFF)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def linear_bf16(x: np.ndarray, w: np.ndarray, threads: int | None = None):
    """x: [M][K] uint16 bf16 codes, w: [N][K] uint16 bf16 codes.

    Returns (y_ref, A, threads_used): fp64 [M][N] each."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    M, K = x.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError("x and w disagree on K")
    y = np.empty((M, N), np.float64)
    a = np.empty((M, N), np.float64)
    t = _load().oracle_linear_bf16(x.ctypes.data, w.ctypes.data, M, N, K, y.ctypes.data,
                                   a.ctypes.data, threads or host_threads())
    if t < 0:
        raise RuntimeError("oracle_linear_bf16 failed")
    return y, a, t


def linear_fp8_bs128(x: np.ndarray, q: np.ndarray, scale: np.ndarray,
                     threads: int | None = None):
    """x: [M][K] uint16 bf16 codes, q: [N][K] uint8 e4m3 codes,
    scale: [ceil(N/128)][ceil(K/128)] float32.

    Returns (y_ref, A, threads_used): fp64 [M][N] each."""
    x = _c(x, np.uint16)
    q = _c(q, np.uint8)
    scale = _c(scale, np.float32)
    M, K = x.shape
    N, K2 = q.shape
    if K != K2:
        raise ValueError("x and q disagree on K")
    if scale.shape != ((N + 127) // 128, (K + 127) // 128):
        raise ValueError("scale must be [ceil(N/128)][ceil(K/128)]")
    y = np.empty((M, N), np.float64)
    a = np.empty((M, N), np.float64)
    t = _load().oracle_linear_fp8_bs128(x.ctypes.data, q.ctypes.data, scale.ctypes.data,
                                        M, N, K, y.ctypes.data, a.ctypes.data,
                                        threads or host_threads())
    if t < 0:
        raise RuntimeError("oracle_linear_fp8_bs128 failed")
    return y, a, t


def bf16_bracket(v: np.ndarray):
    """The two bf16 values around each fp64 value: lo = the largest bf16 value
    <= v, hi = the smallest bf16 value >= v (lo == hi when v is a bf16 value).
    Beyond the largest finite bf16 value, hi is infinity."""
    v = np.asarray(v, np.float64)
    mag = np.abs(v)
    c = bf16_encode(mag).astype(np.int64)          # nearest code of |v| (sign bit clear)
    with np.errstate(invalid="ignore"):            # codes past infinity: unused NaNs
        r = bf16_decode(c.astype(np.uint16))
        below = np.where(r > mag, bf16_decode(np.maximum(c - 1, 0).astype(np.uint16)), r)
        above = np.where(r < mag, bf16_decode(np.minimum(c + 1, 0x7F80).astype(np.uint16)), r)
    return np.where(v < 0, -above, below), np.where(v < 0, -below, above)


def bound(a: np.ndarray) -> np.ndarray:
    """The stated per-output tolerance 2e-3 * A + 1e-6."""
    return REL_TOL * np.asarray(a, np.float64) + ABS_TOL


def accepted(y_ref: np.ndarray, a: np.ndarray):
    """Interval [lo, hi] of results accepted for each output: within the
    stated bound of y_ref, or one of the two bf16 values around y_ref.

    The output is bf16, so no result can be closer to y_ref than its nearest
    bf16 value, and an fp32 sum that lands within rounding distance of the
    midpoint between the two may round either way.  Where an output has
    little cancellation (|y_ref| close to A, e.g. a handful of same-sign
    terms) half a bf16 step can exceed 2e-3 * A; there the two bracketing
    values, and nothing else, are accepted besides the stated interval."""
    b = bound(a)
    y_ref = np.asarray(y_ref, np.float64)
    lo_b, hi_b = bf16_bracket(y_ref)
    return np.minimum(y_ref - b, lo_b), np.maximum(y_ref + b, hi_b)


def check(y_gpu: np.ndarray, y_ref: np.ndarray, a: np.ndarray):
    """Compare a GPU result (any float dtype, [M][N]) with the oracle.

    Returns (ok, worst ratio of the error to the accepted distance on its
    side of y_ref, index of the worst output).  Where 2e-3 * A + 1e-6 is wider
    than bf16 spacing (every large-K output) the ratio is err / bound."""
    y = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    lo, hi = accepted(y_ref, a)
    err = np.abs(y - y_ref)
    ratio = err / np.where(y >= y_ref, hi - y_ref, y_ref - lo)
    if ratio.size == 0:
        return True, 0.0, None
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    worst = float(ratio[idx])
    return bool(np.all(ratio <= 1.0)), worst, idx


def argmax_first(values: np.ndarray) -> np.ndarray:
    """Greedy token of every row of ``values`` [M][N]: the smallest n whose
    value is the largest of the row, NaN counting below every number (-inf
    included), so a row of NaNs gives 0.  The decode step picks its next
    token this way on the device ("Developing a custom Qwen2.5 72B inference
    engine from scratch", section 5, third lever).  A plain scan, row by row."""
    v = np.asarray(values, np.float64)
    out = np.zeros(v.shape[0], np.int64)
    for m in range(v.shape[0]):
        best_i = None                              # no number seen yet
        for n in range(v.shape[1]):
            x = v[m, n]
            if np.isnan(x):
                continue
            if best_i is None or x > v[m, best_i]:
                best_i = n
        out[m] = 0 if best_i is None else best_i
    return out


def greedy_valid(idx: np.ndarray, y_ref: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Whether each chosen token idx[m] is a largest logit of some set of
    outputs each inside its accepted interval [lo, hi] (``accepted``): token
    i can beat every j only if hi[i] >= max_j lo[j].  When the exact winner
    leads every other logit by more than both intervals, this admits it
    alone."""
    lo, hi = accepted(y_ref, a)
    rows = np.arange(np.asarray(y_ref).shape[0])
    return hi[rows, idx] >= np.max(lo, axis=1)


def bf16_encode(v: np.ndarray) -> np.ndarray:
    """bf16 codes of the fp64 values ``v`` rounded to the nearest bf16 value,
    ties to even (8 significant bits; subnormals below 2^-126 on a 2^-133
    grid; beyond the largest finite value, infinity; NaN to 0x7FC0)."""
    v = np.asarray(v, np.float64)
    mag = np.abs(v)
    f, e = np.frexp(mag)                           # mag = f 2^e, f in [0.5, 1)
    normal = mag >= 2.0 ** -126
    # Normal: 8 significant bits, the integer significand in [128, 256].
    sig = np.rint(f * 256.0)                       # numpy rounds halves to even
    r_norm = np.ldexp(sig, e - 8)
    r_sub = np.rint(mag / 2.0 ** -133) * 2.0 ** -133
    r = np.where(normal, r_norm, r_sub)
    r = np.where(r > 3.3895313892515355e38, np.inf, r)   # above (2 - 2^-7) 2^127
    r = np.copysign(r, v)
    # Every rounded value is exact in binary32; its upper half is the code.
    codes = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(v), np.uint16(0x7FC0), codes)


def silu(v: np.ndarray) -> np.ndarray:
    """v / (1 + e^-v) in fp64."""
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def bf16_decode(codes: np.ndarray) -> np.ndarray:
    """fp64 values of bf16 codes (the upper half of a binary32)."""
    c = np.asarray(codes, np.uint16).astype(np.uint32) << 16
    return c.view(np.float32).astype(np.float64)


def mlp_swiglu(x: np.ndarray, w_gate_up, w_down, scales=None, threads: int | None = None):
    """The gated MLP y = down(h), h = bf16(silu(g) * u), [g | u] = bf16(x . W_gate_up^T).

    bf16 weights: w_gate_up [2I][H] and w_down [H][I] bf16 codes.  FP8:
    e4m3 codes with ``scales`` = (s_gate_up, s_down).  Returns (y_ref, A, h
    codes) of the down linear; A bounds its error as for any linear."""
    I = w_down.shape[1]
    if scales is None:
        gu, _, _ = linear_bf16(x, w_gate_up, threads)
    else:
        gu, _, _ = linear_fp8_bs128(x, w_gate_up, scales[0], threads)
    g = bf16_decode(bf16_encode(gu[:, :I]))
    u = bf16_decode(bf16_encode(gu[:, I:]))
    h = bf16_encode(silu(g) * u)
    if scales is None:
        y, a, _ = linear_bf16(h, w_down, threads)
    else:
        y, a, _ = linear_fp8_bs128(h, w_down, scales[1], threads)
    return y, a, h


def moe_linear(x: np.ndarray, ids: np.ndarray, w: np.ndarray, scales=None,
               x_per_route: bool = False, swiglu: bool = False, threads: int | None = None):
    """One linear of a mixture-of-experts layer, over the routes of a batch.

    A router sends each token to its top-k experts, each expert being its own
    small network ("Multi-GPU Inference and Serving at Scale", Example 8); in a
    decode verify step a handful of tokens pass through the weight-only FP8
    expert matmuls ("9% faster GLM-5.3-Flash prefill with GPU-to-GPU IPC",
    section "TileLang: twice as fast, and no faster").  Route r = t * topk + j
    is token t's j-th choice, expert e = ids[t][j]:

        y[r] = x_r . W_e^T                      (an ordinary linear per route)
        x_r  = x[r] if x_per_route else x[t]
        x_r  = bf16(silu(g) * u) of x's row [g | u] when swiglu
        y[r] = 0 when e is outside [0, E)

    x: bf16 codes, [T][K] (or [T * topk][K] per route; 2K columns with swiglu);
    ids: [T][topk] ints; w: [E][N][K] bf16 codes, or e4m3 codes with
    ``scales`` [E][ceil(N/128)][ceil(K/128)] fp32.  Routes of one expert go
    through the linear together; every output is its own dot product.

    Returns (y_ref, A): fp64 [T * topk][N] each (A = 0 on zero rows)."""
    ids = np.asarray(ids)
    T, topk = ids.shape
    E, N, K = w.shape
    routes = T * topk
    x = np.asarray(x)
    if swiglu:
        g = bf16_decode(x[:, :K])
        u = bf16_decode(x[:, K:])
        x = bf16_encode(silu(g) * u)
    if x.shape != ((routes if x_per_route else T), K):
        raise ValueError("x rows or columns do not match the routes and K")
    y = np.zeros((routes, N), np.float64)
    a = np.zeros((routes, N), np.float64)
    flat = ids.reshape(-1)
    for e in range(E):
        rs = np.nonzero(flat == e)[0]
        if rs.size == 0:
            continue
        xr = x[rs] if x_per_route else x[rs // topk]
        if scales is None:
            ye, ae, _ = linear_bf16(xr, w[e], threads)
        else:
            ye, ae, _ = linear_fp8_bs128(xr, w[e], scales[e], threads)
        y[rs] = ye
        a[rs] = ae
    return y, a
