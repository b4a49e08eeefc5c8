"""Device-side twin of the seeded input generator (libskinny_synth.so).

Produces the same bytes as the numpy generator in this package, directly in
GPU memory, for workloads too large to generate on the host (the 80-layer
stack is 140 GB of bf16 weights).  Input generation only."""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from gemv_skinny_gemm_amd import synth

_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libskinny_synth.so")
_lib = None
_tables = {}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise ImportError(f"{_LIB} is not built")
        L = ctypes.CDLL(_LIB)
        vp, ll, u, i = ctypes.c_void_p, ctypes.c_longlong, ctypes.c_uint, ctypes.c_int
        L.synth_normal_bf16.restype = i
        L.synth_normal_bf16.argtypes = [vp, ll, ll, u, u, vp, vp, i, vp]
        L.synth_quantize_bs128.restype = i
        L.synth_quantize_bs128.argtypes = [vp, vp, vp, i, i, vp]
        _lib = L
    return _lib


def _table(sigma: float, device):
    key = (float(sigma), str(device))
    if key not in _tables:
        thr, codes = synth.normal_table(float(sigma))
        _tables[key] = (torch.from_numpy(thr.view(np.int32)).to(device),
                        torch.from_numpy(codes.view(np.int16)).to(device), len(thr))
    return _tables[key]


def _stream():
    return torch.cuda.current_stream().cuda_stream


def normal_bf16_(out: torch.Tensor, seed: int, stream: int, sigma: float, start: int = 0):
    """Fill a contiguous bf16 (or int16) GPU tensor with elements start.. of the sequence."""
    assert out.is_cuda and out.is_contiguous() and out.element_size() == 2
    thr, codes, n = _table(sigma, out.device)
    rc = lib().synth_normal_bf16(out.data_ptr(), start, out.numel(), seed & 0xFFFFFFFF,
                                 stream & 0xFFFFFFFF, thr.data_ptr(), codes.data_ptr(), n,
                                 _stream())
    if rc != 0:
        raise RuntimeError(f"synth_normal_bf16 failed ({rc})")
    return out


def tensor_bf16(seed: int, stream: int, rows: int, cols: int, sigma: float,
                device="cuda") -> torch.Tensor:
    t = torch.empty((rows, cols), dtype=torch.bfloat16, device=device)
    return normal_bf16_(t, seed, stream, sigma)


def quantize_bs128(w: torch.Tensor):
    """bf16 GPU tensor [N][K] -> (uint8 codes [N][K], fp32 scales [ceil(N/128)][ceil(K/128)])."""
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s = torch.empty(((N + 127) // 128, (K + 127) // 128), dtype=torch.float32, device=w.device)
    rc = lib().synth_quantize_bs128(w.data_ptr(), q.data_ptr(), s.data_ptr(), N, K, _stream())
    if rc != 0:
        raise RuntimeError(f"synth_quantize_bs128 failed ({rc})")
    return q, s


def fp8_weight_bs128(seed: int, stream: int, N: int, K: int, sigma: float = 0.02,
                     scratch: torch.Tensor | None = None, device="cuda"):
    """FP8 weights of an [N][K] N(0, sigma^2) tensor, made on the GPU.

    scratch: optional bf16 buffer of at least N*K elements for the unquantized weights."""
    if scratch is None or scratch.numel() < N * K:
        scratch = torch.empty(N * K, dtype=torch.bfloat16, device=device)
    w = scratch[:N * K].view(N, K)
    normal_bf16_(w, seed, stream, sigma)
    return quantize_bs128(w)


def materialise(specs, M: int, copies: int = 1, seed: int = 0):
    """Device tensors and skinny_linear descriptors for `copies` copies of a
    workload (a list of workloads.LinearSpec).  Copy 0 uses each tensor's own
    stream; copy c > 0 offsets the weight stream so every copy is distinct.

    Returns (sets, tensors): sets[c] is the list of descriptors of copy c and
    tensors[c][i] = (x, w, scale or None, y) of linear i."""
    import gemv_skinny_gemm_amd as sg
    from gemv_skinny_gemm_amd import workloads as wl

    max_fp8 = max((s.N * s.K for s in specs if s.dtype == wl.FP8_BS128), default=0)
    scratch = torch.empty(max_fp8, dtype=torch.bfloat16, device="cuda") if max_fp8 else None
    sets, tensors = [], []
    for c in range(copies):
        descs, ts = [], []
        for s in specs:
            wstream = weight_stream(s, c)
            x = tensor_bf16(seed, s.x_stream, M, s.K, wl.X_SIGMA)
            y = torch.zeros((M, s.N), dtype=torch.bfloat16, device="cuda")
            if s.dtype == wl.BF16:
                w = tensor_bf16(seed, wstream, s.N, s.K, wl.W_SIGMA)
                descs.append(sg.make_linear(x, w, y))
                ts.append((x, w, None, y))
            else:
                q, sc = fp8_weight_bs128(seed, wstream, s.N, s.K, wl.W_SIGMA, scratch=scratch)
                descs.append(sg.make_linear(x, q, y, w_scale=sc))
                ts.append((x, q, sc, y))
        sets.append(descs)
        tensors.append(ts)
    torch.cuda.synchronize()
    return sets, tensors


def weight_stream(spec, copy: int = 0) -> int:
    """Philox stream of a weight tensor's copy `copy` (copy 0 = the spec's own)."""
    return (spec.w_stream + copy * 0x9E3779B1) & 0xFFFFFFFF
