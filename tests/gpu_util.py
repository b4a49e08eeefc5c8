"""Shared plumbing of the GPU tests: uploads, downloads and oracle comparison."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    sg.lib()            # raises if the HIP library is not built: no fallback


def dev_bf16(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint16).view(np.int16)) \
        .view(torch.bfloat16).cuda()


def dev_u8(q: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(q, np.uint8)).cuda()


def dev_f32(s: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(s, np.float32)).cuda()


def host_values(y: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> fp64 host values."""
    return y.float().cpu().double().numpy()


def host_codes(y: torch.Tensor) -> np.ndarray:
    return y.cpu().view(torch.int16).numpy().view(np.uint16)


def workspace(M: int, N: int = 1, K: int = 8, dtype: int = sg.BF16) -> torch.Tensor:
    return torch.empty(sg.workspace_bytes(dtype, M, N, K), dtype=torch.uint8, device="cuda")


def out(M: int, N: int) -> torch.Tensor:
    # Filled with NaN so an output the kernels never write cannot pass.
    return torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")


def run_bf16(x, w, M, N, variant=sg.VARIANT_AUTO, waves=0, ws=None):
    xd, wd, yd = dev_bf16(x), dev_bf16(w), out(M, N)
    ws = workspace(M, N, x.shape[1], sg.BF16) if ws is None else ws
    sg.linear_run([sg.make_linear(xd, wd, yd)], M, ws, variant=variant, waves=waves)
    torch.cuda.synchronize()
    return yd


def run_fp8(x, q, s, M, N, variant=sg.VARIANT_AUTO, waves=0, ws=None):
    xd, qd, sd, yd = dev_bf16(x), dev_u8(q), dev_f32(s), out(M, N)
    ws = workspace(M, N, x.shape[1], sg.FP8_BS128) if ws is None else ws
    sg.linear_run([sg.make_linear(xd, qd, yd, w_scale=sd)], M, ws, variant=variant, waves=waves)
    torch.cuda.synchronize()
    return yd


def assert_matches_oracle(y_dev, y_ref, a, what=""):
    """Every output within 2e-3 A + 1e-6 of the oracle, or one of the two bf16
    values around the exact result (oracle.check)."""
    ok, worst, idx = oracle.check(host_values(y_dev), y_ref, a)
    assert ok, f"{what}: worst err/bound {worst:.3g} at {idx}"
    return worst


def variants_for(M):
    return [sg.VARIANT_VECTOR, sg.VARIANT_MFMA] if M <= 8 else [sg.VARIANT_MFMA]
