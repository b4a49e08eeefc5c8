"""The GPU twin of the input generator makes the same bytes as the numpy one."""
import numpy as np
import pytest
import torch

from gemv_skinny_gemm_amd import synth
from tests.gpu_util import host_codes, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    from gemv_skinny_gemm_amd.synth import gpu
    gpu.lib()


@pytest.mark.parametrize("sigma", [0.02, 1.0])
@pytest.mark.parametrize("start,count", [(0, 1), (0, 1000003), (5, 77), (123457, 65536 * 3 + 1)])
def test_normal_bf16_matches_numpy(sigma, start, count):
    from gemv_skinny_gemm_amd.synth import gpu
    t = torch.empty(count, dtype=torch.bfloat16, device="cuda")
    gpu.normal_bf16_(t, 3, 1234567, sigma, start=start)
    torch.cuda.synchronize()
    ref = synth.normal_bf16(3, 1234567, start, count, sigma)
    assert np.array_equal(host_codes(t), ref)


@pytest.mark.parametrize("N,K", [(300, 272), (128, 128), (1000, 3696), (7392, 1024)])
def test_quantize_bs128_matches_numpy(N, K):
    from gemv_skinny_gemm_amd.synth import gpu
    q, s = gpu.fp8_weight_bs128(9, 77, N, K)
    torch.cuda.synchronize()
    q_ref, s_ref, _ = synth.fp8_weight_bs128(9, 77, N, K)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_quantize_handles_zero_blocks_and_extremes():
    from gemv_skinny_gemm_amd.synth import gpu
    N, K = 256, 384
    w = synth.tensor_bf16(1, 2, N, K, 0.02)
    w[0:128, 0:128] = 0
    w[200, 300] = 0x4300                                   # 128.0: one huge weight
    w[201, 301] = 0x0001                                   # a subnormal
    wd = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    q, s = gpu.quantize_bs128(wd)
    q_ref, s_ref = synth.quantize_bs128(w)
    assert np.array_equal(s.cpu().numpy(), s_ref) and np.array_equal(q.cpu().numpy(), q_ref)
