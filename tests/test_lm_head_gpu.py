"""The greedy next token on the device: skinny_argmax_bf16 against the
oracle's argmax on host-made logits (exact: the smallest index of the largest
bf16 value), and skinny_lm_head_argmax at the full vocabulary against the fp64
oracle (logits within the stated bound; the chosen token one the bound
allows, which is the exact winner whenever it leads by more than the bound)."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_amd as sg
import oracle
from gemv_skinny_gemm_amd import synth, workloads as wl
from tests.gpu_util import assert_matches_oracle, dev_bf16, host_codes, host_values, need_gpu, out

pytestmark = pytest.mark.gpu

BF16_ONE = 0x3F80


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def logits_codes(M, N, seed, distinct=17):
    """bf16 codes drawn from a few values (many ties), with NaN and +-inf sprinkled."""
    rng = np.random.default_rng(seed)
    vals = torch.tensor(rng.normal(size=distinct), dtype=torch.float64).to(torch.bfloat16)
    codes = vals.view(torch.int16).numpy().view(np.uint16)[rng.integers(0, distinct, (M, N))]
    flat = codes.reshape(-1)
    k = max(1, flat.size // 997)
    flat[rng.integers(0, flat.size, k)] = 0x7FC0            # NaN
    flat[rng.integers(0, flat.size, k)] = 0xFF80            # -inf
    if flat.size > 50:
        flat[rng.integers(0, flat.size, 1)] = 0x7F80        # +inf somewhere
    return codes


def bf16_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


@pytest.mark.parametrize("M,N", [(1, 1), (1, 7), (3, 8), (16, 1000), (2, 152064), (5, 100003)])
@pytest.mark.parametrize("aligned", [True, False])
def test_argmax_matches_oracle_exactly(M, N, aligned):
    codes = logits_codes(M, N, seed=M * 7919 + N)
    want = oracle.argmax_first(bf16_values(codes))
    flat = np.zeros(M * N + 8, np.uint16)
    off = 0 if aligned else 1                               # 2-byte aligned only: scalar path
    flat[off:off + M * N] = codes.reshape(-1)
    dev = dev_bf16(flat)
    y = dev[off:off + M * N].view(M, N)
    idx = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(sg.argmax_workspace_bytes(M, N), dtype=torch.uint8, device="cuda")
    sg.argmax_bf16(y, idx, ws)
    torch.cuda.synchronize()
    assert idx.cpu().numpy().tolist() == want.tolist()


NAN, NEG_INF = 0x7FC0, 0xFF80


@pytest.mark.parametrize("aligned", [True, False])
def test_argmax_nan_ranks_below_minus_infinity(aligned):
    """NaN loses to every number, -inf included, inside a slice of the first
    pass and across slices (a slice of NaNs against a later slice's -inf); a
    row of NaNs gives 0."""
    N = 9000                                                # three 4096-logit slices
    rows = []
    for head in ([NAN, NEG_INF], [NAN, NAN, NEG_INF, NEG_INF], [NEG_INF, NAN, NEG_INF], []):
        r = np.full(N, NAN, np.uint16)
        r[:len(head)] = head
        rows.append(r)
    r = np.full(N, NAN, np.uint16)
    r[5000] = NEG_INF                                       # the first number is in slice 1
    r[8999] = NEG_INF
    rows.append(r)
    r = np.full(N, NEG_INF, np.uint16)
    r[:4096] = NAN                                          # slice 0 all NaN
    rows.append(r)
    codes = np.stack(rows)
    M = codes.shape[0]
    want = oracle.argmax_first(bf16_values(codes))
    assert want.tolist() == [1, 2, 0, 0, 5000, 4096]
    flat = np.zeros(M * N + 8, np.uint16)
    off = 0 if aligned else 1
    flat[off:off + M * N] = codes.reshape(-1)
    y = dev_bf16(flat)[off:off + M * N].view(M, N)
    idx = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(sg.argmax_workspace_bytes(M, N), dtype=torch.uint8, device="cuda")
    sg.argmax_bf16(y, idx, ws)
    torch.cuda.synchronize()
    assert idx.cpu().numpy().tolist() == want.tolist()


@pytest.mark.parametrize("M", [1, 2])
def test_lm_head_fused_greedy_ties(M):
    """A vocabulary projection large enough for the row kernel's lean
    instance, whose epilogue leaves one greedy pair per workgroup and token
    (then one pass over the pairs): W row n = one-hot at column perm[n], and
    x drawn from a few values, so the logits x[:, perm] tie across many
    workgroups and the smallest index of the largest value must win."""
    N, K = 150000, 4096                                   # 1.2 GB of bf16 weights
    rng = np.random.default_rng(40 + M)
    perm = rng.integers(0, K, N)
    vals = torch.tensor(rng.normal(size=9), dtype=torch.float64).to(torch.bfloat16)
    x = vals.view(torch.int16).numpy().view(np.uint16)[rng.integers(0, 9, (M, K))]
    wd = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    wd[torch.arange(N, device="cuda"), torch.from_numpy(perm).cuda()] = 1.0
    xd, yd = dev_bf16(x), out(M, N)
    tok = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    lin = sg.make_linear(xd, wd, yd)
    ws = torch.empty(sg.lm_head_workspace_bytes(lin, M), dtype=torch.uint8, device="cuda")
    sg.lm_head_argmax(lin, M, tok, ws)
    torch.cuda.synchronize()
    logits = bf16_values(x[:, perm])
    assert np.array_equal(host_values(yd), logits)
    assert tok.cpu().numpy().tolist() == oracle.argmax_first(logits).tolist()
    del wd


def test_lm_head_one_hot_rows_pick_exactly():
    """W row n = one-hot at column perm[n]: the logits are x[:, perm] exactly,
    so the greedy token is decided exactly."""
    M, N, K = 3, 5000, 4096
    perm = np.random.default_rng(3).integers(0, K, N)
    x = synth.tensor_bf16(0, 51, M, K, 1.0)
    w = np.zeros((N, K), np.uint16)
    w[np.arange(N), perm] = BF16_ONE
    xd, wd, yd = dev_bf16(x), dev_bf16(w), out(M, N)
    tok = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    lin = sg.make_linear(xd, wd, yd)
    ws = torch.empty(sg.lm_head_workspace_bytes(lin, M), dtype=torch.uint8, device="cuda")
    sg.lm_head_argmax(lin, M, tok, ws)
    torch.cuda.synchronize()
    want = oracle.argmax_first(bf16_values(x[:, perm]))
    assert tok.cpu().numpy().tolist() == want.tolist()
    assert np.array_equal(host_values(yd), bf16_values(x[:, perm]))


@pytest.mark.parametrize("dtype,M", [(wl.BF16, 1), (wl.BF16, 6), (wl.FP8_BS128, 1)])
def test_lm_head_full_vocabulary(dtype, M):
    """152064 x 8192 head, W ~ N(0, 0.02), x ~ N(0, 1), seed 0.  The weights are
    made on the GPU by the input generator; x and sampled rows (FP8: whole
    scale bands) are regenerated on the host and checked to be identical
    first, then the whole matrix is copied to the host for the oracle."""
    from gemv_skinny_gemm_amd.synth import gpu as sgpu
    spec = wl.lm_head(dtype)[0]
    sets, tensors = sgpu.materialise([spec], M)
    lin = sets[0][0]
    x_dev, w_dev, s_dev, y_dev = tensors[0][0]
    x = synth.tensor_bf16(0, spec.x_stream, M, spec.K, wl.X_SIGMA)
    assert np.array_equal(host_codes(x_dev), x)
    rows = [0, 1, 77777, spec.N - 1]
    if dtype == wl.BF16:
        w_host = synth.tensor_rows_bf16(0, spec.w_stream, rows, spec.K, wl.W_SIGMA)
        assert np.array_equal(host_codes(w_dev[rows]), w_host)
    else:
        for band in sorted(set(r // 128 for r in rows)):
            q, sc, r0 = synth.fp8_weight_bs128(0, spec.w_stream, spec.N, spec.K, wl.W_SIGMA, band, 1)
            assert np.array_equal(w_dev[r0:r0 + q.shape[0]].cpu().numpy(), q)
            assert np.array_equal(s_dev[band:band + 1].cpu().numpy(), sc)
    tok = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(sg.lm_head_workspace_bytes(lin, M), dtype=torch.uint8, device="cuda")
    sg.lm_head_argmax(lin, M, tok, ws)
    torch.cuda.synchronize()
    if dtype == wl.BF16:
        y_ref, a, _ = oracle.linear_bf16(x, host_codes(w_dev))
    else:
        y_ref, a, _ = oracle.linear_fp8_bs128(x, w_dev.cpu().numpy(), s_dev.cpu().numpy())
    assert_matches_oracle(y_dev, y_ref, a, f"lm_head dtype={dtype} M={M}")
    idx = tok.cpu().numpy().astype(np.int64)
    assert np.all((idx >= 0) & (idx < spec.N))
    assert np.all(oracle.greedy_valid(idx, y_ref, a)), (idx, oracle.argmax_first(y_ref))
    del tensors
