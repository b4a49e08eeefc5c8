"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each test fixes the oracle to something the pages or the mathematics decide:
the pages' printed worked examples, exact rational brute force, a library
routine (torch's fp64 matmul and its bf16 / float8_e4m3fn decoders), closed
forms and special cases (identity, permutation, constants)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from gemv_skinny_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

BF16_ONE = 0x3F80


def bf16_codes_of(values):
    """Exact bf16 codes of values that bf16 represents exactly (via torch)."""
    t = torch.tensor(np.asarray(values, np.float64), dtype=torch.float64)
    b = t.to(torch.bfloat16)
    assert torch.equal(b.to(torch.float64), t), "value not exact in bf16"
    return b.view(torch.int16).numpy().view(np.uint16)


def e4m3_codes_of(values):
    t = torch.tensor(np.asarray(values, np.float64), dtype=torch.float64)
    f = t.to(torch.float8_e4m3fn)
    assert torch.equal(f.to(torch.float64), t), "value not exact in e4m3"
    return f.view(torch.uint8).numpy()


def torch_bf16_values(codes):
    c = torch.from_numpy(np.ascontiguousarray(codes, np.uint16).view(np.int16))
    return c.view(torch.bfloat16).to(torch.float64)


def torch_e4m3_values(codes):
    c = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64)


# --- number formats ---------------------------------------------------------

def test_bf16_decode_matches_torch_on_all_codes():
    lib = oracle._load()
    mine = np.array([lib.oracle_bf16_value(c) for c in range(65536)])
    ref = torch_bf16_values(np.arange(65536, dtype=np.uint32).astype(np.uint16)).numpy()
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.all(both_nan | (mine == ref))
    assert np.array_equal(np.signbit(mine[~both_nan]), np.signbit(ref[~both_nan]))


def test_e4m3_decode_matches_torch_and_spec():
    mine = np.array([oracle.e4m3_value(c) for c in range(256)])
    ref = torch_e4m3_values(np.arange(256, dtype=np.uint8)).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(mine[~nan], ref[~nan])
    # Anchors of the OCP E4M3FN definition.
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0xFE) == -448.0
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3_value(0x01) == 2.0 ** -9


# --- brute force in exact rationals -----------------------------------------

def _exact_linear(xv, wv):
    """Exact rational y and A from fp64 input values (each exactly representable)."""
    M, K = xv.shape
    N = wv.shape[0]
    xf = [[Fraction(float(v)) for v in row] for row in xv]
    wf = [[Fraction(float(v)) for v in row] for row in wv]
    y = [[sum((xf[m][k] * wf[n][k] for k in range(K)), Fraction(0)) for n in range(N)]
         for m in range(M)]
    a = [[sum((abs(xf[m][k] * wf[n][k]) for k in range(K)), Fraction(0)) for n in range(N)]
         for m in range(M)]
    return y, a


def _assert_close_to_exact(y, a, y_ex, a_ex, K):
    M, N = y.shape
    for m in range(M):
        for n in range(N):
            ab = float(a_ex[m][n])
            # K-term left-to-right fp64 sum: error at most K * 2^-53 * A.
            tol = K * 2.0 ** -52 * ab
            assert abs(Fraction(float(y[m, n])) - y_ex[m][n]) <= Fraction(tol)
            assert abs(a[m, n] - ab) <= tol


def test_bf16_linear_vs_exact_rationals():
    rng = np.random.default_rng(11)
    M, N, K = 3, 5, 37
    x = bf16_codes_of(torch.randn(M, K, generator=torch.Generator().manual_seed(1),
                                  dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy())
    w = rng.integers(0, 65536, size=(N, K)).astype(np.uint16)
    w[((w >> 7) & 0xFF) == 0xFF] = BF16_ONE                 # no inf/NaN codes
    y, a, _ = oracle.linear_bf16(x, w, threads=2)
    xv = torch_bf16_values(x).numpy()
    wv = torch_bf16_values(w).numpy()
    y_ex, a_ex = _exact_linear(xv, wv)
    # Wide exponent range: results differ from the exact sum only by fp64 rounding.
    _assert_close_to_exact(y, a, y_ex, a_ex, K)


def test_fp8_linear_vs_exact_rationals_with_partial_edge_blocks():
    rng = np.random.default_rng(12)
    M, N, K = 2, 130, 260                                   # 2 x 3 scale blocks, ragged edges
    x = bf16_codes_of(np.round(rng.standard_normal((M, K)) * 64) / 64)
    q = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38                              # no NaN codes
    s = (rng.uniform(0.5, 4.0, size=(2, 3)) * np.array([[1, 2, 4], [8, 16, 32]])).astype(np.float32)
    y, a, _ = oracle.linear_fp8_bs128(x, q, s, threads=3)
    xv = torch_bf16_values(x).numpy()
    wv = torch_e4m3_values(q).numpy() * np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:N, :K]
    y_ex, a_ex = _exact_linear(xv, wv)
    _assert_close_to_exact(y, a, y_ex, a_ex, K)


# --- a library routine: torch fp64 matmul ------------------------------------

def test_bf16_linear_vs_torch_matmul():
    g = torch.Generator().manual_seed(3)
    M, N, K = 4, 300, 520
    xt = torch.randn(M, K, generator=g).to(torch.bfloat16)
    wt = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16)
    x = xt.view(torch.int16).numpy().view(np.uint16)
    w = wt.view(torch.int16).numpy().view(np.uint16)
    y, a, _ = oracle.linear_bf16(x, w)
    ref = (xt.double() @ wt.double().T).numpy()
    ref_a = (xt.double().abs() @ wt.double().abs().T).numpy()
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * ref_a.max())
    assert np.allclose(a, ref_a, rtol=1e-13, atol=0)


def test_fp8_linear_vs_torch_matmul():
    M, N, K = 6, 300, 520
    x = synth.tensor_bf16(0, 5, M, K, 1.0)
    w = synth.tensor_bf16(0, 6, N, K, 0.02)
    q, s = synth.quantize_bs128(w)
    y, a, _ = oracle.linear_fp8_bs128(x, q, s)
    xv = torch_bf16_values(x)
    full = torch.from_numpy(s.astype(np.float64)).repeat_interleave(128, 0).repeat_interleave(128, 1)
    wv = torch_e4m3_values(q) * full[:N, :K]
    ref = (xv @ wv.T).numpy()
    ref_a = (xv.abs() @ wv.abs().T).numpy()
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * ref_a.max())
    assert np.allclose(a, ref_a, rtol=1e-13, atol=0)


def test_scale_index_is_row_block_then_col_block():
    # One nonzero scale block tells a swapped (k-block, n-block) index apart.
    M, N, K = 1, 256, 384
    x = np.full((M, K), BF16_ONE, np.uint16)
    q = np.full((N, K), 0x38, np.uint8)                       # every weight code = 1.0
    s = np.zeros((2, 3), np.float32)
    s[0, 2] = 2.0                                             # rows 0..127, cols 256..383
    y, _, _ = oracle.linear_fp8_bs128(x, q, s)
    assert np.array_equal(y[0, :128], np.full(128, 256.0))
    assert np.array_equal(y[0, 128:], np.zeros(128))


# --- special cases and closed forms -------------------------------------------

def test_identity_bf16_and_fp8():
    K = 256
    x = synth.tensor_bf16(0, 7, 3, K, 1.0)
    w = np.zeros((K, K), np.uint16)
    w[np.arange(K), np.arange(K)] = BF16_ONE
    y, _, _ = oracle.linear_bf16(x, w)
    assert np.array_equal(y, torch_bf16_values(x).numpy())
    q = np.zeros((K, K), np.uint8)
    q[np.arange(K), np.arange(K)] = 0x38
    y8, _, _ = oracle.linear_fp8_bs128(x, q, np.ones((2, 2), np.float32))
    assert np.array_equal(y8, torch_bf16_values(x).numpy())


def test_permutation_bf16():
    K, N = 192, 100
    rng = np.random.default_rng(5)
    perm = rng.permutation(K)[:N]
    x = synth.tensor_bf16(0, 8, 2, K, 1.0)
    w = np.zeros((N, K), np.uint16)
    w[np.arange(N), perm] = BF16_ONE
    y, _, _ = oracle.linear_bf16(x, w)
    assert np.array_equal(y, torch_bf16_values(x).numpy()[:, perm])


def test_constant_closed_form():
    K = 8192
    x = np.full((2, K), 0x3F00, np.uint16)                   # 0.5
    w = np.full((3, K), 0x3E00, np.uint16)                   # 0.125
    y, a, _ = oracle.linear_bf16(x, w)
    assert np.all(y == K * 0.5 * 0.125) and np.all(a == 512.0)
    q = np.full((3, K), 0x30, np.uint8)                      # e4m3 0.5
    s = np.full((1, K // 128), 0.25, np.float32)             # weight 0.125
    y8, _, _ = oracle.linear_fp8_bs128(x, q, s)
    assert np.all(y8 == 512.0)
    x[1] = 0xBF00                                            # -0.5: sign carried through
    y, a, _ = oracle.linear_bf16(x, w)
    assert np.all(y[1] == -512.0) and np.all(a[1] == 512.0)


# --- the pages' printed worked examples --------------------------------------

def test_page_example_column_split():
    d = json.load(open(os.path.join(GOLDEN, "p2_ex2_column_split.json")))
    x = np.array(d["x"], np.float64)
    w_kn = np.array([[((6 * i + j) % 5) - 2 for j in range(6)] for i in range(4)], np.float64)
    assert w_kn.tolist() == d["w_kn"]
    w = w_kn.T                                                  # N x K
    y, _, _ = oracle.linear_bf16(bf16_codes_of(x), bf16_codes_of(w))
    assert y.tolist() == d["y_printed"]
    # Each device's column block is the same product on a slice of W's rows.
    y0, _, _ = oracle.linear_bf16(bf16_codes_of(x), bf16_codes_of(w[:3]))
    y1, _, _ = oracle.linear_bf16(bf16_codes_of(x), bf16_codes_of(w[3:]))
    assert y0.tolist() == d["device0_printed"] and y1.tolist() == d["device1_printed"]
    # FP8 path: the weights -2..2 are exact e4m3 codes; scale 1.
    y8, _, _ = oracle.linear_fp8_bs128(bf16_codes_of(x), e4m3_codes_of(w), np.ones((1, 1), np.float32))
    assert y8.tolist() == d["y_printed"]


def test_page_example_split_k_partials():
    d = json.load(open(os.path.join(GOLDEN, "p2_ex3_mlp_split.json")))
    x = np.array(d["x"], np.float64)
    a_mat = np.array([[((8 * i + j) % 7) - 3 for j in range(8)] for i in range(4)], np.float64)
    b_mat = np.array([[((4 * i + j) % 5) - 2 for j in range(4)] for i in range(8)], np.float64)
    pre, _, _ = oracle.linear_bf16(bf16_codes_of(x), bf16_codes_of(a_mat.T))
    h = np.maximum(pre, 0.0)                                  # the example's ReLU
    wb = b_mat.T                                              # N x K = 4 x 8
    p0, _, _ = oracle.linear_bf16(bf16_codes_of(h[:, :4]), bf16_codes_of(wb[:, :4]))
    p1, _, _ = oracle.linear_bf16(bf16_codes_of(h[:, 4:]), bf16_codes_of(wb[:, 4:]))
    full, _, _ = oracle.linear_bf16(bf16_codes_of(h), bf16_codes_of(wb))
    assert p0.tolist() == d["partial0_printed"]
    assert p1.tolist() == d["partial1_printed"]
    assert (p0 + p1).tolist() == d["sum_printed"]
    assert full.tolist() == d["sum_printed"]


# --- the tolerance check -------------------------------------------------------

def test_check_accepts_inside_and_rejects_outside_bound():
    y_ref = np.array([[1.0, -2.0, 0.0]])
    a = np.array([[10.0, 10.0, 0.0]])
    ok, worst, _ = oracle.check(y_ref + np.array([[0.0199, -0.0199, 0.9e-6]]), y_ref, a)
    assert ok and worst < 1.0
    ok, worst, idx = oracle.check(y_ref + np.array([[0.0, 0.0211, 0.0]]), y_ref, a)
    assert not ok and idx == (0, 1)
    ok, worst, idx = oracle.check(y_ref + np.array([[-0.0211, 0.0, 0.0]]), y_ref, a)
    assert not ok and idx == (0, 0)                 # an error below y_ref counts as much
    # Exactly at the bound is inside: A = 0 leaves the absolute term, 1e-6.
    ok, worst, _ = oracle.check(np.array([[1e-6, -1e-6]]), np.zeros((1, 2)), np.zeros((1, 2)))
    assert ok and worst == 1.0


def test_threads_do_not_change_results():
    x = synth.tensor_bf16(0, 9, 4, 1000, 1.0)
    w = synth.tensor_bf16(0, 10, 77, 1000, 0.02)
    y1, a1, t1 = oracle.linear_bf16(x, w, threads=1)
    y5, a5, t5 = oracle.linear_bf16(x, w, threads=5)
    assert t1 == 1 and t5 == 5
    assert np.array_equal(y1, y5) and np.array_equal(a1, a5)


def test_empty_shapes():
    y, a, _ = oracle.linear_bf16(np.zeros((2, 0), np.uint16), np.zeros((3, 0), np.uint16))
    assert y.shape == (2, 3) and np.all(y == 0) and np.all(a == 0)


def _all_finite_bf16():
    """Every finite bf16 value, sorted (decoded by torch, not the oracle)."""
    codes = np.arange(0x10000, dtype=np.uint32)
    v = torch.from_numpy((codes << 16).astype(np.uint32).view(np.int32)).view(torch.float32)
    v = v.double().numpy()
    return np.unique(v[np.isfinite(v)])


def test_bf16_bracket_is_the_pair_of_neighbours():
    """Brute force against the sorted table of every finite bf16 value: lo is
    the largest value <= v, hi the smallest >= v; torch's round-to-nearest
    result is one of them."""
    table = _all_finite_bf16()
    rng = np.random.default_rng(2)
    v = rng.standard_normal(20000) * 2.0 ** rng.integers(-130, 120, 20000)
    v = np.concatenate([v, table[rng.integers(0, len(table), 2000)], [0.0, -0.0, 1.0, -1.0]])
    lo, hi = oracle.bf16_bracket(v)
    want_hi = table[np.searchsorted(table, v, side="left")]
    want_lo = table[np.searchsorted(table, v, side="right") - 1]
    assert np.array_equal(lo, want_lo) and np.array_equal(hi, want_hi)
    r = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    assert np.all((r == lo) | (r == hi))


def test_check_accepts_the_bf16_neighbours_and_nothing_further():
    """y_ref = 0.07497585 with A = 0.09527504: the stated bound (1.92e-4) is
    below the distance to either bf16 neighbour (0.07470703125 below,
    0.0751953125 above, step 2^-11 there), so exactly those two pass, the
    values one step further do not, and the same holds mirrored."""
    step = 2.0 ** -11
    lo_v, hi_v = 0.07470703125, 0.0751953125
    for sign in (1.0, -1.0):
        y_ref = np.array([[sign * 0.07497585]])
        a = np.array([[0.09527504]])
        for y, want in ((hi_v, True), (lo_v, True), (hi_v + step, False), (lo_v - step, False)):
            ok, _, _ = oracle.check(np.array([[sign * y]]), y_ref, a)
            assert ok == want, (sign, y)
    # A bf16-valued y_ref: only itself, when the bound is below the step.
    y_ref = np.array([[hi_v, -hi_v]])
    a = np.full((1, 2), 0.05)
    assert oracle.check(y_ref, y_ref, a)[0]
    assert not oracle.check(y_ref + np.array([[step, 0.0]]), y_ref, a)[0]
    assert not oracle.check(y_ref - np.array([[0.0, step]]), y_ref, a)[0]


# --- greedy next token ------------------------------------------------------

def test_argmax_first_fixed_cases():
    inf, nan = np.inf, np.nan
    cases = [([[1.0, 3.0, 3.0, 2.0]], [1]),            # ties: the first
             ([[nan, -inf, -5.0]], [2]),                # NaN below every number
             ([[nan, -inf]], [1]),                      # ... -inf included
             ([[nan, nan, -inf, -inf]], [2]),
             ([[-inf, nan, -inf]], [0]),
             ([[nan, nan]], [0]),                       # a row of NaNs
             ([[-inf, -inf, -inf]], [0]),
             ([[0.0, -0.0]], [0]),                      # -0 == +0: the first
             ([[5.0], [-1.0]], [0, 0]),
             ([[1.0, 2.0, inf, inf, nan]], [2])]
    for v, want in cases:
        assert oracle.argmax_first(np.array(v)).tolist() == want


def test_argmax_first_matches_numpy_on_random_rows():
    rng = np.random.default_rng(11)
    v = rng.integers(-20, 20, size=(7, 5000)).astype(np.float64)   # many ties
    assert oracle.argmax_first(v).tolist() == np.argmax(v, axis=1).tolist()


def test_greedy_valid_admits_only_the_winner_when_the_gap_is_wide():
    y_ref = np.array([[1.0, 5.0, 4.9, -2.0]])
    a = np.array([[1.0, 1.0, 1.0, 1.0]])              # bounds 2e-3 + half a bf16 ulp (1/64 at 5)
    assert oracle.greedy_valid(np.array([1]), y_ref, a).tolist() == [True]
    assert oracle.greedy_valid(np.array([2]), y_ref, a).tolist() == [False]
    wide = np.array([[1.0, 5000.0, 5000.0, 1.0]])     # bounds of 10: 4.9 is within reach
    assert oracle.greedy_valid(np.array([2]), y_ref, wide).tolist() == [True]
    assert oracle.greedy_valid(np.array([3]), y_ref, wide).tolist() == [False]
    # 5.0 and 4.99 round to the same bf16 output (spacing 1/32 there), so the
    # runner-up is admissible: the bound carries half an ulp of each.
    close = np.array([[5.0, 4.99]])
    assert oracle.greedy_valid(np.array([1]), close, np.ones((1, 2))).tolist() == [True]
    two = np.array([[5.0, 1.0], [1.0, 2.0]])          # each row takes its own maximum
    assert oracle.greedy_valid(np.array([0, 1]), two, np.ones((2, 2))).tolist() == [True, True]
    assert oracle.greedy_valid(np.array([1, 0]), two, np.ones((2, 2))).tolist() == [False, False]


# --- the gated MLP's activation ---------------------------------------------

def test_bf16_encode_is_the_nearest_code_ties_to_even():
    """Brute force over every finite bf16 value: the nearest one, the even code
    on a tie (halfway points included on purpose)."""
    lib = oracle._load()
    codes = np.arange(0, 0x7F80, dtype=np.uint32)                    # +0 .. largest finite
    vals = np.array([lib.oracle_bf16_value(int(c)) for c in codes])
    rng = np.random.default_rng(21)
    picks = rng.integers(1, len(vals) - 1, 4000)
    mids = (vals[picks] + vals[picks + 1]) / 2                        # exact halfway points
    rand = np.exp(rng.uniform(np.log(1e-40), np.log(3e38), 4000))
    probe = np.concatenate([mids, rand, vals[picks], [0.0, 2.0 ** -133, 1.5 * 2.0 ** -133]])
    for v in probe:
        d = np.abs(vals - v)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        got = int(oracle.bf16_encode(np.array([v]))[0])
        assert got == int(codes[want]), (v, hex(got), hex(int(codes[want])))
        assert int(oracle.bf16_encode(np.array([-v]))[0]) == (got | 0x8000)
    assert oracle.bf16_encode(np.array([1e39, np.nan])).tolist() == [0x7F80, 0x7FC0]


def test_silu_closed_forms():
    v = np.linspace(-30, 30, 601)
    assert np.allclose(oracle.silu(v) - oracle.silu(-v), v, rtol=0, atol=1e-12)   # silu(v) - silu(-v) = v
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([40.0]))[0] - 40.0) < 1e-15
    assert abs(oracle.silu(np.array([-800.0]))[0]) < 1e-300                     # no overflow error
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + np.e ** -1)) < 1e-15


def test_mlp_swiglu_matches_a_direct_computation():
    """Small MLP against fractions-free direct fp64 algebra on exact inputs:
    x and W with few bits make every product and sum exact."""
    rng = np.random.default_rng(23)
    M, H, I = 2, 16, 8
    x = bf16_codes_of(rng.integers(-4, 5, (M, H)) / 4)
    wg = bf16_codes_of(rng.integers(-4, 5, (2 * I, H)) / 8)
    wd = bf16_codes_of(rng.integers(-4, 5, (H, I)) / 8)
    y, a, h = oracle.mlp_swiglu(x, wg, wd)
    xv, wgv, wdv = (torch_bf16_values(c).numpy() for c in (x, wg, wd))
    gu = xv @ wgv.T                                        # exact: few-bit operands
    hv = oracle.silu(gu[:, :I]) * gu[:, I:]
    hb = torch_bf16_values(oracle.bf16_encode(hv)).numpy()
    assert np.array_equal(h, oracle.bf16_encode(hv))
    assert np.allclose(y, hb @ wdv.T, rtol=1e-14, atol=1e-14)
    assert np.allclose(a, np.abs(hb) @ np.abs(wdv).T, rtol=1e-14, atol=1e-14)


def test_mlp_rounds_gate_and_up_to_bf16():
    """g and u are bf16 activations before the SiLU gate: with g = 1 + 2^-9
    exactly (x = [1, 2^-9] against a gate row [1, 1]) and u = 1, bf16(g) = 1
    and h = bf16(silu(1)) = 0.73046875, where an unrounded g would give
    bf16(silu(1 + 2^-9)) = 0.734375; swapping the roles (u = 1 + 2^-9, g = 1)
    pins the rounding of u the same way (bf16(silu(1) (1 + 2^-9)) = 0.734375)."""
    x = bf16_codes_of(np.array([[1.0, 2.0 ** -9]]))
    wd = bf16_codes_of(np.array([[1.0], [2.0]]))                 # H = 2, I = 1
    for gate, up in (([1.0, 1.0], [1.0, 0.0]), ([1.0, 0.0], [1.0, 1.0])):
        wg = bf16_codes_of(np.array([gate, up]))                 # [2I][H]: gate row, then up
        y, a, h = oracle.mlp_swiglu(x, wg, wd)
        assert torch_bf16_values(h).numpy().tolist() == [[0.73046875]]
        assert y.tolist() == [[0.73046875, 1.4609375]]


# --- mixture-of-experts linear ---------------------------------------------

def _moe_exact(xv, ids, wv, x_per_route):
    """Route-by-route exact rational products (Fractions) and |.| sums."""
    T, topk = ids.shape
    E, N, K = wv.shape
    y, a = [], []
    for t in range(T):
        for j in range(topk):
            r = t * topk + j
            e = int(ids[t, j])
            if not 0 <= e < E:
                y.append([Fraction(0)] * N)
                a.append([Fraction(0)] * N)
                continue
            xr = xv[r] if x_per_route else xv[t]
            y.append([sum(Fraction(float(xr[k])) * Fraction(float(wv[e, n, k])) for k in range(K))
                      for n in range(N)])
            a.append([sum(abs(Fraction(float(xr[k])) * Fraction(float(wv[e, n, k]))) for k in range(K))
                      for n in range(N)])
    return y, a


@pytest.mark.parametrize("x_per_route", [False, True])
def test_moe_linear_vs_exact_rationals_bf16(x_per_route):
    """Every route against its expert by brute force, with a duplicate expert
    in one token, an expert no token picks, and ids outside [0, E)."""
    rng = np.random.default_rng(31)
    T, topk, E, N, K = 3, 3, 4, 5, 24
    ids = np.array([[2, 0, 2], [-1, 1, 0], [0, 4, 1]], np.int32)   # expert 3 unused
    x = bf16_codes_of(np.round(rng.standard_normal((T * topk if x_per_route else T, K)) * 32) / 32)
    w = rng.integers(0, 65536, size=(E, N, K)).astype(np.uint16)
    w[((w >> 7) & 0xFF) == 0xFF] = BF16_ONE
    y, a = oracle.moe_linear(x, ids, w, x_per_route=x_per_route, threads=2)
    y_ex, a_ex = _moe_exact(torch_bf16_values(x).numpy(), ids,
                            torch_bf16_values(w.reshape(E * N, K)).numpy().reshape(E, N, K),
                            x_per_route)
    _assert_close_to_exact(y, a, y_ex, a_ex, K)
    assert not y[3].any() and not y[7].any() and not a[3].any()    # ids -1 and 4


def test_moe_linear_vs_exact_rationals_fp8_own_scales():
    """FP8 experts, each with its own block scales (two K blocks, ragged N)."""
    rng = np.random.default_rng(32)
    T, topk, E, N, K = 2, 2, 3, 130, 256
    ids = np.array([[1, 2], [2, 0]], np.int32)
    x = bf16_codes_of(np.round(rng.standard_normal((T, K)) * 16) / 16)
    q = rng.integers(0, 256, size=(E, N, K)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38
    s = rng.uniform(0.25, 4.0, size=(E, 2, 2)).astype(np.float32)
    s *= np.array([1, 2, 4], np.float32)[:, None, None]            # experts' scales differ
    y, a = oracle.moe_linear(x, ids, q, scales=s, threads=3)
    wv = torch_e4m3_values(q.reshape(E * N, K)).numpy().reshape(E, N, K)
    wv = wv * np.repeat(np.repeat(s.astype(np.float64), 128, 1), 128, 2)[:, :N, :K]
    y_ex, a_ex = _moe_exact(torch_bf16_values(x).numpy(), ids, wv, False)
    _assert_close_to_exact(y, a, y_ex, a_ex, K)


def test_moe_linear_scaled_identity_experts():
    """Expert e = (e + 1) I: each route returns its token row times e + 1, bit
    for bit (shared x), and its own row (x per route)."""
    T, topk, E, K = 4, 2, 3, 16
    ids = np.array([[0, 2], [1, 0], [2, 1], [0, 1]], np.int32)
    w = np.stack([bf16_codes_of(np.eye(K) * (e + 1)) for e in range(E)])
    x = bf16_codes_of(np.arange(T * K).reshape(T, K) / 64 - 1)
    y, _ = oracle.moe_linear(x, ids, w)
    xv = torch_bf16_values(x).numpy()
    want = np.stack([xv[t] * (ids[t, j] + 1) for t in range(T) for j in range(topk)])
    assert np.array_equal(y, want)
    xr = bf16_codes_of(np.arange(T * topk * K).reshape(T * topk, K) / 128 - 1)
    y, _ = oracle.moe_linear(xr, ids, w, x_per_route=True)
    xrv = torch_bf16_values(xr).numpy()
    assert np.array_equal(y, xrv * (ids.reshape(-1, 1) + 1))


def test_moe_linear_relabelled_experts_give_the_same_routes():
    rng = np.random.default_rng(33)
    T, topk, E, N, K = 5, 2, 6, 7, 32
    ids = synth.route_topk(0, 77, T, E, topk)
    x = synth.tensor_bf16(0, 78, T, K, 1.0)
    w = synth.tensor_bf16(0, 79, E * N, K, 0.02).reshape(E, N, K)
    perm = rng.permutation(E)                                       # expert e becomes perm[e]
    w2 = np.empty_like(w)
    w2[perm] = w
    y1, a1 = oracle.moe_linear(x, ids, w)
    y2, a2 = oracle.moe_linear(x, perm[ids], w2)
    assert np.array_equal(y1, y2) and np.array_equal(a1, a2)


def test_moe_linear_swiglu_input_per_route():
    """Down projection of the experts: route r's input is bf16(silu(g) u) of
    its own row [g | u]; few-bit values keep the products exact."""
    rng = np.random.default_rng(34)
    T, topk, E, N, I = 2, 2, 3, 4, 8
    ids = np.array([[2, 0], [0, 1]], np.int32)
    gu = bf16_codes_of(rng.integers(-8, 9, (T * topk, 2 * I)) / 4)
    w = bf16_codes_of(rng.integers(-4, 5, (E * N, I)) / 8).reshape(E, N, I)
    y, _ = oracle.moe_linear(gu, ids, w, x_per_route=True, swiglu=True)
    g = torch_bf16_values(gu[:, :I]).numpy()
    u = torch_bf16_values(gu[:, I:]).numpy()
    h = torch_bf16_values(oracle.bf16_encode(g / (1 + np.exp(-g)) * u)).numpy()
    wv = torch_bf16_values(w.reshape(E * N, I)).numpy().reshape(E, N, I)
    want = np.stack([h[r] @ wv[ids.reshape(-1)[r]].T for r in range(T * topk)])
    assert np.allclose(y, want, rtol=1e-14, atol=1e-14)


def test_route_topk_picks_distinct_best_experts():
    ids = synth.route_topk(0, 91, 64, 8, 2)
    assert ids.shape == (64, 2) and ids.dtype == np.int32
    assert all(len(set(r)) == 2 for r in ids.tolist())
    counts = np.bincount(ids.ravel(), minlength=8)
    assert counts.sum() == 128 and counts[:2].min() > counts[2:].max() // 2
