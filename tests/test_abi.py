"""The C-ABI library loads, exports every entry point its header declares, and
rejects bad arguments on the host before touching the GPU (no compute here)."""
import ctypes
import os
import re

import pytest

import gemv_skinny_gemm_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skinny_gemm.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
A = 0x100000          # aligned fake device addresses: never dereferenced by these tests
B = 0x2000000
C = 0x4000000
WS = 0x8000000


def header_define(name):
    m = re.search(r"#define\s+%s\s+(\d+)" % name, open(HEADER).read())
    return int(m.group(1))


MIN_WORKSPACE = header_define("SKINNY_MIN_WORKSPACE_BYTES")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["skinny_workspace_bytes", "skinny_stack_workspace_bytes", "skinny_gemm_bf16",
                 "skinny_gemm_fp8_bs128", "decode_linear_stack", "skinny_linear_run",
                 "skinny_plan_query", "skinny_status_string", "skinny_abi_version",
                 "skinny_launch_count", "skinny_linear_run_timed", "skinny_band_rows"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(sg.lib_path())
    for name in declared_functions():
        assert hasattr(L, name), name


def test_abi_version_and_status_strings():
    assert sg.abi_version() == sg.ABI_VERSION
    assert sg.status_string(0) == "ok"
    for s in range(1, 5):
        assert sg.status_string(s) and sg.status_string(s) != "unknown status"
    assert sg.status_string(99) == "unknown status"


def test_workspace_bytes_is_host_arithmetic():
    # Split-K partial slots: fp32 [slot][M][rows of a row group], one slot per
    # K-chunk of every row group of a split linear.
    one = sg.workspace_bytes(sg.BF16, 4, 1280, 8192)
    assert one > MIN_WORKSPACE and one % (4 * 4 * 64) == 0
    # Proportional to the rows when N is a multiple of every row-group height,
    assert sg.workspace_bytes(sg.BF16, 4, 2560, 8192) == 2 * one
    # never below the minimum, growing with M,
    assert sg.workspace_bytes(sg.BF16, 1, 64, 64) == MIN_WORKSPACE
    for dt in (sg.BF16, sg.FP8_BS128):
        sizes = [sg.workspace_bytes(dt, M, 7392, 8192) for M in range(1, 17)]
        assert sizes == sorted(sizes) and sizes[-1] > sizes[0]
    # and a launch group needs the sum over its linears.
    lins = [sg.Linear(sg.BF16, 1280, 8192, 0, A, None, B, C)] * 3
    assert sg.stack_workspace_bytes(lins, 4) == 3 * one
    assert sg.workspace_bytes(sg.BF16, 0, 1, 8) == 0
    assert sg.workspace_bytes(sg.BF16, 17, 1, 8) == 0
    assert sg.workspace_bytes(7, 1, 1, 8) == 0


def test_table_launch_workspace():
    """A launch of more linears than the kernel arguments hold also needs
    room for its descriptor table and for its partial sums at the largest
    grid; it never needs less than its launches of 32 would."""
    tiny = [sg.Linear(sg.BF16, 16, 64, 0, A, None, B, C)]
    assert sg.stack_workspace_bytes(tiny * 32, 1) == MIN_WORKSPACE        # no split, no table
    t33, t66 = sg.stack_workspace_bytes(tiny * 33, 1), sg.stack_workspace_bytes(tiny * 66, 1)
    assert MIN_WORKSPACE < t33 < t66 and t66 - t33 == 33 * (t33 // 33)  # the table only
    shapes = [(10240, 8192), (8192, 8192), (59136, 8192), (8192, 29568)]
    for dt in (sg.BF16, sg.FP8_BS128):
        scale = None if dt == sg.BF16 else 0x300000
        stack = [sg.Linear(dt, N, K, 0, A, scale, B, C) for N, K in shapes] * 80
        for M in (1, 2, 6, 8, 16):
            full = sg.stack_workspace_bytes(stack, M)
            assert full >= sg.stack_workspace_bytes(stack[:32], M) and full >= 320 * 64


def bf16_call(x=B, w=A, y=C, M=1, N=64, K=64, ws=WS, wsb=None):
    wsb = sg.workspace_bytes(sg.BF16, max(M, 1), 64, 64) if wsb is None else wsb
    return sg.lib().skinny_gemm_bf16(x, w, y, M, N, K, ws, wsb, None)


def fp8_call(x=B, w=A, s=0x300000, y=C, M=1, N=64, K=64, ws=WS, wsb=None):
    wsb = sg.workspace_bytes(sg.FP8_BS128, max(M, 1), 64, 64) if wsb is None else wsb
    return sg.lib().skinny_gemm_fp8_bs128(x, w, s, y, M, N, K, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=0), INVALID), (dict(M=17), INVALID), (dict(N=0), INVALID), (dict(K=0), INVALID),
    (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(y=None), INVALID),
    (dict(K=12), UNSUPPORTED), (dict(w=A + 2), UNSUPPORTED), (dict(x=B + 8), UNSUPPORTED),
    (dict(y=C + 4), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(wsb=MIN_WORKSPACE - 1), WORKSPACE),
    (dict(ws=WS + 8), UNSUPPORTED),
    (dict(y=B), INVALID),                       # y overlaps x
    (dict(y=A + 64), INVALID),                  # y inside W
    (dict(y=WS + 128), INVALID),                # y inside the workspace
    (dict(x=WS + 128), INVALID),                # x inside the workspace
    (dict(w=WS - 64), INVALID),                 # W runs into the workspace
])
def test_bf16_rejects_bad_arguments(kw, status):
    assert bf16_call(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(s=None), INVALID), (dict(K=24), UNSUPPORTED), (dict(s=0x300002), UNSUPPORTED),
    (dict(M=17), INVALID), (dict(wsb=0), WORKSPACE),
    (dict(s=WS + 64), INVALID),                 # scales inside the workspace
])
def test_fp8_rejects_bad_arguments(kw, status):
    assert fp8_call(**kw) == status


def test_stack_rejects_bad_arguments():
    L = sg.lib()
    good = sg.Linear(sg.BF16, 64, 64, 0, A, None, B, C)
    arr = (sg.Linear * 2)(good, sg.Linear(sg.BF16, 64, 64, 0, A, None, B, C))   # same y twice
    wsb = sg.workspace_bytes(sg.BF16, 1, 64, 64)
    assert L.decode_linear_stack(arr, 2, 1, WS, wsb, None) == INVALID
    assert L.decode_linear_stack(arr, 0, 1, WS, wsb, None) == INVALID
    assert L.decode_linear_stack(None, 1, 1, WS, wsb, None) == INVALID
    bad_dtype = (sg.Linear * 1)(sg.Linear(5, 64, 64, 0, A, None, B, C))
    assert L.decode_linear_stack(bad_dtype, 1, 1, WS, wsb, None) == INVALID
    reserved = (sg.Linear * 1)(sg.Linear(sg.BF16, 64, 64, 1, A, None, B, C))
    assert L.decode_linear_stack(reserved, 1, 1, WS, wsb, None) == INVALID
    scale_on_bf16 = (sg.Linear * 1)(sg.Linear(sg.BF16, 64, 64, 0, A, 0x300000, B, C))
    assert L.decode_linear_stack(scale_on_bf16, 1, 1, WS, wsb, None) == INVALID
    plan = sg.Plan(9, 0)
    one = (sg.Linear * 1)(good)
    assert L.skinny_linear_run(one, 1, 1, ctypes.byref(plan), WS, wsb, None) == INVALID
    plan = sg.Plan(sg.VARIANT_VECTOR, 0)
    wsb16 = sg.workspace_bytes(sg.BF16, 16, 64, 64)
    assert L.skinny_linear_run(one, 1, 16, ctypes.byref(plan), WS, wsb16, None) == UNSUPPORTED
    plan = sg.Plan(0, -1)
    assert L.skinny_linear_run(one, 1, 1, ctypes.byref(plan), WS, wsb, None) == INVALID


def test_noalloc_stack_rejects_before_any_device_call():
    """The allocation-free stack accepts a call only if its workspace bound
    fits the static buffer; argument and size errors come back before any
    device call (these fake addresses are never used)."""
    L = sg.lib()
    m = re.search(r"#define\s+SKINNY_STATIC_SCRATCH_BYTES\s+\((\d+)u << (\d+)\)", open(HEADER).read())
    assert int(m.group(1)) << int(m.group(2)) == sg.STATIC_SCRATCH_BYTES
    shapes = [(10240, 8192), (8192, 8192), (59136, 8192), (8192, 29568)] * 8   # 8 TP=1 layers
    big = [sg.Linear(sg.BF16, N, K, 0, A, None, B, C) for N, K in shapes]
    assert sg.stack_workspace_bytes(big, 16) > sg.STATIC_SCRATCH_BYTES
    assert sg.stack_workspace_bytes(big, 1) <= sg.STATIC_SCRATCH_BYTES
    arr = (sg.Linear * len(big))(*big)
    assert L.decode_linear_stack_noalloc(arr, len(big), 16, None) == WORKSPACE
    with pytest.raises(sg.SkinnyError, match="WORKSPACE"):
        sg.decode_linear_stack_noalloc(big, 16, stream=0)
    # Its launches keep to 32 linears, so the bound is that of each 32 (the
    # whole call's bound adds a table launch's partial sums and table).
    stack = big * 10
    assert sg.stack_workspace_bytes(stack, 2) > sg.STATIC_SCRATCH_BYTES
    assert sg.stack_workspace_bytes(stack[:32], 2) <= sg.STATIC_SCRATCH_BYTES
    arr = (sg.Linear * len(stack))(*stack)
    assert L.decode_linear_stack_noalloc(arr, len(stack), 17, None) == INVALID
    one = (sg.Linear * 1)(sg.Linear(sg.BF16, 64, 64, 0, A, None, B, C))
    assert L.decode_linear_stack_noalloc(one, 1, 0, None) == INVALID
    assert L.decode_linear_stack_noalloc(one, 0, 1, None) == INVALID
    assert L.decode_linear_stack_noalloc(None, 1, 1, None) == INVALID
    bad = (sg.Linear * 1)(sg.Linear(sg.BF16, 64, 12, 0, A, None, B, C))
    assert L.decode_linear_stack_noalloc(bad, 1, 1, None) == UNSUPPORTED


def test_band_rows_and_launch_counts():
    for dt in (sg.BF16, sg.FP8_BS128):
        for M in (1, 2, 6, 16):
            assert sg.band_rows(dt, sg.VARIANT_MFMA, M) in (16, 32, 64)
            assert sg.band_rows(dt, sg.VARIANT_AUTO, M) == 0      # depends on the shapes
        assert [sg.band_rows(dt, sg.VARIANT_VECTOR, m) for m in (1, 2, 3, 4, 8)] == [8, 8, 16, 16, 32]
        assert sg.band_rows(dt, sg.VARIANT_VECTOR, 9) == 0
    assert sg.band_rows(sg.BF16, 7, 1) == 0 and sg.band_rows(9, 0, 1) == 0
    lin = sg.Linear(sg.BF16, 64, 64, 0, A, None, B, C)
    fp8 = sg.Linear(sg.FP8_BS128, 64, 64, 0, A, 0x300000, B, C)
    assert sg.launch_count([lin] * 32) == 1
    assert sg.launch_count([lin] * 33) == 1          # one launch per dtype, table in the workspace
    assert sg.launch_count([lin] * 320) == 1
    assert sg.launch_count([lin, fp8, lin]) == 2
    assert sg.launch_count([lin, fp8] * 40) == 2
    assert sg.launch_count([lin] * 4096) == 1 and sg.launch_count([lin] * 4097) == 2
    assert sg.lib().skinny_launch_count(None, 1) == 0


def test_rejects_shapes_beyond_32_bit_indexing():
    wsb = sg.workspace_bytes(sg.BF16, 1, 64, 64)
    assert bf16_call(N=(1 << 26) + 1, wsb=wsb) == UNSUPPORTED
    assert bf16_call(K=(1 << 28) + 8, wsb=wsb) == UNSUPPORTED


def test_argmax_rejects_bad_arguments():
    L = sg.lib()
    wsb = sg.argmax_workspace_bytes(2, 64)
    assert wsb == MIN_WORKSPACE and sg.argmax_workspace_bytes(1, 152064) == 38 * 8
    assert sg.argmax_workspace_bytes(16, 152064) == 16 * 38 * 8      # a pair per 4096 logits
    assert sg.argmax_workspace_bytes(0, 64) == 0 and sg.argmax_workspace_bytes(17, 64) == 0
    Y, I = B, C                                          # y [2][64] at B, idx at C
    assert L.skinny_argmax_bf16(None, 2, 64, I, WS, wsb, None) == INVALID
    assert L.skinny_argmax_bf16(Y, 0, 64, I, WS, wsb, None) == INVALID
    assert L.skinny_argmax_bf16(Y, 17, 64, I, WS, wsb, None) == INVALID
    assert L.skinny_argmax_bf16(Y, 2, 0, I, WS, wsb, None) == INVALID
    assert L.skinny_argmax_bf16(Y, 2, 64, Y + 4, WS, wsb, None) == INVALID          # idx in y
    assert L.skinny_argmax_bf16(Y, 2, 64, WS + 16, WS, wsb, None) == INVALID        # idx in ws
    assert L.skinny_argmax_bf16(Y, 2, 64, I + 2, WS, wsb, None) == UNSUPPORTED      # misaligned
    assert L.skinny_argmax_bf16(Y + 1, 2, 64, I, WS, wsb, None) == UNSUPPORTED
    assert L.skinny_argmax_bf16(Y, 2, 64, I, None, wsb, None) == WORKSPACE
    assert L.skinny_argmax_bf16(Y, 2, 64, I, WS, wsb - 1, None) == WORKSPACE


def test_lm_head_rejects_bad_arguments():
    L = sg.lib()
    head = sg.Linear(sg.BF16, 64, 64, 0, A, None, B, C)
    arr = (sg.Linear * 1)(head)
    wsb = sg.lm_head_workspace_bytes(head, 1)
    assert wsb >= MIN_WORKSPACE and sg.lm_head_workspace_bytes(head, 0) == 0
    T = 0x6000000                                        # next_token
    assert L.skinny_lm_head_argmax(None, 1, T, WS, wsb, None) == INVALID
    assert L.skinny_lm_head_argmax(arr, 1, None, WS, wsb, None) == INVALID
    assert L.skinny_lm_head_argmax(arr, 1, A + 64, WS, wsb, None) == INVALID       # inside W
    assert L.skinny_lm_head_argmax(arr, 1, B, WS, wsb, None) == INVALID            # inside x
    assert L.skinny_lm_head_argmax(arr, 1, C + 4, WS, wsb, None) == INVALID        # inside y
    assert L.skinny_lm_head_argmax(arr, 1, T, WS, 0, None) == WORKSPACE
    assert L.skinny_lm_head_argmax(arr, 17, T, WS, wsb, None) == INVALID


def test_mlp_workspace_and_bad_arguments():
    L = sg.lib()
    mlp = sg.Mlp(sg.BF16, 64, 32, 0, A, None, A + 0x10000, None, B, C)
    wsb = sg.mlp_workspace_bytes(mlp, 2)
    # The [M][2I] bf16 intermediate (rounded to 256 B) comes first.
    assert wsb >= 256 + MIN_WORKSPACE and wsb % 16 == 0
    assert sg.mlp_workspace_bytes(mlp, 0) == 0 and sg.mlp_workspace_bytes(mlp, 17) == 0
    bad = sg.Mlp(sg.BF16, 64, 0, 0, A, None, A + 0x10000, None, B, C)
    assert sg.mlp_workspace_bytes(bad, 1) == 0
    call = lambda m, M=2, ws=WS, n=wsb: L.skinny_mlp_swiglu(ctypes.byref(m), M, ws, n, None)
    assert L.skinny_mlp_swiglu(None, 2, WS, wsb, None) == INVALID
    assert call(mlp, M=0) == INVALID
    assert call(mlp, ws=None) == WORKSPACE
    assert call(mlp, n=wsb - 1) == WORKSPACE
    assert call(sg.Mlp(sg.BF16, 64, 32, 1, A, None, A + 0x10000, None, B, C)) == INVALID  # reserved
    assert call(sg.Mlp(sg.BF16, 64, 12, 0, A, None, A + 0x10000, None, B, C)) == UNSUPPORTED
    assert call(sg.Mlp(sg.BF16, 64, 32, 0, A, None, A + 0x10000, None, B, B)) == INVALID   # y = x
    assert call(sg.Mlp(sg.BF16, 64, 32, 0, A, None, A + 0x10000, None, B, WS + 64)) == INVALID
    assert call(sg.Mlp(sg.BF16, 64, 32, 0, A, None, A + 0x10000, None, WS + 64, C)) == INVALID
    assert call(sg.Mlp(sg.FP8_BS128, 64, 32, 0, A, None, A + 0x10000, None, B, C)) == INVALID


def test_binding_rejects_host_and_strided_tensors():
    """The binding refuses tensors the kernels cannot address as dense device
    memory, before anything reaches the C library."""
    import torch
    x = torch.zeros((2, 64), dtype=torch.bfloat16)
    w = torch.zeros((32, 64), dtype=torch.bfloat16)
    y = torch.zeros((2, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on the GPU"):
        sg.make_linear(x, w, y)
    with pytest.raises(ValueError, match="contiguous"):
        sg.make_linear(x, torch.zeros((64, 32), dtype=torch.bfloat16).t(), y)
    with pytest.raises(ValueError, match="on the GPU"):
        sg.skinny_gemm_bf16(x, w, y, torch.zeros(1024, dtype=torch.uint8))


def test_binding_rejects_mismatched_shapes_and_dtypes():
    """The library sees only pointers, so the binding compares every tensor's
    shape and dtype with what the entry point will read or write, before
    anything reaches the C library (CPU tensors: the shape check comes first)."""
    import torch
    bf, u8, f32, i32 = torch.bfloat16, torch.uint8, torch.float32, torch.int32
    x = torch.zeros((2, 64), dtype=bf)
    w = torch.zeros((32, 64), dtype=bf)
    y = torch.zeros((2, 32), dtype=bf)
    ws = torch.zeros(1024, dtype=torch.uint8)
    bad_linears = [
        dict(x=torch.zeros((2, 48), dtype=bf)),                  # K of x != K of w
        dict(y=torch.zeros((1, 32), dtype=bf)),                  # too few rows of y
        dict(y=torch.zeros((2, 31), dtype=bf)),                  # y narrower than N
        dict(x=torch.zeros((2, 64), dtype=torch.float16)),
        dict(y=torch.zeros((2, 32), dtype=f32)),
        dict(w=torch.zeros((32, 64), dtype=f32)),
    ]
    for kw in bad_linears:
        a = {**dict(x=x, w=w, y=y), **kw}
        with pytest.raises(ValueError, match="shape|dtype"):
            sg.make_linear(a["x"], a["w"], a["y"])
        with pytest.raises(ValueError, match="shape|dtype"):
            sg.skinny_gemm_bf16(a["x"], a["w"], a["y"], ws)
    q = torch.zeros((32, 64), dtype=u8)
    with pytest.raises(ValueError, match="w_scale: shape"):
        sg.make_linear(x, q, y, w_scale=torch.zeros((1, 2), dtype=f32))
    with pytest.raises(ValueError, match="w_scale: dtype"):
        sg.skinny_gemm_fp8_bs128(x, q, torch.zeros((1, 1), dtype=torch.float64), y, ws)
    with pytest.raises(ValueError, match="w: dtype"):
        sg.make_linear(x, w, y, w_scale=torch.zeros((1, 1), dtype=f32))   # bf16 codes as FP8
    # A linear remembers its M: another M is refused.
    lin = sg.Linear(sg.BF16, 32, 64, 0, A, None, B, C)
    lin.rows = 2
    with pytest.raises(ValueError, match="M = 2 called with M = 3"):
        sg.decode_linear_stack([lin], 3, (WS, 1 << 20))
    with pytest.raises(ValueError, match="idx: shape"):
        sg.argmax_bf16(y, torch.zeros(3, dtype=i32), ws)
    with pytest.raises(ValueError, match="idx: dtype"):
        sg.argmax_bf16(y, torch.zeros(2, dtype=torch.int64), ws)
    # Gated MLP: x [M][H], y [M][H], w_gate_up [2I][H], w_down [H][I].
    H, I = 64, 32
    wg, wd = torch.zeros((2 * I, H), dtype=bf), torch.zeros((H, I), dtype=bf)
    xm, ym = torch.zeros((2, H), dtype=bf), torch.zeros((2, H), dtype=bf)
    with pytest.raises(ValueError, match="w_gate_up: shape"):
        sg.make_mlp(xm, torch.zeros((I, H), dtype=bf), wd, ym)
    with pytest.raises(ValueError, match="y: shape"):
        sg.make_mlp(xm, wg, wd, torch.zeros((2, I), dtype=bf))
    # MoE: x [T or T*topk][K or 2K], ids int32 [T][topk], y [T*topk][N].
    E, N, K = 3, 32, 64
    ex = sg.Experts(sg.BF16, E, N, K, A, None)
    ids = torch.zeros((2, 2), dtype=i32)
    xs, yr = torch.zeros((2, K), dtype=bf), torch.zeros((4, N), dtype=bf)
    for kw, what in ((dict(x=torch.zeros((4, K), dtype=bf)), "x: shape"),          # per-route rows, shared flag
                     (dict(y=torch.zeros((2, N), dtype=bf)), "y: shape"),           # a row per token, not per route
                     (dict(ids=torch.zeros((2, 2), dtype=torch.int64)), "ids: dtype")):
        a = {**dict(x=xs, ids=ids, y=yr), **kw}
        with pytest.raises(ValueError, match=what):
            sg.moe_linear(ex, a["x"], a["ids"], a["y"], ws)
    with pytest.raises(ValueError, match="x: shape"):
        sg.moe_linear(ex, xs, ids, yr, ws, swiglu=True)                              # needs 2K columns
    with pytest.raises(ValueError, match="w: shape|w: dtype"):
        sg.make_experts(torch.zeros((E, N, K), dtype=u8))                            # FP8 codes without scales


def test_moe_plan_query():
    """One-token slices of rows of at least four 1 KB segments take the row
    kernel (the verify step's gate_up, K = 4096); short rows (its down,
    K = 1536), two or more tokens and a bf16 x row past the row kernel's
    x window (about 63 KB beside the slice table) take the tile kernel."""
    def variant(dtype, K, T, N=3072, flags=0):
        ex = sg.Experts(dtype, 8, N, K, A, None if dtype == sg.BF16 else A + 0x8000000)
        return sg.moe_plan_query(ex, T, 2, bool(flags & sg.MOE_X_PER_ROUTE),
                                 bool(flags & sg.MOE_SWIGLU)).variant
    for dt in (sg.BF16, sg.FP8_BS128):
        assert variant(dt, 4096, 1) == sg.VARIANT_VECTOR
        assert variant(dt, 4096, 1, flags=sg.MOE_X_PER_ROUTE | sg.MOE_SWIGLU) == sg.VARIANT_VECTOR
        assert variant(dt, 1536, 1, N=4096) == sg.VARIANT_MFMA
        assert variant(dt, 4096, 2) == sg.VARIANT_MFMA
        assert variant(dt, 4096, 6) == sg.VARIANT_MFMA
    assert variant(sg.BF16, 2048, 1) == sg.VARIANT_VECTOR                # 4 segments of 1 KB
    assert variant(sg.BF16, 1536, 1) == sg.VARIANT_MFMA                  # 3
    for dt in (sg.BF16, sg.FP8_BS128):
        assert variant(dt, 31744, 1) == sg.VARIANT_VECTOR                # 62 KB of x
        assert variant(dt, 32768, 1) == sg.VARIANT_MFMA                  # 64 KB: past the window

    def kernel(dtype, K, T, N=3072):
        ex = sg.Experts(dtype, 8, N, K, A, None if dtype == sg.BF16 else A + 0x8000000)
        return sg.KERNEL_NAMES[sg.moe_plan_query(ex, T, 2).kernel]
    for dt in (sg.BF16, sg.FP8_BS128):
        assert kernel(dt, 4096, 1) == "skinny_rows"
        assert kernel(dt, 1536, 1, N=4096) == "skinny_tiles (K-split)"     # the verify step's down
        assert kernel(dt, 4096, 6) in ("skinny_tiles", "skinny_tiles (8-wave)")
    L = sg.lib()
    plan = sg.Plan()
    ex = sg.Experts(sg.BF16, 8, 64, 64, A, None)
    assert L.skinny_moe_plan_query(ctypes.byref(ex), 1, 2, 0, None) == INVALID
    assert L.skinny_moe_plan_query(ctypes.byref(ex), 0, 2, 0, ctypes.byref(plan)) == INVALID
    assert L.skinny_moe_plan_query(ctypes.byref(ex), 1, 2, 4, ctypes.byref(plan)) == INVALID
    bad = sg.Experts(sg.BF16, 8, 64, 60, A, None)
    assert L.skinny_moe_plan_query(ctypes.byref(bad), 1, 2, 0, ctypes.byref(plan)) == UNSUPPORTED


def test_moe_workspace_and_bad_arguments():
    L = sg.lib()
    ex = sg.Experts(sg.FP8_BS128, 8, 3072, 4096, A, A + 0x8000000)
    wsb = sg.moe_workspace_bytes(ex, 6, 2)
    assert wsb >= MIN_WORKSPACE and wsb % 16 == 0
    assert sg.moe_workspace_bytes(ex, 0, 2) == 0 and sg.moe_workspace_bytes(ex, 17, 2) == 0
    assert sg.moe_workspace_bytes(ex, 6, 0) == 0
    assert sg.moe_workspace_bytes(ex, 6, sg.MAX_TOPK + 1) == 0
    assert sg.moe_workspace_bytes(ex, 16, sg.MAX_TOPK) >= wsb          # more routes, more slices
    assert sg.moe_workspace_bytes(sg.Experts(sg.BF16, 8, 64, 64, A, A), 1, 1) == 0  # bf16 + scales
    assert sg.moe_workspace_bytes(sg.Experts(sg.FP8_BS128, 8, 64, 64, A, None), 1, 1) == 0
    assert sg.moe_workspace_bytes(sg.Experts(sg.BF16, 0, 64, 64, A, None), 1, 1) == 0
    X, IDS, Y = 0x20000000, 0x21000000, 0x22000000
    big = 0x40000000                                                      # past the weights

    def call(e=ex, x=X, ids=IDS, T=6, topk=2, flags=0, y=Y, ws=big, n=wsb):
        return L.skinny_moe_linear(ctypes.byref(e) if e is not None else None, x, ids, T, topk,
                                   flags, y, ws, n, None)
    assert call(e=None) == INVALID
    assert call(x=None) == INVALID and call(ids=None) == INVALID and call(y=None) == INVALID
    assert call(T=0) == INVALID and call(T=17) == INVALID and call(topk=17) == INVALID
    assert call(flags=4) == INVALID
    assert call(ws=None) == WORKSPACE and call(n=wsb - 1) == WORKSPACE
    assert call(x=X + 8) == UNSUPPORTED and call(ids=IDS + 2) == UNSUPPORTED
    assert call(e=sg.Experts(sg.FP8_BS128, 8, 3072, 4088, A, A + 0x8000000)) == UNSUPPORTED
    assert call(y=X) == INVALID                                          # y over x
    assert call(y=IDS - 16) == INVALID                                   # y runs into ids
    assert call(y=A + 0x1000) == INVALID                                 # y inside the weights
    assert call(ws=X) == INVALID                                         # workspace over x
    # x per route with SwiGLU: 12 routes x 2K bf16, so y just past 6 x K no longer clears it.
    assert call(y=X + 6 * 4096 * 2, flags=sg.MOE_X_PER_ROUTE | sg.MOE_SWIGLU) == INVALID
    assert L.skinny_moe_linear_timed(ctypes.byref(ex), X, IDS, 6, 2, 0, Y, None, big, wsb,
                                     None) == INVALID


def test_read_probe_loads_and_rejects_bad_arguments():
    """The streaming-read probe library (measurement only) loads and refuses
    invalid arguments on the host, before any device call, in both load modes."""
    from gemv_skinny_gemm_amd import probe
    L = probe.lib()
    for nt in (0, 1):
        assert L.skinny_probe_stream_read(None, 1 << 20, 8192, 8192, 0, 2, 1, nt, 16, None) == -1
        assert L.skinny_probe_stream_read(16, 1 << 20, 8192, 8192, 5, 2, 1, nt, 16, None) == -1
        assert L.skinny_probe_stream_read(16, 1 << 20, 8192, 8192, 0, 3, 1, nt, 16, None) == -1
        assert L.skinny_probe_stream_read_tiles(None, 1 << 20, 8192, 4, 0, 1, nt, 16, None) == -1
        assert L.skinny_probe_stream_read_tiles(16, 1 << 20, 8000, 4, 0, 1, nt, 16, None) == -1
        assert L.skinny_probe_stream_read_tiles(16, 1 << 20, 8192, 6, 0, 1, nt, 16, None) == -1
