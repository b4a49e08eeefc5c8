"""Python binding of the gfx950 skinny-GEMM C ABI (include/skinny_gemm.h).

Argument marshalling only: every step of y = x . W^T runs in the HIP kernels
of ``libskinny_gemm.so``.  PyTorch supplies device memory (``data_ptr()``)
and streams (``torch.cuda.current_stream().cuda_stream``).  There is no
fallback: if the shared library is missing or fails to load, every entry
point raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "BF16", "FP8_BS128", "VARIANT_AUTO", "VARIANT_VECTOR", "VARIANT_MFMA", "MAX_M",
    "SkinnyError", "Linear", "Plan", "lib", "lib_path",
    "workspace_bytes", "stack_workspace_bytes", "skinny_gemm_bf16", "skinny_gemm_fp8_bs128",
    "decode_linear_stack", "decode_linear_stack_noalloc", "STATIC_SCRATCH_BYTES", "linear_run", "linear_run_timed", "launch_count", "band_rows", "plan_query",
    "status_string", "abi_version", "argmax_bf16", "argmax_workspace_bytes", "lm_head_argmax",
    "lm_head_workspace_bytes", "Mlp", "make_mlp", "mlp_workspace_bytes", "mlp_swiglu",
    "Experts", "make_experts", "moe_workspace_bytes", "moe_linear", "moe_linear_timed",
    "moe_plan_query", "moe_mlp_workspace_bytes", "moe_mlp_swiglu", "moe_mlp_swiglu_timed",
    "moe_mlp_set_spin_limit", "moe_mlp_gave_up", "moe_mlp_plan_query", "MOE_MLP_COUNTER_BYTES",
    "MOE_X_PER_ROUTE", "MOE_SWIGLU", "MAX_TOPK", "KERNEL_NAMES",
]

BF16 = 0
FP8_BS128 = 1
VARIANT_AUTO = 0
VARIANT_VECTOR = 1
VARIANT_MFMA = 2
MAX_M = 16
MAX_LINEARS_PER_LAUNCH = 32    # descriptors in a launch's arguments; more go in a table
MAX_TOPK = 16
MOE_X_PER_ROUTE = 1
MOE_SWIGLU = 2
ABI_VERSION = 2
# enum skinny_kernel (skinny_plan.kernel): the main kernel's form, by the name
# of its HIP function (and instance).
KERNEL_NAMES = {1: "skinny_rows", 2: "skinny_rows (lean)", 3: "skinny_rows_flat",
                4: "skinny_tiles", 5: "skinny_tiles (8-wave)", 6: "skinny_tiles (K-split)",
                7: "skinny_moe_mlp1"}
STATIC_SCRATCH_BYTES = 64 << 20
MOE_MLP_COUNTER_BYTES = 256   # moe_mlp_swiglu's workspace: counter and flag, then gate_up outputs

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libskinny_gemm.so"

STATUS_NAMES = {0: "SKINNY_OK", 1: "SKINNY_ERR_INVALID_ARG", 2: "SKINNY_ERR_UNSUPPORTED",
                3: "SKINNY_ERR_WORKSPACE", 4: "SKINNY_ERR_HIP"}


class SkinnyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


class Linear(ctypes.Structure):
    """struct skinny_linear"""
    _fields_ = [("dtype", ctypes.c_int), ("N", ctypes.c_int), ("K", ctypes.c_int),
                ("reserved", ctypes.c_int), ("w", ctypes.c_void_p), ("w_scale", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class Mlp(ctypes.Structure):
    """struct skinny_mlp"""
    _fields_ = [("dtype", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int),
                ("reserved", ctypes.c_int), ("w_gate_up", ctypes.c_void_p),
                ("s_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_down", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class Experts(ctypes.Structure):
    """struct skinny_experts"""
    _fields_ = [("dtype", ctypes.c_int), ("E", ctypes.c_int), ("N", ctypes.c_int),
                ("K", ctypes.c_int), ("w", ctypes.c_void_p), ("w_scale", ctypes.c_void_p)]


class Plan(ctypes.Structure):
    """struct skinny_plan"""
    _fields_ = [("variant", ctypes.c_int), ("waves", ctypes.c_int), ("kernel", ctypes.c_int),
                ("reserved", ctypes.c_int * 5)]


_lib = None


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def _bind(path: str):
    """Load a built library and declare the C signatures of include/skinny_gemm.h."""
    L = ctypes.CDLL(path)
    sz, vp, i = ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
    lp = ctypes.POINTER(Linear)
    L.skinny_workspace_bytes.restype = sz
    L.skinny_workspace_bytes.argtypes = [i, i, i, i]
    L.skinny_stack_workspace_bytes.restype = sz
    L.skinny_stack_workspace_bytes.argtypes = [lp, i, i]
    L.skinny_gemm_bf16.restype = i
    L.skinny_gemm_bf16.argtypes = [vp, vp, vp, i, i, i, vp, sz, vp]
    L.skinny_gemm_fp8_bs128.restype = i
    L.skinny_gemm_fp8_bs128.argtypes = [vp, vp, vp, vp, i, i, i, vp, sz, vp]
    L.decode_linear_stack.restype = i
    L.decode_linear_stack.argtypes = [lp, i, i, vp, sz, vp]
    L.decode_linear_stack_noalloc.restype = i
    L.decode_linear_stack_noalloc.argtypes = [lp, i, i, vp]
    L.skinny_linear_run.restype = i
    L.skinny_linear_run.argtypes = [lp, i, i, ctypes.POINTER(Plan), vp, sz, vp]
    L.skinny_launch_count.restype = i
    L.skinny_launch_count.argtypes = [lp, i]
    L.skinny_linear_run_timed.restype = i
    L.skinny_linear_run_timed.argtypes = [lp, i, i, ctypes.POINTER(Plan),
                                          ctypes.POINTER(ctypes.c_void_p), i, vp, sz, vp]
    L.skinny_band_rows.restype = i
    L.skinny_band_rows.argtypes = [i, i, i]
    L.skinny_plan_query.restype = i
    L.skinny_plan_query.argtypes = [lp, i, i, ctypes.POINTER(Plan)]
    L.skinny_argmax_workspace_bytes.restype = sz
    L.skinny_argmax_workspace_bytes.argtypes = [i, i]
    L.skinny_argmax_bf16.restype = i
    L.skinny_argmax_bf16.argtypes = [vp, i, i, vp, vp, sz, vp]
    L.skinny_lm_head_workspace_bytes.restype = sz
    L.skinny_lm_head_workspace_bytes.argtypes = [lp, i]
    L.skinny_lm_head_argmax.restype = i
    L.skinny_lm_head_argmax.argtypes = [lp, i, vp, vp, sz, vp]
    mp = ctypes.POINTER(Mlp)
    L.skinny_mlp_workspace_bytes.restype = sz
    L.skinny_mlp_workspace_bytes.argtypes = [mp, i]
    L.skinny_mlp_swiglu.restype = i
    L.skinny_mlp_swiglu.argtypes = [mp, i, vp, sz, vp]
    ep = ctypes.POINTER(Experts)
    L.skinny_moe_workspace_bytes.restype = sz
    L.skinny_moe_workspace_bytes.argtypes = [ep, i, i, i]
    L.skinny_moe_linear.restype = i
    L.skinny_moe_linear.argtypes = [ep, vp, vp, i, i, i, vp, vp, sz, vp]
    L.skinny_moe_linear_timed.restype = i
    L.skinny_moe_linear_timed.argtypes = [ep, vp, vp, i, i, i, vp, ctypes.POINTER(vp), vp, sz, vp]
    L.skinny_moe_plan_query.restype = i
    L.skinny_moe_plan_query.argtypes = [ep, i, i, i, ctypes.POINTER(Plan)]
    L.skinny_moe_mlp_workspace_bytes.restype = sz
    L.skinny_moe_mlp_workspace_bytes.argtypes = [ep, ep, i, i]
    L.skinny_moe_mlp_swiglu.restype = i
    L.skinny_moe_mlp_swiglu.argtypes = [ep, ep, vp, vp, i, i, vp, vp, sz, vp]
    L.skinny_moe_mlp_swiglu_timed.restype = i
    L.skinny_moe_mlp_swiglu_timed.argtypes = [ep, ep, vp, vp, i, i, vp, ctypes.POINTER(vp), vp,
                                              sz, vp]
    L.skinny_moe_mlp_plan_query.restype = i
    L.skinny_moe_mlp_plan_query.argtypes = [ep, ep, i, i, ctypes.POINTER(Plan)]
    L.skinny_moe_mlp_set_spin_limit.restype = None
    L.skinny_moe_mlp_set_spin_limit.argtypes = [ctypes.c_longlong]
    L.skinny_status_string.restype = ctypes.c_char_p
    L.skinny_status_string.argtypes = [i]
    L.skinny_abi_version.restype = i
    L.skinny_abi_version.argtypes = []
    if L.skinny_abi_version() != ABI_VERSION:
        raise ImportError(f"{path}: ABI version {L.skinny_abi_version()} != {ABI_VERSION}")
    return L


def lib():
    """The loaded C library.  Raises if it is not built: there is no fallback."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run __graft_entry__.build() or "
                              "python -m gemv_skinny_gemm_amd._build")
        _lib = _bind(path)
    return _lib


def _ptr(t) -> int | None:
    """Device address of a torch tensor, or an int address as given (None = NULL).
    The library reads and writes dense row-major device memory, so a tensor must
    be contiguous and on the GPU."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous (row-major)")
    if t.device.type != "cuda":
        raise ValueError(f"tensors passed to the library must be on the GPU, not {t.device}")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise SkinnyError(status, where)


def status_string(status: int) -> str:
    return lib().skinny_status_string(int(status)).decode()


def abi_version() -> int:
    return lib().skinny_abi_version()


def workspace_bytes(dtype: int, M: int, N: int, K: int) -> int:
    return lib().skinny_workspace_bytes(dtype, M, N, K)


def _linear_array(linears):
    arr = (Linear * len(linears))()
    for i, L in enumerate(linears):
        arr[i] = L
    return arr


def stack_workspace_bytes(linears, M: int) -> int:
    arr = _linear_array(linears)
    return lib().skinny_stack_workspace_bytes(arr, len(linears), M)


def _shape2(t):
    if isinstance(t, int):
        raise TypeError("pass tensors, or call the raw C entry points through lib()")
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    return int(t.shape[0]), int(t.shape[1])


def _dtype_name(t) -> str:
    return str(t.dtype).replace("torch.", "")


def _need(t, shape, dtypes, what):
    """Refuse a tensor whose shape or dtype does not match what the C entry
    point will read or write: the library sees only pointers, so a short or
    mistyped buffer would be read or written past its end."""
    if isinstance(t, int) or t is None:
        return
    if tuple(int(v) for v in t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if _dtype_name(t) not in dtypes:
        raise ValueError(f"{what}: dtype {_dtype_name(t)}, expected one of {sorted(dtypes)}")


_BF16 = {"bfloat16"}
_FP8 = {"uint8", "float8_e4m3fn"}
_F32 = {"float32"}
_I32 = {"int32"}


def _scale_shape(N: int, K: int):
    return ((N + 127) // 128, (K + 127) // 128)


def _ws(workspace):
    if workspace is None:
        return None, 0
    if isinstance(workspace, tuple):
        return workspace
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def skinny_gemm_bf16(x, w, y, workspace, stream=None):
    """y[M][N] = x[M][K] . w[N][K]^T (bf16 tensors on the GPU; y written in place)."""
    M, K = _shape2(x)
    N, _ = _shape2(w)
    _need(x, (M, K), _BF16, "x")
    _need(w, (N, K), _BF16, "w")
    _need(y, (M, N), _BF16, "y")
    wp, wb = _ws(workspace)
    _check(lib().skinny_gemm_bf16(_ptr(x), _ptr(w), _ptr(y), M, N, K, wp, wb, _stream(stream)),
           "skinny_gemm_bf16")
    return y


def skinny_gemm_fp8_bs128(x, w_fp8, w_scale, y, workspace, stream=None):
    """y = x . (e4m3(w_fp8) * block scale)^T; w_fp8 [N][K] uint8 / float8_e4m3fn,
    w_scale [ceil(N/128)][ceil(K/128)] float32."""
    M, K = _shape2(x)
    N, _ = _shape2(w_fp8)
    _need(x, (M, K), _BF16, "x")
    _need(w_fp8, (N, K), _FP8, "w_fp8")
    _need(w_scale, _scale_shape(N, K), _F32, "w_scale")
    _need(y, (M, N), _BF16, "y")
    wp, wb = _ws(workspace)
    _check(lib().skinny_gemm_fp8_bs128(_ptr(x), _ptr(w_fp8), _ptr(w_scale), _ptr(y), M, N, K,
                                        wp, wb, _stream(stream)), "skinny_gemm_fp8_bs128")
    return y


def make_linear(x, w, y, w_scale=None, dtype=None) -> Linear:
    """A skinny_linear from GPU tensors x [M][K], w [N][K], y [M][N] (w_scale for FP8).

    Shapes and dtypes are checked here; the Linear remembers M (as ``rows``)
    so that a call with another M is refused before it reaches the library."""
    N, K = _shape2(w)
    if dtype is None:
        dtype = FP8_BS128 if w_scale is not None else BF16
    M = None
    if not isinstance(x, int):
        M, _ = _shape2(x)
        _need(x, (M, K), _BF16, "x")
        _need(y, (M, N), _BF16, "y")
    _need(w, (N, K), _BF16 if dtype == BF16 else _FP8, "w")
    if dtype == FP8_BS128:
        _need(w_scale, _scale_shape(N, K), _F32, "w_scale")
    lin = Linear(dtype, N, K, 0, _ptr(w), _ptr(w_scale), _ptr(x), _ptr(y))
    lin.rows = M
    return lin


def _check_rows(linears, M: int):
    for L in linears:
        rows = getattr(L, "rows", None)
        if rows is not None and rows != M:
            raise ValueError(f"a linear made for M = {rows} called with M = {M}")


def decode_linear_stack(linears, M: int, workspace, stream=None):
    """Run independent linears (a list of Linear) that share M."""
    _check_rows(linears, M)
    arr = _linear_array(linears)
    wp, wb = _ws(workspace)
    _check(lib().decode_linear_stack(arr, len(linears), M, wp, wb, _stream(stream)),
           "decode_linear_stack")


def decode_linear_stack_noalloc(linears, M: int, stream=None):
    """decode_linear_stack without a workspace: the partial sums go to the
    library's static device buffer (STATIC_SCRATCH_BYTES per GPU), shared by
    every call on that GPU, so calls that may overlap on one GPU race."""
    _check_rows(linears, M)
    arr = _linear_array(linears)
    _check(lib().decode_linear_stack_noalloc(arr, len(linears), M, _stream(stream)),
           "decode_linear_stack_noalloc")


def linear_run(linears, M: int, workspace, variant: int = VARIANT_AUTO, waves: int = 0,
               stream=None):
    """decode_linear_stack with a forced variant and/or persistent wave count."""
    _check_rows(linears, M)
    arr = _linear_array(linears)
    plan = Plan(variant, waves)
    wp, wb = _ws(workspace)
    _check(lib().skinny_linear_run(arr, len(linears), M, ctypes.byref(plan), wp, wb,
                                   _stream(stream)), "skinny_linear_run")


def band_rows(dtype: int, variant: int, M: int) -> int:
    """Rows per band of the main kernel: the workspace slot layout is [slot][M][band_rows]."""
    return lib().skinny_band_rows(dtype, variant, M)


def launch_count(linears) -> int:
    arr = _linear_array(linears)
    return lib().skinny_launch_count(arr, len(linears))


def linear_run_timed(linears, M: int, workspace, events, variant: int = VARIANT_AUTO,
                     waves: int = 0, stream=None):
    """linear_run recording events[2g] / events[2g+1] (hipEvent_t addresses) around
    main-kernel launch g."""
    _check_rows(linears, M)
    arr = _linear_array(linears)
    plan = Plan(variant, waves)
    ev = (ctypes.c_void_p * len(events))(*events)
    wp, wb = _ws(workspace)
    _check(lib().skinny_linear_run_timed(arr, len(linears), M, ctypes.byref(plan), ev, len(events),
                                         wp, wb, _stream(stream)), "skinny_linear_run_timed")


def plan_query(linears, M: int) -> Plan:
    arr = _linear_array(linears)
    plan = Plan()
    _check(lib().skinny_plan_query(arr, len(linears), M, ctypes.byref(plan)), "skinny_plan_query")
    return plan


def argmax_workspace_bytes(M: int, N: int) -> int:
    return lib().skinny_argmax_workspace_bytes(M, N)


def argmax_bf16(y, idx, workspace, stream=None):
    """idx[m] = smallest index of the largest value of y[m] (bf16 [M][N] and
    int32 [M] tensors on the GPU; idx written in place)."""
    M, N = _shape2(y)
    _need(y, (M, N), _BF16, "y")
    _need(idx, (M,), _I32, "idx")
    wp, wb = _ws(workspace)
    _check(lib().skinny_argmax_bf16(_ptr(y), M, N, _ptr(idx), wp, wb, _stream(stream)),
           "skinny_argmax_bf16")
    return idx


def lm_head_workspace_bytes(head: Linear, M: int) -> int:
    return lib().skinny_lm_head_workspace_bytes(_linear_array([head]), M)


def lm_head_argmax(head: Linear, M: int, next_token, workspace, stream=None):
    """Run the vocabulary projection `head` (its y = logits) and write the
    greedy token of each of the M rows into next_token (int32 [M] on the GPU)."""
    _check_rows([head], M)
    _need(next_token, (M,), _I32, "next_token")
    arr = _linear_array([head])
    wp, wb = _ws(workspace)
    _check(lib().skinny_lm_head_argmax(arr, M, _ptr(next_token), wp, wb, _stream(stream)),
           "skinny_lm_head_argmax")
    return next_token


def make_mlp(x, w_gate_up, w_down, y, s_gate_up=None, s_down=None) -> Mlp:
    """A skinny_mlp from GPU tensors x [M][H], w_gate_up [2I][H] (gate rows
    first), w_down [H][I], y [M][H] (scales for FP8)."""
    H, I = _shape2(w_down)
    dtype = FP8_BS128 if s_gate_up is not None else BF16
    wd = _BF16 if dtype == BF16 else _FP8
    _need(w_gate_up, (2 * I, H), wd, "w_gate_up")
    _need(w_down, (H, I), wd, "w_down")
    if dtype == FP8_BS128:
        _need(s_gate_up, _scale_shape(2 * I, H), _F32, "s_gate_up")
        _need(s_down, _scale_shape(H, I), _F32, "s_down")
    M = None
    if not isinstance(x, int):
        M, _ = _shape2(x)
        _need(x, (M, H), _BF16, "x")
        _need(y, (M, H), _BF16, "y")
    mlp = Mlp(dtype, H, I, 0, _ptr(w_gate_up), _ptr(s_gate_up), _ptr(w_down), _ptr(s_down),
              _ptr(x), _ptr(y))
    mlp.rows = M
    return mlp


def mlp_workspace_bytes(mlp: Mlp, M: int) -> int:
    return lib().skinny_mlp_workspace_bytes(ctypes.byref(mlp), M)


def mlp_swiglu(mlp: Mlp, M: int, workspace, stream=None):
    """y = down(silu(gate) * up) with [gate | up] = x . W_gate_up^T."""
    _check_rows([mlp], M)
    wp, wb = _ws(workspace)
    _check(lib().skinny_mlp_swiglu(ctypes.byref(mlp), M, wp, wb, _stream(stream)),
           "skinny_mlp_swiglu")


def make_experts(w, w_scale=None) -> Experts:
    """A skinny_experts from GPU tensors w [E][N][K] (bf16, or uint8 E4M3FN
    codes with w_scale [E][ceil(N/128)][ceil(K/128)] fp32)."""
    if isinstance(w, int) or w.dim() != 3:
        raise ValueError("w must be a 3-D tensor [E][N][K]")
    E, N, K = (int(v) for v in w.shape)
    _need(w, (E, N, K), _BF16 if w_scale is None else _FP8, "w")
    if w_scale is not None:
        _need(w_scale, (E, *_scale_shape(N, K)), _F32, "w_scale")
    return Experts(FP8_BS128 if w_scale is not None else BF16, E, N, K, _ptr(w), _ptr(w_scale))


def _moe_flags(x_per_route: bool, swiglu: bool) -> int:
    return (MOE_X_PER_ROUTE if x_per_route else 0) | (MOE_SWIGLU if swiglu else 0)


def _check_moe(experts: Experts, x, ids, y, x_per_route: bool, swiglu: bool):
    T, topk = _shape2(ids)
    _need(ids, (T, topk), _I32, "ids")
    _need(x, ((T * topk if x_per_route else T), (2 if swiglu else 1) * experts.K), _BF16, "x")
    _need(y, (T * topk, experts.N), _BF16, "y")
    return T, topk


def moe_workspace_bytes(experts: Experts, T: int, topk: int, x_per_route: bool = False,
                        swiglu: bool = False) -> int:
    return lib().skinny_moe_workspace_bytes(ctypes.byref(experts), T, topk,
                                            _moe_flags(x_per_route, swiglu))


def moe_linear(experts: Experts, x, ids, y, workspace, x_per_route: bool = False,
               swiglu: bool = False, stream=None):
    """y[t * topk + j] = x_r . W_{ids[t][j]}^T for the T x topk routes of ids
    (int32 [T][topk] on the GPU); x_r = x[t], or x[r] with x_per_route, or
    silu(g) * u of that row [g | u] with swiglu."""
    T, topk = _check_moe(experts, x, ids, y, x_per_route, swiglu)
    wp, wb = _ws(workspace)
    _check(lib().skinny_moe_linear(ctypes.byref(experts), _ptr(x), _ptr(ids), T, topk,
                                   _moe_flags(x_per_route, swiglu), _ptr(y), wp, wb,
                                   _stream(stream)), "skinny_moe_linear")
    return y


def moe_linear_timed(experts: Experts, x, ids, y, workspace, events, x_per_route: bool = False,
                     swiglu: bool = False, stream=None):
    """moe_linear recording the two hipEvent_t handles in `events` around its
    main launch."""
    T, topk = _check_moe(experts, x, ids, y, x_per_route, swiglu)
    wp, wb = _ws(workspace)
    ev = (ctypes.c_void_p * 2)(*events)
    _check(lib().skinny_moe_linear_timed(ctypes.byref(experts), _ptr(x), _ptr(ids), T, topk,
                                         _moe_flags(x_per_route, swiglu), _ptr(y), ev, wp, wb,
                                         _stream(stream)), "skinny_moe_linear_timed")
    return y


def _check_moe_mlp(gate_up: Experts, down: Experts, x, ids, y):
    T, topk = _shape2(ids)
    _need(ids, (T, topk), _I32, "ids")
    _need(x, (T, gate_up.K), _BF16, "x")
    _need(y, (T * topk, down.N), _BF16, "y")
    return T, topk


def moe_mlp_workspace_bytes(gate_up: Experts, down: Experts, T: int, topk: int) -> int:
    """Bytes of workspace moe_mlp_swiglu needs; allocate it zeroed (its first
    256 bytes are counters that must start at zero)."""
    return lib().skinny_moe_mlp_workspace_bytes(ctypes.byref(gate_up), ctypes.byref(down), T,
                                                topk)


def moe_mlp_swiglu(gate_up: Experts, down: Experts, x, ids, y, workspace, stream=None):
    """y[r] = bf16(silu(g) * u) . Wdown_e^T with [g | u] = x[t] . Wgate_up_e^T
    (bf16) for route r = t * topk + j, e = ids[t][j]; one launch for one token."""
    T, topk = _check_moe_mlp(gate_up, down, x, ids, y)
    wp, wb = _ws(workspace)
    _check(lib().skinny_moe_mlp_swiglu(ctypes.byref(gate_up), ctypes.byref(down), _ptr(x),
                                       _ptr(ids), T, topk, _ptr(y), wp, wb, _stream(stream)),
           "skinny_moe_mlp_swiglu")
    return y


def moe_mlp_swiglu_timed(gate_up: Experts, down: Experts, x, ids, y, workspace, events,
                         stream=None):
    """moe_mlp_swiglu recording the two hipEvent_t handles in `events` around
    its main launch (the one launch for one token, else gate_up's)."""
    T, topk = _check_moe_mlp(gate_up, down, x, ids, y)
    wp, wb = _ws(workspace)
    ev = (ctypes.c_void_p * 2)(*events)
    _check(lib().skinny_moe_mlp_swiglu_timed(ctypes.byref(gate_up), ctypes.byref(down), _ptr(x),
                                             _ptr(ids), T, topk, _ptr(y), ev, wp, wb,
                                             _stream(stream)), "skinny_moe_mlp_swiglu_timed")
    return y


def moe_mlp_plan_query(gate_up: Experts, down: Experts, T: int, topk: int) -> Plan:
    """The main launch moe_mlp_swiglu makes (kernel 7 = the one launch)."""
    plan = Plan()
    _check(lib().skinny_moe_mlp_plan_query(ctypes.byref(gate_up), ctypes.byref(down), T, topk,
                                           ctypes.byref(plan)), "skinny_moe_mlp_plan_query")
    return plan


def moe_mlp_set_spin_limit(polls: int) -> None:
    """Polls before the one-token launch's wait gives up (< 0: it does not
    wait); for tests of that path."""
    lib().skinny_moe_mlp_set_spin_limit(int(polls))


def moe_mlp_gave_up(workspace) -> bool:
    """Whether a wait of the one-token launch on this workspace gave up (its
    counter word 2; synchronizes with the device)."""
    import torch
    return bool(int(workspace[:16].view(torch.int32)[2].item()))


def moe_plan_query(experts: Experts, T: int, topk: int, x_per_route: bool = False,
                   swiglu: bool = False) -> Plan:
    """The main kernel moe_linear takes for these experts and T x topk routes
    (variant VARIANT_VECTOR or VARIANT_MFMA)."""
    plan = Plan()
    _check(lib().skinny_moe_plan_query(ctypes.byref(experts), T, topk,
                                       _moe_flags(x_per_route, swiglu), ctypes.byref(plan)),
           "skinny_moe_plan_query")
    return plan
