"""ctypes binding of libdgemm.so: the C ABI of include/dgemm.h, by the same names.

This layer only marshals arguments: it reads shapes, row pitches and data
pointers from torch tensors and passes them, with the tensor's current HIP
stream, to the library.  Every arithmetic step runs in the library's kernels.
There is no fallback: if libdgemm.so is missing or fails to load, importing
this module raises.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdgemm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "or python -m dense_gemm_matrix_amd.build")
_lib = ctypes.CDLL(LIB_PATH)

_c_int, _c_void_p = ctypes.c_int, ctypes.c_void_p
for _f in (_lib.gemm_f32, _lib.gemm_f32_3xbf16):
    _f.argtypes = [_c_int, _c_int, _c_int, _c_void_p, _c_int, _c_void_p, _c_int,
                   _c_void_p, _c_int, _c_void_p]
for _f in (_lib.gemm_bf16, _lib.gemm_f16):
    _f.argtypes = [_c_int, _c_int, _c_int, _c_void_p, _c_int, _c_void_p, _c_int,
                   _c_void_p, _c_int, _c_int, _c_void_p]
for _f in (_lib.gemm_f32, _lib.gemm_f32_3xbf16, _lib.gemm_bf16, _lib.gemm_f16):
    _f.restype = _c_int
_lib.dgemm_status_string.argtypes = [_c_int]
_lib.dgemm_status_string.restype = ctypes.c_char_p
_P = ctypes.POINTER(ctypes.c_int)
_lib.dgemm_tile_map.argtypes = [_c_int, _c_int, _c_int, _c_int, _P, _P, _P, _P, _P]
_lib.dgemm_tile_map.restype = _c_int
_c_float, _c_size_t = ctypes.c_float, ctypes.c_size_t
_lib.gemm_ex.argtypes = [_c_int, _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_int, _c_void_p,
                         _c_int, _c_void_p, _c_int, _c_float, _c_float, _c_void_p, _c_int,
                         _c_void_p, _c_size_t, _c_void_p]
_lib.gemm_ex.restype = _c_int
_lib.gemm_ex_static.argtypes = [_c_int, _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_int,
                                _c_void_p, _c_int, _c_void_p, _c_int, _c_float, _c_float,
                                _c_void_p, _c_int, _c_size_t, _c_void_p]
_lib.gemm_ex_static.restype = _c_int
_lib.gemm_ex_plan.argtypes = [_c_int, _c_int, _c_int, _c_int, _c_int, _c_size_t, _P, _P, _P,
                              ctypes.POINTER(_c_size_t)]
_lib.gemm_ex_plan.restype = _c_int
_lib.dgemm_set_plan_override.argtypes = [_c_int, _c_int, _c_int, _c_int]
_lib.dgemm_set_plan_override.restype = _c_int
_lib.dgemm_set_stream_k_wait_us.argtypes = [ctypes.c_double]
_lib.dgemm_set_stream_k_wait_us.restype = _c_int
_lib.dgemm_stream_k_schedule.argtypes = [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _P,
                                         _c_int, _P]
_lib.dgemm_stream_k_schedule.restype = _c_int

DGEMM_OK = 0
DGEMM_ERR_INVALID_VALUE = 1
DGEMM_ERR_LEADING_DIM = 2
DGEMM_ERR_MISALIGNED = 3
DGEMM_ERR_ALIAS = 4
DGEMM_ERR_TOO_LARGE = 5
DGEMM_ERR_DEVICE = 6
DGEMM_ERR_LAUNCH = 7
DGEMM_ERR_SCRATCH_SIZE = 8
DGEMM_STATIC_SCRATCH_BYTES = 32 << 20
DGEMM_OUT_F32 = 0
DGEMM_OUT_SAME = 1
DGEMM_ACT_NONE = 0
DGEMM_ACT_RELU = 1
DGEMM_PLAN_AUTO = 0
DGEMM_PLAN_GRID = 1
DGEMM_PLAN_STREAM_K = 2
DGEMM_PLAN_NO_STREAM_K = 3
SK_ROLES = ("piece", "recompute", "reduce")
IN_CODES = {"f32": 0, "bf16": 1, "f16": 2, "f32x3": 3}
_TORCH_IN = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}


class DgemmError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(dgemm_status_string(status))


def dgemm_status_string(status: int) -> str:
    return _lib.dgemm_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != DGEMM_OK:
        raise DgemmError(status)


def _pitch(t: torch.Tensor, row_len: int) -> int:
    """Row pitch in elements.  A matrix with at most one row never steps to a
    second row, so its pitch is free: it is given as the row length rounded up
    to 16 bytes, which the ABI's alignment rule accepts."""
    if t.dim() != 2:
        raise ValueError("operands must be 2-D")
    rows, cols = t.shape
    pitch, inner = t.stride()
    if rows > 0 and cols > 1 and inner != 1:
        raise ValueError("operands must be row-major with unit inner stride")
    if rows > 1:
        return pitch
    per16 = 16 // t.element_size()
    return (max(row_len, 1) + per16 - 1) // per16 * per16


def _shapes(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor):
    """(M, N, K) after checking that A, B and C are 2-D, conformable and on one
    GPU: the library launches on C's device and would otherwise be handed another
    device's pointers."""
    if A.dim() != 2 or B.dim() != 2 or C.dim() != 2:
        raise ValueError("operands must be 2-D")
    M, K = A.shape
    K2, N = B.shape
    if K != K2 or tuple(C.shape) != (M, N):
        raise ValueError(f"shapes {tuple(A.shape)} x {tuple(B.shape)} -> {tuple(C.shape)}")
    if not (A.is_cuda and B.is_cuda and C.is_cuda):
        raise ValueError("operands must be device tensors")
    if not (A.get_device() == B.get_device() == C.get_device()):
        raise ValueError(f"operands on different devices: {A.device}, {B.device}, {C.device}")
    return M, N, K


# The calling thread's current stream on a device, as a raw handle: torch's
# accessor for it when present (it skips building a Stream object, 2 us of a
# 10 us call), else the public API.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(C: torch.Tensor, stream):
    if stream is None:
        if _raw_stream is not None:
            return ctypes.c_void_p(_raw_stream(C.get_device()))
        stream = torch.cuda.current_stream(C.device)
    return ctypes.c_void_p(stream.cuda_stream)


class _on_device:
    """Makes C's device current for the call (the library launches on the
    current device), skipping torch's device switch when it already is."""
    __slots__ = ("idx", "prev")

    def __init__(self, t: torch.Tensor):
        self.idx = t.get_device()

    def __enter__(self):
        self.prev = torch.cuda.current_device()
        if self.idx is not None and self.idx != self.prev:
            torch.cuda.set_device(self.idx)
        else:
            self.prev = None

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)
        return False


def gemm_f32(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, stream=None) -> None:
    """C = A @ B for fp32 A [M,K], B [K,N], C [M,N]; enqueued on `stream`."""
    M, N, K = _shapes(A, B, C)
    if not (A.dtype == B.dtype == C.dtype == torch.float32):
        raise TypeError("gemm_f32 takes float32 A, B and C")
    with _on_device(C):
        _check(_lib.gemm_f32(M, N, K, A.data_ptr(), _pitch(A, K), B.data_ptr(), _pitch(B, N),
                             C.data_ptr(), _pitch(C, N), _stream(C, stream)))


def gemm_f32_3xbf16(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, stream=None) -> None:
    """C = A @ B for fp32 A, B, C on bf16 matrix units (each input split in two
    bf16 parts, three products per term); error within 1e-4 * sum|a*b|."""
    M, N, K = _shapes(A, B, C)
    if not (A.dtype == B.dtype == C.dtype == torch.float32):
        raise TypeError("gemm_f32_3xbf16 takes float32 A, B and C")
    with _on_device(C):
        _check(_lib.gemm_f32_3xbf16(M, N, K, A.data_ptr(), _pitch(A, K), B.data_ptr(),
                                    _pitch(B, N), C.data_ptr(), _pitch(C, N), _stream(C, stream)))


def _gemm16(fn, dtype, A, B, C, stream):
    M, N, K = _shapes(A, B, C)
    if A.dtype != dtype or B.dtype != dtype:
        raise TypeError(f"inputs must be {dtype}")
    if C.dtype == torch.float32:
        out = DGEMM_OUT_F32
    elif C.dtype == dtype:
        out = DGEMM_OUT_SAME
    else:
        raise TypeError(f"C must be float32 or {dtype}")
    with _on_device(C):
        _check(fn(M, N, K, A.data_ptr(), _pitch(A, K), B.data_ptr(), _pitch(B, N),
                  C.data_ptr(), _pitch(C, N), out, _stream(C, stream)))


def gemm_bf16(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, stream=None) -> None:
    """C = A @ B for bf16 A, B; C is float32 or bfloat16 (rounded once, nearest even)."""
    _gemm16(_lib.gemm_bf16, torch.bfloat16, A, B, C, stream)


def gemm_f16(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, stream=None) -> None:
    """C = A @ B for fp16 A, B; C is float32 or float16 (rounded once, nearest even)."""
    _gemm16(_lib.gemm_f16, torch.float16, A, B, C, stream)


def gemm_ex_plan(in_fmt: str, M: int, N: int, K: int, workspace_bytes: int,
                 out_same: bool = False) -> dict:
    """Host query of the plan gemm_ex uses with `workspace_bytes` available."""
    v = [ctypes.c_int(-1) for _ in range(3)]
    used = _c_size_t(0)
    out = DGEMM_OUT_SAME if out_same else DGEMM_OUT_F32
    _check(_lib.gemm_ex_plan(IN_CODES[in_fmt], out, M, N, K, int(workspace_bytes),
                             *[ctypes.byref(x) for x in v], ctypes.byref(used)))
    return {"tile_rows": v[0].value, "tile_cols": v[1].value, "splits": v[2].value,
            "stream_k": v[2].value == 0, "workspace_bytes": used.value}


def dgemm_set_plan_override(kind: int, tile_rows: int = 0, tile_cols: int = 0,
                            splits: int = 1) -> None:
    """Process-wide plan override of gemm_ex / gemm_ex_static / gemm_ex_plan
    (DGEMM_PLAN_AUTO clears it); for tests and tuning."""
    _check(_lib.dgemm_set_plan_override(int(kind), int(tile_rows), int(tile_cols), int(splits)))


def dgemm_set_stream_k_wait_us(us: float) -> None:
    """Longest wait of a Stream-K workgroup for another's partial sums, in
    microseconds (< 0: the default; 0: never wait, compute missing ones)."""
    _check(_lib.dgemm_set_stream_k_wait_us(float(us)))


def dgemm_stream_k_schedule(in_fmt: str, M: int, N: int, K: int, wg: int,
                            partials_present: bool = True) -> list:
    """Host query of the items Stream-K workgroup `wg` runs, in order: a list
    of dicts (role, tile_m, tile_n, k_begin, k_end, slot, first, last, lo, hi)."""
    n = ctypes.c_int(0)
    st = _lib.dgemm_stream_k_schedule(IN_CODES[in_fmt], M, N, K, wg, int(partials_present),
                                      None, 0, ctypes.byref(n))
    if n.value == 0:
        _check(st)
        return []
    buf = (ctypes.c_int * (10 * n.value))()
    _check(_lib.dgemm_stream_k_schedule(IN_CODES[in_fmt], M, N, K, wg, int(partials_present),
                                        buf, n.value, ctypes.byref(n)))
    keys = ("role", "tile_m", "tile_n", "k_begin", "k_end", "slot", "first", "last", "lo", "hi")
    out = []
    for i in range(n.value):
        d = dict(zip(keys, buf[10 * i: 10 * i + 10]))
        d["role"] = SK_ROLES[d["role"]]
        out.append(d)
    return out


def _ex_args(A, B, C, bias, in_fmt):
    """(M, N, K, input code, output code, bias pointer) for gemm_ex and gemm_ex_static."""
    M, N, K = _shapes(A, B, C)
    fmt = in_fmt or _TORCH_IN.get(A.dtype)
    if fmt is None or B.dtype != A.dtype or (fmt == "f32x3" and A.dtype != torch.float32):
        raise TypeError("unsupported input dtypes")
    if C.dtype == torch.float32:
        out = DGEMM_OUT_F32
    elif C.dtype == A.dtype:
        out = DGEMM_OUT_SAME
    else:
        raise TypeError("C must be float32 or the input dtype")
    bias_ptr = None
    if bias is not None:
        if bias.dtype != torch.float32 or bias.dim() != 1 or bias.numel() != N \
                or not bias.is_contiguous() or bias.device != C.device:
            raise ValueError("bias must be a contiguous float32 device vector of length N")
        bias_ptr = bias.data_ptr()
    return M, N, K, IN_CODES[fmt], out, bias_ptr


def gemm_ex_static(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, *, alpha: float = 1.0,
                   beta: float = 0.0, bias: torch.Tensor = None, relu: bool = False,
                   scratch_bytes: int = DGEMM_STATIC_SCRATCH_BYTES, in_fmt: str = None,
                   stream=None) -> None:
    """gemm_ex with the library's static device scratch as the split-K workspace
    (scratch_bytes of it); allocates nothing.  Calls that overlap in time on one
    GPU share that scratch and must be ordered (one stream)."""
    M, N, K, code, out, bias_ptr = _ex_args(A, B, C, bias, in_fmt)
    with _on_device(C):
        _check(_lib.gemm_ex_static(code, out, M, N, K, A.data_ptr(), _pitch(A, K),
                                   B.data_ptr(), _pitch(B, N), C.data_ptr(), _pitch(C, N),
                                   float(alpha), float(beta), bias_ptr,
                                   DGEMM_ACT_RELU if relu else DGEMM_ACT_NONE,
                                   int(scratch_bytes), _stream(C, stream)))


def gemm_ex(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, *, alpha: float = 1.0,
            beta: float = 0.0, bias: torch.Tensor = None, relu: bool = False,
            workspace: torch.Tensor = None, in_fmt: str = None, stream=None) -> None:
    """C = act(alpha * A @ B + beta * C + bias) through the library's gemm_ex.

    `workspace` (a device tensor, any dtype) lends scratch memory for a split-K
    plan; None means no split.  `in_fmt` picks "f32x3" for fp32 data on the
    3 x bf16 path; by default it follows A's dtype."""
    M, N, K, code, out, bias_ptr = _ex_args(A, B, C, bias, in_fmt)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if workspace.device != C.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on C's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with _on_device(C):
        _check(_lib.gemm_ex(code, out, M, N, K, A.data_ptr(), _pitch(A, K),
                            B.data_ptr(), _pitch(B, N), C.data_ptr(), _pitch(C, N),
                            float(alpha), float(beta), bias_ptr,
                            DGEMM_ACT_RELU if relu else DGEMM_ACT_NONE, ws_ptr, ws_bytes,
                            _stream(C, stream)))


def matmul(A: torch.Tensor, B: torch.Tensor, out_dtype=None, *, bias: torch.Tensor = None,
           relu: bool = False, alpha: float = 1.0, split_k: bool = True,
           stream=None) -> torch.Tensor:
    """Allocates C (torch allocator) and computes C = act(alpha * A @ B + bias).

    C and, with split_k, the workspace a split-K plan asks for are taken from
    torch's allocator on the stream the kernels run on (`stream`, else the
    current one).  The workspace is released on return; the allocator hands
    that block out again only to later work on the same stream, which runs after
    these kernels.  C belongs to that stream too: a caller that goes on to use
    it on another stream orders the two streams (or calls C.record_stream)."""
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("operands must be 2-D")
    if A.dtype not in _TORCH_IN or B.dtype != A.dtype:
        raise TypeError(f"unsupported input dtypes {A.dtype}, {B.dtype}")
    if out_dtype is None:
        out_dtype = A.dtype
    if out_dtype not in (torch.float32, A.dtype):
        raise TypeError(f"out_dtype must be float32 or {A.dtype}")
    if stream is not None and stream != torch.cuda.current_stream(A.device):
        with torch.cuda.stream(stream):
            return matmul(A, B, out_dtype, bias=bias, relu=relu, alpha=alpha, split_k=split_k)
    C = torch.empty((A.shape[0], B.shape[1]), dtype=out_dtype, device=A.device)
    ws = None
    if split_k:
        fmt = _TORCH_IN[A.dtype]
        plan = gemm_ex_plan(fmt, A.shape[0], B.shape[1], A.shape[1], 1 << 40,
                            out_same=(out_dtype == A.dtype and fmt != "f32"))
        if plan["workspace_bytes"] > 0:
            ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=A.device)
    gemm_ex(A, B, C, alpha=alpha, bias=bias, relu=relu, workspace=ws)
    return C


def dgemm_tile_map(M: int, N: int, in_fmt: str, wg: int = -1) -> dict:
    """Host query of the workgroup -> tile mapping (no GPU needed)."""
    v = [ctypes.c_int(-1) for _ in range(5)]
    _check(_lib.dgemm_tile_map(M, N, IN_CODES[in_fmt], wg, *[ctypes.byref(x) for x in v]))
    return {"tile_rows": v[0].value, "tile_cols": v[1].value, "num_wg": v[2].value,
            "tile_m": v[3].value, "tile_n": v[4].value}


def raw():
    """The loaded ctypes library (for tests of the raw C ABI)."""
    return _lib
