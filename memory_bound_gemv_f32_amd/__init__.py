"""Python binding of libgemv (dense GEMV for MI355X / gfx950).

Marshalling only: every step of the computation runs in the HIP kernels of
``libgemv.so``; this module passes device pointers, sizes and the current
HIP stream through ctypes.  There is no CPU fallback: importing this package
without a built ``libgemv.so`` raises ``ImportError``.

Two levels:

* the C ABI under the same names (``gemv_f32``, ``gemv_f16``, ``gemv_bf16``,
  ``gemv_batched_*``, ``gemv_multi_*``, ``gemv_gate_up_silu_*``,
  ``gemv_splitk_*``, ``gemv_q8_*``, ``gemv_plan``, ``gemv_run_family``, ...), taking integer
  addresses and returning the ``gemv_status_t`` code;
* tensor helpers ``gemv``, ``gemv_batched``, ``gemv_multi``,
  ``gemv_gate_up_silu``, ``gemv_splitk`` and ``gemv_q8`` that check dtype, shape,
  strides and device, call the matching entry point on
  ``torch.cuda.current_stream()`` and raise ``GemvError`` on a failure code.

Layout of the tensor helpers: ``A`` is (M, K) with unit column stride and row
stride ``lda = A.stride(0) >= K`` (so a column slice of a wider matrix works);
``x`` is (K,); for the batched form ``X`` is (nvec, K) contiguous, which is the
K×nvec column-major matrix of the C ABI, and the result is (nvec, M)
contiguous, i.e. Y as M×nvec column-major.
"""

from __future__ import annotations

import ctypes
import os
from pathlib import Path

# torch ships its own HIP runtime under the same soname (libamdhip64.so.7) as
# the system one that libgemv is linked against.  Whichever loads first is the
# one the process uses, so torch goes first: libgemv then launches on the
# runtime that owns torch's streams and allocations.
try:
    import torch as _torch_runtime  # noqa: F401
except ImportError:  # a C-only user of the library has no torch
    _torch_runtime = None

PACKAGE = Path(__file__).resolve().parent
# LIBGEMV_LIBRARY: another build of the same library (e.g. for comparing two
# builds in one process tree); the in-tree build by default
LIBRARY = Path(os.environ.get("LIBGEMV_LIBRARY", PACKAGE / "libgemv.so"))

if not LIBRARY.exists():
    raise ImportError(
        f"{LIBRARY} is not built; run `python memory_bound_gemv_f32_amd/build.py` "
        "(there is no fallback implementation)")

_lib = ctypes.CDLL(str(LIBRARY))

GEMV_SUCCESS = 0
GEMV_ERROR_INVALID_VALUE = 1
GEMV_ERROR_LAUNCH_FAILURE = 2

DTYPE_F32, DTYPE_F16, DTYPE_BF16 = 0, 1, 2
DTYPE_CODES = {"f32": DTYPE_F32, "f16": DTYPE_F16, "bf16": DTYPE_BF16}

FAMILY_AUTO = -1
FAMILY_ROWS_PER_WAVE = 0
FAMILY_WAVE_PER_ROW = 1
FAMILY_GROUP_PER_ROW = 2
FAMILY_BATCHED = 3
FAMILY_BATCHED_MFMA = 4
FAMILY_GATED_SILU = 5
FAMILY_SPLIT_K = 6
MAX_SEGMENTS = 8
FAMILY_NAMES = {
    FAMILY_ROWS_PER_WAVE: "rows_per_wave",
    FAMILY_WAVE_PER_ROW: "wave_per_row",
    FAMILY_GROUP_PER_ROW: "group_per_row",
    FAMILY_BATCHED: "batched",
    FAMILY_BATCHED_MFMA: "batched_mfma",
    FAMILY_GATED_SILU: "gated_silu",
    FAMILY_SPLIT_K: "split_k",
}


class GemvPlan(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int) for name in (
        "family", "vector_loads", "chunk_elems", "lanes_per_row",
        "rows_per_wave", "row_tiles", "waves_per_group", "rows_per_group",
        "batch", "passes", "block", "lds_bytes", "splits", "slice_elems",
        "x_in_registers", "rounding_chain", "column_blocks")] + [
        ("grid", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class GemvSegment(ctypes.Structure):
    """gemv_segment_t: one matrix of a multi-GEMV."""
    _fields_ = [("A", ctypes.c_void_p), ("lda", ctypes.c_int), ("M", ctypes.c_int),
                ("bias", ctypes.c_void_p), ("y", ctypes.c_void_p)]


_vp, _i, _st = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p


def _bind(name, argtypes, restype=ctypes.c_int):
    fn = getattr(_lib, name)
    fn.argtypes = argtypes
    fn.restype = restype
    return fn


gemv_status_string = _bind("gemv_status_string", [_i], ctypes.c_char_p)
gemv_last_hip_error = _bind("gemv_last_hip_error", [])
gemv_last_hip_error_string = _bind("gemv_last_hip_error_string", [], ctypes.c_char_p)
gemv_f32 = _bind("gemv_f32", [_vp, _i, _vp, _vp, _vp, _i, _i, _st])
gemv_f16 = _bind("gemv_f16", [_vp, _i, _vp, _vp, _vp, _i, _i, _st])
gemv_bf16 = _bind("gemv_bf16", [_vp, _i, _vp, _vp, _vp, _i, _i, _st])
gemv_batched_f16 = _bind("gemv_batched_f16", [_vp, _i, _vp, _vp, _vp, _i, _i, _i, _st])
gemv_batched_bf16 = _bind("gemv_batched_bf16", [_vp, _i, _vp, _vp, _vp, _i, _i, _i, _st])
gemv_multi_f32 = _bind("gemv_multi_f32", [ctypes.POINTER(GemvSegment), _i, _vp, _i, _st])
gemv_multi_f16 = _bind("gemv_multi_f16", [ctypes.POINTER(GemvSegment), _i, _vp, _i, _st])
gemv_multi_bf16 = _bind("gemv_multi_bf16", [ctypes.POINTER(GemvSegment), _i, _vp, _i, _st])
gemv_gate_up_silu_f32 = _bind("gemv_gate_up_silu_f32", [_vp, _vp, _i, _vp, _vp, _i, _i, _st])
gemv_gate_up_silu_f16 = _bind("gemv_gate_up_silu_f16", [_vp, _vp, _i, _vp, _vp, _i, _i, _st])
gemv_gate_up_silu_bf16 = _bind("gemv_gate_up_silu_bf16", [_vp, _vp, _i, _vp, _vp, _i, _i, _st])
_sz = ctypes.c_size_t
gemv_splitk_workspace_size = _bind("gemv_splitk_workspace_size", [_i, _i, _i, _i, ctypes.POINTER(_sz)])
gemv_splitk_f32 = _bind("gemv_splitk_f32", [_vp, _i, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _st])
gemv_splitk_f16 = _bind("gemv_splitk_f16", [_vp, _i, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _st])
gemv_splitk_bf16 = _bind("gemv_splitk_bf16", [_vp, _i, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _st])
gemv_splitk_noalloc = _bind("gemv_splitk_noalloc", [_i, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _st])
NOALLOC_SCRATCH_BYTES = 256 * 1024
gemv_q8_f32 = _bind("gemv_q8_f32", [_vp, _i, _vp, _vp, _vp, _vp, _i, _i, _st])
gemv_q8_f16 = _bind("gemv_q8_f16", [_vp, _i, _vp, _vp, _vp, _vp, _i, _i, _st])
gemv_q8_bf16 = _bind("gemv_q8_bf16", [_vp, _i, _vp, _vp, _vp, _vp, _i, _i, _st])
gemv_q8_run_family = _bind("gemv_q8_run_family", [_i, _i, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _st])
gemv_plan_q8 = _bind("gemv_plan_q8", [_i, _i, _i, _i, _vp, _vp, _i, ctypes.POINTER(GemvPlan)])
gemv_read_probe = _bind("gemv_read_probe", [_vp, _sz, _vp, _st])
gemv_read_probe_variant = _bind("gemv_read_probe_variant",
                                [_vp, _sz, _vp, _i, _i, _i, _i, _vp, _sz, _st])
gemv_plan = _bind("gemv_plan", [_i, _i, _i, _i, _i, _vp, _vp, _i, ctypes.POINTER(GemvPlan)])
gemv_plan_splitk = _bind("gemv_plan_splitk", [_i, _i, _i, _i, _i, _vp, _vp, ctypes.POINTER(GemvPlan)])
gemv_run_family = _bind("gemv_run_family", [_i, _i, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _st])
gemv_test_refused_launch = _bind("gemv_test_refused_launch", [_st])

EXPORTED = ("gemv_status_string", "gemv_last_hip_error",
            "gemv_last_hip_error_string", "gemv_f32", "gemv_f16", "gemv_bf16",
            "gemv_batched_f16", "gemv_batched_bf16", "gemv_multi_f32",
            "gemv_multi_f16", "gemv_multi_bf16", "gemv_gate_up_silu_f32",
            "gemv_gate_up_silu_f16", "gemv_gate_up_silu_bf16",
            "gemv_splitk_workspace_size", "gemv_splitk_f32", "gemv_splitk_f16",
            "gemv_splitk_bf16", "gemv_splitk_noalloc", "gemv_q8_f32", "gemv_q8_f16", "gemv_q8_bf16",
            "gemv_q8_run_family", "gemv_plan_q8", "gemv_read_probe",
            "gemv_read_probe_variant", "gemv_plan",
            "gemv_plan_splitk", "gemv_run_family", "gemv_test_refused_launch")


class GemvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {gemv_status_string(status).decode()}"
        if status == GEMV_ERROR_LAUNCH_FAILURE:
            msg += f" ({gemv_last_hip_error_string().decode()})"
        super().__init__(msg)


def plan(dtype: str, M: int, K: int, lda: int | None = None, nvec: int = 1,
         A_addr: int = 0, X_addr: int = 0, family: int = FAMILY_AUTO) -> dict:
    """The mapping libgemv would launch (host-only; no GPU needed)."""
    out = GemvPlan()
    rc = gemv_plan(DTYPE_CODES[dtype], M, K, K if lda is None else lda, nvec,
                   A_addr, X_addr, family, ctypes.byref(out))
    if rc != GEMV_SUCCESS:
        raise GemvError(rc, "gemv_plan")
    return out.as_dict()


def plan_splitk(dtype: str, M: int, K: int, lda: int | None = None, splits: int = 0,
                A_addr: int = 0, x_addr: int = 0) -> dict:
    """The mapping gemv_splitk_* would launch (host-only)."""
    out = GemvPlan()
    rc = gemv_plan_splitk(DTYPE_CODES[dtype], M, K, K if lda is None else lda, splits,
                          A_addr, x_addr, ctypes.byref(out))
    if rc != GEMV_SUCCESS:
        raise GemvError(rc, "gemv_plan_splitk")
    return out.as_dict()


def plan_q8(xdtype: str, M: int, K: int, ldq: int | None = None, Q_addr: int = 0,
            x_addr: int = 0, family: int = FAMILY_AUTO) -> dict:
    """The mapping gemv_q8_* would launch for int8 weights and x of type
    ``xdtype`` (host-only)."""
    out = GemvPlan()
    rc = gemv_plan_q8(DTYPE_CODES[xdtype], M, K, K if ldq is None else ldq, Q_addr, x_addr,
                      family, ctypes.byref(out))
    if rc != GEMV_SUCCESS:
        raise GemvError(rc, "gemv_plan_q8")
    return out.as_dict()


def splitk_workspace_size(dtype: str, M: int, K: int, splits: int = 0) -> int:
    """Workspace bytes gemv_splitk_* needs (0: a single slice, none needed)."""
    n = ctypes.c_size_t(0)
    rc = gemv_splitk_workspace_size(DTYPE_CODES[dtype], M, K, splits, ctypes.byref(n))
    if rc != GEMV_SUCCESS:
        raise GemvError(rc, "gemv_splitk_workspace_size")
    return n.value


# ---------------------------------------------------------------------------
# tensor helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch  # noqa: PLC0415 - torch only allocates memory and streams
    return torch


def _dtype_name(t) -> str:
    torch = _torch()
    names = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}
    if t.dtype not in names:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32, float16 or bfloat16")
    return names[t.dtype]


def _stream_handle(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _check_matrix(A):
    if A.dim() != 2:
        raise ValueError("A must be 2-D (M, K)")
    if not A.is_cuda:
        raise ValueError("A must be a device tensor")
    M, K = A.shape
    if K > 1 and A.stride(1) != 1:
        raise ValueError("A must have unit column stride")
    # with one row, or no columns, the row pitch is never used: pass K, the
    # tightest value (so 16-byte alignment depends only on the pointers)
    lda = A.stride(0) if (M > 1 and K > 0) else K
    if lda < K:
        raise ValueError("A's row stride is smaller than K")
    return M, K, lda


def _check_out(out, shape, device):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    if out.dtype != torch.float32 or tuple(out.shape) != tuple(shape) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous float32 tensor of shape {tuple(shape)}")
    if out.device != device:
        raise ValueError("out is on another device")
    return out


def _check_bias(bias, M, device):
    torch = _torch()
    if bias is None:
        return None
    if bias.dtype != torch.float32 or bias.dim() != 1 or bias.shape[0] != M or not bias.is_contiguous():
        raise ValueError("bias must be a contiguous float32 tensor of shape (M,)")
    if bias.device != device:
        raise ValueError("bias is on another device")
    return bias


def gemv(A, x, bias=None, out=None, *, family: int = FAMILY_AUTO, stream=None):
    """y = A @ x (+ bias) in fp32 on A's device; returns y (M,) float32."""
    M, K, lda = _check_matrix(A)
    dt = _dtype_name(A)
    if x.dtype != A.dtype or x.dim() != 1 or x.shape[0] != K or not x.is_contiguous():
        raise ValueError("x must be a contiguous (K,) tensor of A's dtype")
    if x.device != A.device:
        raise ValueError("x is on another device")
    bias = _check_bias(bias, M, A.device)
    y = _check_out(out, (M,), A.device)
    args = (A.data_ptr(), lda, x.data_ptr(),
            bias.data_ptr() if bias is not None else None, y.data_ptr(), M, K)
    if family == FAMILY_AUTO:
        fn = {"f32": gemv_f32, "f16": gemv_f16, "bf16": gemv_bf16}[dt]
        rc = fn(*args, _stream_handle(stream))
        where = fn.__name__
    else:
        rc = gemv_run_family(DTYPE_CODES[dt], family, args[0], lda, args[2],
                             args[3], args[4], M, K, 1, _stream_handle(stream))
        where = "gemv_run_family"
    if rc != GEMV_SUCCESS:
        raise GemvError(rc, where)
    return y


def gemv_batched(A, X, bias=None, out=None, *, family: int = FAMILY_AUTO,
                 stream=None):
    """Y = A @ X (+ bias) for X of shape (nvec, K), 1 <= nvec <= 64, fp16 or
    bf16; returns Y of shape (nvec, M) float32 (column j = output for X[j])."""
    M, K, lda = _check_matrix(A)
    dt = _dtype_name(A)
    if X.dtype != A.dtype or X.dim() != 2 or X.shape[1] != K or not X.is_contiguous():
        raise ValueError("X must be a contiguous (nvec, K) tensor of A's dtype")
    if X.device != A.device:
        raise ValueError("X is on another device")
    nvec = X.shape[0]
    bias = _check_bias(bias, M, A.device)
    Y = _check_out(out, (nvec, M), A.device)
    bptr = bias.data_ptr() if bias is not None else None
    if family == FAMILY_AUTO:
        if dt == "f32":
            raise TypeError("the batched entry points take float16 or bfloat16")
        fn = {"f16": gemv_batched_f16, "bf16": gemv_batched_bf16}[dt]
        rc = fn(A.data_ptr(), lda, X.data_ptr(), bptr, Y.data_ptr(), M, K, nvec,
                _stream_handle(stream))
        where = fn.__name__
    else:
        rc = gemv_run_family(DTYPE_CODES[dt], family, A.data_ptr(), lda,
                             X.data_ptr(), bptr, Y.data_ptr(), M, K, nvec,
                             _stream_handle(stream))
        where = "gemv_run_family"
    if rc != GEMV_SUCCESS:
        raise GemvError(rc, where)
    return Y


def gemv_splitk(A, x, bias=None, out=None, *, splits: int = 0, workspace=None, stream=None):
    """y = A @ x (+ bias) by split-K (for few, long rows); returns y (M,)
    float32.  ``workspace``: a device tensor of at least
    ``splitk_workspace_size(...)`` bytes, allocated here through torch when
    not given."""
    torch = _torch()
    M, K, lda = _check_matrix(A)
    dt = _dtype_name(A)
    if x.dtype != A.dtype or x.dim() != 1 or x.shape[0] != K or not x.is_contiguous():
        raise ValueError("x must be a contiguous (K,) tensor of A's dtype")
    if x.device != A.device:
        raise ValueError("x is on another device")
    bias = _check_bias(bias, M, A.device)
    y = _check_out(out, (M,), A.device)
    need = splitk_workspace_size(dt, M, K, splits)
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=A.device)
    if workspace.device != A.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on A's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    fn = {"f32": gemv_splitk_f32, "f16": gemv_splitk_f16, "bf16": gemv_splitk_bf16}[dt]
    rc = fn(A.data_ptr(), lda, x.data_ptr(), bias.data_ptr() if bias is not None else None,
            y.data_ptr(), M, K, splits, workspace.data_ptr(), ws_bytes, _stream_handle(stream))
    if rc != GEMV_SUCCESS:
        raise GemvError(rc, fn.__name__)
    return y


def gemv_q8(Q, scale, x, bias=None, out=None, *, family: int = FAMILY_AUTO, stream=None):
    """Weight-only int8: y = scale * (Q @ x) (+ bias) with Q int8 (M, K)
    (unit column stride, row stride ldq), scale float32 (M,), x (K,) float32,
    float16 or bfloat16; returns y (M,) float32."""
    torch = _torch()
    if Q.dtype != torch.int8:
        raise TypeError("Q must be int8")
    M, K, ldq = _check_matrix(Q)
    if x.dim() != 1 or x.shape[0] != K or not x.is_contiguous() or x.device != Q.device:
        raise ValueError("x must be a contiguous (K,) tensor on Q's device")
    dt = _dtype_name(x)
    if (scale.dtype != torch.float32 or scale.dim() != 1 or scale.shape[0] != M
            or not scale.is_contiguous() or scale.device != Q.device):
        raise ValueError("scale must be a contiguous float32 (M,) tensor on Q's device")
    bias = _check_bias(bias, M, Q.device)
    y = _check_out(out, (M,), Q.device)
    bptr = bias.data_ptr() if bias is not None else None
    if family == FAMILY_AUTO:
        fn = {"f32": gemv_q8_f32, "f16": gemv_q8_f16, "bf16": gemv_q8_bf16}[dt]
        rc = fn(Q.data_ptr(), ldq, scale.data_ptr(), x.data_ptr(), bptr, y.data_ptr(), M, K,
                _stream_handle(stream))
        where = fn.__name__
    else:
        rc = gemv_q8_run_family(DTYPE_CODES[dt], family, Q.data_ptr(), ldq, scale.data_ptr(),
                                x.data_ptr(), bptr, y.data_ptr(), M, K, _stream_handle(stream))
        where = "gemv_q8_run_family"
    if rc != GEMV_SUCCESS:
        raise GemvError(rc, where)
    return y


def segment_table(segments) -> "ctypes.Array":
    """A gemv_segment_t array from (A_addr, lda, M, bias_addr_or_None, y_addr)
    tuples."""
    arr = (GemvSegment * len(segments))()
    for i, (A, lda, M, bias, y) in enumerate(segments):
        arr[i] = GemvSegment(A, lda, M, bias, y)
    return arr


def gemv_multi(As, x, biases=None, outs=None, *, stream=None):
    """y_i = A_i @ x (+ bias_i) for up to 8 matrices with the same K and dtype,
    in one launch; returns the list of y_i (float32)."""
    if not 1 <= len(As) <= MAX_SEGMENTS:
        raise ValueError(f"between 1 and {MAX_SEGMENTS} matrices")
    dt = _dtype_name(As[0])
    K = As[0].shape[1] if As[0].dim() == 2 else -1
    if x.dtype != As[0].dtype or x.dim() != 1 or x.shape[0] != K or not x.is_contiguous():
        raise ValueError("x must be a contiguous (K,) tensor of the matrices' dtype")
    biases = list(biases) if biases is not None else [None] * len(As)
    outs = list(outs) if outs is not None else [None] * len(As)
    segs, ys = [], []
    for A, b, o in zip(As, biases, outs):
        M, Ki, lda = _check_matrix(A)
        if A.dtype != As[0].dtype or Ki != K or A.device != x.device:
            raise ValueError("every matrix must have x's dtype, K and device")
        b = _check_bias(b, M, A.device)
        y = _check_out(o, (M,), A.device)
        ys.append(y)
        segs.append((A.data_ptr(), lda, M, b.data_ptr() if b is not None else None, y.data_ptr()))
    table = segment_table(segs)
    fn = {"f32": gemv_multi_f32, "f16": gemv_multi_f16, "bf16": gemv_multi_bf16}[dt]
    rc = fn(table, len(segs), x.data_ptr(), K, _stream_handle(stream))
    if rc != GEMV_SUCCESS:
        raise GemvError(rc, fn.__name__)
    return ys


def gemv_gate_up_silu(A_gate, A_up, x, out=None, *, stream=None):
    """h = silu(A_gate @ x) * (A_up @ x) in one pass over both matrices
    (same shape, dtype and row stride); returns h (M,) float32."""
    M, K, lda = _check_matrix(A_gate)
    M2, K2, lda2 = _check_matrix(A_up)
    if (M2, K2) != (M, K) or A_up.dtype != A_gate.dtype or A_up.device != A_gate.device:
        raise ValueError("A_gate and A_up must have the same shape, dtype and device")
    if lda2 != lda and M > 1:
        raise ValueError("A_gate and A_up must have the same row stride")
    dt = _dtype_name(A_gate)
    if x.dtype != A_gate.dtype or x.dim() != 1 or x.shape[0] != K or not x.is_contiguous():
        raise ValueError("x must be a contiguous (K,) tensor of the matrices' dtype")
    h = _check_out(out, (M,), A_gate.device)
    fn = {"f32": gemv_gate_up_silu_f32, "f16": gemv_gate_up_silu_f16,
          "bf16": gemv_gate_up_silu_bf16}[dt]
    rc = fn(A_gate.data_ptr(), A_up.data_ptr(), lda, x.data_ptr(), h.data_ptr(), M, K,
            _stream_handle(stream))
    if rc != GEMV_SUCCESS:
        raise GemvError(rc, fn.__name__)
    return h
