"""Python binding of libsparq24 (ctypes): argument marshalling only.

Every step of every call runs in the HIP kernels of ``libsparq24.so``; this
module builds the C descriptors from torch tensors, allocates outputs and
workspace with torch (device memory only) and passes the current HIP stream.
There is no fallback: if the library is missing or a call fails, an exception
is raised.

The operations follow Qin, "Is 2:4 Sparsity Still Worth It?" (paper-daily.com
English summary, sections 2-4); the C header ``include/sparq24.h`` documents
each one.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_int32, c_int64, c_size_t, c_uint8, c_void_p
from typing import Optional, Sequence, Tuple, Union

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparq24.so")

F32, BF16, F16 = 0, 1, 2
MAGNITUDE, WANDA = 0, 1
Q_NONE, Q_INT, Q_FP8, Q_MXFP4, Q_NVFP4 = 0, 1, 2, 3, 4

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "bad shape", 4: "misaligned",
          5: "workspace", 6: "no device", 7: "launch failed"}


class Sparq24Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({STATUS.get(status, '?')})")
        self.status = status


class CTensor(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("dtype", c_int32), ("batch", c_int64), ("rows", c_int64),
                ("k", c_int64), ("batch_stride", c_int64), ("row_stride", c_int64),
                ("k_stride", c_int64)]


class CQSpec(ctypes.Structure):
    _fields_ = [("fmt", c_int32), ("bits", c_int32), ("tensor_amax_in", c_void_p)]


class CSide(ctypes.Structure):
    _fields_ = [("pattern", c_int32), ("q", CQSpec)]


#: Every symbol the C header declares.
SYMBOLS = ("sparq24_prune_compress", "sparq24_quantize", "sparq24_prune_quantize",
           "sparq24_error_energy", "sparq24_predict_R", "sparq24_col_l2norm", "sparq24_copy",
           "sparq24_prune_compress_pairs48", "sparq24_prune_quantize_pairs48",
           "sparq24_predict_R_pairs48", "sparq24_hadamard", "sparq24_quantize_rot",
           "sparq24_prune_quantize_rot", "sparq24_predict_R_rot", "sparq24_operator_error",
           "sparq24_sparse_gemm", "sparq24_dense_gemm", "sparq24_fp8_gemm",
           "sparq24_bits_per_element", "sparq24_status_string", "sparq24_version",
           "sparq24_predict_R_noalloc")

_lib = None


def lib(path: Optional[str] = None):
    """Load libsparq24.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} not found: build it with `python -m pruning_quantization_amd.build`")
    L = ctypes.CDLL(p)
    T, Q = POINTER(CTensor), POINTER(CQSpec)
    sig = {
        "sparq24_prune_compress": [T, c_int32, c_void_p, c_void_p, c_void_p, c_void_p],
        "sparq24_quantize": [T, Q, c_void_p, c_void_p, c_void_p, c_void_p, POINTER(c_size_t), c_void_p],
        "sparq24_prune_quantize": [T, c_int32, c_void_p, Q, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, POINTER(c_size_t), c_void_p],
        "sparq24_prune_quantize_pairs48": [T, Q, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           POINTER(c_size_t), c_void_p],
        "sparq24_error_energy": [T, c_int32, c_void_p, Q, Q, c_int64, c_void_p, c_void_p,
                                 POINTER(c_size_t), c_void_p],
        "sparq24_predict_R": [T, c_int32, c_void_p, Q, Q, c_int32, c_int64, c_void_p, c_void_p,
                              POINTER(c_size_t), c_void_p],
        "sparq24_predict_R_noalloc": [T, c_int32, c_void_p, Q, Q, c_int32, c_int64, c_void_p,
                                      c_void_p],
        "sparq24_col_l2norm": [T, c_void_p, c_void_p, POINTER(c_size_t), c_void_p],
        "sparq24_copy": [c_void_p, c_void_p, c_size_t, c_void_p],
        "sparq24_prune_compress_pairs48": [T, c_void_p, c_void_p, c_void_p],
        "sparq24_predict_R_pairs48": [T, Q, Q, c_int32, c_int64, c_void_p, c_void_p,
                                      POINTER(c_size_t), c_void_p],
        "sparq24_hadamard": [T, c_int32, c_void_p, c_void_p, POINTER(c_size_t), c_void_p],
        "sparq24_operator_error": [T, T, POINTER(CSide), c_int32, c_void_p, c_void_p,
                                   POINTER(c_size_t), c_void_p],
        "sparq24_sparse_gemm": [c_void_p, c_void_p, c_int64, c_int64, T, c_void_p, c_void_p],
        "sparq24_dense_gemm": [T, T, c_void_p, c_void_p],
        "sparq24_fp8_gemm": [c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_int64, c_int64,
                             c_void_p, c_void_p],
        "sparq24_quantize_rot": [T, c_int32, Q, c_void_p, c_void_p, c_void_p, c_void_p,
                                 POINTER(c_size_t), c_void_p],
        "sparq24_prune_quantize_rot": [T, c_int32, c_int32, Q, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, POINTER(c_size_t), c_void_p],
        "sparq24_predict_R_rot": [T, c_int32, c_int32, Q, Q, c_int32, c_int64, c_void_p, c_void_p,
                                  POINTER(c_size_t), c_void_p],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = c_int32
    L.sparq24_bits_per_element.argtypes = [Q, c_int32, c_int64, c_int32, c_int64]
    L.sparq24_bits_per_element.restype = c_double
    L.sparq24_status_string.argtypes = [c_int32]
    L.sparq24_status_string.restype = ctypes.c_char_p
    L.sparq24_version.argtypes = []
    L.sparq24_version.restype = ctypes.c_char_p
    if path is None:
        _lib = L
    return L


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise Sparq24Error(fn, st)


# ---------------------------------------------------------------------------
# Descriptors
# ---------------------------------------------------------------------------

_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


def describe(x: torch.Tensor, axis: int = -1) -> Tuple[CTensor, Tuple[int, ...]]:
    """C descriptor of ``x`` with the reduction axis ``axis``.

    The reduction axis is either the last dim (K-contiguous rows, leading dims
    are rows) or the second to last with a unit-stride last dim (transposed:
    the last dim indexes rows, dims before the axis are batches).  Returns the
    descriptor and the output shape prefix (batch..., rows)."""
    if x.dtype not in _DT:
        raise TypeError(f"unsupported dtype {x.dtype}")
    nd = x.dim()
    axis = axis % nd
    c = CTensor()
    c.data = x.data_ptr()
    c.dtype = _DT[x.dtype]
    if axis == nd - 1:
        lead = x.shape[:-1]
        c.k = x.shape[-1]
        c.k_stride = x.stride(-1) if x.shape[-1] > 1 else 1
        if nd == 1:
            c.batch, c.rows, c.batch_stride, c.row_stride = 1, 1, 0, c.k
        elif nd == 2:
            c.batch, c.rows = 1, x.shape[0]
            c.batch_stride, c.row_stride = 0, x.stride(0)
        else:
            y = x.reshape(-1, x.shape[-2], x.shape[-1]) if nd > 3 else x
            if nd > 3 and y.data_ptr() != x.data_ptr():
                raise ValueError("leading dims must be collapsible")
            c.batch, c.rows = y.shape[0], y.shape[1]
            c.batch_stride, c.row_stride = y.stride(0), y.stride(1)
        return c, tuple(lead)
    if axis == nd - 2 and x.stride(-1) == 1:
        c.k = x.shape[axis]
        c.k_stride = x.stride(axis)
        c.rows = x.shape[-1]
        c.row_stride = 1
        lead = x.shape[:axis]
        if len(lead) == 0:
            c.batch, c.batch_stride = 1, 0
        elif len(lead) == 1:
            c.batch, c.batch_stride = lead[0], x.stride(0)
        else:
            raise ValueError("at most one batch dim before a transposed reduction axis")
        return c, tuple(lead) + (x.shape[-1],)
    raise ValueError("reduction axis must be the last dim, or the second to last with the last dim contiguous")


QLike = Union[str, Tuple[str, int], CQSpec]


def qspec(q: QLike, tensor_amax: Optional[torch.Tensor] = None) -> CQSpec:
    """("int", b) | "fp8" | "mxfp4" | "nvfp4" | "none" -> C spec."""
    if isinstance(q, CQSpec):
        return q
    if isinstance(q, tuple):
        name, bits = q
    else:
        name, bits = q, 0
    fmt = {"none": Q_NONE, "int": Q_INT, "fp8": Q_FP8, "mxfp4": Q_MXFP4, "nvfp4": Q_NVFP4}[name]
    s = CQSpec()
    s.fmt, s.bits = fmt, int(bits)
    s.tensor_amax_in = tensor_amax.data_ptr() if tensor_amax is not None else None
    return s


def _stream(x: torch.Tensor) -> int:
    return torch.cuda.current_stream(x.device).cuda_stream


def _score(score: str) -> int:
    return {"magnitude": MAGNITUDE, "wanda": WANDA}[score]


def _ptr(t: Optional[torch.Tensor]):
    return t.data_ptr() if t is not None else None


def _norm_ptr(score: str, col_norm: Optional[torch.Tensor]):
    if score == "wanda":
        if col_norm is None or col_norm.dtype != torch.float32 or not col_norm.is_contiguous():
            raise ValueError("wanda needs a contiguous fp32 col_norm")
        return col_norm.data_ptr()
    return None


def _workspace(x: torch.Tensor, query):
    """Query the workspace size and allocate it; returns (ws tensor or None,
    the ws_bytes argument to pass: a c_size_t, or None when none is needed)."""
    n = c_size_t(0)
    query(None, ctypes.byref(n))
    if n.value == 0:
        return None, None
    return torch.empty(int(n.value), dtype=torch.uint8, device=x.device), n


def _wsarg(n):
    return ctypes.byref(n) if n is not None else None


def _code_dtype(q: CQSpec):
    if q.fmt == Q_INT:
        return torch.int8 if q.bits <= 8 else torch.int16
    return torch.uint8


# ---------------------------------------------------------------------------
# Calls
# ---------------------------------------------------------------------------


def prune_compress(x: torch.Tensor, axis: int = -1, score: str = "magnitude",
                   col_norm: Optional[torch.Tensor] = None,
                   out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """2:4 prune-and-compress along ``axis`` -> (values [..., K/2] in x.dtype,
    meta uint8 [..., K/8])."""
    c, lead = describe(x, axis)
    k = int(c.k)
    if out is None:
        vals = torch.empty(*lead, k // 2, dtype=x.dtype, device=x.device)
        meta = torch.empty(*lead, k // 8, dtype=torch.uint8, device=x.device)
    else:
        vals, meta = out
    st = lib().sparq24_prune_compress(ctypes.byref(c), _score(score), _norm_ptr(score, col_norm),
                                      vals.data_ptr(), meta.data_ptr(), _stream(x))
    _check("sparq24_prune_compress", st)
    return vals, meta


def _pq_outputs(x, lead, k, qs, meta_div):
    dev = x.device
    meta = torch.empty(*lead, k // meta_div, dtype=torch.uint8, device=dev)
    if qs.fmt in (Q_INT, Q_FP8):
        codes = torch.empty(*lead, k // 2, dtype=_code_dtype(qs), device=dev)
        return codes, meta, torch.empty(*lead, dtype=torch.float32, device=dev)
    codes = torch.empty(*lead, k // 4, dtype=torch.uint8, device=dev)
    if qs.fmt == Q_MXFP4:
        return codes, meta, torch.empty(*lead, k // 64, dtype=torch.uint8, device=dev)
    return (codes, meta, torch.empty(*lead, k // 32, dtype=torch.uint8, device=dev),
            torch.empty(1, dtype=torch.float32, device=dev))


def _prune_quantize(name, head, x, lead, c, qs, meta_div, out, workspace):
    """Shared marshalling of the fused prune + quantize calls; ``head`` are the
    arguments between the tensor and the qspec."""
    k = int(c.k)
    fn = getattr(lib(), name)
    s = _stream(x)
    outs = _pq_outputs(x, lead, k, qs, meta_div) if out is None else tuple(out)
    codes, meta, scales = outs[:3]
    ts = outs[3] if len(outs) > 3 else None
    if workspace is None:
        ws, n = _workspace(x, lambda w, nb: fn(ctypes.byref(c), *head, ctypes.byref(qs), None, None,
                                               None, None, w, nb, s))
    else:
        ws, n = workspace, (c_size_t(workspace.numel()) if workspace is not None else None)
    st = fn(ctypes.byref(c), *head, ctypes.byref(qs), codes.data_ptr(), meta.data_ptr(),
            scales.data_ptr(), _ptr(ts), _ptr(ws), _wsarg(n), s)
    _check(name, st)
    return outs


def prune_quantize(x: torch.Tensor, q: QLike, axis: int = -1, score: str = "magnitude",
                   col_norm: Optional[torch.Tensor] = None,
                   tensor_amax: Optional[torch.Tensor] = None, out=None, workspace=None):
    """Fused 2:4 prune + compress + quantization of the kept values.
    INT/FP8 -> (codes [..., K/2], meta uint8 [..., K/8], scales fp32 [...]);
    MXFP4 -> (codes [..., K/4], meta, e8m0 [..., K/64]); NVFP4 -> (codes
    [..., K/4], meta, e4m3 [..., K/32], tensor scale fp32 [1])."""
    c, lead = describe(x, axis)
    qs = qspec(q, tensor_amax)
    return _prune_quantize("sparq24_prune_quantize", (_score(score), _norm_ptr(score, col_norm)),
                           x, lead, c, qs, 8, out, workspace)


def prune_quantize_pairs48(x: torch.Tensor, q: QLike, axis: int = -1,
                           tensor_amax: Optional[torch.Tensor] = None, out=None, workspace=None):
    """Pairwise 4:8 prune + quantization of the kept values (with NVFP4: the
    sparse FP4 operand).  Outputs as :func:`prune_quantize` with meta
    [..., K/16]."""
    c, lead = describe(x, axis)
    qs = qspec(q, tensor_amax)
    return _prune_quantize("sparq24_prune_quantize_pairs48", (), x, lead, c, qs, 16, out,
                           workspace)


def _quantize(name, head, x, lead, c, qs, out, workspace):
    k = int(c.k)
    fn = getattr(lib(), name)
    s = _stream(x)
    if out is None:
        if qs.fmt in (Q_INT, Q_FP8):
            codes = torch.empty(*lead, k, dtype=_code_dtype(qs), device=x.device)
            scales = torch.empty(*lead, dtype=torch.float32, device=x.device)
        elif qs.fmt == Q_MXFP4:
            codes = torch.empty(*lead, k // 2, dtype=torch.uint8, device=x.device)
            scales = torch.empty(*lead, k // 32, dtype=torch.uint8, device=x.device)
        else:
            codes = torch.empty(*lead, k // 2, dtype=torch.uint8, device=x.device)
            scales = torch.empty(*lead, k // 16, dtype=torch.uint8, device=x.device)
        ts = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        codes, scales, ts = out
    if workspace is None:
        ws, n = _workspace(x, lambda w, nb: fn(ctypes.byref(c), *head, ctypes.byref(qs), None, None,
                                               None, w, nb, s))
    else:
        ws, n = workspace, (c_size_t(workspace.numel()) if workspace is not None else None)
    st = fn(ctypes.byref(c), *head, ctypes.byref(qs), codes.data_ptr(), scales.data_ptr(),
            ts.data_ptr(), _ptr(ws), _wsarg(n), s)
    _check(name, st)
    if qs.fmt == Q_NVFP4:
        return codes, scales, ts
    return codes, scales


_PATTERNS = {"2:4": 0, "pairs4:8": 1}


def prune_quantize_rot(x: torch.Tensor, block: int, q: QLike, pattern: str = "2:4", axis: int = -1,
                       tensor_amax: Optional[torch.Tensor] = None, out=None, workspace=None):
    """Magnitude prune (2:4 or pairwise 4:8) + quantization of the kept values
    of the block-Hadamard-rotated operand (rotation fused).  Outputs as
    :func:`prune_quantize` / :func:`prune_quantize_pairs48`."""
    c, lead = describe(x, axis)
    qs = qspec(q, tensor_amax)
    return _prune_quantize("sparq24_prune_quantize_rot", (int(block), _PATTERNS[pattern]), x, lead,
                           c, qs, 8 if pattern == "2:4" else 16, out, workspace)


def hadamard(x: torch.Tensor, block: int, axis: int = -1, out: Optional[torch.Tensor] = None,
             workspace=None):
    """Block Hadamard rotation along ``axis`` -> [..., K] in x.dtype (the
    rotated axis last)."""
    c, lead = describe(x, axis)
    k = int(c.k)
    L = lib()
    s = _stream(x)
    if out is None:
        out = torch.empty(*lead, k, dtype=x.dtype, device=x.device)
    if workspace is None:
        ws, n = _workspace(x, lambda w, nb: L.sparq24_hadamard(ctypes.byref(c), int(block), None, w,
                                                               nb, s))
    else:
        ws, n = workspace, (c_size_t(workspace.numel()) if workspace is not None else None)
    st = L.sparq24_hadamard(ctypes.byref(c), int(block), out.data_ptr(), _ptr(ws), _wsarg(n), s)
    _check("sparq24_hadamard", st)
    return out


def quantize(x: torch.Tensor, q: QLike, axis: int = -1,
             tensor_amax: Optional[torch.Tensor] = None, out=None, workspace=None):
    """Dense quantization.  INT/FP8 -> (codes [..., K], scales fp32 [...]);
    MXFP4 -> (codes [..., K/2], e8m0 [..., K/32]); NVFP4 -> (codes [..., K/2],
    e4m3 block scales [..., K/16], tensor scale fp32 [1])."""
    c, lead = describe(x, axis)
    return _quantize("sparq24_quantize", (), x, lead, c, qspec(q, tensor_amax), out, workspace)


def quantize_rot(x: torch.Tensor, block: int, q: QLike, axis: int = -1,
                 tensor_amax: Optional[torch.Tensor] = None, out=None, workspace=None):
    """:func:`quantize` of the block-Hadamard-rotated operand (rotation fused)."""
    c, lead = describe(x, axis)
    return _quantize("sparq24_quantize_rot", (int(block),), x, lead, c, qspec(q, tensor_amax),
                     out, workspace)


def _qarray(qs: Sequence[QLike]):
    arr = (CQSpec * len(qs))()
    for i, q in enumerate(qs):
        arr[i] = qspec(q)
    return arr


def error_energy(x: torch.Tensor, kept: QLike, dense: QLike, axis: int = -1,
                 score: str = "magnitude", col_norm: Optional[torch.Tensor] = None,
                 rows_per_block: int = 0, out: Optional[torch.Tensor] = None, workspace=None):
    """Raw error energies per block -> fp64 [nblk, 4] = (sum x^2, sum dropped
    x^2, kept error, dense error)."""
    c, _ = describe(x, axis)
    kq, dq = qspec(kept), qspec(dense)
    L = lib()
    s = _stream(x)
    nrows = int(c.batch) * int(c.rows)
    rpb = rows_per_block or nrows
    nblk = (nrows + rpb - 1) // rpb
    if out is None:
        out = torch.empty(nblk, 4, dtype=torch.float64, device=x.device)
    npt = _norm_ptr(score, col_norm)
    if workspace is None:
        ws, n = _workspace(x, lambda w, nb: L.sparq24_error_energy(
            ctypes.byref(c), _score(score), npt, ctypes.byref(kq), ctypes.byref(dq),
            rows_per_block, None, w, nb, s))
    else:
        ws, n = workspace, (c_size_t(workspace.numel()) if workspace is not None else None)
    st = L.sparq24_error_energy(ctypes.byref(c), _score(score), npt, ctypes.byref(kq),
                                ctypes.byref(dq), rows_per_block, out.data_ptr(), _ptr(ws),
                                _wsarg(n), s)
    _check("sparq24_error_energy", st)
    return out


def predict_R(x: torch.Tensor, kept: Sequence[QLike], dense: Sequence[QLike], axis: int = -1,
              score: str = "magnitude", col_norm: Optional[torch.Tensor] = None,
              rows_per_block: int = 0, out: Optional[torch.Tensor] = None, workspace=None):
    """Predicted R -> fp64 [nblk, npairs, 5] = (E_prune, E_qkept, E_2:4,
    E_dense, R)."""
    if len(kept) != len(dense):
        raise ValueError("kept and dense must pair up")
    c, _ = describe(x, axis)
    ka, da = _qarray(kept), _qarray(dense)
    L = lib()
    s = _stream(x)
    nrows = int(c.batch) * int(c.rows)
    rpb = rows_per_block or nrows
    nblk = (nrows + rpb - 1) // rpb
    npairs = len(kept)
    if out is None:
        out = torch.empty(nblk, npairs, 5, dtype=torch.float64, device=x.device)
    npt = _norm_ptr(score, col_norm)
    if workspace is None:
        ws, n = _workspace(x, lambda w, nb: L.sparq24_predict_R(
            ctypes.byref(c), _score(score), npt, ka, da, npairs, rows_per_block, None, w, nb, s))
    else:
        ws, n = workspace, (c_size_t(workspace.numel()) if workspace is not None else None)
    st = L.sparq24_predict_R(ctypes.byref(c), _score(score), npt, ka, da, npairs, rows_per_block,
                             out.data_ptr(), _ptr(ws), _wsarg(n), s)
    _check("sparq24_predict_R", st)
    return out


def predict_R_noalloc(x: torch.Tensor, kept: Sequence[QLike], dense: Sequence[QLike],
                      axis: int = -1, score: str = "magnitude",
                      col_norm: Optional[torch.Tensor] = None, rows_per_block: int = 0,
                      out: Optional[torch.Tensor] = None):
    """:func:`predict_R` through the allocation-free entry point (its workspace
    is the library's static device array); ``out`` may be preallocated."""
    if len(kept) != len(dense):
        raise ValueError("kept and dense must pair up")
    c, _ = describe(x, axis)
    ka, da = _qarray(kept), _qarray(dense)
    nrows = int(c.batch) * int(c.rows)
    rpb = rows_per_block or nrows
    nblk = (nrows + rpb - 1) // rpb
    if out is None:
        out = torch.empty(nblk, len(kept), 5, dtype=torch.float64, device=x.device)
    st = lib().sparq24_predict_R_noalloc(ctypes.byref(c), _score(score), _norm_ptr(score, col_norm),
                                         ka, da, len(kept), rows_per_block, out.data_ptr(),
                                         _stream(x))
    _check("sparq24_predict_R_noalloc", st)
    return out


def prune_compress_pairs48(x: torch.Tensor, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Pairwise 4:8 prune-and-compress along the last dim -> (values [..., K/2],
    meta uint8 [..., K/16])."""
    c, lead = describe(x, -1)
    k = int(c.k)
    if out is None:
        vals = torch.empty(*lead, k // 2, dtype=x.dtype, device=x.device)
        meta = torch.empty(*lead, k // 16, dtype=torch.uint8, device=x.device)
    else:
        vals, meta = out
    st = lib().sparq24_prune_compress_pairs48(ctypes.byref(c), vals.data_ptr(), meta.data_ptr(),
                                              _stream(x))
    _check("sparq24_prune_compress_pairs48", st)
    return vals, meta


def predict_R_pairs48(x: torch.Tensor, kept: Sequence[QLike], dense: Sequence[QLike],
                      axis: int = -1, rows_per_block: int = 0,
                      out: Optional[torch.Tensor] = None, workspace=None):
    """Predicted R of pairwise 4:8 vs dense quantizers -> fp64 [nblk, npairs, 5]."""
    if len(kept) != len(dense):
        raise ValueError("kept and dense must pair up")
    c, _ = describe(x, axis)
    ka, da = _qarray(kept), _qarray(dense)
    L = lib()
    s = _stream(x)
    nrows = int(c.batch) * int(c.rows)
    rpb = rows_per_block or nrows
    nblk = (nrows + rpb - 1) // rpb
    npairs = len(kept)
    if out is None:
        out = torch.empty(nblk, npairs, 5, dtype=torch.float64, device=x.device)
    if workspace is None:
        ws, n = _workspace(x, lambda w, nb: L.sparq24_predict_R_pairs48(
            ctypes.byref(c), ka, da, npairs, rows_per_block, None, w, nb, s))
    else:
        ws, n = workspace, (c_size_t(workspace.numel()) if workspace is not None else None)
    st = L.sparq24_predict_R_pairs48(ctypes.byref(c), ka, da, npairs, rows_per_block,
                                     out.data_ptr(), _ptr(ws), _wsarg(n), s)
    _check("sparq24_predict_R_pairs48", st)
    return out


def predict_R_rot(x: torch.Tensor, block: int, kept: Sequence[QLike], dense: Sequence[QLike],
                  pattern: str = "2:4", axis: int = -1, rows_per_block: int = 0,
                  out: Optional[torch.Tensor] = None, workspace=None):
    """Predicted R of the block-Hadamard-rotated operand (rotation fused) ->
    fp64 [nblk, npairs, 5]."""
    if len(kept) != len(dense):
        raise ValueError("kept and dense must pair up")
    c, _ = describe(x, axis)
    ka, da = _qarray(kept), _qarray(dense)
    L = lib()
    s = _stream(x)
    nrows = int(c.batch) * int(c.rows)
    rpb = rows_per_block or nrows
    nblk = (nrows + rpb - 1) // rpb
    npairs = len(kept)
    pat = _PATTERNS[pattern]
    if out is None:
        out = torch.empty(nblk, npairs, 5, dtype=torch.float64, device=x.device)
    if workspace is None:
        ws, n = _workspace(x, lambda w, nb: L.sparq24_predict_R_rot(
            ctypes.byref(c), int(block), pat, ka, da, npairs, rows_per_block, None, w, nb, s))
    else:
        ws, n = workspace, (c_size_t(workspace.numel()) if workspace is not None else None)
    st = L.sparq24_predict_R_rot(ctypes.byref(c), int(block), pat, ka, da, npairs, rows_per_block,
                                 out.data_ptr(), _ptr(ws), _wsarg(n), s)
    _check("sparq24_predict_R_rot", st)
    return out


def operator_error(a: torch.Tensor, b: torch.Tensor, sides: Sequence[Tuple[str, QLike]],
                   out: Optional[torch.Tensor] = None, workspace=None):
    """Operator-level output error of Y = A B^T (A [M, K], B [N, K], bf16) ->
    fp64 [M, 1 + S]: column 0 the reference output energy per row, column
    1 + s side s's output error energy per row.  A side is (pattern, q) with
    pattern "dense", "2:4" or "pairs4:8"."""
    ca, _ = describe(a, -1)
    cb, _ = describe(b, -1)
    pats = {"2:4": 0, "pairs4:8": 1, "dense": 2}
    arr = (CSide * len(sides))()
    for i, (pat, q) in enumerate(sides):
        arr[i].pattern = pats[pat]
        arr[i].q = qspec(q)
    M = int(ca.batch) * int(ca.rows)
    L = lib()
    s = _stream(a)
    if out is None:
        out = torch.empty(M, 1 + len(sides), dtype=torch.float64, device=a.device)
    if workspace is None:
        ws, n = _workspace(a, lambda w, nb: L.sparq24_operator_error(
            ctypes.byref(ca), ctypes.byref(cb), arr, len(sides), None, w, nb, s))
    else:
        ws, n = workspace, (c_size_t(workspace.numel()) if workspace is not None else None)
    st = L.sparq24_operator_error(ctypes.byref(ca), ctypes.byref(cb), arr, len(sides),
                                  out.data_ptr(), _ptr(ws), _wsarg(n), s)
    _check("sparq24_operator_error", st)
    return out


def sparse_gemm(values: torch.Tensor, meta: torch.Tensor, b: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A B^T (fp32 [M, N]) with A the 2:4-compressed output of
    :func:`prune_compress` (bf16 values [M, K/2], meta [M, K/8]) and B bf16
    [N, K], on the sparse MFMA."""
    m, k = int(values.shape[0]), int(values.shape[1]) * 2
    cb, _ = describe(b, -1)
    n = int(cb.batch) * int(cb.rows)
    if out is None:
        out = torch.empty(m, n, dtype=torch.float32, device=b.device)
    st = lib().sparq24_sparse_gemm(values.data_ptr(), meta.data_ptr(), m, k, ctypes.byref(cb),
                                   out.data_ptr(), _stream(b))
    _check("sparq24_sparse_gemm", st)
    return out


def dense_gemm(a: torch.Tensor, b: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A B^T (fp32 [M, N]) for bf16 A [M, K] and B [N, K], same tile."""
    ca, _ = describe(a, -1)
    cb, _ = describe(b, -1)
    m, n = int(ca.batch) * int(ca.rows), int(cb.batch) * int(cb.rows)
    if out is None:
        out = torch.empty(m, n, dtype=torch.float32, device=a.device)
    st = lib().sparq24_dense_gemm(ctypes.byref(ca), ctypes.byref(cb), out.data_ptr(), _stream(a))
    _check("sparq24_dense_gemm", st)
    return out


def fp8_gemm(codes_a: torch.Tensor, scale_a: torch.Tensor, codes_b: torch.Tensor,
             scale_b: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = diag(scale_a) (A B^T) diag(scale_b) (fp32 [M, N]) from the e4m3
    codes [M, K], [N, K] and per-row scales of :func:`quantize` (FP8)."""
    m, k = int(codes_a.shape[0]), int(codes_a.shape[1])
    n = int(codes_b.shape[0])
    if out is None:
        out = torch.empty(m, n, dtype=torch.float32, device=codes_a.device)
    st = lib().sparq24_fp8_gemm(codes_a.data_ptr(), scale_a.data_ptr(), m, codes_b.data_ptr(),
                                scale_b.data_ptr(), n, k, out.data_ptr(), _stream(codes_a))
    _check("sparq24_fp8_gemm", st)
    return out


def col_l2norm(x: torch.Tensor, out: Optional[torch.Tensor] = None, workspace=None):
    """Per-channel L2 norms of an activation [tokens, channels] -> fp32 [channels]."""
    c, _ = describe(x, -1)
    L = lib()
    s = _stream(x)
    if out is None:
        out = torch.empty(int(c.k), dtype=torch.float32, device=x.device)
    if workspace is None:
        ws, n = _workspace(x, lambda w, nb: L.sparq24_col_l2norm(ctypes.byref(c), None, w, nb, s))
    else:
        ws, n = workspace, (c_size_t(workspace.numel()) if workspace is not None else None)
    st = L.sparq24_col_l2norm(ctypes.byref(c), out.data_ptr(), _ptr(ws), _wsarg(n), s)
    _check("sparq24_col_l2norm", st)
    return out


def copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """Plain device copy through the library's bandwidth-baseline kernel."""
    nbytes = src.numel() * src.element_size()
    st = lib().sparq24_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream(src))
    _check("sparq24_copy", st)


def bits_per_element(q: QLike, sparse24: bool = False, row_len: int = 0, value_bits: int = 0,
                     tensor_elems: int = 0, pattern: Optional[str] = None) -> float:
    """Storage bits charged per original element (host arithmetic in the
    library).  ``pattern``: "dense", "2:4" or "pairs4:8" (``sparse24=True`` is
    "2:4")."""
    qs = qspec(q)
    if pattern is None:
        pattern = "2:4" if sparse24 else "dense"
    code = {"dense": 0, "2:4": 1, "pairs4:8": 2}[pattern]
    return lib().sparq24_bits_per_element(ctypes.byref(qs), code, row_len, value_bits,
                                          tensor_elems)


def version() -> str:
    return lib().sparq24_version().decode()
