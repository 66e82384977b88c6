"""Thin Python binding of libiq.so (see include/iq.h).

Argument marshalling only: every step runs in the HIP library.  Tensors must
be contiguous device tensors of the current HIP device; work is enqueued on
torch's current stream.  If libiq.so is missing this module raises -- there is
no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libiq.so")

FORMATS = ("IQ2_XXS", "IQ2_XS", "IQ2_S", "IQ1_S", "IQ1_M")
FMT = {n: i for i, n in enumerate(FORMATS)}
DTYPE = {torch.float32: 0, torch.bfloat16: 1}

STATUS_NONFINITE, STATUS_OVERFLOW, STATUS_BADCHOICE, STATUS_BADIMP, STATUS_BADID = 1, 2, 4, 8, 16
ERRORS = {-1: "IQ_ERR_FMT", -2: "IQ_ERR_DTYPE", -3: "IQ_ERR_NULL", -4: "IQ_ERR_SHAPE", -5: "IQ_ERR_ARG",
          -6: "IQ_ERR_HIP"}

# C ABI signatures, by exported name
_P, _I, _I64, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
SIGNATURES = {
    "iq_format_info": ([_I, _P], _I),
    "iq_imatrix_collect": ([_P, _I, _I64, _I64, _P, _I, _I, _I, _P, _P, _P, _P], _I),
    "iq_hessian_collect": ([_P, _I, _I64, _I64, _P, _I, _I, _I, _P, _P, _P], _I),
    "iq_imatrix_merge": ([_P, _P, _I, _I64, _P, _P, _P, _P], _I),
    "iq_imatrix_importance": ([_P, _P, _I, _I64, _F, _P, _P, _P], _I),
    "iq_quantize": ([_I, _P, _I, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P], _I),
    "iq_quantize_every_choice": ([_I, _P, _I, _I64, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "iq_choice_search": ([_I, _P, _I, _I64, _I64, _I64, _P, _P, _P, _F, _P, _P, _P, _P], _I),
    "iq_dequantize": ([_I, _P, _I64, _I64, _P, _P, _I, _P], _I),
    "iq_time_next_search": ([_P, _P], _I),
    "iq_error_string": ([_I], ctypes.c_char_p),
}


class IQError(RuntimeError):
    pass


class _FormatInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("block_values", "block_bytes", "grid_size", "choice_groups", "num_choices", "groups_per_choice")]


_lib = None


def lib():
    """Load libiq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise IQError(f"{LIB_PATH} is missing: build it with `python -m ggml_iq_codebook_imatrix_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        raise IQError(f"{what}: {ERRORS.get(rc, rc)} ({lib().iq_error_string(rc).decode()})")


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        if fmt not in FMT:
            raise IQError(f"unknown format {fmt!r}")
        return FMT[fmt]
    return int(fmt)


def _dev(t: torch.Tensor | None, name: str, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise IQError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise IQError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise IQError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def format_info(fmt) -> dict:
    info = _FormatInfo()
    _check(lib().iq_format_info(_fmt(fmt), ctypes.byref(info)), "iq_format_info")
    return {n: getattr(info, n) for n, _ in _FormatInfo._fields_}


def new_status(device=None) -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=device or "cuda")


def read_status(status: torch.Tensor) -> int:
    torch.cuda.synchronize(status.device)
    return int(status.item())


def imatrix_collect(x: torch.Tensor, ids: torch.Tensor | None = None, num_experts: int = 1,
                    chunk_rows: int = 1024, sums: torch.Tensor | None = None,
                    counts: torch.Tensor | None = None, status: torch.Tensor | None = None):
    """Accumulate per-expert sum of x^2 and token counts. Returns (sums [E,K] f32, counts [E] i64)."""
    if x.dim() != 2:
        raise IQError("x must be [T, K]")
    T, K = x.shape
    E = int(num_experts)
    if sums is None:
        sums = torch.zeros((E, K), dtype=torch.float32, device=x.device)
    if counts is None:
        counts = torch.zeros((E,), dtype=torch.int64, device=x.device)
    top_k = 0
    if ids is not None:
        if ids.dim() != 2 or ids.shape[0] != T:
            raise IQError("ids must be [T, top_k]")
        top_k = ids.shape[1]
    if tuple(sums.shape) != (E, K) or tuple(counts.shape) != (E,):
        raise IQError("sums must be [E, K] and counts [E]")
    if x.dtype not in DTYPE:
        raise IQError(f"unsupported dtype {x.dtype}")
    rc = lib().iq_imatrix_collect(_dev(x, "x"), DTYPE[x.dtype], T, K, _dev(ids, "ids", torch.int32), top_k, E,
                                  int(chunk_rows), _dev(sums, "sums", torch.float32),
                                  _dev(counts, "counts", torch.int64), _dev(status, "status", torch.int32),
                                  _stream())
    _check(rc, "iq_imatrix_collect")
    return sums, counts


def hessian_collect(x: torch.Tensor, ids: torch.Tensor | None = None, num_experts: int = 1,
                    chunk_rows: int = 1024, hess: torch.Tensor | None = None,
                    status: torch.Tensor | None = None) -> torch.Tensor:
    """Accumulate each expert's 256-column diagonal blocks of X^T X -> hess [E, K/256, 256, 256] f32."""
    if x.dim() != 2:
        raise IQError("x must be [T, K]")
    T, K = x.shape
    E = int(num_experts)
    if K % 256:
        raise IQError("K must be a multiple of 256")
    if hess is None:
        hess = torch.zeros((E, K // 256, 256, 256), dtype=torch.float32, device=x.device)
    top_k = 0
    if ids is not None:
        if ids.dim() != 2 or ids.shape[0] != T:
            raise IQError("ids must be [T, top_k]")
        top_k = ids.shape[1]
    if tuple(hess.shape) != (E, K // 256, 256, 256):
        raise IQError("hess must be [E, K/256, 256, 256]")
    if x.dtype not in DTYPE:
        raise IQError(f"unsupported dtype {x.dtype}")
    rc = lib().iq_hessian_collect(_dev(x, "x"), DTYPE[x.dtype], T, K, _dev(ids, "ids", torch.int32), top_k, E,
                                  int(chunk_rows), _dev(hess, "hess", torch.float32),
                                  _dev(status, "status", torch.int32), _stream())
    _check(rc, "iq_hessian_collect")
    return hess


def imatrix_merge(src_sums: torch.Tensor, src_counts: torch.Tensor, sums: torch.Tensor, counts: torch.Tensor,
                  status: torch.Tensor | None = None):
    """Add one collection's statistics into another's in place: sums += src_sums,
    counts += src_counts.  Returns (sums, counts)."""
    if src_sums.dim() != 2:
        raise IQError("src_sums must be [E, K]")
    E, K = src_sums.shape
    if tuple(sums.shape) != (E, K) or tuple(src_counts.shape) != (E,) or tuple(counts.shape) != (E,):
        raise IQError("sums must be [E, K] and counts [E], like the source")
    rc = lib().iq_imatrix_merge(_dev(src_sums, "src_sums", torch.float32), _dev(src_counts, "src_counts", torch.int64),
                                E, K, _dev(sums, "sums", torch.float32), _dev(counts, "counts", torch.int64),
                                _dev(status, "status", torch.int32), _stream())
    _check(rc, "iq_imatrix_merge")
    return sums, counts


def imatrix_importance(sums: torch.Tensor, counts: torch.Tensor, floor_rel: float = 1e-6,
                       out: torch.Tensor | None = None, status: torch.Tensor | None = None) -> torch.Tensor:
    """a = sqrt(max(sums/count, floor_rel * mean)) per expert; idle experts get ones."""
    E, K = sums.shape
    if out is None:
        out = torch.empty((E, K), dtype=torch.float32, device=sums.device)
    rc = lib().iq_imatrix_importance(_dev(sums, "sums", torch.float32), _dev(counts, "counts", torch.int64), E, K,
                                     float(floor_rel), _dev(out, "out", torch.float32),
                                     _dev(status, "status", torch.int32), _stream())
    _check(rc, "iq_imatrix_importance")
    return out


def quantize(fmt, w: torch.Tensor, grid: torch.Tensor, importance: torch.Tensor | None = None,
             rows_per_expert: int | None = None, choices: torch.Tensor | None = None,
             out: torch.Tensor | None = None, status: torch.Tensor | None = None,
             check: bool = False) -> torch.Tensor:
    """Encode w [rows, cols] -> uint8 [rows, cols/256, block_bytes]."""
    f = _fmt(fmt)
    if w.dim() != 2:
        raise IQError("w must be [rows, cols]")
    rows, cols = w.shape
    info = format_info(f)
    if tuple(grid.shape) != (info["grid_size"], 8):
        raise IQError(f"grid must be [{info['grid_size']}, 8]")
    rpe = (rows or 1) if rows_per_expert is None else int(rows_per_expert)
    if importance is not None and (rpe < 1 or importance.dim() != 2 or importance.shape[1] != cols
                                   or importance.shape[0] * rpe != rows):
        raise IQError("importance must be [rows / rows_per_expert, cols]")
    if choices is not None:
        want = (rows, cols // 256, info["choice_groups"])
        if tuple(choices.shape) != want or choices.dtype != torch.uint8:
            raise IQError(f"choices must be uint8 {want}")
    if out is None:
        out = torch.empty((rows, cols // 256, info["block_bytes"]), dtype=torch.uint8, device=w.device)
    if w.dtype not in DTYPE:
        raise IQError(f"unsupported dtype {w.dtype}")
    if check and status is None:
        status = new_status(w.device)
    rc = lib().iq_quantize(f, _dev(w, "w"), DTYPE[w.dtype], rows, cols, rpe, _dev(grid, "grid", torch.float32),
                           _dev(importance, "importance", torch.float32), _dev(choices, "choices", torch.uint8),
                           _dev(out, "out", torch.uint8), _dev(status, "status", torch.int32), _stream())
    _check(rc, "iq_quantize")
    if check:
        st = read_status(status)
        if st:
            raise IQError(f"iq_quantize device status {st:#x}")
    return out


def quantize_every_choice(fmt, w: torch.Tensor, grid: torch.Tensor, importance: torch.Tensor | None = None,
                          rows_per_expert: int | None = None, out: torch.Tensor | None = None,
                          status: torch.Tensor | None = None) -> torch.Tensor:
    """Encode w under every choice: uint8 [num_choices, rows, cols/256, block_bytes],
    out[c] == quantize(fmt, w, grid, importance, choices=full(c))."""
    f = _fmt(fmt)
    if w.dim() != 2:
        raise IQError("w must be [rows, cols]")
    rows, cols = w.shape
    info = format_info(f)
    if tuple(grid.shape) != (info["grid_size"], 8):
        raise IQError(f"grid must be [{info['grid_size']}, 8]")
    rpe = (rows or 1) if rows_per_expert is None else int(rows_per_expert)
    if importance is not None and (rpe < 1 or importance.dim() != 2 or importance.shape[1] != cols
                                   or importance.shape[0] * rpe != rows):
        raise IQError("importance must be [rows / rows_per_expert, cols]")
    if out is None:
        out = torch.empty((info["num_choices"], rows, cols // 256, info["block_bytes"]), dtype=torch.uint8,
                          device=w.device)
    if w.dtype not in DTYPE:
        raise IQError(f"unsupported dtype {w.dtype}")
    rc = lib().iq_quantize_every_choice(f, _dev(w, "w"), DTYPE[w.dtype], rows, cols, rpe,
                                        _dev(grid, "grid", torch.float32),
                                        _dev(importance, "importance", torch.float32),
                                        _dev(out, "out", torch.uint8), _dev(status, "status", torch.int32),
                                        _stream())
    _check(rc, "iq_quantize_every_choice")
    return out


def choice_search(fmt, w: torch.Tensor, grid: torch.Tensor, hess: torch.Tensor,
                  importance: torch.Tensor | None = None, rows_per_expert: int | None = None,
                  perc_damp: float = 0.3, out: torch.Tensor | None = None,
                  status: torch.Tensor | None = None, payload: torch.Tensor | bool | None = None):
    """Local-Hessian choice search -> uint8 choices [rows, cols/256, choice_groups];
    hess: [rows / rows_per_expert, cols/256, 256, 256] f32 diagonal Hessian blocks.
    With `payload` (True, or a uint8 [rows, cols/256, block_bytes] tensor to fill)
    the payload under the picks is written as well and (choices, payload) returned."""
    f = _fmt(fmt)
    if w.dim() != 2:
        raise IQError("w must be [rows, cols]")
    rows, cols = w.shape
    info = format_info(f)
    rpe = (rows or 1) if rows_per_expert is None else int(rows_per_expert)
    if tuple(grid.shape) != (info["grid_size"], 8):
        raise IQError(f"grid must be [{info['grid_size']}, 8]")
    if rpe < 1 or rows % rpe or tuple(hess.shape) != (rows // rpe, cols // 256, 256, 256):
        raise IQError("hess must be [rows / rows_per_expert, cols/256, 256, 256]")
    if importance is not None and (importance.dim() != 2 or importance.shape[1] != cols
                                   or importance.shape[0] * rpe != rows):
        raise IQError("importance must be [rows / rows_per_expert, cols]")
    if out is None:
        out = torch.empty((rows, cols // 256, info["choice_groups"]), dtype=torch.uint8, device=w.device)
    if w.dtype not in DTYPE:
        raise IQError(f"unsupported dtype {w.dtype}")
    if payload is True:
        payload = torch.empty((rows, cols // 256, info["block_bytes"]), dtype=torch.uint8, device=w.device)
    elif payload is False:
        payload = None
    if payload is not None and tuple(payload.shape) != (rows, cols // 256, info["block_bytes"]):
        raise IQError(f"payload must be [rows, cols/256, {info['block_bytes']}]")
    rc = lib().iq_choice_search(f, _dev(w, "w"), DTYPE[w.dtype], rows, cols, rpe, _dev(grid, "grid", torch.float32),
                                _dev(importance, "importance", torch.float32), _dev(hess, "hess", torch.float32),
                                float(perc_damp), _dev(out, "out", torch.uint8), _dev(payload, "payload", torch.uint8),
                                _dev(status, "status", torch.int32), _stream())
    _check(rc, "iq_choice_search")
    return out if payload is None else (out, payload)


def time_next_search(start, stop):
    """Profiling hook: the next quantize() on this thread records the two
    torch.cuda.Event objects around its search kernel (events are materialised
    here by a first record)."""
    for e in (start, stop):
        e.record()
    _check(lib().iq_time_next_search(ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event)),
           "iq_time_next_search")


def dequantize(fmt, packed: torch.Tensor, grid: torch.Tensor, dtype=torch.float32,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """Decode uint8 [rows, cols/256, block_bytes] -> [rows, cols]."""
    f = _fmt(fmt)
    rows, nb = packed.shape[0], packed.shape[1]
    cols = nb * 256
    if out is None:
        out = torch.empty((rows, cols), dtype=dtype, device=packed.device)
    rc = lib().iq_dequantize(f, _dev(packed, "packed", torch.uint8), rows, cols, _dev(grid, "grid", torch.float32),
                             _dev(out, "out"), DTYPE[out.dtype], _stream())
    _check(rc, "iq_dequantize")
    return out
