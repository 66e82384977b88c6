"""Thin Python binding of libiq.so (see include/iq.h).

Argument marshalling only: every step runs in the HIP library.  Each wrapper
checks the shape, dtype and device of every tensor it is given (IQError before
any launch), allocates missing outputs and the call's workspace with torch
(the library itself allocates nothing), and enqueues the work on torch's
current stream.  If libiq.so is missing this module raises -- there is no CPU
fallback.
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
          -6: "IQ_ERR_HIP", -7: "IQ_ERR_WORKSPACE"}

# C ABI signatures, by exported name
_P, _I, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "iq_format_info": ([_I, _P], _I),
    "iq_imatrix_collect_workspace_size": ([_I64, _I64, _I, _I, _I, _P], _I),
    "iq_imatrix_collect": ([_P, _I, _I64, _I64, _P, _I, _I, _I, _P, _P, _P, _SZ, _P, _P], _I),
    "iq_hessian_collect_workspace_size": ([_I64, _I64, _I, _I, _I, _P], _I),
    "iq_hessian_collect": ([_P, _I, _I64, _I64, _P, _I, _I, _I, _P, _P, _SZ, _P, _P], _I),
    "iq_imatrix_merge": ([_P, _P, _I, _I64, _P, _P, _P, _P], _I),
    "iq_imatrix_importance": ([_P, _P, _I, _I64, _F, _P, _P, _P], _I),
    "iq_quantize_workspace_size": ([_I, _I64, _I64, _I64, _I, _P], _I),
    "iq_quantize": ([_I, _P, _I, _I64, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P, _P], _I),
    "iq_quantize_noalloc": ([_I, _P, _I, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P], _I),
    "iq_quantize_timed": ([_I, _P, _I, _I64, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P, _P, _P, _P], _I),
    "iq_quantize_every_choice": ([_I, _P, _I, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P, _P], _I),
    "iq_choice_search_workspace_size": ([_I, _I64, _I64, _I64, _I, _P], _I),
    "iq_choice_search": ([_I, _P, _I, _I64, _I64, _I64, _P, _P, _P, _F, _P, _P, _P, _SZ, _P, _P], _I),
    "iq_dequantize": ([_I, _P, _I64, _I64, _P, _P, _I, _P], _I),
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
    if int(fmt) not in range(len(FORMATS)):
        raise IQError(f"unknown format {fmt!r}")
    return int(fmt)


# --------------------------------------------------------------------------
# Argument checks: shape and dtype first (no device needed), then placement.
# --------------------------------------------------------------------------
def _need(t, name: str, shape=None, dtype=None):
    """t must be a tensor of `shape` (a tuple, None entries free) and dtype."""
    if not isinstance(t, torch.Tensor):
        raise IQError(f"{name} must be a tensor")
    if shape is not None and (t.dim() != len(shape) or
                              any(s is not None and int(d) != int(s) for d, s in zip(t.shape, shape))):
        want = "[" + ", ".join("*" if s is None else str(s) for s in shape) + "]"
        raise IQError(f"{name} has shape {list(t.shape)}, expected {want}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise IQError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t


def _ptr(t, name: str, device):
    """Device pointer of t, which must be a contiguous tensor on `device`."""
    if t is None:
        return None
    if not t.is_cuda:
        raise IQError(f"{name} must be a device tensor")
    if t.device != device:
        raise IQError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise IQError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _device_of(t: torch.Tensor):
    """The device of the call's main tensor; it must be the current device,
    since the library launches on the current device."""
    if not t.is_cuda:
        raise IQError("tensors must be device tensors")
    if t.device.index != torch.cuda.current_device():
        raise IQError(f"tensors are on {t.device} but the current device is cuda:{torch.cuda.current_device()}")
    return t.device


def _status_ok(status):
    if status is not None:
        _need(status, "status", (None,), torch.int32)
        if status.numel() < 1:
            raise IQError("status must hold at least one int32")


def _workspace(nbytes: int, device, workspace):
    """The caller's workspace (a uint8 device tensor of at least nbytes) or a
    new one from torch's allocator; returns (tensor, pointer, size)."""
    if nbytes == 0:
        return None, None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _need(workspace, "workspace", None, torch.uint8)
    if workspace.numel() < nbytes:
        raise IQError(f"workspace holds {workspace.numel()} bytes, the call needs {nbytes}")
    return workspace, _ptr(workspace, "workspace", device), workspace.numel()


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


def _size_query(fn, *args) -> int:
    out = ctypes.c_size_t(0)
    _check(getattr(lib(), fn)(*args, ctypes.byref(out)), fn)
    return int(out.value)


# --------------------------------------------------------------------------
# Workspace queries
# --------------------------------------------------------------------------
def collect_workspace_size(T: int, K: int, top_k: int = 0, num_experts: int = 1, chunk_rows: int = 1024) -> int:
    return _size_query("iq_imatrix_collect_workspace_size", int(T), int(K), int(top_k), int(num_experts),
                       int(chunk_rows))


def hessian_workspace_size(T: int, K: int, top_k: int = 0, num_experts: int = 1, chunk_rows: int = 1024) -> int:
    return _size_query("iq_hessian_collect_workspace_size", int(T), int(K), int(top_k), int(num_experts),
                       int(chunk_rows))


def quantize_workspace_size(fmt, rows: int, cols: int, rows_per_expert: int | None = None,
                            weighted: bool = True) -> int:
    rpe = (rows or 1) if rows_per_expert is None else int(rows_per_expert)
    return _size_query("iq_quantize_workspace_size", _fmt(fmt), int(rows), int(cols), rpe, int(bool(weighted)))


def choice_search_workspace_size(fmt, rows: int, cols: int, rows_per_expert: int | None = None,
                                 weighted: bool = True) -> int:
    rpe = (rows or 1) if rows_per_expert is None else int(rows_per_expert)
    return _size_query("iq_choice_search_workspace_size", _fmt(fmt), int(rows), int(cols), rpe,
                       int(bool(weighted)))


# --------------------------------------------------------------------------
# Collection
# --------------------------------------------------------------------------
def _collect_args(x, ids):
    _need(x, "x", (None, None), tuple(DTYPE))
    T, K = x.shape
    top_k = 0
    if ids is not None:
        _need(ids, "ids", (T, None), torch.int32)
        top_k = ids.shape[1]
    return T, K, top_k


def imatrix_collect(x: torch.Tensor, ids: torch.Tensor | None = None, num_experts: int = 1,
                    chunk_rows: int = 1024, sums: torch.Tensor | None = None,
                    counts: torch.Tensor | None = None, status: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None):
    """Accumulate per-expert sum of x^2 and token counts. Returns (sums [E,K] f32, counts [E] i64)."""
    T, K, top_k = _collect_args(x, ids)
    E = int(num_experts)
    if sums is not None:
        _need(sums, "sums", (E, K), torch.float32)
    if counts is not None:
        _need(counts, "counts", (E,), torch.int64)
    _status_ok(status)
    dev = _device_of(x)
    if sums is None:
        sums = torch.zeros((E, K), dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.zeros((E,), dtype=torch.int64, device=dev)
    ws, wp, wn = _workspace(collect_workspace_size(T, K, top_k if ids is not None else 0, E, chunk_rows), dev,
                            workspace)
    rc = lib().iq_imatrix_collect(_ptr(x, "x", dev), DTYPE[x.dtype], T, K, _ptr(ids, "ids", dev), top_k, E,
                                  int(chunk_rows), _ptr(sums, "sums", dev), _ptr(counts, "counts", dev), wp, wn,
                                  _ptr(status, "status", dev), _stream())
    _check(rc, "iq_imatrix_collect")
    return sums, counts


def hessian_collect(x: torch.Tensor, ids: torch.Tensor | None = None, num_experts: int = 1,
                    chunk_rows: int = 1024, hess: torch.Tensor | None = None,
                    status: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Accumulate each expert's 256-column diagonal blocks of X^T X -> hess [E, K/256, 256, 256] f32."""
    T, K, top_k = _collect_args(x, ids)
    E = int(num_experts)
    if K % 256:
        raise IQError("K must be a multiple of 256")
    if hess is not None:
        _need(hess, "hess", (E, K // 256, 256, 256), torch.float32)
    _status_ok(status)
    dev = _device_of(x)
    if hess is None:
        hess = torch.zeros((E, K // 256, 256, 256), dtype=torch.float32, device=dev)
    ws, wp, wn = _workspace(hessian_workspace_size(T, K, top_k if ids is not None else 0, E, chunk_rows), dev,
                            workspace)
    rc = lib().iq_hessian_collect(_ptr(x, "x", dev), DTYPE[x.dtype], T, K, _ptr(ids, "ids", dev), top_k, E,
                                  int(chunk_rows), _ptr(hess, "hess", dev), wp, wn, _ptr(status, "status", dev),
                                  _stream())
    _check(rc, "iq_hessian_collect")
    return hess


def imatrix_merge(src_sums: torch.Tensor, src_counts: torch.Tensor, sums: torch.Tensor, counts: torch.Tensor,
                  status: torch.Tensor | None = None):
    """Add one collection's statistics into another's in place: sums += src_sums,
    counts += src_counts.  Returns (sums, counts)."""
    _need(src_sums, "src_sums", (None, None), torch.float32)
    E, K = src_sums.shape
    _need(src_counts, "src_counts", (E,), torch.int64)
    _need(sums, "sums", (E, K), torch.float32)
    _need(counts, "counts", (E,), torch.int64)
    _status_ok(status)
    dev = _device_of(sums)
    rc = lib().iq_imatrix_merge(_ptr(src_sums, "src_sums", dev), _ptr(src_counts, "src_counts", dev), E, K,
                                _ptr(sums, "sums", dev), _ptr(counts, "counts", dev), _ptr(status, "status", dev),
                                _stream())
    _check(rc, "iq_imatrix_merge")
    return sums, counts


def imatrix_importance(sums: torch.Tensor, counts: torch.Tensor, floor_rel: float = 1e-6,
                       out: torch.Tensor | None = None, status: torch.Tensor | None = None) -> torch.Tensor:
    """a = sqrt(max(sums/count, floor_rel * mean)) per expert; idle experts get ones."""
    _need(sums, "sums", (None, None), torch.float32)
    E, K = sums.shape
    _need(counts, "counts", (E,), torch.int64)
    if out is not None:
        _need(out, "out", (E, K), torch.float32)
    _status_ok(status)
    dev = _device_of(sums)
    if out is None:
        out = torch.empty((E, K), dtype=torch.float32, device=dev)
    rc = lib().iq_imatrix_importance(_ptr(sums, "sums", dev), _ptr(counts, "counts", dev), E, K, float(floor_rel),
                                     _ptr(out, "out", dev), _ptr(status, "status", dev), _stream())
    _check(rc, "iq_imatrix_importance")
    return out


# --------------------------------------------------------------------------
# Encode / decode
# --------------------------------------------------------------------------
def _encode_args(fmt, w, grid, importance, rows_per_expert):
    f = _fmt(fmt)
    _need(w, "w", (None, None), tuple(DTYPE))
    rows, cols = w.shape
    if cols % 256:
        raise IQError(f"w has {cols} columns, not a multiple of 256")
    info = format_info(f)
    _need(grid, "grid", (info["grid_size"], 8), torch.float32)
    rpe = (rows or 1) if rows_per_expert is None else int(rows_per_expert)
    if rpe < 1 or rows % rpe:
        raise IQError(f"rows_per_expert {rpe} does not divide rows {rows}")
    if importance is not None:
        _need(importance, "importance", (rows // rpe, cols), torch.float32)
    return f, rows, cols, rpe, info


def quantize(fmt, w: torch.Tensor, grid: torch.Tensor, importance: torch.Tensor | None = None,
             rows_per_expert: int | None = None, choices: torch.Tensor | None = None,
             out: torch.Tensor | None = None, status: torch.Tensor | None = None,
             check: bool = False, workspace: torch.Tensor | None = None, events=None) -> torch.Tensor:
    """Encode w [rows, cols] -> uint8 [rows, cols/256, block_bytes].
    events: optional (start, stop) torch.cuda.Event pair recorded around the
    search kernel alone (iq_quantize_timed)."""
    f, rows, cols, rpe, info = _encode_args(fmt, w, grid, importance, rows_per_expert)
    nb = cols // 256
    if choices is not None:
        _need(choices, "choices", (rows, nb, info["choice_groups"]), torch.uint8)
    if out is not None:
        _need(out, "out", (rows, nb, info["block_bytes"]), torch.uint8)
    _status_ok(status)
    dev = _device_of(w)
    if out is None:
        out = torch.empty((rows, nb, info["block_bytes"]), dtype=torch.uint8, device=dev)
    if check and status is None:
        status = new_status(dev)
    ws, wp, wn = _workspace(quantize_workspace_size(f, rows, cols, rpe, importance is not None), dev, workspace)
    args = (f, _ptr(w, "w", dev), DTYPE[w.dtype], rows, cols, rpe, _ptr(grid, "grid", dev),
            _ptr(importance, "importance", dev), _ptr(choices, "choices", dev), _ptr(out, "out", dev), wp, wn,
            _ptr(status, "status", dev))
    if events is None:
        rc = lib().iq_quantize(*args, _stream())
        _check(rc, "iq_quantize")
    else:
        start, stop = events
        for e in (start, stop):
            e.record()  # materialises the event on the current device
        rc = lib().iq_quantize_timed(*args, ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event),
                                     _stream())
        _check(rc, "iq_quantize_timed")
    if check:
        st = read_status(status)
        if st:
            raise IQError(f"iq_quantize device status {st:#x}")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # IQ_NOALLOC_SCRATCH_BYTES


def quantize_noalloc(fmt, w: torch.Tensor, grid: torch.Tensor, importance: torch.Tensor | None = None,
                     rows_per_expert: int | None = None, choices: torch.Tensor | None = None,
                     out: torch.Tensor | None = None, status: torch.Tensor | None = None) -> torch.Tensor:
    """quantize() through iq_quantize_noalloc: the library works in its static
    device scratch, so apart from `out` when it is not given nothing is
    allocated.  Calls that overlap on one GPU race (they share the scratch)."""
    f, rows, cols, rpe, info = _encode_args(fmt, w, grid, importance, rows_per_expert)
    nb = cols // 256
    if choices is not None:
        _need(choices, "choices", (rows, nb, info["choice_groups"]), torch.uint8)
    if out is not None:
        _need(out, "out", (rows, nb, info["block_bytes"]), torch.uint8)
    _status_ok(status)
    dev = _device_of(w)
    if out is None:
        out = torch.empty((rows, nb, info["block_bytes"]), dtype=torch.uint8, device=dev)
    rc = lib().iq_quantize_noalloc(f, _ptr(w, "w", dev), DTYPE[w.dtype], rows, cols, rpe, _ptr(grid, "grid", dev),
                                   _ptr(importance, "importance", dev), _ptr(choices, "choices", dev),
                                   _ptr(out, "out", dev), _ptr(status, "status", dev), _stream())
    _check(rc, "iq_quantize_noalloc")
    return out


def quantize_every_choice(fmt, w: torch.Tensor, grid: torch.Tensor, importance: torch.Tensor | None = None,
                          rows_per_expert: int | None = None, out: torch.Tensor | None = None,
                          status: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Encode w under every choice: uint8 [num_choices, rows, cols/256, block_bytes],
    out[c] == quantize(fmt, w, grid, importance, choices=full(c))."""
    f, rows, cols, rpe, info = _encode_args(fmt, w, grid, importance, rows_per_expert)
    shape = (info["num_choices"], rows, cols // 256, info["block_bytes"])
    if out is not None:
        _need(out, "out", shape, torch.uint8)
    _status_ok(status)
    dev = _device_of(w)
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=dev)
    ws, wp, wn = _workspace(quantize_workspace_size(f, rows, cols, rpe, importance is not None), dev, workspace)
    rc = lib().iq_quantize_every_choice(f, _ptr(w, "w", dev), DTYPE[w.dtype], rows, cols, rpe,
                                        _ptr(grid, "grid", dev), _ptr(importance, "importance", dev),
                                        _ptr(out, "out", dev), wp, wn, _ptr(status, "status", dev), _stream())
    _check(rc, "iq_quantize_every_choice")
    return out


def choice_search(fmt, w: torch.Tensor, grid: torch.Tensor, hess: torch.Tensor,
                  importance: torch.Tensor | None = None, rows_per_expert: int | None = None,
                  perc_damp: float = 0.3, out: torch.Tensor | None = None,
                  status: torch.Tensor | None = None, payload: torch.Tensor | bool | None = None,
                  workspace: torch.Tensor | None = None):
    """Local-Hessian choice search -> uint8 choices [rows, cols/256, choice_groups];
    hess: [rows / rows_per_expert, cols/256, 256, 256] f32 diagonal Hessian blocks.
    With `payload` (True, or a uint8 [rows, cols/256, block_bytes] tensor to fill)
    the payload under the picks is written as well and (choices, payload) returned."""
    f, rows, cols, rpe, info = _encode_args(fmt, w, grid, importance, rows_per_expert)
    nb = cols // 256
    _need(hess, "hess", (rows // rpe, nb, 256, 256), torch.float32)
    if out is not None:
        _need(out, "out", (rows, nb, info["choice_groups"]), torch.uint8)
    if isinstance(payload, torch.Tensor):
        _need(payload, "payload", (rows, nb, info["block_bytes"]), torch.uint8)
    _status_ok(status)
    dev = _device_of(w)
    if out is None:
        out = torch.empty((rows, nb, info["choice_groups"]), dtype=torch.uint8, device=dev)
    if payload is True:
        payload = torch.empty((rows, nb, info["block_bytes"]), dtype=torch.uint8, device=dev)
    elif payload is False:
        payload = None
    ws, wp, wn = _workspace(choice_search_workspace_size(f, rows, cols, rpe, importance is not None), dev,
                            workspace)
    rc = lib().iq_choice_search(f, _ptr(w, "w", dev), DTYPE[w.dtype], rows, cols, rpe, _ptr(grid, "grid", dev),
                                _ptr(importance, "importance", dev), _ptr(hess, "hess", dev), float(perc_damp),
                                _ptr(out, "out", dev), _ptr(payload, "payload", dev), wp, wn,
                                _ptr(status, "status", dev), _stream())
    _check(rc, "iq_choice_search")
    return out if payload is None else (out, payload)


def dequantize(fmt, packed: torch.Tensor, grid: torch.Tensor, dtype=torch.float32,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """Decode uint8 [rows, cols/256, block_bytes] -> [rows, cols]."""
    f = _fmt(fmt)
    info = format_info(f)
    _need(packed, "packed", (None, None, info["block_bytes"]), torch.uint8)
    _need(grid, "grid", (info["grid_size"], 8), torch.float32)
    rows, nb = packed.shape[0], packed.shape[1]
    cols = nb * 256
    if out is not None:
        _need(out, "out", (rows, cols), tuple(DTYPE))
    elif dtype not in DTYPE:
        raise IQError(f"unsupported output dtype {dtype}")
    dev = _device_of(packed)
    if out is None:
        out = torch.empty((rows, cols), dtype=dtype, device=dev)
    rc = lib().iq_dequantize(f, _ptr(packed, "packed", dev), rows, cols, _ptr(grid, "grid", dev),
                             _ptr(out, "out", dev), DTYPE[out.dtype], _stream())
    _check(rc, "iq_dequantize")
    return out
