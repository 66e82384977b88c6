"""CPU oracle for importance-weighted GGML IQ encoding and imatrix collection.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package; the product path never
does.  The arithmetic lives in ``iq_oracle.c`` (plain scalar C, fp32 with
explicit fmaf and contraction off, fp64 for collection) and ``brute.py``
(fp64 exhaustive search on tiny inputs).  It shares no code with the HIP
library; only the seeded input generators are common to both.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "iq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FORMATS = ("IQ2_XXS", "IQ2_XS", "IQ2_S", "IQ1_S", "IQ1_M")
FMT = {n: i for i, n in enumerate(FORMATS)}

ST_NONFINITE, ST_OVERFLOW, ST_BADCHOICE, ST_BADIMP, ST_BADID = 1, 2, 4, 8, 16

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (contraction off, no fast math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-pthread", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        L.orc_geometry.argtypes = [ci, P]
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_collect.argtypes = [P, i64, i64, P, ci, ci, P, P]
        L.orc_importance.argtypes = [P, P, ci, i64, ctypes.c_float, P]
        L.orc_merge.argtypes = [P, P, ci, i64, P, P]
        L.orc_hessian_collect.argtypes = [P, i64, i64, P, ci, ci, P]
        L.orc_mean.argtypes = [P, i64]
        L.orc_mean.restype = ctypes.c_float
        L.orc_anchor.argtypes = [ci, P, P]
        L.orc_anchor.restype = ctypes.c_uint16
        L.orc_encode_block.argtypes = [ci, P, P, P, ci, P, ci, P]
        L.orc_group_minima.argtypes = [ci, P, P, P, ci, ctypes.c_uint16, P, P]
        L.orc_quantize.argtypes = [ci, P, i64, i64, i64, P, i64, P, P, P, P, ci]
        L.orc_dequantize.argtypes = [ci, P, i64, i64, P, P]
        L.orc_choice_search.argtypes = [ci, P, i64, i64, i64, P, i64, P, P, P, ctypes.c_float, P, ci]
        L.orc_damping.argtypes = [P, ctypes.c_float]
        L.orc_damping.restype = ctypes.c_float
        L.orc_pack_flat.argtypes = [ci, P, P]
        L.orc_unpack_flat.argtypes = [ci, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def fmt_id(fmt) -> int:
    return FMT[fmt] if isinstance(fmt, str) else int(fmt)


def geometry(fmt) -> dict:
    out = np.zeros(5, dtype=np.int32)
    if lib().orc_geometry(fmt_id(fmt), _p(out)) != 0:
        raise ValueError(fmt)
    return dict(block_bytes=int(out[0]), grid_n=int(out[1]), groups_per_unit=int(out[2]),
                units=int(out[3]), num_choices=int(out[4]))


def f32_to_f16_bits(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib().orc_f32_to_f16(float(v)) for v in x], dtype=np.uint16)


def f16_bits_to_f32(h) -> np.ndarray:
    h = np.asarray(h, dtype=np.uint16).ravel()
    return np.array([lib().orc_f16_to_f32(int(v)) for v in h], dtype=np.float32)


def collect(x, ids=None, num_experts: int = 1, sums=None, counts=None):
    """fp64 per-expert sum of squares and counts. Returns (sums [E,K] f64, counts [E] i64, status)."""
    x = _f32(x)
    T, K = x.shape
    E = 1 if ids is None else int(num_experts)
    sums = np.zeros((E, K), dtype=np.float64) if sums is None else sums
    counts = np.zeros(E, dtype=np.int64) if counts is None else counts
    top_k = 0
    if ids is not None:
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        top_k = ids.shape[1]
    st = lib().orc_collect(_p(x), T, K, _p(ids), top_k, E, _p(sums), _p(counts))
    return sums, counts, st


def hessian_collect(x, ids=None, num_experts: int = 1, hess=None):
    """fp64 [E, K/256, 256, 256] diagonal blocks of each expert's X^T X (accumulated)."""
    x = _f32(x)
    T, K = x.shape
    E = 1 if ids is None else int(num_experts)
    hess = np.zeros((E, K // 256, 256, 256), dtype=np.float64) if hess is None else hess
    top_k = 0
    if ids is not None:
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        top_k = ids.shape[1]
    st = lib().orc_hessian_collect(_p(x), T, K, _p(ids), top_k, E, _p(hess))
    return hess, st


def merge(src_sums, src_counts, sums, counts):
    """Add one collection's statistics into another's (fp32 sums, int64 counts);
    returns (sums, counts, status)."""
    src = _f32(src_sums)
    sc = np.ascontiguousarray(src_counts, dtype=np.int64)
    out_s = np.array(sums, dtype=np.float32, copy=True)
    out_c = np.array(counts, dtype=np.int64, copy=True)
    E, K = src.shape
    assert out_s.shape == (E, K) and sc.shape == out_c.shape == (E,)
    st = lib().orc_merge(_p(src), _p(sc), E, K, _p(out_s), _p(out_c))
    return out_s, out_c, st


def importance(sums32, counts, floor_rel: float = 1e-6):
    s = _f32(sums32)
    E, K = s.shape
    c = np.ascontiguousarray(counts, dtype=np.int64)
    out = np.empty((E, K), dtype=np.float32)
    st = lib().orc_importance(_p(s), _p(c), E, K, float(floor_rel), _p(out))
    return out, st


def mean(m):
    """The floor's mean of the m_j (fp32 result)."""
    m = _f32(m).ravel()
    return float(lib().orc_mean(_p(m), m.size))


def anchor(fmt, block):
    b = _f32(block).ravel()
    assert b.size == 256
    st = ctypes.c_int(0)
    h = lib().orc_anchor(fmt_id(fmt), _p(b), ctypes.byref(st))
    return int(h), st.value


def encode_block(fmt, x, a, grid, choices=None, d16=None):
    f = fmt_id(fmt)
    geo = geometry(f)
    x, a, g = _f32(x).ravel(), _f32(a).ravel(), _f32(grid)
    ch = None if choices is None else np.ascontiguousarray(choices, dtype=np.uint8).ravel()
    out = np.zeros(geo["block_bytes"], dtype=np.uint8)
    st = lib().orc_encode_block(f, _p(x), _p(a), _p(g), g.shape[0], _p(ch),
                                -1 if d16 is None else int(d16), _p(out))
    return out, st


def group_minima(fmt, x, a, grid, d16):
    """Per group and slot (IQ2: choice c; IQ1: h*8+ls): first-min reduced error and entry."""
    x, a, g = _f32(x).ravel(), _f32(a).ravel(), _f32(grid)
    best = np.zeros((32, 16), dtype=np.float32)
    bestk = np.zeros((32, 16), dtype=np.int32)
    lib().orc_group_minima(fmt_id(fmt), _p(x), _p(a), _p(g), g.shape[0], int(d16), _p(best), _p(bestk))
    return best, bestk


def quantize(fmt, w, grid, importance=None, rows_per_expert=None, choices=None, row_ids=None,
             threads: int | None = None):
    """Encode w [rows, cols]. Returns (payload uint8 [n_rows, cols/256, block_bytes], status).

    importance: [E, cols] (row r uses expert r // rows_per_expert) or None (flat).
    row_ids: encode only these rows (the payload then holds them in that order)."""
    f = fmt_id(fmt)
    geo = geometry(f)
    w = _f32(w)
    rows, cols = w.shape
    rpe = rows if rows_per_expert is None else int(rows_per_expert)
    imp = None if importance is None else _f32(importance)
    ch = None if choices is None else np.ascontiguousarray(choices, dtype=np.uint8)
    rid = None if row_ids is None else np.ascontiguousarray(row_ids, dtype=np.int64)
    n = rows if rid is None else rid.size
    out = np.zeros((n, cols // 256, geo["block_bytes"]), dtype=np.uint8)
    threads = threads or os.cpu_count() or 1
    st = lib().orc_quantize(f, _p(w), rows, cols, rpe, _p(rid), n, _p(_f32(grid)), _p(imp), _p(ch),
                            _p(out), int(threads))
    if st < 0:
        raise ValueError("oracle rejected the shapes")
    return out, st


def quantize_every_choice(fmt, w, grid, importance=None, rows_per_expert=None, row_ids=None,
                          threads: int | None = None):
    """[num_choices, n_rows, cols/256, block_bytes]: for each choice c, the encode with
    every unit fixed to c (ModelOpt PR #3159 description: the PyTorch encoders loop over
    forced choices; packed[c] == quantize(choices=full(c)))."""
    geo = geometry(fmt)
    rows, cols = np.asarray(w).shape
    outs, st = [], 0
    for c in range(geo["num_choices"]):
        ch = np.full((rows, cols // 256, geo["units"]), c, np.uint8)
        p, s = quantize(fmt, w, grid, importance, rows_per_expert, choices=ch, row_ids=row_ids, threads=threads)
        outs.append(p)
        st |= s
    return np.stack(outs), st


def choice_search(fmt, w, grid, hess, importance=None, rows_per_expert=None, perc_damp: float = 0.3,
                  row_ids=None, threads: int | None = None):
    """Local-Hessian choice search (ModelOpt PR #3158). hess: [E, cols/256, 256, 256]
    diagonal blocks of each expert's input Hessian.  Returns uint8 choices
    [n_rows, cols/256, units] to feed quantize(choices=...)."""
    f = fmt_id(fmt)
    geo = geometry(f)
    w = _f32(w)
    rows, cols = w.shape
    rpe = rows if rows_per_expert is None else int(rows_per_expert)
    imp = None if importance is None else _f32(importance)
    h = _f32(hess)
    assert h.shape == (rows // rpe, cols // 256, 256, 256)
    rid = None if row_ids is None else np.ascontiguousarray(row_ids, dtype=np.int64)
    n = rows if rid is None else rid.size
    out = np.zeros((n, cols // 256, geo["units"]), dtype=np.uint8)
    threads = threads or os.cpu_count() or 1
    st = lib().orc_choice_search(f, _p(w), rows, cols, rpe, _p(rid), n, _p(_f32(grid)), _p(imp), _p(h),
                                 float(perc_damp), _p(out), int(threads))
    if st < 0:
        raise ValueError("oracle rejected the shapes")
    return out, st


def damping(H, perc_damp: float = 0.3) -> float:
    return float(lib().orc_damping(_p(_f32(H)), float(perc_damp)))


def dequantize(fmt, packed, rows, cols, grid):
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    y = np.empty((rows, cols), dtype=np.float32)
    if lib().orc_dequantize(fmt_id(fmt), _p(p), rows, cols, _p(_f32(grid)), _p(y)) != 0:
        raise ValueError("bad shape")
    return y


def pack_fields(fmt, fields: dict) -> np.ndarray:
    """fields: d (int), k [32], mask [32], h [32], ls [16] -> block bytes."""
    v = np.zeros(113, dtype=np.int32)
    v[0] = fields.get("d", 0)
    v[1:33] = fields.get("k", np.zeros(32))
    v[33:65] = fields.get("mask", np.zeros(32))
    v[65:97] = fields.get("h", np.zeros(32))
    v[97:113] = fields.get("ls", np.zeros(16))
    out = np.zeros(geometry(fmt)["block_bytes"], dtype=np.uint8)
    lib().orc_pack_flat(fmt_id(fmt), _p(v), _p(out))
    return out


def unpack_fields(fmt, block) -> dict:
    b = np.ascontiguousarray(block, dtype=np.uint8)
    v = np.zeros(113, dtype=np.int32)
    lib().orc_unpack_flat(fmt_id(fmt), _p(b), _p(v))
    return dict(d=int(v[0]), k=v[1:33].copy(), mask=v[33:65].copy(), h=v[65:97].copy(), ls=v[97:113].copy())


def weighted_mse(w, w_hat, a_rows):
    """sum a (w - w_hat)^2 / sum a w^2 in fp64 (a broadcast per row)."""
    w = np.asarray(w, dtype=np.float64)
    d = w - np.asarray(w_hat, dtype=np.float64)
    a = np.asarray(a_rows, dtype=np.float64)
    return float((a * d * d).sum() / (a * w * w).sum())
