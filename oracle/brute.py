"""Exhaustive fp64 search over one block, for pinning the oracle on small inputs.

TEST INFRASTRUCTURE ONLY.  For every choice, every grid entry and every
admissible sign pattern (IQ2) or shift (IQ1), it evaluates the weighted squared
error sum_j a_j (x_j - x^_j)^2 directly, in fp64, from the values the decoder
would produce (fp32 s * g, as in the pages' dequantize_row semantics), and
keeps the first minimum in a fixed candidate order.  It shares nothing with
the oracle's reduced-form search in iq_oracle.c: no expansion into P and G
terms, no parity shortcut, no first-min scans over fp32 values.

Candidate order (the tie rules the pages state or that the oracle reads into
them): choice ascending ("lowest choice"); within a group, IQ1_M shift before
entry ("a tie still prefers the lower shift and then the lower entry", ModelOpt
PR #2513 IQ1_M body and the modelopt_recipes IQ1_M encoder commit); entry
ascending; IQ2 sign patterns by the number of elements whose sign differs from
the input, then by the lowest differing element.
"""
from __future__ import annotations

import numpy as np

IQ2_NCHOICE = 16
GEO = {  # groups per unit, units per block, choices per unit
    "IQ2_XXS": (4, 8, 16), "IQ2_XS": (2, 16, 16), "IQ2_S": (2, 16, 16),
    "IQ1_S": (4, 8, 16), "IQ1_M": (2, 16, 8),
}


def _f16_to_f32(h: int) -> float:
    return float(np.array([h], dtype=np.uint16).view(np.float16)[0])


def _masks(fmt: str, neg: int):
    """Admissible sign masks (bit j = element j negative) in candidate order."""
    if fmt == "IQ2_S":
        cands = range(256)
    else:  # 7-bit sign index + parity bit: even popcount only
        cands = [m for m in range(256) if bin(m).count("1") % 2 == 0]

    def key(m):
        diff = m ^ neg
        pos = tuple(j for j in range(8) if (diff >> j) & 1)
        return (len(pos), pos)

    return sorted(cands, key=key)


def _iq2_scale(d: float, c: int) -> np.float32:
    return np.float32(np.float32(d) * np.float32((2 * c + 1) / 8.0))


def _iq1_scale(d: float, ls: int) -> np.float32:
    return np.float32(np.float32(d) * np.float32(2 * ls + 1))


def group_table(fmt: str, x8, a8, grid, d: float):
    """Errors of every candidate for one group.

    IQ2: err[c, k, m_idx] with masks in candidate order (list returned).
    IQ1: err[h, ls, k]."""
    x8 = np.asarray(x8, dtype=np.float64)
    a8 = np.asarray(a8, dtype=np.float64)
    g = np.asarray(grid, dtype=np.float32)
    if fmt.startswith("IQ2"):
        neg = sum(1 << j for j in range(8) if x8[j] < 0)
        masks = _masks(fmt, neg)
        sgn = np.array([[-1.0 if (m >> j) & 1 else 1.0 for j in range(8)] for m in masks])  # [M, 8]
        errs = np.empty((IQ2_NCHOICE, g.shape[0], len(masks)))
        for c in range(IQ2_NCHOICE):
            s = _iq2_scale(d, c)
            v = (s * g).astype(np.float32).astype(np.float64)                 # [N, 8] decoded magnitudes
            w_hat = v[:, None, :] * sgn[None, :, :]                            # [N, M, 8]
            errs[c] = (a8 * (x8 - w_hat) ** 2).sum(axis=-1)
        return errs, masks
    errs = np.empty((2, 8, g.shape[0]))
    for h, delta in enumerate((0.125, -0.125)):
        u = (g + np.float32(delta)).astype(np.float32)
        for ls in range(8):
            s = _iq1_scale(d, ls)
            w_hat = (s * u).astype(np.float32).astype(np.float64)
            errs[h, ls] = (a8 * (x8 - w_hat) ** 2).sum(axis=-1)
    return errs, None


def _first_min(vals):
    """index of the first minimum of a 1-d sequence."""
    vals = np.asarray(vals)
    return int(np.flatnonzero(vals == vals.min())[0])


def _n_min(vals):
    vals = np.asarray(vals)
    return int((vals == vals.min()).sum())


def search_block(fmt: str, x, a, grid, d16: int, choices=None):
    """Exhaustive search of one 256-value block at scale fp16 d16.

    Returns dict(choice [units], k [32], mask [32], h [32], unit_err [units, NC],
    group_best [32, NC] (per-choice best error of the group), err (total)).
    """
    gpu, units, nc = GEO[fmt]
    d = _f16_to_f32(d16)
    x = np.asarray(x, dtype=np.float32)
    a = np.asarray(a, dtype=np.float32)
    # per group: best candidate and error for every unit choice
    gbest = np.empty((32, nc))
    gpick = [[None] * nc for _ in range(32)]
    ties = 0  # (group, choice) pairs whose minimum is attained by more than one candidate
    for gi in range(32):
        errs, masks = group_table(fmt, x[8 * gi:8 * gi + 8], a[8 * gi:8 * gi + 8], grid, d)
        for c in range(nc):
            if fmt.startswith("IQ2"):
                e = errs[c]                                   # [N, M]
                flat = e.reshape(-1)                          # order: k, then mask order
                i = _first_min(flat)
                ties += _n_min(flat) > 1
                k, mi = divmod(i, e.shape[1])
                gbest[gi, c] = flat[i]
                gpick[gi][c] = (k, masks[mi], 0)
            elif fmt == "IQ1_S":
                h, ls = c >> 3, c & 7
                e = errs[h, ls]
                k = _first_min(e)
                ties += _n_min(e) > 1
                gbest[gi, c] = e[k]
                gpick[gi][c] = (k, 0, h)
            else:  # IQ1_M: per group shift then entry
                e = errs[:, c, :].reshape(-1)                 # order: h, then k
                i = _first_min(e)
                ties += _n_min(e) > 1
                h, k = divmod(i, errs.shape[2])
                gbest[gi, c] = e[i]
                gpick[gi][c] = (k, 0, h)
    unit_err = np.empty((units, nc))
    out = dict(choice=np.zeros(units, dtype=np.int64), k=np.zeros(32, dtype=np.int64),
               mask=np.zeros(32, dtype=np.int64), h=np.zeros(32, dtype=np.int64))
    total = 0.0
    for u in range(units):
        gs = range(u * gpu, (u + 1) * gpu)
        unit_err[u] = [sum(gbest[g, c] for g in gs) for c in range(nc)]
        c = int(choices[u]) if choices is not None else _first_min(unit_err[u])
        out["choice"][u] = c
        total += unit_err[u, c]
        for g in gs:
            k, m, h = gpick[g][c]
            out["k"][g], out["mask"][g], out["h"][g] = k, m, h
    out["unit_err"] = unit_err
    out["group_best"] = gbest
    out["err"] = total
    out["group_ties"] = ties
    out["choice_ties"] = int(sum(_n_min(unit_err[u]) > 1 for u in range(units)))
    return out


def decoded_error(x, a, w_hat) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float((np.asarray(a, dtype=np.float64) * (x - np.asarray(w_hat, dtype=np.float64)) ** 2).sum())


__all__ = ["search_block", "group_table", "decoded_error", "GEO"]
