"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module only draws data.  It holds none of the encoder's or the
collector's arithmetic, so both sides can take their inputs from it without
sharing any of the method.  Every array comes from numpy's PCG64 with an
explicit seed, so a (seed, shape) pair names the data exactly.

The workloads stand in for the pages' real weights and calibration activations
(a 5632x2048 weight measured on ModelOpt PR #2513's commit messages; the
4,096-token, 1,024-row-chunk collection of PR #2735's description): weights
~ N(0, 0.02^2) with optional 1 % outliers at 8 sigma, activations whose column
scales sigma_j are lognormal(0, 1), top-k routing drawn from a Zipf(1.1)
popularity law with a fixed set of experts that no token reaches.
"""
from __future__ import annotations

import numpy as np

# Codebook alphabets: IQ2 grids hold magnitudes, IQ1 grids signed values.
IQ2_ALPHABET = (1.0, 3.0, 5.0)
IQ1_ALPHABET = (-1.0, 0.0, 1.0)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# ----------------------------------------------------------------------------
# bfloat16 storage helpers (data preparation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array holding exactly the bfloat16-representable values of x."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ----------------------------------------------------------------------------
# Codebooks
# ----------------------------------------------------------------------------
def grid(n: int, alphabet, seed: int) -> np.ndarray:
    """n distinct 8-tuples over a 3-letter alphabet, float32 [n, 8].

    Codes are drawn without replacement from the 3^8 base-3 codes and sorted
    ascending; digit j of a code (least significant first) picks element j.
    """
    codes = np.sort(rng(seed).choice(3 ** 8, size=n, replace=False))
    digits = (codes[:, None] // (3 ** np.arange(8))[None, :]) % 3
    return np.asarray(alphabet, dtype=np.float32)[digits]


def grid_iq2(n: int, seed: int) -> np.ndarray:
    return grid(n, IQ2_ALPHABET, seed)


def grid_iq1(n: int, seed: int) -> np.ndarray:
    return grid(n, IQ1_ALPHABET, seed)


# ----------------------------------------------------------------------------
# Weights, activations, routing
# ----------------------------------------------------------------------------
def weight(rows: int, cols: int, seed: int, outlier_seed: int | None = None,
           std: float = 0.02, outlier_frac: float = 0.01, outlier_sigmas: float = 8.0,
           bf16: bool = True) -> np.ndarray:
    """float32 [rows, cols] ~ N(0, std^2); with outlier_seed, a Bernoulli(outlier_frac)
    set of positions is replaced by +-outlier_sigmas*std (sign of the original draw)."""
    w = (rng(seed).standard_normal((rows, cols), dtype=np.float32) * np.float32(std))
    if outlier_seed is not None:
        mask = rng(outlier_seed).random((rows, cols), dtype=np.float32) < outlier_frac
        w = np.where(mask, np.copysign(np.float32(outlier_sigmas * std), w), w).astype(np.float32)
    return round_to_bf16(w) if bf16 else w


def column_sigmas(K: int, seed: int) -> np.ndarray:
    """sigma_j = exp(N(0, 1)): the per-column activation scale law."""
    return np.exp(rng(seed).standard_normal(K)).astype(np.float32)


def activations(T: int, K: int, sigma_seed: int, z_seed: int, bf16: bool = True) -> np.ndarray:
    """float32 [T, K], x_tj = sigma_j * z_tj with z ~ N(0, 1)."""
    sig = column_sigmas(K, sigma_seed)
    z = rng(z_seed).standard_normal((T, K), dtype=np.float32)
    x = (z * sig[None, :]).astype(np.float32)
    return round_to_bf16(x) if bf16 else x


def routing(T: int, top_k: int, num_experts: int, seed: int, n_idle: int = 5,
            zipf_s: float = 1.1) -> np.ndarray:
    """int32 [T, top_k] expert ids, top_k distinct ids per token.

    A seeded permutation sets n_idle experts aside (no token reaches them); the
    others are ranked by a second permutation and drawn with p ~ rank^-zipf_s via
    Gumbel-top-k on log p.
    """
    g = rng(seed)
    perm = g.permutation(num_experts)
    active = perm[n_idle:]
    ranks = g.permutation(active.size) + 1
    logp = -zipf_s * np.log(ranks.astype(np.float64))
    gumbel = -np.log(-np.log(g.random((T, active.size))))
    top = np.argsort(-(logp[None, :] + gumbel), axis=1, kind="stable")[:, :top_k]
    return active[top].astype(np.int32)


def importance_like(K: int, seed: int) -> np.ndarray:
    """A positive float32 importance row with the configs' dynamic range
    (sqrt of lognormal second moments); used where a test feeds importance
    directly instead of collecting it."""
    s = column_sigmas(K, seed)
    return s.astype(np.float32)


# ----------------------------------------------------------------------------
# The five named workloads (shapes, seeds)
# ----------------------------------------------------------------------------
WORKLOADS = {
    # one 256x512 fp32 weight, IQ2_XXS layout, 512 fp32 tokens
    "iq2_xxs_256x512": dict(fmt="IQ2_XXS", rows=256, cols=512, w_seed=101, w_outlier_seed=None,
                            bf16=False, T=512, sigma_seed=102, z_seed=103, grid_seed=201),
    # dense path: collect 4096 bf16 tokens into 2048 columns, IQ2_XS encode of 5632x2048
    "iq2_xs_5632x2048": dict(fmt="IQ2_XS", rows=5632, cols=2048, w_seed=113, w_outlier_seed=114,
                             bf16=True, T=4096, sigma_seed=111, z_seed=112, grid_seed=202),
    "iq2_s_5632x2048": dict(fmt="IQ2_S", rows=5632, cols=2048, w_seed=113, w_outlier_seed=114,
                            bf16=True, T=4096, sigma_seed=111, z_seed=112, grid_seed=203),
    "iq2_xxs_5632x2048": dict(fmt="IQ2_XXS", rows=5632, cols=2048, w_seed=113, w_outlier_seed=114,
                              bf16=True, T=4096, sigma_seed=111, z_seed=112, grid_seed=201),
    "iq1_s_5632x2048": dict(fmt="IQ1_S", rows=5632, cols=2048, w_seed=113, w_outlier_seed=114,
                            bf16=True, T=4096, sigma_seed=123, z_seed=125, grid_seed=204),
    "iq1_m_5632x2048": dict(fmt="IQ1_M", rows=5632, cols=2048, w_seed=113, w_outlier_seed=114,
                            bf16=True, T=4096, sigma_seed=123, z_seed=125, grid_seed=204),
    "iq1_s_17408x5120": dict(fmt="IQ1_S", rows=17408, cols=5120, w_seed=121, w_outlier_seed=122,
                             bf16=True, T=4096, sigma_seed=124, z_seed=126, grid_seed=204),
    "iq1_m_17408x5120": dict(fmt="IQ1_M", rows=17408, cols=5120, w_seed=121, w_outlier_seed=122,
                             bf16=True, T=4096, sigma_seed=124, z_seed=126, grid_seed=204),
}

GRID_SIZES = {"IQ2_XXS": 256, "IQ2_XS": 512, "IQ2_S": 1024, "IQ1_S": 2048, "IQ1_M": 2048}

# fused-MoE workload: 128 experts of 768x2048, 4096 tokens, top-8 routing
MOE = dict(fmt="IQ2_XXS", experts=128, rows_per_expert=768, cols=2048, w_seed=131,
           T=4096, top_k=8, x_sigma_seed=132, x_z_seed=134, ids_seed=133, n_idle=5, grid_seed=201)


def grid_for(fmt: str, seed: int) -> np.ndarray:
    n = GRID_SIZES[fmt]
    return grid_iq1(n, seed) if fmt.startswith("IQ1") else grid_iq2(n, seed)


def workload(name: str, rows: int | None = None):
    """(w [rows, cols] f32, x [T, cols] f32, grid [N, 8] f32, spec) for a named workload.

    rows=None gives the full weight; a smaller rows draws the full matrix's first rows
    only when it is cheap to do so (callers that need a row subset of a large weight
    should slice the full draw)."""
    spec = dict(WORKLOADS[name])
    w = weight(spec["rows"], spec["cols"], spec["w_seed"], spec["w_outlier_seed"], bf16=spec["bf16"])
    if rows is not None:
        w = np.ascontiguousarray(w[:rows])
    x = activations(spec["T"], spec["cols"], spec["sigma_seed"], spec["z_seed"], bf16=spec["bf16"])
    g = grid_for(spec["fmt"], spec["grid_seed"])
    return w, x, g, spec


def moe_workload(experts: int | None = None):
    """(w [E*rpe, cols], x [T, cols], ids [T, top_k], grid, spec) for the fused-MoE workload."""
    spec = dict(MOE)
    E = spec["experts"] if experts is None else experts
    w = weight(E * spec["rows_per_expert"], spec["cols"], spec["w_seed"], None, bf16=True)
    x = activations(spec["T"], spec["cols"], spec["x_sigma_seed"], spec["x_z_seed"], bf16=True)
    ids = routing(spec["T"], spec["top_k"], spec["experts"], spec["ids_seed"], spec["n_idle"])
    g = grid_for(spec["fmt"], spec["grid_seed"])
    return w, x, ids, g, spec
