"""Statistics files: collected imatrix statistics saved, loaded and merged.

"MoE expert coverage in imatrix calibration" (Facts list) describes the GGUF
imatrix format as storing each tensor's ``in_sum2`` and ``counts`` so that
files can be merged, and the collector's report of experts with partial or no
data.  This module keeps that naming in a safetensors container (it is not the
GGUF binary format): for a weight named ``name``,

  ``name.in_sum2``  float32 [E, K]  per-expert sums of x_j^2 (E = 1 for a dense weight)
  ``name.counts``   int64   [E]     (token, slot) pairs each expert saw

Saving and loading are host file IO; merging runs on the device through
``iq_imatrix_merge`` (sums added in fp32, counts exactly), in the order given.
"""
from __future__ import annotations

import torch
from safetensors.torch import load_file, save_file

from . import api

SUMS, COUNTS = ".in_sum2", ".counts"


def save(path: str, stats: dict) -> None:
    """Write {name: (sums [E, K] f32, counts [E] int64)} to ``path``."""
    tensors = {}
    for name, (sums, counts) in stats.items():
        if sums.dim() != 2 or counts.dim() != 1 or counts.shape[0] != sums.shape[0]:
            raise api.IQError(f"{name}: sums must be [E, K] and counts [E]")
        tensors[name + SUMS] = sums.detach().to("cpu", torch.float32).contiguous()
        tensors[name + COUNTS] = counts.detach().to("cpu", torch.int64).contiguous()
    save_file(tensors, path)


def load(path: str, device=None) -> dict:
    """Read a statistics file -> {name: (sums, counts)} (on ``device`` if given)."""
    raw = load_file(path)
    out = {}
    for key in raw:
        if key.endswith(SUMS):
            name = key[: -len(SUMS)]
            if name + COUNTS not in raw:
                raise api.IQError(f"{path}: {name} has sums but no counts")
            sums, counts = raw[key], raw[name + COUNTS]
            if sums.dtype != torch.float32 or counts.dtype != torch.int64 or sums.dim() != 2 \
                    or tuple(counts.shape) != (sums.shape[0],):
                raise api.IQError(f"{path}: {name} must hold f32 [E, K] sums and int64 [E] counts")
            if device is not None:
                sums, counts = sums.to(device), counts.to(device)
            out[name] = (sums, counts)
    return out


def merge_files(paths, device="cuda", status: torch.Tensor | None = None) -> dict:
    """Merge statistics files in the given order on ``device``: a weight present
    in several files gets the sum of its statistics; shapes must agree."""
    merged: dict = {}
    for p in paths:
        for name, (sums, counts) in load(p, device).items():
            if name not in merged:
                merged[name] = (sums.clone(), counts.clone())
                continue
            dst_s, dst_c = merged[name]
            if dst_s.shape != sums.shape:
                raise api.IQError(f"{name}: {tuple(sums.shape)} in {p} differs from {tuple(dst_s.shape)}")
            api.imatrix_merge(sums, counts, dst_s, dst_c, status=status)
    return merged


def coverage(counts: torch.Tensor) -> dict:
    """How many experts saw data: the figure behind the collector's
    partial-data report (an expert with count 0 is encoded with flat weights)."""
    c = counts.detach().to("cpu")
    n = int(c.numel())
    seen = int((c > 0).sum())
    return {"experts": n, "with_data": seen, "fraction": seen / n if n else 0.0}
