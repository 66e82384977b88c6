"""bench.py's work model and roofline fractions (no GPU).

The search FLOP per launch is counted here from the operations the exhaustive
search performs, written per (row, group, entry) and per (expert, column group,
entry), and compared with bench.search_flop; the odd-parity count of the IQ2_XS
workload weight is taken from numpy.  The documented per-launch figure for the
5632x2048 IQ2_XS weight (53.51 GFLOP) follows from both.
"""
import numpy as np
import pytest

import bench
from ggml_iq_codebook_imatrix_amd import inputs

FMA, MUL, MIN, ADD = 2, 1, 1, 1


def per_entry(fmt):
    """FLOP per (row, group, entry) for every group, and extra for an odd group."""
    chain = 8 * FMA                                 # the -2P (IQ1: Q) chain over 8 values
    cands = 16 * (FMA + MIN)                        # 16 candidates: scale * G + P, running minimum
    shifts = 2 * FMA if fmt.startswith("IQ1") else 0
    parity = 8 * MUL + 7 * MIN + 1 * FMA if fmt in ("IQ2_XXS", "IQ2_XS") else 0
    return chain + cands + shifts, parity


def per_norm(fmt):
    """FLOP per (expert, column group, entry): the weighted norm sum_j a_j g_j^2
    (IQ1: for each of the two shifts, of (g_j + delta)^2)."""
    one = 8 * MUL + 8 * FMA                         # g^2, then a * g^2 accumulated
    return 2 * (8 * ADD + one) if fmt.startswith("IQ1") else one


@pytest.mark.parametrize("fmt", ["IQ2_XXS", "IQ2_XS", "IQ2_S", "IQ1_S", "IQ1_M"])
def test_search_flop_is_the_counted_operations(fmt):
    rows, cols, E, odd = 320, 1024, 2, 1234
    n = bench.GRID_N[fmt]
    base, parity = per_entry(fmt)
    want = n * (rows * cols // 8 * base + odd * parity) + n * E * (cols // 8) * per_norm(fmt)
    assert bench.search_flop(fmt, rows, cols, E, odd) == want


def test_workload_flop_per_launch():
    torch = pytest.importorskip("torch")
    w32, _, _, _ = inputs.workload("iq2_xs_5632x2048")
    wb = inputs.round_to_bf16(w32)
    odd_np = int(((wb.reshape(wb.shape[0], -1, 8) < 0).sum(-1) % 2).sum())
    odd = bench.odd_parity_groups(torch.from_numpy(wb))
    assert odd == odd_np
    flop = bench.search_flop("IQ2_XS", 5632, 2048, 1, odd)
    assert round(flop / 1e9, 2) == 53.51


def test_fractions_refuse_values_above_one():
    assert bench.frac(78.65, 157.3, "x") == 0.5
    with pytest.raises(RuntimeError):
        bench.frac(160.0, 157.3, "x")
    assert bench.frac_measured(50.0, 100.0) == 0.5
    assert bench.frac_measured(101.0, 100.0) is None


def test_best_ceiling_keeps_the_higher_run():
    lo = {"ceiling_TFLOP_s": 99.7, "clock_GHz": 1.90}
    hi = {"ceiling_TFLOP_s": 118.6, "clock_GHz": 2.09}
    assert bench.best_ceiling(lo, hi) is hi and bench.best_ceiling(hi, lo) is hi


def test_more_than_one_gpu_is_refused_with_a_message():
    """bench.py measures one GPU: asked for more it says so and exits with code 2,
    before touching torch or a device."""
    import os
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
