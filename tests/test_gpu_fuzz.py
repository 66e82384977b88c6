"""Seeded random configurations of the encoder, the every-choice encode and the
local-Hessian choice search, each against the CPU oracle byte for byte.

Every case draws its layout, expert count, rows per expert (so ragged 64-row
tiles and one-row experts occur), width, dtype, weighting (importance per
expert, flat, or importance with dead columns), caller choices, and row
magnitudes (zero rows, and rows scaled by 2^-20 .. 2^20, so fp16 block scales
underflow to subnormals or overflow and the block is refused on both sides).
"""
import numpy as np
import pytest

from ggml_iq_codebook_imatrix_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FORMATS = ("IQ2_XXS", "IQ2_XS", "IQ2_S", "IQ1_S", "IQ1_M")
UNITS = {"IQ2_XXS": 8, "IQ2_XS": 16, "IQ2_S": 16, "IQ1_S": 8, "IQ1_M": 16}
CHOICES = {"IQ2_XXS": 16, "IQ2_XS": 16, "IQ2_S": 16, "IQ1_S": 16, "IQ1_M": 8}


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ggml_iq_codebook_imatrix_amd import api as a
    a.lib()  # raises if the HIP library is missing: no fallback
    return a


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_w(w32, dtype):
    if dtype == "bf16":
        return torch.from_numpy(inputs.f32_to_bf16_bits(w32).view(np.int16)).cuda().view(torch.bfloat16)
    return dev(w32.astype(np.float32))


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def draw_case(seed):
    """One random configuration: (fmt, w fp32 [rows, cols] exactly representable
    in the dtype, dtype, rows per expert, importance [E, cols] or None, grid)."""
    g = inputs.rng(seed)
    fmt = FORMATS[int(g.integers(len(FORMATS)))]
    E = int(g.integers(1, 4))
    rpe = int(g.choice([1, 7, 63, 64, 65, 100, 130]))
    nb = int(g.integers(1, 4))
    rows, cols = E * rpe, 256 * nb
    dtype = "bf16" if g.random() < 0.6 else "f32"
    w = inputs.weight(rows, cols, seed + 1, seed + 2, bf16=False)
    scale = np.exp2(g.integers(-20, 21, size=(rows, 1))).astype(np.float32)
    w = (w * scale).astype(np.float32)
    w[g.random(rows) < 0.05] = 0.0
    if dtype == "bf16":
        w = inputs.round_to_bf16(w)
    kind = g.choice(["weighted", "flat", "dead_columns"])
    imp = None
    if kind != "flat":
        imp = np.stack([inputs.importance_like(cols, seed + 10 + e) for e in range(E)]).astype(np.float32)
        if kind == "dead_columns":
            imp[:, g.random(cols) < 0.2] = 0.0
    grid = inputs.grid_for(fmt, 201 + FORMATS.index(fmt) if fmt != "IQ1_M" else 204)
    return fmt, w, dtype, rpe, imp, grid, g


@pytest.mark.parametrize("seed", range(5000, 5024))
def test_encode_fuzz(api, orc, seed):
    fmt, w, dtype, rpe, imp, grid, g = draw_case(seed)
    rows, cols = w.shape
    choices = None
    if g.random() < 0.4:
        choices = g.integers(0, CHOICES[fmt], size=(rows, cols // 256, UNITS[fmt])).astype(np.uint8)
    say("encode", seed, fmt, w.shape, dtype, rpe, imp is not None, choices is not None)
    st = api.new_status()
    got = host(api.quantize(fmt, dev_w(w, dtype), dev(grid), None if imp is None else dev(imp), rpe,
                            None if choices is None else dev(choices), status=st))
    want, st_want = orc.quantize(fmt, w, grid, imp, rows_per_expert=rpe, choices=choices)
    bad = np.argwhere((got != want).any(axis=-1))
    assert bad.size == 0, f"{len(bad)} blocks differ, first {bad[:5].tolist()}"
    assert int(host(st)[0]) == st_want


@pytest.mark.parametrize("seed", range(6000, 6006))
def test_every_choice_fuzz(api, orc, seed):
    fmt, w, dtype, rpe, imp, grid, _ = draw_case(seed)
    say("every choice", seed, fmt, w.shape, dtype, rpe, imp is not None)
    got = host(api.quantize_every_choice(fmt, dev_w(w, dtype), dev(grid), None if imp is None else dev(imp), rpe))
    want, _ = orc.quantize_every_choice(fmt, w, grid, imp, rows_per_expert=rpe)
    bad = np.argwhere((got != want).any(axis=-1))
    assert bad.size == 0, f"{len(bad)} blocks differ, first {bad[:5].tolist()}"


@pytest.mark.parametrize("seed", range(7000, 7006))
def test_choice_search_fuzz(api, orc, seed):
    fmt, w, dtype, rpe, imp, grid, g = draw_case(seed)
    rows, cols = w.shape
    E, nb = rows // rpe, cols // 256
    # each expert's blocks: X^T X of a few correlated tokens plus a diagonal
    hess = np.empty((E, nb, 256, 256), np.float32)
    for e in range(E):
        for b in range(nb):
            x = g.standard_normal((24, 256)).astype(np.float32) * np.exp(g.normal(0, 1, 256)).astype(np.float32)
            h = x.T.astype(np.float64) @ x.astype(np.float64) + np.diag(g.random(256) * 0.1)
            hess[e, b] = h.astype(np.float32)
    pd = float(g.choice([0.0, 0.01, 0.3]))
    say("choice search", seed, fmt, w.shape, dtype, rpe, imp is not None, pd)
    ch, pay = api.choice_search(fmt, dev_w(w, dtype), dev(grid), dev(hess), None if imp is None else dev(imp),
                                rows_per_expert=rpe, perc_damp=pd, payload=True)
    want, _ = orc.choice_search(fmt, w, grid, hess, imp, rows_per_expert=rpe, perc_damp=pd)
    got = host(ch)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} picks differ, first {bad[:5].tolist()}"
    pw, _ = orc.quantize(fmt, w, grid, imp, rows_per_expert=rpe, choices=want)
    bad = np.argwhere((host(pay) != pw).any(axis=-1))
    assert bad.size == 0, f"{len(bad)} blocks differ, first {bad[:5].tolist()}"
