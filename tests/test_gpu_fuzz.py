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


def draw_tie_case(seed):
    """A configuration whose values make exact ties likely: small integer
    multiples of a power of two, one constant magnitude with random signs, or a
    sparse set of equal spikes, with flat or small-integer importance; so the
    first-minimum rules (lower choice, lower shift, lower entry) decide many
    picks on both sides."""
    g = inputs.rng(seed)
    fmt = FORMATS[int(g.integers(len(FORMATS)))]
    E = int(g.integers(1, 4))
    rpe = int(g.choice([1, 31, 64, 65, 129]))
    nb = int(g.integers(1, 3))
    rows, cols = E * rpe, 256 * nb
    fam = g.choice(["ints", "const", "spiky"])
    if fam == "ints":
        w = g.integers(-3, 4, size=(rows, cols)).astype(np.float32) * np.float32(2.0 ** int(g.integers(-8, 3)))
    elif fam == "const":
        w = np.sign(g.standard_normal((rows, cols))).astype(np.float32) * np.float32(0.25)
    else:
        w = g.standard_normal((rows, cols)).astype(np.float32) * np.float32(1e-3)
        m = g.random((rows, cols)) < 0.02
        w[m] = np.sign(g.standard_normal(int(m.sum()))).astype(np.float32)
    w[g.random(rows) < 0.05] = 0.0
    dtype = "bf16" if g.random() < 0.5 else "f32"
    if dtype == "bf16":
        w = inputs.round_to_bf16(w)
    imp = None if g.random() < 0.5 else g.integers(1, 4, size=(E, cols)).astype(np.float32)
    grid = inputs.grid_for(fmt, int(g.integers(200, 100000)))
    return fmt, w, dtype, rpe, imp, grid, g, fam


@pytest.mark.parametrize("seed", range(8000, 8012))
def test_encode_fuzz_ties(api, orc, seed):
    fmt, w, dtype, rpe, imp, grid, g, fam = draw_tie_case(seed)
    rows, cols = w.shape
    choices = None
    if g.random() < 0.3:
        choices = g.integers(0, CHOICES[fmt], size=(rows, cols // 256, UNITS[fmt])).astype(np.uint8)
    say("encode ties", seed, fmt, w.shape, dtype, rpe, fam, imp is not None, choices is not None)
    st = api.new_status()
    got = host(api.quantize(fmt, dev_w(w, dtype), dev(grid), None if imp is None else dev(imp), rpe,
                            None if choices is None else dev(choices), status=st))
    want, st_want = orc.quantize(fmt, w, grid, imp, rows_per_expert=rpe, choices=choices)
    bad = np.argwhere((got != want).any(axis=-1))
    assert bad.size == 0, f"{len(bad)} blocks differ, first {bad[:5].tolist()}"
    assert int(host(st)[0]) == st_want
    ev = host(api.quantize_every_choice(fmt, dev_w(w, dtype), dev(grid), None if imp is None else dev(imp), rpe))
    want_ev, _ = orc.quantize_every_choice(fmt, w, grid, imp, rows_per_expert=rpe)
    assert np.array_equal(ev, want_ev)


@pytest.mark.parametrize("seed", range(8100, 8104))
def test_choice_search_fuzz_ties(api, orc, seed):
    """Integer Hessian blocks (X^T X of small integer tokens) on tie-prone
    weights: the fp32 sums are exact, so the picks' ties are exact too."""
    fmt, w, dtype, rpe, imp, grid, g, fam = draw_tie_case(seed)
    rows, cols = w.shape
    E, nb = rows // rpe, cols // 256
    hess = np.empty((E, nb, 256, 256), np.float32)
    for e in range(E):
        for b in range(nb):
            x = g.integers(-2, 3, size=(8, 256)).astype(np.float64)
            hess[e, b] = (x.T @ x).astype(np.float32)
    pd = float(g.choice([0.0, 0.3]))
    say("choice search ties", seed, fmt, w.shape, dtype, rpe, fam, imp is not None, pd)
    ch, pay = api.choice_search(fmt, dev_w(w, dtype), dev(grid), dev(hess), None if imp is None else dev(imp),
                                rows_per_expert=rpe, perc_damp=pd, payload=True)
    want, _ = orc.choice_search(fmt, w, grid, hess, imp, rows_per_expert=rpe, perc_damp=pd)
    assert np.array_equal(host(ch), want)
    pw, _ = orc.quantize(fmt, w, grid, imp, rows_per_expert=rpe, choices=want)
    assert np.array_equal(host(pay), pw)


@pytest.mark.parametrize("seed", range(8200, 8206))
def test_collect_importance_merge_fuzz(api, orc, seed):
    """Random token counts, widths (not multiples of 8), expert counts, top-k
    with repeated ids and chunk sizes: counts exact, sums exact on integer
    tokens (else within 1e-5 of the fp64 sums), importance and merge bit-exact
    on the device's own statistics."""
    g = inputs.rng(seed)
    T, K, E = int(g.integers(1, 3000)), int(g.integers(1, 700)), int(g.integers(1, 9))
    routed = g.random() < 0.6
    top_k = int(g.integers(1, 5)) if routed else 0
    chunk = int(g.choice([1, 7, 100, 1024, 1500]))
    ints = g.random() < 0.5
    x = (g.integers(-4, 5, size=(T, K)).astype(np.float32) if ints else
         g.standard_normal((T, K)).astype(np.float32) * np.exp(g.normal(0, 2, K)).astype(np.float32))
    dtype = "bf16" if g.random() < 0.5 else "f32"
    if dtype == "bf16":
        x = inputs.round_to_bf16(x)
    ids = g.integers(0, E, size=(T, top_k)).astype(np.int32) if routed else None
    Ee = E if routed else 1
    say("collect", seed, T, K, Ee, top_k, chunk, dtype, ints)
    s, c = api.imatrix_collect(dev_w(x, dtype), None if ids is None else dev(ids), Ee, chunk_rows=chunk)
    so, co, _ = orc.collect(x, ids, Ee)
    assert np.array_equal(host(c), co)
    sg = host(s).astype(np.float64)
    if ints:
        assert np.array_equal(sg, so)
    else:
        assert np.all(np.abs(sg - so) <= 1e-5 * so)
    fr = float(g.choice([1e-6, 0.0, 0.5]))
    imp = host(api.imatrix_importance(s, c, floor_rel=fr))
    imp_o, _ = orc.importance(host(s), host(c), floor_rel=fr)
    assert np.array_equal(imp.view(np.uint32), imp_o.view(np.uint32))
    s2 = dev((g.standard_normal((Ee, K)) ** 2).astype(np.float32))
    c2 = dev(g.integers(0, 100, Ee).astype(np.int64))
    before_s, before_c = host(s).copy(), host(c).copy()
    api.imatrix_merge(s2, c2, s, c)
    ms, mc, _ = orc.merge(host(s2), host(c2), before_s, before_c)
    assert np.array_equal(host(s).view(np.uint32), ms.view(np.uint32))
    assert np.array_equal(host(c), mc)


@pytest.mark.parametrize("seed", range(8300, 8304))
def test_hessian_fuzz_integer_tokens(api, orc, seed):
    """Random routed / dense Hessian blocks on small integer tokens (every fp32
    sum exact): equal to the fp64 oracle element for element."""
    g = inputs.rng(seed)
    T, K, E = int(g.integers(1, 700)), 256 * int(g.integers(1, 3)), int(g.integers(1, 5))
    routed = g.random() < 0.6
    top_k = int(g.integers(1, 4)) if routed else 0
    x = g.integers(-3, 4, size=(T, K)).astype(np.float32)
    dtype = "bf16" if g.random() < 0.5 else "f32"
    ids = g.integers(0, E, size=(T, top_k)).astype(np.int32) if routed else None
    Ee = E if routed else 1
    chunk = int(g.choice([32, 100, 1024]))
    say("hessian", seed, T, K, Ee, top_k, dtype, chunk)
    hg = host(api.hessian_collect(dev_w(x, dtype), None if ids is None else dev(ids), Ee, chunk_rows=chunk))
    ho, _ = orc.hessian_collect(x, ids, Ee)
    assert np.array_equal(hg.astype(np.float64), ho)
