"""iq_quantize_noalloc (the entry point for callers that cannot allocate)
against iq_quantize with a caller workspace, through the C ABI: byte-identical
payloads and status on two calls in a row, the second smaller, for weighted,
flat, fixed-choice and per-expert encodes; a call too large for the static
scratch is refused before anything runs."""
import numpy as np
import pytest

from ggml_iq_codebook_imatrix_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GRID_SEED = {"IQ2_XXS": 201, "IQ2_XS": 202, "IQ2_S": 203, "IQ1_S": 204, "IQ1_M": 204}


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ggml_iq_codebook_imatrix_amd import api as a
    a.lib()
    return a


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(w32):
    return torch.from_numpy(inputs.f32_to_bf16_bits(w32).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("fmt", ["IQ2_XXS", "IQ2_XS", "IQ2_S", "IQ1_S", "IQ1_M"])
def test_noalloc_matches_workspace_call(api, fmt):
    print("[case] noalloc", fmt, flush=True)
    grid = dev(inputs.grid_for(fmt, GRID_SEED[fmt]))
    info = api.format_info(fmt)
    w = inputs.weight(300, 1024, 5100, 5101)
    w[3, :256] = 0.0
    wd = dev_bf16(w)
    imp = dev(inputs.importance_like(1024, 5102)[None, :])
    ch = dev(inputs.rng(5103).integers(0, info["num_choices"], (300, 4, info["choice_groups"])).astype(np.uint8))
    for rows, kw in ((300, dict(importance=imp)), (130, dict(importance=imp)), (300, dict()),
                     (130, dict(importance=imp, choices=ch[:130])), (96, dict(importance=imp[:, :512]))):
        cols = 512 if kw.get("importance") is not None and kw["importance"].shape[1] == 512 else 1024
        x = wd[:rows, :cols].contiguous()
        s1, s2 = api.new_status(), api.new_status()
        want = api.quantize(fmt, x, grid, rows_per_expert=None, status=s1, **kw)
        got = api.quantize_noalloc(fmt, x, grid, status=s2, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (fmt, rows, cols, sorted(kw))
        assert int(s1.item()) == int(s2.item())


def test_noalloc_experts_and_refusal(api):
    print("[case] noalloc experts", flush=True)
    fmt = "IQ2_XXS"
    grid = dev(inputs.grid_for(fmt, 201))
    w = dev_bf16(inputs.weight(4 * 72, 512, 5200, 5201))
    imp = dev(np.stack([inputs.importance_like(512, 5202 + e) for e in range(4)]))
    for rows, e in ((4 * 72, 4), (2 * 72, 2)):
        want = api.quantize(fmt, w[:rows], grid, imp[:e], rows_per_expert=72)
        got = api.quantize_noalloc(fmt, w[:rows], grid, imp[:e], rows_per_expert=72)
        assert torch.equal(got, want)
    # 256 experts x 2048 columns of IQ2_XS tables need 128 MiB: refused, output untouched
    big_rows, cols = 256 * 8, 2048
    assert api.quantize_workspace_size("IQ2_XS", big_rows, cols, 8) > api.NOALLOC_SCRATCH_BYTES
    wb = torch.zeros((big_rows, cols), dtype=torch.bfloat16, device="cuda")
    ib = torch.ones((256, cols), dtype=torch.float32, device="cuda")
    out = torch.full((big_rows, cols // 256, 74), 7, dtype=torch.uint8, device="cuda")
    with pytest.raises(api.IQError, match="IQ_ERR_WORKSPACE"):
        api.quantize_noalloc("IQ2_XS", wb, dev(inputs.grid_for("IQ2_XS", 202)), ib, rows_per_expert=8, out=out)
    assert bool((out == 7).all().item())
    # after the refusal the entry point still works
    got = api.quantize_noalloc(fmt, w[:72], grid, imp[:1])
    assert torch.equal(got, api.quantize(fmt, w[:72], grid, imp[:1]))
