"""Statistics files: the in_sum2 / counts layout, round trip and coverage (host
only), and merging files on the GPU equals merging the statistics in memory."""
import numpy as np
import pytest
import torch

from ggml_iq_codebook_imatrix_amd import imatrix_file, inputs


def stats(seed, E, K):
    g = inputs.rng(seed)
    return (torch.from_numpy((g.lognormal(0, 1, (E, K)) * 10).astype(np.float32)),
            torch.from_numpy(g.integers(0, 300, E).astype(np.int64)))


def test_file_layout_and_round_trip(tmp_path):
    from safetensors.torch import load_file
    s = {"blk.0.ffn_down_exps": stats(1, 8, 512), "blk.0.attn_q": stats(2, 1, 256)}
    p = str(tmp_path / "a.safetensors")
    imatrix_file.save(p, s)
    raw = load_file(p)
    assert sorted(raw) == sorted(["blk.0.ffn_down_exps.in_sum2", "blk.0.ffn_down_exps.counts",
                                  "blk.0.attn_q.in_sum2", "blk.0.attn_q.counts"])
    back = imatrix_file.load(p)
    for name, (a, c) in s.items():
        assert torch.equal(back[name][0], a) and torch.equal(back[name][1], c)


def test_coverage_counts_experts_with_data():
    c = torch.tensor([0, 5, 0, 1, 9, 0, 0, 2], dtype=torch.int64)
    assert imatrix_file.coverage(c) == {"experts": 8, "with_data": 4, "fraction": 0.5}


@pytest.mark.gpu
def test_merge_files_equals_merge_in_memory(tmp_path, orc):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    a, b, c = stats(3, 6, 1024), stats(4, 6, 1024), stats(5, 2, 256)
    pa, pb = str(tmp_path / "a.safetensors"), str(tmp_path / "b.safetensors")
    imatrix_file.save(pa, {"w1": a, "w2": c})
    imatrix_file.save(pb, {"w1": b})
    merged = imatrix_file.merge_files([pa, pb])
    torch.cuda.synchronize()
    want_s, want_c, _ = orc.merge(b[0].numpy(), b[1].numpy(), a[0].numpy(), a[1].numpy())
    assert np.array_equal(merged["w1"][0].cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(merged["w1"][1].cpu().numpy(), want_c)
    assert torch.equal(merged["w2"][0].cpu(), c[0]) and torch.equal(merged["w2"][1].cpu(), c[1])
