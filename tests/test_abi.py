"""C ABI checks that need no GPU: the library loads, exports every entry point
include/iq.h declares, its format table agrees with the oracle's independent
one, and host-side validation rejects bad arguments before anything runs."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "iq.h")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(iq_\w+)\s*\(", txt, flags=re.M)))


@pytest.fixture(scope="module")
def api():
    from ggml_iq_codebook_imatrix_amd import api as a
    if not os.path.exists(a.LIB_PATH):
        from ggml_iq_codebook_imatrix_amd import build
        build.build()
    return a


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["iq_format_info", "iq_imatrix_collect", "iq_imatrix_collect_workspace_size", "iq_hessian_collect",
         "iq_hessian_collect_workspace_size", "iq_imatrix_merge", "iq_imatrix_importance", "iq_quantize",
         "iq_quantize_workspace_size", "iq_quantize_noalloc", "iq_quantize_timed", "iq_quantize_every_choice", "iq_choice_search",
         "iq_choice_search_workspace_size", "iq_dequantize", "iq_error_string"])


def test_library_exports_every_declared_symbol(api):
    lib = api.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (iq_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
        assert name in api.SIGNATURES


def test_library_allocates_nothing(api):
    """The library imports no allocator: every buffer, workspaces included, is the caller's."""
    out = subprocess.run(["nm", "-D", "--undefined-only", api.LIB_PATH], capture_output=True, text=True).stdout
    imported = set(re.findall(r"\b(hip\w+)", out))
    assert imported, out
    assert not {n for n in imported if "Malloc" in n or "Free" in n or "Alloc" in n or "Memcpy" in n}, imported


def test_workspace_sizes(api):
    L = api.lib()
    q = api.quantize_workspace_size
    # weighted norms: one table per (expert, 8-column group); flat: one table
    assert q("IQ2_XS", 5632, 2048, weighted=True) > q("IQ2_XS", 5632, 2048, weighted=False)
    assert q("IQ2_XXS", 0, 512) == 0
    assert q("IQ2_XXS", 98304, 2048, 768) > q("IQ2_XXS", 98304, 2048)  # 128 experts' tables
    assert api.choice_search_workspace_size("IQ2_XS", 5632, 2048) > 16 * 5632 * 8 * 32 * 4
    # collection scratch does not grow with the number of tokens
    c = api.collect_workspace_size
    assert c(0, 2048) == 0
    assert c(10 ** 4, 7168, 8, 256) == c(10 ** 6, 7168, 8, 256) == c(10 ** 8, 7168, 8, 256)
    assert c(10 ** 7, 2048) == c(10 ** 9, 2048)
    assert c(65536, 7168, 8, 256) < 64 << 20
    assert api.hessian_workspace_size(4096, 2048, 8, 128) > 0
    n = ctypes.c_size_t()
    assert L.iq_quantize_workspace_size(5, 64, 256, 64, 1, ctypes.byref(n)) == -1
    assert L.iq_quantize_workspace_size(0, 64, 300, 64, 1, ctypes.byref(n)) == -4
    assert L.iq_quantize_workspace_size(0, 64, 256, 64, 1, None) == -3
    assert L.iq_imatrix_collect_workspace_size(-1, 8, 0, 1, 1024, ctypes.byref(n)) == -5
    assert L.iq_hessian_collect_workspace_size(16, 300, 0, 1, 1024, ctypes.byref(n)) == -4


def test_binding_checks_buffers_before_any_launch(api):
    """Shapes and dtypes of every caller-supplied tensor are checked before the
    call reaches the library (these CPU tensors would be refused later anyway:
    the shape check must come first)."""
    import torch
    E = api.IQError
    w = torch.zeros(64, 512, dtype=torch.bfloat16)
    g2 = torch.zeros(512, 8)
    with pytest.raises(E, match="grid"):
        api.quantize("IQ2_XS", w, torch.zeros(256, 8))
    with pytest.raises(E, match="out"):
        api.quantize("IQ2_XS", w, g2, out=torch.zeros(64, 2, 66, dtype=torch.uint8))
    with pytest.raises(E, match="choices"):
        api.quantize("IQ2_XS", w, g2, choices=torch.zeros(64, 2, 8, dtype=torch.uint8))
    with pytest.raises(E, match="importance"):
        api.quantize("IQ2_XS", w, g2, torch.zeros(2, 512))
    with pytest.raises(E, match="columns"):
        api.quantize("IQ2_XS", torch.zeros(64, 300), g2)
    with pytest.raises(E, match="out"):
        api.quantize_every_choice("IQ2_XS", w, g2, out=torch.zeros(15, 64, 2, 74, dtype=torch.uint8))
    h = torch.zeros(1, 2, 256, 256)
    with pytest.raises(E, match="hess"):
        api.choice_search("IQ2_XS", w, g2, torch.zeros(1, 1, 256, 256))
    with pytest.raises(E, match="out"):
        api.choice_search("IQ2_XS", w, g2, h, out=torch.zeros(64, 2, 8, dtype=torch.uint8))
    with pytest.raises(E, match="payload"):
        api.choice_search("IQ2_XS", w, g2, h, payload=torch.zeros(64, 2, 66, dtype=torch.uint8))
    p = torch.zeros(64, 2, 66, dtype=torch.uint8)
    with pytest.raises(E, match="packed"):
        api.dequantize("IQ2_S", p, torch.zeros(1024, 8))           # 66-byte blocks read as 82-byte ones
    with pytest.raises(E, match="out"):
        api.dequantize("IQ2_XXS", p, torch.zeros(256, 8), out=torch.zeros(64, 256))
    with pytest.raises(E, match="dtype"):
        api.dequantize("IQ2_XXS", p, torch.zeros(256, 8), dtype=torch.float16)
    with pytest.raises(E, match="counts"):
        api.imatrix_importance(torch.zeros(2, 8), torch.zeros(3, dtype=torch.int64))
    with pytest.raises(E, match="out"):
        api.imatrix_importance(torch.zeros(2, 8), torch.zeros(2, dtype=torch.int64), out=torch.zeros(2, 7))
    x = torch.zeros(16, 512, dtype=torch.bfloat16)
    with pytest.raises(E, match="ids"):
        api.imatrix_collect(x, torch.zeros(15, 2, dtype=torch.int32), 4)
    with pytest.raises(E, match="sums"):
        api.imatrix_collect(x, sums=torch.zeros(1, 256))
    with pytest.raises(E, match="hess"):
        api.hessian_collect(x, hess=torch.zeros(1, 1, 256, 256))
    with pytest.raises(E, match="src_counts"):
        api.imatrix_merge(torch.zeros(2, 8), torch.zeros(1, dtype=torch.int64), torch.zeros(2, 8),
                          torch.zeros(2, dtype=torch.int64))
    with pytest.raises(E, match="status"):
        api.quantize("IQ2_XS", w, g2, status=torch.zeros(1, dtype=torch.int64))
    with pytest.raises(E, match="device"):                       # right shapes: now the placement check
        api.quantize("IQ2_XS", w, g2)


def test_format_table_matches_oracle(api, orc):
    for fmt in api.FORMATS:
        info = api.format_info(fmt)
        geo = orc.geometry(fmt)
        assert info["block_values"] == 256
        assert info["block_bytes"] == geo["block_bytes"]
        assert info["grid_size"] == geo["grid_n"]
        assert info["choice_groups"] == geo["units"]
        assert info["num_choices"] == geo["num_choices"]
        assert info["groups_per_choice"] == geo["groups_per_unit"]


def test_host_validation_quantize(api):
    L = api.lib()
    q = lambda fmt=0, w=FAKE, dt=1, rows=64, cols=512, rpe=64, grid=FAKE, out=FAKE: L.iq_quantize(
        fmt, w, dt, rows, cols, rpe, grid, None, None, out, FAKE, 1 << 40, None, None)
    assert q(fmt=5) == -1 and q(fmt=-1) == -1
    assert q(dt=2) == -2
    assert q(w=None) == -3 and q(grid=None) == -3 and q(out=None) == -3
    assert q(cols=300) == -4 and q(cols=0) == -4 and q(rows=-1) == -4
    assert q(rpe=0) == -4 and q(rpe=48) == -4
    ev = lambda fmt=0, cols=512, out=FAKE: L.iq_quantize_every_choice(fmt, FAKE, 1, 64, cols, 64, FAKE, None, out,
                                                                      FAKE, 1 << 40, None, None)
    assert ev(fmt=7) == -1 and ev(cols=100) == -4 and ev(out=None) == -3
    cs = lambda fmt=0, hess=FAKE, ch=FAKE, damp=0.3, rpe=64: L.iq_choice_search(fmt, FAKE, 1, 64, 512, rpe, FAKE, None,
                                                                              hess, damp, ch, None, FAKE, 1 << 40,
                                                                              None, None)
    assert cs(fmt=9) == -1 and cs(hess=None) == -3 and cs(ch=None) == -3 and cs(rpe=7) == -4
    assert cs(damp=-1.0) == -5 and cs(damp=float("inf")) == -5
    assert L.iq_format_info(0, None) == -3
    assert api.lib().iq_error_string(-4) == b"invalid shape"
    assert q(rows=1 << 41) == -4 and q(cols=256 * (1 << 25)) == -4


def test_host_validation_collect_importance_decode(api):
    L = api.lib()
    c = lambda x=FAKE, dt=1, T=16, K=64, ids=None, top_k=0, E=1, chunk=1024, sums=FAKE, counts=FAKE: \
        L.iq_imatrix_collect(x, dt, T, K, ids, top_k, E, chunk, sums, counts, FAKE, 1 << 40, None, None)
    assert c(dt=7) == -2
    assert c(x=None) == -3 and c(sums=None) == -3 and c(counts=None) == -3
    assert c(T=-1) == -5 and c(K=0) == -5 and c(chunk=0) == -5 and c(E=0) == -5
    assert c(E=4) == -5                           # dense needs one statistic
    assert c(ids=FAKE, top_k=0, E=4) == -5
    h = lambda x=FAKE, dt=1, T=16, K=512, ids=None, top_k=0, E=1, chunk=1024, hess=FAKE: \
        L.iq_hessian_collect(x, dt, T, K, ids, top_k, E, chunk, hess, FAKE, 1 << 40, None, None)
    assert h(dt=5) == -2 and h(x=None) == -3 and h(hess=None) == -3
    assert h(K=300) == -4 and h(T=-1) == -5 and h(E=2) == -5 and h(ids=FAKE, top_k=0, E=2) == -5
    assert h(chunk=0) == -5 and h(ids=FAKE, top_k=2, E=1 << 22) == -5 and h(T=1 << 31) == -5
    assert h(T=0) == 0                            # nothing to add: returns before any launch
    imp = lambda s=FAKE, cnt=FAKE, E=1, K=8, fl=1e-6, out=FAKE: L.iq_imatrix_importance(s, cnt, E, K, fl, out,
                                                                                       None, None)
    assert imp(s=None) == -3 and imp(out=None) == -3
    assert imp(E=0) == -5 and imp(K=0) == -5 and imp(fl=-1.0) == -5 and imp(fl=float("nan")) == -5
    F2, F3 = ctypes.c_void_p(0x2000), ctypes.c_void_p(0x9000)
    m = lambda s=FAKE, sc=F2, E=2, K=8, d=F3, dc=ctypes.c_void_p(0xA000): L.iq_imatrix_merge(s, sc, E, K, d, dc,
                                                                                            None, None)
    assert m(s=None) == -3 and m(sc=None) == -3 and m(d=None) == -3 and m(dc=None) == -3
    assert m(E=0) == -5 and m(K=0) == -5
    assert m(d=ctypes.c_void_p(0x1020)) == -5      # source sums overlap the accumulator
    assert m(dc=ctypes.c_void_p(0x2008)) == -5     # source counts overlap the accumulator
    d = lambda fmt=0, p=FAKE, rows=4, cols=256, grid=FAKE, out=FAKE, dt=0: L.iq_dequantize(
        fmt, p, rows, cols, grid, out, dt, None)
    assert d(fmt=9) == -1 and d(dt=3) == -2 and d(p=None) == -3 and d(cols=100) == -4


def test_binding_fails_loudly_without_library(api, monkeypatch, tmp_path):
    monkeypatch.setattr(api, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(api, "_lib", None)
    with pytest.raises(api.IQError):
        api.lib()
