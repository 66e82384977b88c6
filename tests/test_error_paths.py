"""Launch error paths of the C ABI, on the CPU.

A test build of libiq links the library's own objects against a stand-in for
the HIP runtime's launch calls (tests/hip_launch_stub.c), so kernels never run
and any chosen launch can fail.  Every entry point must return IQ_ERR_HIP at
the first failed launch and enqueue nothing after it, and a call rejected on
the host (bad workspace, bad arguments) must launch nothing at all."""
import ctypes
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "ggml_iq_codebook_imatrix_amd", "_build")
STUB = os.path.join(ROOT, "tests", "hip_launch_stub.c")
F = ctypes.c_void_p(0x100000)  # stands for device memory; never dereferenced
BIG = 1 << 40                  # workspace bytes: large enough for every call here


@pytest.fixture(scope="module")
def stubbed(api, tmp_path_factory):
    objs = sorted(glob.glob(os.path.join(BUILD, "iq_*.hip.o")))
    assert objs, "build the library first"
    d = tmp_path_factory.mktemp("stub")
    so = str(d / "libiq_stubbed.so")
    subprocess.run(["gcc", "-O1", "-fPIC", "-c", STUB, "-o", str(d / "stub.o")], check=True)
    subprocess.run(["gcc", "-shared", "-o", so, *objs, str(d / "stub.o"), "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-Bsymbolic", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    L = ctypes.CDLL(so)
    for name, (args, res) in api.SIGNATURES.items():
        getattr(L, name).argtypes = args
        getattr(L, name).restype = res
    return L


@pytest.fixture(scope="module")
def api():
    from ggml_iq_codebook_imatrix_amd import api as a
    if not os.path.exists(a.LIB_PATH):
        from ggml_iq_codebook_imatrix_amd import build
        build.build()
    return a


def run_failing(L, call):
    """Count the call's launches, then fail each launch in turn."""
    L.stub_reset(0)
    assert call() == 0
    n = L.stub_launches()
    assert n > 0
    for k in range(1, n + 1):
        L.stub_reset(k)
        assert call() == -6, k            # IQ_ERR_HIP
        assert L.stub_launches() == k, k  # nothing enqueued after the failed launch
    return n


CALLS = {
    "quantize": lambda L: L.iq_quantize(1, F, 1, 200, 512, 200, F, F, None, F, F, BIG, None, None),
    "quantize_fixed": lambda L: L.iq_quantize(4, F, 1, 200, 512, 100, F, None, F, F, F, BIG, F, None),
    "every_choice": lambda L: L.iq_quantize_every_choice(0, F, 0, 64, 256, 64, F, F, F, F, BIG, None, None),
    "choice_search": lambda L: L.iq_choice_search(2, F, 1, 130, 512, 65, F, F, F, 0.3, F, F, F, BIG, None, None),
    "collect_dense": lambda L: L.iq_imatrix_collect(F, 1, 70000, 2048, None, 0, 1, 1024, F, F, F, BIG, None, None),
    "collect_routed": lambda L: L.iq_imatrix_collect(F, 1, 20000, 2048, F, 8, 128, 1024, F, F, F, BIG, None, None),
    "hessian_dense": lambda L: L.iq_hessian_collect(F, 1, 4096, 2048, None, 0, 1, 1024, F, F, BIG, None, None),
    "hessian_routed": lambda L: L.iq_hessian_collect(F, 1, 4096, 2048, F, 8, 128, 1024, F, F, BIG, None, None),
    "importance": lambda L: L.iq_imatrix_importance(F, F, 4, 2048, 1e-6, F, None, None),
    "merge": lambda L: L.iq_imatrix_merge(F, F, 4, 2048, ctypes.c_void_p(0x900000), ctypes.c_void_p(0xA00000),
                                          None, None),
    "decode": lambda L: L.iq_dequantize(3, F, 64, 512, F, F, 1, None),
}
LAUNCHES = {"quantize": 3, "quantize_fixed": 3, "every_choice": 3, "choice_search": 5, "hessian_dense": 2,
            "hessian_routed": 6, "importance": 1, "merge": 1, "decode": 1}


@pytest.mark.parametrize("name", sorted(CALLS))
def test_first_failed_launch_stops_the_call(stubbed, name):
    n = run_failing(stubbed, lambda: CALLS[name](stubbed))
    if name in LAUNCHES:
        assert n == LAUNCHES[name]
    if name == "collect_dense":        # 69 chunks in windows of 1,024: one window
        assert n == 2
    if name == "collect_routed":       # 20 chunks in windows of 8: route, slices, combine each
        assert n == 9


def test_timed_quantize_records_both_events_around_the_search(stubbed):
    L = stubbed
    L.stub_reset(0)
    assert L.iq_quantize_timed(0, F, 1, 64, 256, 64, F, F, None, F, F, BIG, None, F, F, None) == 0
    assert L.stub_launches() == 3 and L.stub_events() == 2
    L.stub_reset(3)                    # the search launch fails: its stop event is not recorded
    assert L.iq_quantize_timed(0, F, 1, 64, 256, 64, F, F, None, F, F, BIG, None, F, F, None) == -6
    assert L.stub_events() == 1
    L.stub_reset(0)
    assert L.iq_quantize_timed(0, F, 1, 64, 256, 64, F, F, None, F, F, BIG, None, None, F, None) == -3
    assert L.stub_launches() == 0


def test_host_rejections_launch_nothing(stubbed, api):
    L = stubbed
    need = ctypes.c_size_t()
    assert L.iq_quantize_workspace_size(1, 200, 512, 200, 1, ctypes.byref(need)) == 0
    cases = [
        lambda: L.iq_quantize(1, F, 1, 200, 512, 200, F, F, None, F, None, BIG, None, None),            # no workspace
        lambda: L.iq_quantize(1, F, 1, 200, 512, 200, F, F, None, F, F, need.value - 1, None, None),    # too small
        lambda: L.iq_quantize(1, F, 1, 200, 300, 200, F, F, None, F, F, BIG, None, None),               # shape
        lambda: L.iq_choice_search(2, F, 1, 130, 512, 65, F, F, F, -1.0, F, F, F, BIG, None, None),     # damping
        lambda: L.iq_imatrix_collect(F, 1, 70000, 2048, None, 0, 1, 1024, F, F, F, 16, None, None),     # too small
        lambda: L.iq_hessian_collect(F, 1, 4096, 2048, F, 8, 128, 1024, F, None, BIG, None, None),      # no workspace
    ]
    codes = []
    for c in cases:
        L.stub_reset(0)
        codes.append(c())
        assert L.stub_launches() == 0
    assert codes == [-3, -7, -4, -5, -7, -3]
    # a workspace of exactly the queried size is accepted
    L.stub_reset(0)
    assert L.iq_quantize(1, F, 1, 200, 512, 200, F, F, None, F, F, need.value, None, None) == 0
