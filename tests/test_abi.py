"""Host-side checks of the C ABI (no kernel launches): the library loads,
exports every symbol the header declares, validates arguments and sizes its
workspaces.  Runs without a GPU."""
import ctypes
import os
import re

import pytest

import free_block_sparse_major_amd as fb
import synthgen as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparsepr.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sparsepr_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fb.LIB_PATH):
        from free_block_sparse_major_amd.build import build
        build()
    return fb.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(fb.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert fb.sparsepr_version() == 10000
    for s, text in [(0, b"ok"), (1, b"invalid argument"), (2, b"unsupported shape or dtype"),
                    (3, b"workspace too small"), (4, b"HIP launch error")]:
        assert lib.sparsepr_status_string(s) == text
    assert lib.sparsepr_status_string(99) == b"unknown status"


def test_dims_struct_layout():
    assert ctypes.sizeof(fb.Dims) == 8 * 4 + 4 * 8


def test_workspace_sizes(lib):
    for name in ("tiny_fp32", "cogvideox", "wan", "hunyuan"):
        w = sg.workload(name)
        dims = fb.make_dims(w.heads, w.n, w.n, w.head_dim, fb.BF16 if w.dtype == "bf16" else fb.F32,
                            w.c_q, w.c_k)
        for which in range(4):
            nb = fb.workspace_bytes(which, dims, w.m, w.r)
            assert nb > 0
        assert fb.workspace_bytes(fb.CALL_CORRECT, dims) == 0
        # route scratch holds one fp64 score per cell
        assert fb.workspace_bytes(fb.CALL_ROUTE_CELLS, dims) >= 8 * w.heads * w.c_q * w.c_k
    bad = fb.make_dims(1, 100, 100, 96, fb.BF16, 4, 4)
    assert fb.workspace_bytes(fb.CALL_ROUTE_CELLS, bad) == 0
    ok = fb.make_dims(1, 100, 100, 64, fb.BF16, 4, 4)
    assert fb.workspace_bytes(fb.CALL_PROBE_FIT, ok, m=65) == 0
    assert fb.workspace_bytes(fb.CALL_PROBE_FIT, ok, m=64, rank=65) == 0


def _layout_status(lib, dims, null=False, ws_bytes=1 << 30, addr=4096):
    p = ctypes.c_void_p(0 if null else addr)
    args = [p] * 15
    return lib.sparsepr_partition_layout(ctypes.byref(dims), *args, ctypes.c_void_p(4096),
                                         ws_bytes, None)


def test_argument_validation_before_launch(lib):
    """Every rejected call returns before touching the device."""
    good = fb.make_dims(2, 300, 300, 64, fb.BF16, 8, 8)
    assert _layout_status(lib, fb.make_dims(2, 300, 300, 96, fb.BF16, 8, 8)) == fb.ERR_UNSUPPORTED
    assert _layout_status(lib, fb.make_dims(2, 300, 300, 64, 7, 8, 8)) == fb.ERR_UNSUPPORTED
    assert _layout_status(lib, fb.make_dims(2, 300, 300, 64, fb.BF16, 2000, 8)) == fb.ERR_UNSUPPORTED
    assert _layout_status(lib, fb.make_dims(0, 300, 300, 64, fb.BF16, 8, 8)) == fb.ERR_INVALID
    assert _layout_status(lib, fb.make_dims(2, 0, 300, 64, fb.BF16, 8, 8)) == fb.ERR_INVALID
    assert _layout_status(lib, fb.make_dims(2, 300, 300, 64, fb.BF16, 8, 8,
                                            q_strides=(300 * 64, 60))) == fb.ERR_INVALID
    assert _layout_status(lib, good, null=True) == fb.ERR_INVALID
    # q, k, v read in 16-byte chunks: a base 4 bytes past a boundary is refused
    assert _layout_status(lib, good, addr=4100) == fb.ERR_INVALID
    assert _layout_status(lib, good, ws_bytes=16) == fb.ERR_WORKSPACE
    P = ctypes.c_void_p(4096)
    # probe_fit: m out of range, rank out of range, lambda 0 with rank > 0
    for m, rank, lam in [(0, 16, 0.1), (65, 16, 0.1), (64, -1, 0.1), (64, 65, 0.1), (64, 16, 0.0),
                         (64, 16, float("nan"))]:
        st = lib.sparsepr_probe_fit(ctypes.byref(good), m, rank, lam, *([P] * 10),
                                    ctypes.c_float(0.125), *([P] * 7), P, 1 << 30, None)
        assert st == fb.ERR_INVALID, (m, rank, lam)
    # correct: unsupported output dtype, misaligned output stride
    st = lib.sparsepr_correct(ctypes.byref(good), 64, 16, *([P] * 8), 5, 300 * 64, 64, None, 0, None)
    assert st == fb.ERR_UNSUPPORTED
    st = lib.sparsepr_correct(ctypes.byref(good), 64, 16, *([P] * 8), fb.F32, 300 * 64, 65, None, 0,
                              None)
    assert st == fb.ERR_INVALID
    # route: workspace too small
    st = lib.sparsepr_route_cells(ctypes.byref(good), P, P, P, P, 100, P, P, P, P, 8, None)
    assert st == fb.ERR_WORKSPACE
    # partition across calls: warm flag, missing init on a first call, missing
    # state, rank above 64, workspace too small
    def part_ex(warm=0, init=P, state=P, r_k=16, ws_bytes=1 << 30):
        return lib.sparsepr_rcp_partition_ex(ctypes.byref(good), 64, r_k, 16, 2, warm, P, P, init,
                                             init, state, state, state, state, P, P, None, None, P,
                                             ws_bytes, None)
    assert part_ex(warm=2) == fb.ERR_INVALID
    assert part_ex(init=None) == fb.ERR_INVALID
    assert part_ex(state=None) == fb.ERR_INVALID
    assert part_ex(warm=1, state=None) == fb.ERR_INVALID
    assert part_ex(r_k=65) == fb.ERR_INVALID
    assert part_ex(ws_bytes=16) == fb.ERR_WORKSPACE
    # split probe fit: m out of range, a missing centroid (no features), a
    # feature width out of range, a small workspace; the fit half as probe_fit
    def select(m=64, cen=P, feat=None, fd=0, ws_bytes=1 << 30):
        return lib.sparsepr_probe_select(ctypes.byref(good), m, P, P, cen, feat, fd, P, P, P, P,
                                         ws_bytes, None)
    assert select(m=0) == fb.ERR_INVALID
    assert select(m=65) == fb.ERR_INVALID
    assert select(cen=None) == fb.ERR_INVALID
    assert select(cen=None, feat=P, fd=65) == fb.ERR_INVALID
    assert select(ws_bytes=16) == fb.ERR_WORKSPACE
    def fit_sel(m=64, rank=16, lam=0.1, est=fb.EST_FULL, corr_g=None, ws_bytes=1 << 30):
        return lib.sparsepr_probe_fit_selected(ctypes.byref(good), m, rank, lam, est, *([P] * 8),
                                               ctypes.c_float(0.125), *([P] * 6), corr_g, P,
                                               ws_bytes, None)
    for m, rank, lam in [(0, 16, 0.1), (65, 16, 0.1), (64, -1, 0.1), (64, 65, 0.1), (64, 16, 0.0)]:
        assert fit_sel(m, rank, lam) == fb.ERR_INVALID, (m, rank, lam)
    assert fit_sel(est=fb.EST_MEAN) == fb.ERR_INVALID   # corr_g required
    assert fit_sel(est=7) == fb.ERR_INVALID
    assert fit_sel(ws_bytes=16) == fb.ERR_WORKSPACE


def test_debug_check_and_size_limits(lib):
    """The debug check refuses a missing error word, a row-pointer array
    without columns and an m outside 1..64 before launching; shapes whose
    per-head K/V bytes reach 2^32 are refused as unsupported (the bf16 kernels
    address a head through 32-bit buffer offsets)."""
    good = fb.make_dims(2, 300, 300, 64, fb.BF16, 8, 8)
    P = ctypes.c_void_p(4096)
    N = None

    def dbg(m=64, rowptr=P, col=P, err=P, probes=P):
        return lib.sparsepr_debug_check(ctypes.byref(good), m, N, N, N, N, N, N, rowptr, col, N,
                                        probes, N, err, None)
    assert dbg(err=None) == fb.ERR_INVALID
    assert dbg(col=None) == fb.ERR_INVALID
    assert dbg(m=0) == fb.ERR_INVALID
    assert dbg(m=65) == fb.ERR_INVALID
    assert lib.sparsepr_debug_check(ctypes.byref(fb.make_dims(1, 10, 10, 96, fb.BF16, 2, 2)), 1,
                                    *([N] * 11), P, None) == fb.ERR_UNSUPPORTED
    # 2^32 / (128 * 2) = 16777216 keys: the first refused count for bf16, d = 128
    assert _layout_status(lib, fb.make_dims(1, 1000, 16777216, 128, fb.BF16, 8, 8)) == \
        fb.ERR_UNSUPPORTED
    assert fb.workspace_bytes(fb.CALL_SPARSE_ATTN,
                              fb.make_dims(1, 1000, 16777215, 128, fb.BF16, 8, 8)) > 0
    assert _layout_status(lib, fb.make_dims(1, 1000, 8388608, 128, fb.F32, 8, 8)) == \
        fb.ERR_UNSUPPORTED
    assert _layout_status(lib, fb.make_dims(1, 8388608, 1000, 128, fb.BF16, 8, 8)) == \
        fb.ERR_UNSUPPORTED


def test_budget_matches_oracle_closed_form():
    import oracle
    for rho, n, m in [("0.26", 4096, 64), ("0.22", 75600, 64), ("0.26", 118800, 64), ("0.3", 50, 64)]:
        assert fb.routed_pair_budget(rho, n, n, m) == oracle.routed_pair_budget(rho, n, n, m)


def test_product_path_does_not_load_the_oracle():
    """The package (binding and build helper) never imports the CPU oracle:
    every step of a call runs in libsparsepr.so."""
    import subprocess
    import sys
    code = ("import sys; import free_block_sparse_major_amd as fb; "
            "import free_block_sparse_major_amd.build; "
            "print(any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "False"


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, cwd=root, timeout=120)
    assert out.returncode == 2
    assert "one GPU" in out.stderr
