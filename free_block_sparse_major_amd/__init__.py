"""MI355X-native SparsePR attention call: thin Python binding of libsparsepr.

The five ABI calls keep their C names and only marshal arguments (torch
tensors -> device pointers, current HIP stream); every step of the path runs
in the HIP kernels of libsparsepr.so.  There is no CPU fallback: importing
works without a GPU, but every call raises if the library is missing.

`SparsePRCall` allocates the per-call buffers once (torch device memory) and
chains the five calls; probe fitting runs on a side stream concurrently with
the sparse attention, joined before the correction.
"""
from __future__ import annotations

import ctypes
import math
import os
from fractions import Fraction

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparsepr.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
BF16, F32 = 0, 1
(CALL_PARTITION_LAYOUT, CALL_ROUTE_CELLS, CALL_SPARSE_ATTN, CALL_PROBE_FIT, CALL_CORRECT,
 CALL_RCP_PARTITION, CALL_PROBE_FIT_EX, CALL_ROUTE_CELLS_EX, CALL_SPARSE_ATTN_CORRECT) = range(9)
ROUTE_GLOBAL, ROUTE_PER_GROUP = range(2)
ROUTE_RULES = {"global": ROUTE_GLOBAL, "per_group": ROUTE_PER_GROUP}
EST_FULL, EST_MEAN, EST_SCALAR, EST_DIAGONAL = range(4)
ESTIMATORS = {"full": EST_FULL, "mean": EST_MEAN, "scalar": EST_SCALAR, "diagonal": EST_DIAGONAL}
EXPORTED = (
    "sparsepr_partition_layout", "sparsepr_route_cells", "sparsepr_sparse_attn",
    "sparsepr_probe_fit", "sparsepr_correct", "sparsepr_workspace_bytes",
    "sparsepr_status_string", "sparsepr_version", "sparsepr_rcp_partition",
    "sparsepr_probe_fit_ex", "sparsepr_correct_ex", "sparsepr_route_cells_ex",
    "sparsepr_rcp_partition_ex", "sparsepr_debug_check", "sparsepr_sparse_attn_noalloc",
    "sparsepr_sparse_attn_correct", "sparsepr_probe_select", "sparsepr_probe_fit_selected",
)


class Dims(ctypes.Structure):
    _fields_ = [
        ("heads", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_k", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("c_q", ctypes.c_int32),
        ("c_k", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("q_stride_head", ctypes.c_int64), ("q_stride_tok", ctypes.c_int64),
        ("kv_stride_head", ctypes.c_int64), ("kv_stride_tok", ctypes.c_int64),
    ]


class SparsePRError(RuntimeError):
    pass


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libsparsepr.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise SparsePRError(f"{path} is missing: build it with `python -m "
                            "free_block_sparse_major_amd.build` (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double
    DP = ctypes.POINTER(Dims)
    lib.sparsepr_workspace_bytes.argtypes = [I32, DP, I32, I32]
    lib.sparsepr_workspace_bytes.restype = SZ
    lib.sparsepr_status_string.argtypes = [I32]
    lib.sparsepr_status_string.restype = ctypes.c_char_p
    lib.sparsepr_version.argtypes = []
    lib.sparsepr_version.restype = I32
    lib.sparsepr_partition_layout.argtypes = [DP] + [P] * 15 + [P, SZ, P]
    lib.sparsepr_partition_layout.restype = I32
    lib.sparsepr_route_cells.argtypes = [DP, P, P, P, P, I64, P, P, P, P, SZ, P]
    lib.sparsepr_route_cells.restype = I32
    lib.sparsepr_sparse_attn.argtypes = [DP, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, SZ, P]
    lib.sparsepr_sparse_attn.restype = I32
    lib.sparsepr_sparse_attn_noalloc.argtypes = [DP, P, P, P, P, P, P, P, P, ctypes.c_float, P,
                                                 P, P]
    lib.sparsepr_sparse_attn_noalloc.restype = I32
    # dims, m, rank, offsets_q, offsets_kv, cell_rowptr, cell_col, q_g, k_g, v_g, v_shift,
    # scale, perm_q, probe_tokens, o_probe_dense, corr_a, corr_psi_t, corr_c, corr_g, out,
    # out_dtype, out_stride_head, out_stride_tok, lse, ws, ws_bytes, stream
    lib.sparsepr_sparse_attn_correct.argtypes = ([DP, I32, I32] + [P] * 8 + [ctypes.c_float]
                                                 + [P] * 8 + [I32, I64, I64, P, P, SZ, P])
    lib.sparsepr_sparse_attn_correct.restype = I32
    lib.sparsepr_probe_fit.argtypes = ([DP, I32, I32, D] + [P] * 10 + [ctypes.c_float] + [P] * 7
                                       + [P, SZ, P])
    lib.sparsepr_probe_fit.restype = I32
    lib.sparsepr_correct.argtypes = [DP, I32, I32] + [P] * 8 + [I32, I64, I64, P, SZ, P]
    lib.sparsepr_correct.restype = I32
    lib.sparsepr_rcp_partition.argtypes = [DP, I32, I32, I32, I32] + [P] * 8 + [P, SZ, P]
    lib.sparsepr_rcp_partition.restype = I32
    lib.sparsepr_probe_fit_ex.argtypes = ([DP, I32, I32, D, I32] + [P] * 7 + [I32] + [P] * 4
                                          + [ctypes.c_float] + [P] * 8 + [P, SZ, P])
    lib.sparsepr_probe_fit_ex.restype = I32
    lib.sparsepr_probe_select.argtypes = [DP, I32] + [P] * 4 + [I32] + [P] * 3 + [P, SZ, P]
    lib.sparsepr_probe_select.restype = I32
    lib.sparsepr_probe_fit_selected.argtypes = ([DP, I32, I32, D, I32] + [P] * 8
                                                + [ctypes.c_float] + [P] * 7 + [P, SZ, P])
    lib.sparsepr_probe_fit_selected.restype = I32
    lib.sparsepr_correct_ex.argtypes = [DP, I32, I32] + [P] * 9 + [I32, I64, I64, P, SZ, P]
    lib.sparsepr_correct_ex.restype = I32
    lib.sparsepr_route_cells_ex.argtypes = [DP, I32, P, P, P, P, I64, P, P, P, P, SZ, P]
    lib.sparsepr_route_cells_ex.restype = I32
    # dims, m_s, r_k, r_q, iters, warm, q, k, init_q, init_k, basis_q, basis_k, cent_q, cent_k,
    # labels_q, labels_kv, phi_q, phi_k, ws, ws_bytes, stream
    lib.sparsepr_rcp_partition_ex.argtypes = [DP, I32, I32, I32, I32, I32] + [P] * 12 + [P, SZ, P]
    lib.sparsepr_rcp_partition_ex.restype = I32
    # dims, m, labels_q, labels_kv, offsets_q, offsets_kv, perm_q, perm_kv, cell_rowptr,
    # cell_col, routed_pairs, probe_rows, probe_tokens, error_word, stream
    lib.sparsepr_debug_check.argtypes = [DP, I32] + [P] * 12 + [P]
    lib.sparsepr_debug_check.restype = I32
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, name):
    if status != OK:
        msg = load_library().sparsepr_status_string(status).decode()
        raise SparsePRError(f"{name}: {msg} (status {status})")


def make_dims(heads, n_q, n_k, head_dim, dtype, c_q, c_k, q_strides=None, kv_strides=None):
    """q_strides / kv_strides: (stride_head, stride_tok) in elements; default [H][N][d]."""
    qs = q_strides or (n_q * head_dim, head_dim)
    ks = kv_strides or (n_k * head_dim, head_dim)
    return Dims(heads, n_q, n_k, head_dim, dtype, c_q, c_k, 0, qs[0], qs[1], ks[0], ks[1])


def workspace_bytes(which, dims, m=64, rank=16):
    return int(load_library().sparsepr_workspace_bytes(which, ctypes.byref(dims), m, rank))


def sparsepr_version():
    return int(load_library().sparsepr_version())


# ----------------------------------------------------------------------------
# the five ABI calls (argument marshalling only)
# ----------------------------------------------------------------------------

def sparsepr_partition_layout(dims, labels_q, labels_kv, q, k, v, perm_q, offsets_q, perm_kv,
                              offsets_kv, q_g, k_g, v_g, v_shift, centroid_q, centroid_k, ws,
                              stream=None):
    st = load_library().sparsepr_partition_layout(
        ctypes.byref(dims), _ptr(labels_q), _ptr(labels_kv), _ptr(q), _ptr(k), _ptr(v),
        _ptr(perm_q), _ptr(offsets_q), _ptr(perm_kv), _ptr(offsets_kv), _ptr(q_g), _ptr(k_g),
        _ptr(v_g), _ptr(v_shift), _ptr(centroid_q), _ptr(centroid_k), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st, "sparsepr_partition_layout")


def sparsepr_route_cells(dims, offsets_q, offsets_kv, centroid_q, centroid_k, budget, cell_rowptr,
                         cell_col, routed_pairs, ws, stream=None):
    st = load_library().sparsepr_route_cells(
        ctypes.byref(dims), _ptr(offsets_q), _ptr(offsets_kv), _ptr(centroid_q), _ptr(centroid_k),
        int(budget), _ptr(cell_rowptr), _ptr(cell_col), _ptr(routed_pairs), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st, "sparsepr_route_cells")


def sparsepr_route_cells_ex(dims, rule, offsets_q, offsets_kv, centroid_q, centroid_k, budget,
                            cell_rowptr, cell_col, routed_pairs, ws, stream=None):
    st = load_library().sparsepr_route_cells_ex(
        ctypes.byref(dims), int(rule), _ptr(offsets_q), _ptr(offsets_kv), _ptr(centroid_q),
        _ptr(centroid_k), int(budget), _ptr(cell_rowptr), _ptr(cell_col), _ptr(routed_pairs),
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st, "sparsepr_route_cells_ex")


def sparsepr_sparse_attn(dims, offsets_q, offsets_kv, cell_rowptr, cell_col, q_g, k_g, v_g,
                         v_shift, softmax_scale, o_sp, lse, ws, stream=None):
    st = load_library().sparsepr_sparse_attn(
        ctypes.byref(dims), _ptr(offsets_q), _ptr(offsets_kv), _ptr(cell_rowptr), _ptr(cell_col),
        _ptr(q_g), _ptr(k_g), _ptr(v_g), _ptr(v_shift), ctypes.c_float(softmax_scale), _ptr(o_sp), _ptr(lse),
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st, "sparsepr_sparse_attn")


def sparsepr_sparse_attn_noalloc(dims, offsets_q, offsets_kv, cell_rowptr, cell_col, q_g, k_g,
                                 v_g, v_shift, softmax_scale, o_sp, lse, stream=None):
    st = load_library().sparsepr_sparse_attn_noalloc(
        ctypes.byref(dims), _ptr(offsets_q), _ptr(offsets_kv), _ptr(cell_rowptr), _ptr(cell_col),
        _ptr(q_g), _ptr(k_g), _ptr(v_g), _ptr(v_shift), ctypes.c_float(softmax_scale),
        _ptr(o_sp), _ptr(lse), _stream(stream))
    _check(st, "sparsepr_sparse_attn_noalloc")


def sparsepr_sparse_attn_correct(dims, m, rank, offsets_q, offsets_kv, cell_rowptr, cell_col,
                                 q_g, k_g, v_g, v_shift, softmax_scale, perm_q, probe_tokens,
                                 o_probe_dense, corr_a, corr_psi_t, corr_c, corr_g, out,
                                 out_dtype, out_stride_head, out_stride_tok, lse, ws,
                                 stream=None):
    st = load_library().sparsepr_sparse_attn_correct(
        ctypes.byref(dims), int(m), int(rank), _ptr(offsets_q), _ptr(offsets_kv),
        _ptr(cell_rowptr), _ptr(cell_col), _ptr(q_g), _ptr(k_g), _ptr(v_g), _ptr(v_shift),
        ctypes.c_float(softmax_scale), _ptr(perm_q), _ptr(probe_tokens), _ptr(o_probe_dense),
        _ptr(corr_a), _ptr(corr_psi_t), _ptr(corr_c), _ptr(corr_g), _ptr(out), int(out_dtype),
        int(out_stride_head), int(out_stride_tok), _ptr(lse), _ptr(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st, "sparsepr_sparse_attn_correct")


def sparsepr_probe_fit(dims, m, rank, lam, offsets_q, offsets_kv, perm_q, cell_rowptr, cell_col,
                       centroid_q, q_g, k_g, v_g, v_shift, softmax_scale, probe_rows, probe_tokens,
                       o_probe_dense, o_probe_sparse, corr_a, corr_psi_t, corr_c, ws, stream=None):
    st = load_library().sparsepr_probe_fit(
        ctypes.byref(dims), int(m), int(rank), float(lam), _ptr(offsets_q), _ptr(offsets_kv),
        _ptr(perm_q), _ptr(cell_rowptr), _ptr(cell_col), _ptr(centroid_q), _ptr(q_g), _ptr(k_g),
        _ptr(v_g), _ptr(v_shift), ctypes.c_float(softmax_scale), _ptr(probe_rows), _ptr(probe_tokens),
        _ptr(o_probe_dense), _ptr(o_probe_sparse), _ptr(corr_a), _ptr(corr_psi_t), _ptr(corr_c),
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st, "sparsepr_probe_fit")


def sparsepr_correct(dims, m, rank, perm_q, o_sp, probe_tokens, o_probe_dense, corr_a, corr_psi_t,
                     corr_c, out, out_dtype, out_stride_head, out_stride_tok, stream=None):
    st = load_library().sparsepr_correct(
        ctypes.byref(dims), int(m), int(rank), _ptr(perm_q), _ptr(o_sp), _ptr(probe_tokens),
        _ptr(o_probe_dense), _ptr(corr_a), _ptr(corr_psi_t), _ptr(corr_c), _ptr(out),
        int(out_dtype), int(out_stride_head), int(out_stride_tok), None, 0, _stream(stream))
    _check(st, "sparsepr_correct")


def sparsepr_rcp_partition(dims, m_s, r_k, r_q, iters, q, k, init_q, init_k, labels_q,
                           labels_kv, phi_q, phi_k, ws, stream=None):
    st = load_library().sparsepr_rcp_partition(
        ctypes.byref(dims), int(m_s), int(r_k), int(r_q), int(iters), _ptr(q), _ptr(k),
        _ptr(init_q), _ptr(init_k), _ptr(labels_q), _ptr(labels_kv), _ptr(phi_q), _ptr(phi_k),
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st, "sparsepr_rcp_partition")


def sparsepr_rcp_partition_ex(dims, m_s, r_k, r_q, iters, warm, q, k, init_q, init_k, basis_q,
                              basis_k, cent_q, cent_k, labels_q, labels_kv, phi_q, phi_k, ws,
                              stream=None):
    st = load_library().sparsepr_rcp_partition_ex(
        ctypes.byref(dims), int(m_s), int(r_k), int(r_q), int(iters), int(warm), _ptr(q), _ptr(k),
        _ptr(init_q), _ptr(init_k), _ptr(basis_q), _ptr(basis_k), _ptr(cent_q), _ptr(cent_k),
        _ptr(labels_q), _ptr(labels_kv), _ptr(phi_q), _ptr(phi_k),
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st, "sparsepr_rcp_partition_ex")


def sparsepr_probe_fit_ex(dims, m, rank, lam, estimator, offsets_q, offsets_kv, perm_q,
                          cell_rowptr, cell_col, centroid_q, probe_feat, feat_dim, q_g, k_g, v_g,
                          v_shift, softmax_scale, probe_rows, probe_tokens, o_probe_dense,
                          o_probe_sparse, corr_a, corr_psi_t, corr_c, corr_g, ws, stream=None):
    st = load_library().sparsepr_probe_fit_ex(
        ctypes.byref(dims), int(m), int(rank), float(lam), int(estimator), _ptr(offsets_q),
        _ptr(offsets_kv), _ptr(perm_q), _ptr(cell_rowptr), _ptr(cell_col), _ptr(centroid_q),
        _ptr(probe_feat), int(feat_dim), _ptr(q_g), _ptr(k_g), _ptr(v_g), _ptr(v_shift),
        ctypes.c_float(softmax_scale), _ptr(probe_rows), _ptr(probe_tokens), _ptr(o_probe_dense),
        _ptr(o_probe_sparse), _ptr(corr_a), _ptr(corr_psi_t), _ptr(corr_c), _ptr(corr_g),
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st, "sparsepr_probe_fit_ex")


def sparsepr_probe_select(dims, m, offsets_q, perm_q, centroid_q, probe_feat, feat_dim, q_g,
                          probe_rows, probe_tokens, ws, stream=None):
    st = load_library().sparsepr_probe_select(
        ctypes.byref(dims), int(m), _ptr(offsets_q), _ptr(perm_q), _ptr(centroid_q),
        _ptr(probe_feat), int(feat_dim), _ptr(q_g), _ptr(probe_rows), _ptr(probe_tokens),
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st, "sparsepr_probe_select")


def sparsepr_probe_fit_selected(dims, m, rank, lam, estimator, offsets_q, offsets_kv,
                                cell_rowptr, cell_col, q_g, k_g, v_g, v_shift, softmax_scale,
                                probe_rows, o_probe_dense, o_probe_sparse, corr_a, corr_psi_t,
                                corr_c, corr_g, ws, stream=None):
    st = load_library().sparsepr_probe_fit_selected(
        ctypes.byref(dims), int(m), int(rank), float(lam), int(estimator), _ptr(offsets_q),
        _ptr(offsets_kv), _ptr(cell_rowptr), _ptr(cell_col), _ptr(q_g), _ptr(k_g), _ptr(v_g),
        _ptr(v_shift), ctypes.c_float(softmax_scale), _ptr(probe_rows), _ptr(o_probe_dense),
        _ptr(o_probe_sparse), _ptr(corr_a), _ptr(corr_psi_t), _ptr(corr_c), _ptr(corr_g),
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check(st, "sparsepr_probe_fit_selected")


def sparsepr_correct_ex(dims, m, rank, perm_q, o_sp, probe_tokens, o_probe_dense, corr_a,
                        corr_psi_t, corr_c, corr_g, out, out_dtype, out_stride_head,
                        out_stride_tok, stream=None):
    st = load_library().sparsepr_correct_ex(
        ctypes.byref(dims), int(m), int(rank), _ptr(perm_q), _ptr(o_sp), _ptr(probe_tokens),
        _ptr(o_probe_dense), _ptr(corr_a), _ptr(corr_psi_t), _ptr(corr_c), _ptr(corr_g),
        _ptr(out), int(out_dtype), int(out_stride_head), int(out_stride_tok), None, 0,
        _stream(stream))
    _check(st, "sparsepr_correct_ex")


def sparsepr_debug_check(dims, m, labels_q, labels_kv, offsets_q, offsets_kv, perm_q, perm_kv,
                         cell_rowptr, cell_col, routed_pairs, probe_rows, probe_tokens,
                         error_word, stream=None):
    st = load_library().sparsepr_debug_check(
        ctypes.byref(dims), int(m), _ptr(labels_q), _ptr(labels_kv), _ptr(offsets_q),
        _ptr(offsets_kv), _ptr(perm_q), _ptr(perm_kv), _ptr(cell_rowptr), _ptr(cell_col),
        _ptr(routed_pairs), _ptr(probe_rows), _ptr(probe_tokens), _ptr(error_word),
        _stream(stream))
    _check(st, "sparsepr_debug_check")


DBG_LABELS, DBG_OFFSETS, DBG_PERM, DBG_ROWPTR, DBG_CELLS, DBG_ROUTE, DBG_PROBES = (
    1, 2, 4, 8, 16, 32, 64)


class RcpPartition:
    """Buffers for sparsepr_rcp_partition of one shape: labels_q, labels_kv
    (int32 [H][N]), phi_q (fp32 [H][N_q][r_q]) and optionally phi_k.

    With keep_state=True the partition keeps the state of later calls
    (sparsepr_rcp_partition_ex): the first call starts from init rows, and
    every call after it (warm=True) from the state the previous one left."""

    def __init__(self, heads, n_q, n_k, head_dim, dtype, c_q, c_k, m_s=256, r_k=48, r_q=64,
                 iters=10, device="cuda", q_strides=None, kv_strides=None, keep_phi_k=False,
                 keep_state=False):
        load_library()
        self.dims = make_dims(heads, n_q, n_k, head_dim, dtype, c_q, c_k, q_strides, kv_strides)
        self.m_s, self.r_k, self.r_q, self.iters = m_s, r_k, r_q, iters
        dev = torch.device(device)
        self.labels_q = torch.empty(heads, n_q, dtype=torch.int32, device=dev)
        self.labels_kv = torch.empty(heads, n_k, dtype=torch.int32, device=dev)
        self.phi_q = torch.empty(heads, n_q, r_q, dtype=torch.float32, device=dev)
        self.phi_k = (torch.empty(heads, n_k, r_k, dtype=torch.float32, device=dev)
                      if keep_phi_k else None)
        nb = workspace_bytes(CALL_RCP_PARTITION, self.dims)
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.keep_state = keep_state
        self.has_state = False
        if keep_state:
            f32 = torch.float32
            self.basis_q = torch.empty(heads, head_dim, r_q, dtype=f32, device=dev)
            self.basis_k = torch.empty(heads, head_dim, r_k, dtype=f32, device=dev)
            self.cent_q = torch.empty(heads, c_q, head_dim, dtype=f32, device=dev)
            self.cent_k = torch.empty(heads, c_k, head_dim, dtype=f32, device=dev)

    def __call__(self, q, k, init_q=None, init_k=None, warm=False, iters=None, stream=None):
        iters = self.iters if iters is None else iters
        if not self.keep_state:
            if warm:
                raise ValueError("warm calls need keep_state=True")
            sparsepr_rcp_partition(self.dims, self.m_s, self.r_k, self.r_q, iters, q, k, init_q,
                                   init_k, self.labels_q, self.labels_kv, self.phi_q, self.phi_k,
                                   self.ws, stream)
            return self.labels_q, self.labels_kv
        if warm and not self.has_state:
            raise ValueError("a warm call needs the state of an earlier call")
        sparsepr_rcp_partition_ex(self.dims, self.m_s, self.r_k, self.r_q, iters, int(warm), q, k,
                                  init_q, init_k, self.basis_q, self.basis_k, self.cent_q,
                                  self.cent_k, self.labels_q, self.labels_kv, self.phi_q,
                                  self.phi_k, self.ws, stream)
        self.has_state = True
        return self.labels_q, self.labels_kv


# ----------------------------------------------------------------------------
# budget (host, exact rational) and the chained call
# ----------------------------------------------------------------------------

def routed_pair_budget(rho, n_q, n_k, m):
    """ceil((rho*N_q - M_eff)*N_k), clamped at 0 (probe cost reserved)."""
    m_eff = min(m, n_q)
    return max(0, math.ceil((Fraction(rho) * n_q - m_eff) * n_k))


def key_token_budget(rho, n_q, n_k, m):
    """Key tokens per query of the per-group rule: ceil((rho*N_q - M_eff)*N_k/N_q), >= 0."""
    m_eff = min(m, n_q)
    return max(0, math.ceil((Fraction(rho) * n_q - m_eff) * n_k / n_q))


class _HeadOffset:
    """A device address `h0` heads into a tensor with the given head stride
    (elements); passed to the ABI like a tensor."""

    def __init__(self, t, h0, stride_head):
        self._p = t.data_ptr() + int(h0) * int(stride_head) * t.element_size()

    def data_ptr(self):
        return self._p


_PER_HEAD = ("perm_q", "perm_kv", "offsets_q", "offsets_kv", "q_g", "k_g", "v_g", "v_shift",
             "centroid_q", "centroid_k", "cell_rowptr", "cell_col", "routed_pairs", "o_sp", "lse",
             "probe_rows", "probe_tokens", "o_probe_dense", "o_probe_sparse", "corr_a",
             "corr_psi_t", "corr_c", "corr_g", "out")


class _Heads:
    """Heads h0..h1 of a call: their dims, views of the call's buffers and a
    workspace set."""

    def __init__(self, call, h0, h1, ws):
        self.h0, self.h1 = h0, h1
        d = call.dims
        self.dims = Dims(h1 - h0, d.n_q, d.n_k, d.head_dim, d.dtype, d.c_q, d.c_k, 0,
                         d.q_stride_head, d.q_stride_tok, d.kv_stride_head, d.kv_stride_tok)
        for name in _PER_HEAD:
            setattr(self, name, getattr(call, name)[h0:h1])
        self.ws_layout, self.ws_route, self.ws_attn, self.ws_probe = ws[:4]
        self.ws_attn_correct = ws[4] if len(ws) > 4 else None


class SparsePRCall:
    """Device buffers and stream plumbing for repeated calls of one shape.

    Inputs are torch tensors on the GPU: q [H][N_q][d], k, v [H][N_k][d]
    (bf16 or f32, or any layout with contiguous last dim given via strides),
    labels int32 [H][N].  Outputs stay resident on the device.

    head_chunks > 1 (or a list of head counts) splits a call into that many
    ranges of heads, issued on
    two alternating streams (with the probe fits on a third), so that the
    layout and routing of one range run while the attention of the previous
    one does; every head is computed exactly as in a whole call.

    fused=True runs the probe-first order: the probe fit before the attention,
    and the attention writes the corrected output in token order
    (sparsepr_sparse_attn_correct), so O_sp is neither stored nor read.
    lead_unfused=True (fused order over head ranges, overlap on) lets the
    first range attend as soon as it is routed, storing O_sp, and take the
    correction kernel once its fit is done, so that fit runs beside the
    attention instead of in front of it."""

    def __init__(self, heads, n_q, n_k, head_dim, dtype, c_q, c_k, m=64, rank=16, lam=0.1,
                 rho="0.26", budget=None, out_dtype=F32, device="cuda", q_strides=None,
                 kv_strides=None, overlap=True, feat_dim=0, estimator="full",
                 route_rule="global", head_chunks=1, fused=False, lead_unfused=False):
        load_library()
        self.dims = make_dims(heads, n_q, n_k, head_dim, dtype, c_q, c_k, q_strides, kv_strides)
        self.m, self.rank, self.lam = m, rank, lam
        self.route_rule = ROUTE_RULES[route_rule]
        if budget is not None:
            self.budget = int(budget)
        elif self.route_rule == ROUTE_GLOBAL:
            self.budget = routed_pair_budget(rho, n_q, n_k, m)
        else:
            self.budget = key_token_budget(rho, n_q, n_k, m)
        self.scale = 1.0 / math.sqrt(head_dim)
        self.out_dtype = out_dtype
        self.overlap = overlap
        # probe features (response-coupled partitions): set self.probe_feat to
        # an fp32 [H][N_q][feat_dim] tensor before the call
        self.feat_dim = int(feat_dim)
        self.probe_feat = None
        # residual estimator (full ridge with projection, or mean / scalar / diagonal)
        self.estimator = ESTIMATORS[estimator]
        H, d = heads, head_dim
        dev = torch.device(device)
        tdt = torch.bfloat16 if dtype == BF16 else torch.float32
        i32 = dict(dtype=torch.int32, device=dev)
        self.perm_q = torch.empty(H, n_q, **i32)
        self.perm_kv = torch.empty(H, n_k, **i32)
        self.offsets_q = torch.empty(H, c_q + 1, **i32)
        self.offsets_kv = torch.empty(H, c_k + 1, **i32)
        self.q_g = torch.empty(H, n_q, d, dtype=tdt, device=dev)
        self.k_g = torch.empty(H, n_k, d, dtype=tdt, device=dev)
        vdt = torch.float16 if dtype == BF16 else torch.float32
        self.v_g = torch.empty(H, n_k, d, dtype=vdt, device=dev)
        self.v_shift = torch.empty(H, dtype=torch.int32, device=dev)
        self.centroid_q = torch.empty(H, c_q, d, dtype=torch.float64, device=dev)
        self.centroid_k = torch.empty(H, c_k, d, dtype=torch.float64, device=dev)
        self.cell_rowptr = torch.empty(H, c_q + 1, **i32)
        self.cell_col = torch.empty(H, c_q * c_k, **i32)
        self.routed_pairs = torch.empty(H, dtype=torch.int64, device=dev)
        self.o_sp = torch.empty(H, n_q, d, dtype=torch.float32, device=dev)
        self.lse = torch.empty(H, n_q, dtype=torch.float32, device=dev)
        self.probe_rows = torch.empty(H, m, **i32)
        self.probe_tokens = torch.empty(H, m, **i32)
        self.o_probe_dense = torch.empty(H, m, d, dtype=torch.float32, device=dev)
        self.o_probe_sparse = torch.empty(H, m, d, dtype=torch.float32, device=dev)
        self.corr_a = torch.empty(H, d, max(rank, 1), dtype=torch.float32, device=dev)
        self.corr_psi_t = torch.empty(H, max(rank, 1), d, dtype=torch.float32, device=dev)
        self.corr_c = torch.empty(H, d, dtype=torch.float32, device=dev)
        self.corr_g = torch.zeros(H, d, dtype=torch.float32, device=dev)
        odt = torch.bfloat16 if out_dtype == BF16 else torch.float32
        self.out = torch.empty(H, n_q, d, dtype=odt, device=dev)
        self._ex = bool(feat_dim) or self.estimator != EST_FULL

        self.fused = bool(fused)
        # fused order over head ranges: the first range instead attends as soon
        # as it is routed and takes the correction kernel once its fit is done
        self.lead_unfused = bool(lead_unfused) and self.fused and overlap

        def ws_set(dims):
            def ws(which):
                nb = workspace_bytes(which, dims, m, rank)
                return torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
            wss = (ws(CALL_PARTITION_LAYOUT),
                   ws(CALL_ROUTE_CELLS if self.route_rule == ROUTE_GLOBAL else CALL_ROUTE_CELLS_EX),
                   ws(CALL_SPARSE_ATTN),
                   ws(CALL_PROBE_FIT_EX if self._ex else CALL_PROBE_FIT))
            if self.fused:
                wss += (ws(CALL_SPARSE_ATTN_CORRECT),)
            return wss

        self._whole = _Heads(self, 0, H, ws_set(self.dims))
        self.ws_attn_correct = self._whole.ws_attn_correct
        self.ws_layout, self.ws_route, self.ws_attn, self.ws_probe = (
            self._whole.ws_layout, self._whole.ws_route, self._whole.ws_attn, self._whole.ws_probe)
        self.side = torch.cuda.Stream(device=dev) if overlap else None
        self.ev_laid = torch.cuda.Event()
        self.ev_routed = torch.cuda.Event()
        self.ev_fit = torch.cuda.Event()
        # head ranges of a chunked call: two workspace sets, used alternately
        self.chunks = None
        if isinstance(head_chunks, (list, tuple)):
            # explicit head counts per range, in order
            sizes = [int(x) for x in head_chunks]
            if any(x < 1 for x in sizes) or sum(sizes) != H:
                raise ValueError("head_chunks counts must be positive and sum to the heads")
            k = len(sizes)
            bounds = [0]
            for x in sizes:
                bounds.append(bounds[-1] + x)
        else:
            k = max(1, min(int(head_chunks), H))
            bounds = [H * i // k for i in range(k + 1)]
        if k > 1:
            hc = max(b - a for a, b in zip(bounds, bounds[1:]))
            cdims = make_dims(hc, n_q, n_k, head_dim, dtype, c_q, c_k, q_strides, kv_strides)
            sets = (ws_set(cdims), ws_set(cdims))
            self.chunks = [_Heads(self, a, b, sets[i % 2])
                           for i, (a, b) in enumerate(zip(bounds, bounds[1:]))]
            self.stream_b = torch.cuda.Stream(device=dev)
            self.ev_start = torch.cuda.Event()
            self.ev_b_done = torch.cuda.Event()
            self.ev_laid_c = [torch.cuda.Event() for _ in self.chunks]
            self.ev_routed_c = [torch.cuda.Event() for _ in self.chunks]
            self.ev_fit_c = [torch.cuda.Event() for _ in self.chunks]

    # individual stages (all heads, or the head range `part`) ---------------
    def layout(self, labels_q, labels_kv, q, k, v, stream=None, part=None):
        p = part or self._whole
        d = self.dims
        sparsepr_partition_layout(p.dims, labels_q[p.h0:p.h1], labels_kv[p.h0:p.h1],
                                  _HeadOffset(q, p.h0, d.q_stride_head),
                                  _HeadOffset(k, p.h0, d.kv_stride_head),
                                  _HeadOffset(v, p.h0, d.kv_stride_head), p.perm_q,
                                  p.offsets_q, p.perm_kv, p.offsets_kv, p.q_g,
                                  p.k_g, p.v_g, p.v_shift, p.centroid_q,
                                  p.centroid_k,
                                  p.ws_layout, stream)

    def route(self, stream=None, part=None):
        p = part or self._whole
        if self.route_rule != ROUTE_GLOBAL:
            sparsepr_route_cells_ex(p.dims, self.route_rule, p.offsets_q, p.offsets_kv,
                                    p.centroid_q, p.centroid_k, self.budget,
                                    p.cell_rowptr, p.cell_col, p.routed_pairs,
                                    p.ws_route, stream)
            return
        sparsepr_route_cells(p.dims, p.offsets_q, p.offsets_kv, p.centroid_q,
                             p.centroid_k, self.budget, p.cell_rowptr, p.cell_col,
                             p.routed_pairs, p.ws_route, stream)

    def attend(self, stream=None, part=None):
        p = part or self._whole
        sparsepr_sparse_attn(p.dims, p.offsets_q, p.offsets_kv, p.cell_rowptr,
                             p.cell_col, p.q_g, p.k_g, p.v_g, p.v_shift,
                             self.scale, p.o_sp,
                             p.lse, p.ws_attn, stream)

    def probe_fit(self, stream=None, part=None):
        p = part or self._whole
        if self._ex:
            if self.feat_dim and self.probe_feat is None:
                raise SparsePRError("probe_feat is not set")
            feat = self.probe_feat[p.h0:p.h1] if self.feat_dim else None
            sparsepr_probe_fit_ex(p.dims, self.m, self.rank, self.lam, self.estimator,
                                  p.offsets_q, p.offsets_kv, p.perm_q, p.cell_rowptr,
                                  p.cell_col, p.centroid_q, feat, self.feat_dim,
                                  p.q_g, p.k_g, p.v_g, p.v_shift, self.scale,
                                  p.probe_rows, p.probe_tokens, p.o_probe_dense,
                                  p.o_probe_sparse, p.corr_a, p.corr_psi_t, p.corr_c,
                                  p.corr_g, p.ws_probe, stream)
            return
        sparsepr_probe_fit(p.dims, self.m, self.rank, self.lam, p.offsets_q,
                           p.offsets_kv, p.perm_q, p.cell_rowptr, p.cell_col,
                           p.centroid_q, p.q_g, p.k_g, p.v_g, p.v_shift,
                           self.scale,
                           p.probe_rows, p.probe_tokens, p.o_probe_dense,
                           p.o_probe_sparse, p.corr_a, p.corr_psi_t, p.corr_c,
                           p.ws_probe, stream)

    def probe_select(self, stream=None, part=None):
        """The probe selection alone (reads only the layout's outputs)."""
        p = part or self._whole
        if self.feat_dim and self.probe_feat is None:
            raise SparsePRError("probe_feat is not set")
        feat = self.probe_feat[p.h0:p.h1] if self.feat_dim else None
        sparsepr_probe_select(p.dims, self.m, p.offsets_q, p.perm_q, p.centroid_q, feat,
                              self.feat_dim, p.q_g, p.probe_rows, p.probe_tokens, p.ws_probe,
                              stream)

    def probe_fit_selected(self, stream=None, part=None):
        """Exact probe rows, merge and fit for the probes probe_select chose."""
        p = part or self._whole
        sparsepr_probe_fit_selected(p.dims, self.m, self.rank, self.lam, self.estimator,
                                    p.offsets_q, p.offsets_kv, p.cell_rowptr, p.cell_col,
                                    p.q_g, p.k_g, p.v_g, p.v_shift, self.scale, p.probe_rows,
                                    p.o_probe_dense, p.o_probe_sparse, p.corr_a, p.corr_psi_t,
                                    p.corr_c, p.corr_g if self.estimator != EST_FULL else None,
                                    p.ws_probe, stream)

    def correct(self, stream=None, part=None):
        p = part or self._whole
        if self.estimator != EST_FULL:
            sparsepr_correct_ex(p.dims, self.m, self.rank, p.perm_q, p.o_sp,
                                p.probe_tokens, p.o_probe_dense, p.corr_a,
                                p.corr_psi_t, p.corr_c, p.corr_g, p.out,
                                self.out_dtype, p.out.stride(0), p.out.stride(1), stream)
            return
        sparsepr_correct(p.dims, self.m, self.rank, p.perm_q, p.o_sp, p.probe_tokens,
                         p.o_probe_dense, p.corr_a, p.corr_psi_t, p.corr_c, p.out,
                         self.out_dtype, p.out.stride(0), p.out.stride(1), stream)

    def attend_correct(self, stream=None, part=None):
        """The attention with the correction in its epilogue (fused order)."""
        p = part or self._whole
        sparsepr_sparse_attn_correct(p.dims, self.m, self.rank, p.offsets_q, p.offsets_kv,
                                     p.cell_rowptr, p.cell_col, p.q_g, p.k_g, p.v_g, p.v_shift,
                                     self.scale, p.perm_q, p.probe_tokens, p.o_probe_dense,
                                     p.corr_a, p.corr_psi_t, p.corr_c,
                                     p.corr_g if self.estimator != EST_FULL else None, p.out,
                                     self.out_dtype, p.out.stride(0), p.out.stride(1), p.lse,
                                     p.ws_attn_correct, stream)

    def __call__(self, labels_q, labels_kv, q, k, v):
        """One whole attention call on the current stream.  With overlap on,
        the probe selection runs on the side stream while the cells are
        routed, and the rest of the probe fit beside the attention (usual
        order) or before it (fused order).  Returns the output tensor."""
        if self.chunks is not None:
            if self.fused:
                return self._chunked_fused(labels_q, labels_kv, q, k, v)
            return self._chunked(labels_q, labels_kv, q, k, v)
        main = torch.cuda.current_stream()
        self.layout(labels_q, labels_kv, q, k, v)
        if self.side is None:
            self.route()
            if self.fused:
                self.probe_fit()
                self.attend_correct()
                return self.out
            self.attend()
            self.probe_fit()
            self.correct()
            return self.out
        # the probe selection runs on the side stream while the cells are
        # routed; the rest of the fit once the routing is done
        self.ev_laid.record(main)
        self.side.wait_event(self.ev_laid)
        self.probe_select(self.side)
        self.route()
        self.ev_routed.record(main)
        self.side.wait_event(self.ev_routed)
        self.probe_fit_selected(self.side)
        self.ev_fit.record(self.side)
        if self.fused:
            main.wait_event(self.ev_fit)
            self.attend_correct()
            return self.out
        self.attend()
        main.wait_event(self.ev_fit)
        self.correct()
        return self.out

    def capture(self, labels_q, labels_kv, q, k, v):
        """Records one whole call on these input tensors into a HIP graph
        (torch.cuda.CUDAGraph); `replay()` then reruns it with one launch.
        The library allocates nothing and issues no memset, so every kernel
        of the call is captured; the inputs must stay at the same addresses
        (copy new values into them before a replay)."""
        self(labels_q, labels_kv, q, k, v)   # warm-up outside the capture
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self(labels_q, labels_kv, q, k, v)
        torch.cuda.synchronize()
        return self.graph

    def replay(self):
        """Reruns the captured call (see `capture`); returns the output tensor."""
        self.graph.replay()
        return self.out

    def _chunked_fused(self, labels_q, labels_kv, q, k, v):
        """Fused order over head ranges: layout and routing of every range on
        the current stream, the probe selection of each range on the side
        stream once it is laid out and the rest of its fit once it is routed,
        and the attention with the correction of
        range i on stream_b (even i) or the current stream (odd i) once its
        fit is done.  The fit of range i runs while later ranges are laid out
        and routed or while earlier ranges are attended, and two attention
        launches overlap each other's tails (with lead_unfused, range 0 attends
        once it is routed and is corrected after its fit).  Attention launches
        on one stream share a workspace set; the two streams use different sets."""
        main = torch.cuda.current_stream()
        side = self.side if self.side is not None else main
        self.ev_start.record(main)
        self.stream_b.wait_event(self.ev_start)
        side.wait_event(self.ev_start)
        for i, p in enumerate(self.chunks):
            self.layout(labels_q, labels_kv, q, k, v, stream=main, part=p)
            if side is main:
                self.route(stream=main, part=p)
                self.probe_fit(stream=main, part=p)
            else:
                # selection beside the routing, the rest of the fit after it
                self.ev_laid_c[i].record(main)
                side.wait_event(self.ev_laid_c[i])
                self.probe_select(stream=side, part=p)
                self.route(stream=main, part=p)
                self.ev_routed_c[i].record(main)
                side.wait_event(self.ev_routed_c[i])
                self.probe_fit_selected(stream=side, part=p)
            self.ev_fit_c[i].record(side)
        for i, p in enumerate(self.chunks):
            s = self.stream_b if i % 2 == 0 else main
            if i == 0 and self.lead_unfused and side is not main:
                s.wait_event(self.ev_routed_c[i])
                self.attend(stream=s, part=p)
                s.wait_event(self.ev_fit_c[i])
                self.correct(stream=s, part=p)
                continue
            s.wait_event(self.ev_fit_c[i])
            self.attend_correct(stream=s, part=p)
        self.ev_b_done.record(self.stream_b)
        main.wait_event(self.ev_b_done)
        return self.out

    def _chunked(self, labels_q, labels_kv, q, k, v):
        """Head ranges on the current stream and stream_b in turn.  A range
        reuses the workspace set of the range two before it, which ran on the
        same stream (and whose probe fit ran earlier on the in-order side
        stream), so stream order alone keeps the sets from being shared."""
        main = torch.cuda.current_stream()
        self.ev_start.record(main)
        self.stream_b.wait_event(self.ev_start)
        if self.side is not None:
            self.side.wait_event(self.ev_start)
        for i, p in enumerate(self.chunks):
            s = main if i % 2 == 0 else self.stream_b
            self.layout(labels_q, labels_kv, q, k, v, stream=s, part=p)
            if self.side is not None:
                self.ev_laid_c[i].record(s)
                self.side.wait_event(self.ev_laid_c[i])
                self.probe_select(stream=self.side, part=p)
                self.route(stream=s, part=p)
                self.ev_routed_c[i].record(s)
                self.side.wait_event(self.ev_routed_c[i])
                self.probe_fit_selected(stream=self.side, part=p)
                self.ev_fit_c[i].record(self.side)
                self.attend(stream=s, part=p)
                s.wait_event(self.ev_fit_c[i])
            else:
                self.route(stream=s, part=p)
                self.attend(stream=s, part=p)
                self.probe_fit(stream=s, part=p)
            self.correct(stream=s, part=p)
        self.ev_b_done.record(self.stream_b)
        main.wait_event(self.ev_b_done)
        return self.out
