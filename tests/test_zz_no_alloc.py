"""The attention entry point that allocates nothing
(sparsepr_sparse_attn_noalloc) against sparsepr_sparse_attn on the same
inputs: identical kernels, so identical outputs, bit for bit.  Two calls in a
row, the second on a smaller input, so the second reuses the device array
the first one filled."""
import numpy as np
import pytest

import synthgen as sg
from harness import say, upload

pytestmark = pytest.mark.gpu


def _prepared(w):
    """A call run through layout and routing (its attention inputs)."""
    import torch
    import free_block_sparse_major_amd as fb
    data = sg.make_call(w)
    q, k, v, lq, lk = upload(w, data)
    call = fb.SparsePRCall(w.heads, w.n, w.n, w.head_dim,
                           fb.BF16 if w.dtype == "bf16" else fb.F32, w.c_q, w.c_k, m=w.m,
                           rank=w.r, rho=w.rho)
    call.layout(lq, lk, q, k, v)
    call.route()
    torch.cuda.synchronize()
    return call


def _both(call):
    import torch
    import free_block_sparse_major_amd as fb
    H, n, d = call.o_sp.shape
    ref_o = torch.full_like(call.o_sp, float("nan"))
    ref_l = torch.full_like(call.lse, float("nan"))
    fb.sparsepr_sparse_attn(call.dims, call.offsets_q, call.offsets_kv, call.cell_rowptr,
                            call.cell_col, call.q_g, call.k_g, call.v_g, call.v_shift, call.scale,
                            ref_o, ref_l, call.ws_attn)
    o = torch.full_like(call.o_sp, float("nan"))
    l = torch.full_like(call.lse, float("nan"))
    fb.sparsepr_sparse_attn_noalloc(call.dims, call.offsets_q, call.offsets_kv, call.cell_rowptr,
                                    call.cell_col, call.q_g, call.k_g, call.v_g, call.v_shift,
                                    call.scale, o, l)
    torch.cuda.synchronize()
    return ref_o.cpu().numpy(), ref_l.cpu().numpy(), o.cpu().numpy(), l.cpu().numpy()


def test_noalloc_attention_matches_workspace_entry_point():
    big = sg.small_workload(name="noalloc_big", heads=4, n=4000, head_dim=128, components=24,
                            kv_split=3, rho="0.3", seed=81)
    small = sg.small_workload(name="noalloc_small", heads=2, n=900, head_dim=64, components=10,
                              kv_split=2, rho="0.35", seed=82)
    for w in (big, small):
        say(f"[noalloc] {w}")
        ro, rl, o, l = _both(_prepared(w))
        assert not np.isnan(ro).any() and not np.isnan(rl).any()
        assert np.array_equal(o, ro)
        assert np.array_equal(l, rl)


def test_noalloc_refuses_tables_beyond_its_array():
    import free_block_sparse_major_amd as fb
    lib = fb.load_library()
    import ctypes
    dims = fb.make_dims(65, 1000, 1000, 64, fb.BF16, 1024, 8)   # 65 * 1024 + 1 > 65537
    P = ctypes.c_void_p(4096)
    st = lib.sparsepr_sparse_attn_noalloc(ctypes.byref(dims), P, P, P, P, P, P, P, P,
                                          ctypes.c_float(0.125), P, P, None)
    assert st == fb.ERR_UNSUPPORTED
