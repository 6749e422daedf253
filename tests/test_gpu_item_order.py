"""GPU check of the longest-first order of the attention's work items.

The entry points with a workspace launch the items from an ordered list
(sorted by cost per head, the last two heads together, when there are at
least 8 items per compute unit by the bound; sorted over all heads in one
block when there are fewer), dealt to the XCDs; the entry point without a
workspace launches them in (head, group, tile) order.  Both must write every
row, bit-identically (the order changes which block computes an item, not
how).  O_sp is filled with NaN first, so a row no item covers shows."""
import numpy as np
import pytest

import synthgen as sg
from harness import compare_head, oracle_head, say, upload

pytestmark = pytest.mark.gpu

CASES = {
    "h2": sg.small_workload(name="ord2", heads=2, n=40000, head_dim=64, components=1024,
                            rho="0.22", seed=121),
    "h3": sg.small_workload(name="ord3", heads=3, n=30000, head_dim=128, components=1024,
                            rho="0.22", seed=122),
    "h5": sg.small_workload(name="ord5", heads=5, n=20000, head_dim=64, components=512,
                            kv_split=2, rho="0.26", seed=123),
    # few items per compute unit: one list over all heads
    "few6": sg.small_workload(name="ordfew6", heads=6, n=17550, head_dim=64, components=64,
                              rho="0.26", seed=124),
    "few3": sg.small_workload(name="ordfew3", heads=3, n=9000, head_dim=128, components=256,
                              kv_split=4, rho="0.22", seed=125),
}
# cases whose list is ordered over all heads (fewer than 8 items per unit)
FEW = {"few6", "few3"}


@pytest.mark.parametrize("name", list(CASES))
def test_ordered_items_match_natural_order(name):
    import torch
    import free_block_sparse_major_amd as fb
    w = CASES[name]
    say(f"[item order {name}] {w}")
    data = sg.make_call(w)
    q, k, v, lq, lk = upload(w, data)
    call = fb.SparsePRCall(w.heads, w.n, w.n, w.head_dim, fb.BF16, w.c_q, w.c_k, m=w.m,
                           rank=w.r, rho=w.rho)
    # the list of the intended kind is used at this shape
    from test_gpu_large import item_waves, sample_rows
    tq = 32 * item_waves(w.heads, w.n, w.c_q)
    bound = w.heads * (-(-w.n // tq) + w.c_q)
    if name in FEW:
        assert bound < 8 * 256 and w.heads * w.c_q <= 2048
    else:
        assert bound >= 8 * 256
    call.o_sp.fill_(float("nan"))
    call(lq, lk, q, k, v)
    o2 = torch.full_like(call.o_sp, float("nan"))
    l2 = torch.full_like(call.lse, float("nan"))
    fb.sparsepr_sparse_attn_noalloc(call.dims, call.offsets_q, call.offsets_kv, call.cell_rowptr,
                                    call.cell_col, call.q_g, call.k_g, call.v_g, call.v_shift,
                                    call.scale, o2, l2)
    torch.cuda.synchronize()
    assert not torch.isnan(call.o_sp).any()
    assert torch.equal(call.o_sp, o2)
    assert torch.equal(call.lse, l2)
    # and the rows are right: head 0 against the oracle on sampled rows
    fetch = lambda t: (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy()
    g = {key: fetch(getattr(call, key))
         for key in ("perm_q", "perm_kv", "offsets_q", "offsets_kv", "centroid_q", "centroid_k",
                     "cell_rowptr", "cell_col", "routed_pairs", "o_sp", "lse", "probe_rows",
                     "probe_tokens", "o_probe_dense", "o_probe_sparse", "corr_a", "corr_psi_t",
                     "corr_c", "corr_g", "out")}
    g["q_g"] = call.q_g.float().cpu().numpy()
    g["k_g"] = call.k_g.float().cpu().numpy()
    g["v_g"] = call.v_g.float().cpu().numpy()
    g["v_shift"] = call.v_shift.cpu().numpy()
    g["budget"] = call.budget
    g["call"] = call
    hd = data[0]
    rows = sample_rows(hd["labels_q"], w.c_q, 1200, seed=77)
    r = oracle_head(w, hd, rows=rows)
    errs = compare_head(w, g, 0, r, hd=hd)
    say(f"[item order {name}] head 0: {errs}")
