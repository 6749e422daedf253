"""sparsepr_debug_check on the GPU: a valid call reports 0, and every kind of
corrupted integer data sets its bit.  The corrupted arrays are copies given
to the check alone; no other kernel sees them."""
import numpy as np
import pytest

import synthgen as sg
from harness import say, upload

pytestmark = pytest.mark.gpu


def _check(fb, call, m, **over):
    import torch
    err = torch.full((1,), 0xdead, dtype=torch.int32, device="cuda")
    a = dict(labels_q=call._lq, labels_kv=call._lk, offsets_q=call.offsets_q,
             offsets_kv=call.offsets_kv, perm_q=call.perm_q, perm_kv=call.perm_kv,
             cell_rowptr=call.cell_rowptr, cell_col=call.cell_col,
             routed_pairs=call.routed_pairs, probe_rows=call.probe_rows,
             probe_tokens=call.probe_tokens)
    a.update(over)
    fb.sparsepr_debug_check(call.dims, m, a["labels_q"], a["labels_kv"], a["offsets_q"],
                            a["offsets_kv"], a["perm_q"], a["perm_kv"], a["cell_rowptr"],
                            a["cell_col"], a["routed_pairs"], a["probe_rows"],
                            a["probe_tokens"], err)
    torch.cuda.synchronize()
    return int(err.item()) & 0xffffffff


def test_debug_check_valid_and_corrupted():
    import torch
    import free_block_sparse_major_amd as fb
    w = sg.small_workload(name="dbg", heads=2, n=1500, head_dim=64, components=12, kv_split=2,
                          rho="0.3", seed=71)
    data = sg.make_call(w)
    q, k, v, lq, lk = upload(w, data)
    call = fb.SparsePRCall(w.heads, w.n, w.n, w.head_dim, fb.BF16, w.c_q, w.c_k, m=w.m,
                           rank=w.r, rho=w.rho)
    call(lq, lk, q, k, v)
    torch.cuda.synchronize()
    call._lq, call._lk = lq, lk
    assert _check(fb, call, w.m) == 0
    # nothing to check but the error word: 0
    none = {k: None for k in ("labels_q", "labels_kv", "offsets_q", "offsets_kv", "perm_q",
                              "perm_kv", "cell_rowptr", "cell_col", "routed_pairs",
                              "probe_rows", "probe_tokens")}
    assert _check(fb, call, w.m, **none) == 0

    def bad(name, t, bit):
        got = _check(fb, call, w.m, **{name: t})
        say(f"[debug_check] {name}: 0x{got:x}")
        assert got & bit, (name, got, bit)

    lab = lq.clone(); lab[1, 7] = w.c_q
    bad("labels_q", lab, fb.DBG_LABELS)
    lab = lk.clone(); lab[0, 3] = -1
    bad("labels_kv", lab, fb.DBG_LABELS)
    off = call.offsets_q.clone(); off[0, 3] = off[0, 5] + 1
    bad("offsets_q", off, fb.DBG_OFFSETS)
    off = call.offsets_kv.clone(); off[1, -1] = w.n + 1
    bad("offsets_kv", off, fb.DBG_OFFSETS)
    perm = call.perm_q.clone(); perm[0, [10, 11]] = perm[0, [11, 10]]
    bad("perm_q", perm, fb.DBG_PERM)
    perm = call.perm_kv.clone(); perm[1, 0] = w.n + 5
    bad("perm_kv", perm, fb.DBG_PERM)
    rp = call.cell_rowptr.clone(); rp[0, 2] = w.c_q * w.c_k + 1
    bad("cell_rowptr", rp, fb.DBG_ROWPTR)
    col = call.cell_col.clone()
    r0 = int(call.cell_rowptr[0, 0]); col[0, r0] = w.c_k
    bad("cell_col", col, fb.DBG_CELLS)
    col = call.cell_col.clone()
    a = int(np.argmax(np.diff(call.cell_rowptr[1].cpu().numpy())))
    r0 = int(call.cell_rowptr[1, a])
    col[1, [r0, r0 + 1]] = col[1, [r0 + 1, r0]]
    bad("cell_col", col, fb.DBG_CELLS)
    rpairs = call.routed_pairs.clone(); rpairs[1] = -1
    bad("routed_pairs", rpairs, fb.DBG_ROUTE)
    pr = call.probe_rows.clone(); pr[0, 5] = pr[0, 4]
    bad("probe_rows", pr, fb.DBG_PROBES)
    pr = call.probe_rows.clone(); pr[1, 0] = w.n
    bad("probe_rows", pr, fb.DBG_PROBES)
    pt = call.probe_tokens.clone(); pt[1, 9] = (pt[1, 9] + 1) % w.n
    bad("probe_tokens", pt, fb.DBG_PROBES)
    # the original buffers are untouched by all of this
    assert _check(fb, call, w.m) == 0
