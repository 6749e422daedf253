"""A call split into head ranges (SparsePRCall(head_chunks=k), ranges issued
on alternating streams) computes every head exactly as a whole call: all
outputs are compared bit for bit with those of the unsplit call on the same
inputs.  Every step of the path is per head ([paper] App. A.2: the fit is per
query head), so the split changes only the order of launches."""
import numpy as np
import pytest

import synthgen as sg
from harness import say, upload

pytestmark = pytest.mark.gpu

OUTPUTS = ("perm_q", "offsets_q", "perm_kv", "offsets_kv", "v_shift", "cell_rowptr", "cell_col",
           "routed_pairs", "o_sp", "lse", "probe_rows", "probe_tokens", "o_probe_dense",
           "corr_a", "corr_psi_t", "corr_c", "corr_g", "out")


def _run(w, tensors, chunks, layout="hnd", feat=None, **kw):
    import torch
    import free_block_sparse_major_amd as fb
    q, k, v, lq, lk = tensors
    strides = dict(q_strides=(w.head_dim, w.heads * w.head_dim),
                   kv_strides=(w.head_dim, w.heads * w.head_dim)) if layout == "nhd" else {}
    call = fb.SparsePRCall(w.heads, w.n, w.n, w.head_dim, fb.BF16 if w.dtype == "bf16" else fb.F32,
                           w.c_q, w.c_k, m=w.m, rank=w.r, lam=w.lam, rho=w.rho, out_dtype=fb.BF16,
                           head_chunks=chunks, feat_dim=0 if feat is None else feat.shape[2],
                           **strides, **kw)
    if feat is not None:
        call.probe_feat = feat
    for _ in range(2):          # a repeated call reuses the workspace sets
        call(lq, lk, q, k, v)
    torch.cuda.synchronize()
    return {name: getattr(call, name).cpu().clone() for name in OUTPUTS}


def _same(a, b):
    import torch
    for name in OUTPUTS:
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("heads,chunks", [(6, 3), (7, 3), (5, 5)])
def test_chunked_call_is_bitwise_the_whole_call(heads, chunks):
    w = sg.small_workload(name=f"chunks_{heads}", heads=heads, n=3200, head_dim=128,
                          components=16, kv_split=2, grid=(4, 20, 40), rho="0.26", seed=61)
    tensors = upload(w, sg.make_call(w))
    whole = _run(w, tensors, 1)
    split = _run(w, tensors, chunks)
    _same(whole, split)
    say(f"[chunks] H={heads} k={chunks}: identical")


def test_chunked_call_with_options_and_strided_inputs():
    import torch
    w = sg.small_workload(name="chunks_opt", heads=6, n=3200, head_dim=64, components=16,
                          kv_split=2, grid=(4, 20, 40), rho="0.3", seed=62)
    heads = sg.make_call(w)
    tensors = upload(w, heads, layout="nhd")
    rng = np.random.default_rng(7)
    feat = torch.from_numpy(rng.standard_normal((w.heads, w.n, 16), dtype=np.float32)).to("cuda")
    for kw in (dict(route_rule="per_group"), dict(estimator="diagonal")):
        whole = _run(w, tensors, 1, layout="nhd", feat=feat, **kw)
        split = _run(w, tensors, 4, layout="nhd", feat=feat, **kw)
        _same(whole, split)
        say(f"[chunks] options {kw}: identical")


def test_fused_ranges_with_unfused_first_range():
    # lead_unfused: the first range attends as soon as it is routed and takes
    # the correction kernel after its fit (the usual order on those heads); the
    # later ranges keep the correction in the attention epilogue
    w = sg.small_workload(name="chunks_lead", heads=5, n=3200, head_dim=128, components=16,
                          kv_split=2, grid=(4, 20, 40), rho="0.26", seed=63)
    tensors = upload(w, sg.make_call(w))
    usual = _run(w, tensors, 1)
    fused = _run(w, tensors, 1, fused=True)
    mixed = _run(w, tensors, [2, 3], fused=True, lead_unfused=True)
    shared = [n for n in OUTPUTS if n not in ("o_sp", "out", "lse")]
    for name in shared:
        assert torch_equal(usual[name], mixed[name]), name
    assert torch_equal(usual["lse"][:2], mixed["lse"][:2])
    assert torch_equal(usual["o_sp"][:2], mixed["o_sp"][:2])
    assert torch_equal(usual["out"][:2], mixed["out"][:2]), "first range: usual order"
    assert torch_equal(fused["out"][2:], mixed["out"][2:]), "later ranges: fused order"
    say("[chunks] unfused first range: heads 0-1 as the usual order, 2-4 as the fused order")


def torch_equal(a, b):
    import torch
    return torch.equal(a, b)
