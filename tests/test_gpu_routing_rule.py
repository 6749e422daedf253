"""GPU parity of the pages' per-group routing rule ([paper] §4.3): every query
group keeps the shortest score-ordered prefix of non-empty K/V groups that
reaches a common key-token budget per query (centroid-logit score, ties to
the smaller b, at least the top cell).  Cells and pair counts are bit-exact;
the rest of the call is compared as usual."""
import numpy as np
import pytest

import synthgen as sg
from harness import compare_head, oracle_head, run_gpu, say, upload_arrays

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("head_dim,dtype,rho", [(128, "bf16", "0.26"), (64, "bf16", "0.12"),
                                               (64, "f32", "0.3")])
def test_per_group_rule(head_dim, dtype, rho):
    w = sg.small_workload(name=f"pg_{head_dim}_{dtype}", heads=2, n=3200, head_dim=head_dim,
                          dtype=dtype, components=16, kv_split=3, grid=(4, 20, 40), rho=rho,
                          seed=61)
    heads = sg.make_call(w)
    g = run_gpu(w, heads, route_rule="per_group")
    for h in range(w.heads):
        r = oracle_head(w, heads[h], route_rule="per_group")
        assert g["budget"] == r["budget"]
        errs = compare_head(w, g, h, r, hd=heads[h])
        say(f"[per_group {dtype} d={head_dim} rho={rho}] head {h}: {errs}")


def test_per_group_rule_edge_budgets():
    # budget 0 keeps each group's top cell; a budget of every key keeps all
    w = sg.small_workload(name="pg_edges", heads=1, n=900, head_dim=64, components=6,
                          kv_split=2, rho="0.3", seed=62)
    heads = sg.make_call(w)
    for budget in (0, w.n):
        g = run_gpu(w, heads, budget=budget, route_rule="per_group")
        r = oracle_head(w, heads[0], budget=budget, route_rule="per_group")
        errs = compare_head(w, g, 0, r, hd=heads[0])
        say(f"[per_group budget {budget}] {errs}")
        counts = np.diff(g["cell_rowptr"][0])
        if budget == 0:
            assert np.all(counts[np.diff(r["offsets_q"]) > 0] == 1)


def test_per_group_rule_full_size_sampled():
    w = sg.workload("wan")
    arr = sg.make_call_arrays(w)
    tensors = upload_arrays(w, arr)
    del arr
    from test_gpu_large import sample_rows
    g = run_gpu(w, None, tensors=tensors, fetch_heads=[0, 39], route_rule="per_group")
    pos = sg.position_code(w.grid, w.head_dim)
    say(f"[per_group wan] routed pairs {int(g['call'].routed_pairs.sum())}, key budget {g['budget']}")
    for j, h in enumerate([0, 39]):
        hd = sg.make_head(w, h, pos=pos)
        rows = sample_rows(hd["labels_q"], w.c_q, 1500, seed=3000 + h)
        r = oracle_head(w, hd, rows=rows, route_rule="per_group")
        errs = compare_head(w, g, j, r, hd=hd)
        say(f"[per_group wan] head {h}: {errs}")
