"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.  Integers (permutations, offsets, cell tables, routed
pair counts, probe indices) must match bit for bit; floating outputs within
relative Frobenius 2e-3 for bf16 inputs and 1e-5 for fp32 inputs."""
import numpy as np
import pytest

import oracle
import synthgen as sg
from harness import compare_head, oracle_head, rel_fro, run_gpu, say, tol_for

pytestmark = pytest.mark.gpu

# name -> workload, variant, kwargs for run_gpu/oracle
CASES = {
    "tiny_fp32_full": (sg.workload("tiny_fp32"), "default", {}),
    "bf16_d64_small": (sg.small_workload(heads=2, n=700, head_dim=64, components=8, rho="0.3",
                                         seed=21), "default", {}),
    "bf16_d128_kvsplit_grid": (sg.small_workload(heads=3, n=2000, head_dim=128, components=16,
                                                 kv_split=4, grid=(2, 10, 100), rho="0.25",
                                                 seed=22), "default", {}),
    "f32_d128_kvsplit": (sg.small_workload(heads=2, n=1500, head_dim=128, dtype="f32",
                                           components=12, kv_split=2, rho="0.3", seed=23),
                         "default", {}),
    "bf16_fewer_rows_than_probes": (sg.small_workload(heads=2, n=50, head_dim=64, components=5,
                                                      rho="0.5", seed=24), "default", {}),
    "bf16_empty_groups": (sg.small_workload(heads=2, n=130, head_dim=64, components=100,
                                            kv_split=2, rho="0.4", seed=25), "default", {}),
    "bf16_near_exact": (sg.small_workload(heads=2, n=1200, head_dim=128, components=10,
                                          rho="0.3", seed=26), "near_exact", {}),
    "bf16_odd_m_rank0": (sg.small_workload(heads=1, n=900, head_dim=64, components=7, m=33, r=0,
                                           rho="0.35", seed=27), "default", {}),
    "bf16_rank_cap": (sg.small_workload(heads=1, n=900, head_dim=64, components=7, m=20, r=64,
                                        rho="0.35", seed=28), "default", {}),
    "bf16_strided_nhd": (sg.small_workload(heads=3, n=640, head_dim=64, components=6, rho="0.3",
                                           seed=29), "default", {"layout": "nhd"}),
    "bf16_budget_zero": (sg.small_workload(heads=2, n=600, head_dim=64, components=6, rho="0.3",
                                           seed=30), "default", {"budget": 0}),
    # the largest group counts on both sides (1024 query groups, 1024 K/V groups),
    # a few rows each and some groups empty
    "bf16_max_groups": (sg.small_workload(heads=1, n=4096, head_dim=64, components=1024,
                                          kv_split=1, rho="0.3", seed=35), "default", {}),
}


def _run_case(name, check_fit=True):
    w, variant, kw = CASES[name]
    say(f"[case {name}] {w}")
    data = sg.make_call(w, variant)
    g = run_gpu(w, data, **kw)
    budget = kw.get("budget")
    tol = tol_for(w)
    worst = {}
    for h, hd in enumerate(data):
        r = oracle_head(w, hd, budget=budget)
        errs = compare_head(w, g, h, r, hd=hd)
        for k2, v in errs.items():
            worst[k2] = max(worst.get(k2, 0.0), v)
    say(f"[case {name}] errors {worst}")
    if check_fit:
        assert worst["T"] <= tol and worst["c"] <= tol, worst
    return worst


@pytest.mark.parametrize("name", list(CASES))
def test_parity_case(name):
    _run_case(name)


def test_full_density_equals_dense():
    """One query group and one K/V group with every cell selected: the call
    is dense attention (SparsePR paper §3), the residual is 0 and the
    correction reduces to 0."""
    w = sg.small_workload(heads=2, n=1000, head_dim=128, components=1, rho="1", seed=31)
    say(f"[case dense_one_group] {w}")
    data = sg.make_call(w)
    g = run_gpu(w, data, budget=w.n * w.n)
    for h, hd in enumerate(data):
        dense, _ = oracle.dense_attention_rows(hd["q"], hd["k"], hd["v"], 1 / np.sqrt(w.head_dim))
        assert rel_fro(g["out"][h], dense) <= 2e-3
        assert np.abs(g["corr_c"][h]).max() < 1e-4


def test_bf16_output_is_rounded_fp32_output():
    w = sg.small_workload(heads=2, n=800, head_dim=128, components=8, rho="0.3", seed=32)
    say(f"[case bf16_out] {w}")
    data = sg.make_call(w)
    g32 = run_gpu(w, data, out_dtype="f32")
    g16 = run_gpu(w, data, out_dtype="bf16")
    ref = sg.bf16_bits_to_f32(sg.f32_to_bf16_bits(g32["out"].astype(np.float32)))
    assert np.array_equal(g16["out"], ref)


def test_serial_and_overlapped_streams_agree():
    w = sg.small_workload(heads=2, n=900, head_dim=64, components=8, rho="0.3", seed=33)
    say(f"[case streams] {w}")
    data = sg.make_call(w)
    a = run_gpu(w, data, overlap=True)
    b = run_gpu(w, data, overlap=False)
    for key in ("out", "o_sp", "corr_a", "corr_c", "probe_tokens", "cell_rowptr"):
        assert np.array_equal(a[key], b[key]), key
    for h in range(w.heads):
        n_cells = a["cell_rowptr"][h][-1]
        assert np.array_equal(a["cell_col"][h][:n_cells], b["cell_col"][h][:n_cells])


def test_repeat_calls_are_deterministic():
    w = sg.small_workload(heads=2, n=900, head_dim=128, components=8, kv_split=2, rho="0.3",
                          seed=34)
    say(f"[case repeat] {w}")
    import torch
    from harness import upload
    import free_block_sparse_major_amd as fb
    data = sg.make_call(w)
    q, k, v, lq, lk = upload(w, data)
    call = fb.SparsePRCall(w.heads, w.n, w.n, w.head_dim, fb.BF16, w.c_q, w.c_k, rho=w.rho)
    o1 = call(lq, lk, q, k, v).clone()
    o2 = call(lq, lk, q, k, v).clone()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("rule", ["global", "per_group"])
def test_routing_with_unaligned_centroids(rule):
    # the score kernel moves centroid rows in 16-byte pairs only when both
    # arrays are 16-byte aligned; centroids at an 8-byte offset take the
    # one-double path and give the same cells
    import torch
    import free_block_sparse_major_amd as fb
    w = sg.small_workload(name="unal", heads=2, n=2000, head_dim=64, components=12, kv_split=2,
                          rho="0.3", seed=141)
    g = run_gpu(w, sg.make_call(w), route_rule=rule)
    call = g["call"]

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        assert v.data_ptr() % 16 == 8
        return v
    cq, ck = shifted(call.centroid_q), shifted(call.centroid_k)
    rowptr = torch.empty_like(call.cell_rowptr)
    col = torch.full_like(call.cell_col, -1)
    pairs = torch.empty_like(call.routed_pairs)
    if rule == "global":
        fb.sparsepr_route_cells(call.dims, call.offsets_q, call.offsets_kv, cq, ck, call.budget,
                                rowptr, col, pairs, call.ws_route)
    else:
        fb.sparsepr_route_cells_ex(call.dims, fb.ROUTE_RULES[rule], call.offsets_q,
                                   call.offsets_kv, cq, ck, call.budget, rowptr, col, pairs,
                                   call.ws_route)
    torch.cuda.synchronize()
    assert torch.equal(rowptr, call.cell_rowptr)
    assert torch.equal(pairs, call.routed_pairs)
    for h in range(w.heads):
        used = int(rowptr[h][-1])
        assert torch.equal(col[h][:used], call.cell_col[h][:used])
