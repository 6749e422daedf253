"""Shared helpers of the GPU parity tests: draw inputs, run the HIP path
through the C ABI, run the oracle on the same inputs, compare."""
from __future__ import annotations

import math
import sys

import numpy as np

import oracle
import synthgen as sg


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def ari(a, b):
    """Adjusted Rand index of two labelings (pair counting)."""
    a = np.asarray(a)
    b = np.asarray(b)
    n = a.size
    _, ai = np.unique(a, return_inverse=True)
    _, bi = np.unique(b, return_inverse=True)
    cont = np.zeros((ai.max() + 1, bi.max() + 1), np.int64)
    np.add.at(cont, (ai, bi), 1)
    comb = lambda m: m * (m - 1) / 2.0
    idx = comb(cont).sum()
    ea, eb = comb(cont.sum(axis=1)).sum(), comb(cont.sum(axis=0)).sum()
    exp = ea * eb / comb(n)
    den = 0.5 * (ea + eb) - exp
    return float((idx - exp) / den) if den != 0 else 1.0


def tol_for(w):
    return 1e-5 if w.dtype == "f32" else 2e-3


def upload(w, heads_data, layout="hnd"):
    """Device tensors q, k, v (bf16 or f32) and int32 labels for all heads.
    layout 'hnd' -> [H][N][d]; 'nhd' -> [N][H][d] (strided model layout)."""
    import torch
    H = len(heads_data)
    if w.dtype == "bf16":
        def stack(name):
            bits = np.stack([hd[name + "_bits"] for hd in heads_data])
            t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
            return t
    else:
        def stack(name):
            return torch.from_numpy(np.stack([hd[name] for hd in heads_data]))
    q, k, v = (stack(n) for n in ("q", "k", "v"))
    if layout == "nhd":
        q, k, v = (t.transpose(0, 1).contiguous() for t in (q, k, v))
    lq = torch.from_numpy(np.stack([hd["labels_q"] for hd in heads_data]))
    lk = torch.from_numpy(np.stack([hd["labels_kv"] for hd in heads_data]))
    dev = torch.device("cuda")
    return (q.to(dev), k.to(dev), v.to(dev), lq.to(dev), lk.to(dev))


def upload_arrays(w, arr):
    """Device tensors from packed [H][N][d] arrays (synthgen.make_call_arrays)."""
    import torch
    dev = torch.device("cuda")
    if w.dtype == "bf16":
        cv = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        cv = lambda a: torch.from_numpy(a).to(dev)
    return (cv(arr["q"]), cv(arr["k"]), cv(arr["v"]), torch.from_numpy(arr["labels_q"]).to(dev),
            torch.from_numpy(arr["labels_kv"]).to(dev))


def run_gpu(w, heads_data, budget=None, rank=None, m=None, layout="hnd", out_dtype="f32",
            overlap=True, tensors=None, fetch_heads=None, probe_feat=None, estimator="full",
            route_rule="global", fused=False, head_chunks=1):
    """Runs the whole call.  Inputs come from per-head dicts (`heads_data`) or,
    for large shapes, from already uploaded `tensors` (heads_data is then
    None).  `fetch_heads` limits the per-head outputs copied back."""
    import torch
    import free_block_sparse_major_amd as fb
    if tensors is None:
        H = len(heads_data)
        q, k, v, lq, lk = upload(w, heads_data, layout)
    else:
        H = w.heads
        q, k, v, lq, lk = tensors
    d = w.head_dim
    strides = None
    if layout == "nhd":
        strides = (d, H * d)
    call = fb.SparsePRCall(H, w.n, w.n, d, fb.BF16 if w.dtype == "bf16" else fb.F32, w.c_q, w.c_k,
                           m=w.m if m is None else m, rank=w.r if rank is None else rank,
                           lam=w.lam, rho=w.rho, budget=budget,
                           out_dtype=fb.F32 if out_dtype == "f32" else fb.BF16,
                           q_strides=strides, kv_strides=strides, overlap=overlap,
                           feat_dim=0 if probe_feat is None else probe_feat.shape[-1],
                           estimator=estimator, route_rule=route_rule, fused=fused,
                           head_chunks=head_chunks)
    call.probe_feat = probe_feat
    if fused:
        # the fused order stores no O_sp: mark the buffer so a stray read shows
        call.o_sp.fill_(float("nan"))
    call(lq, lk, q, k, v)
    torch.cuda.synchronize()
    g = {name: getattr(call, name) for name in (
        "perm_q", "perm_kv", "offsets_q", "offsets_kv", "centroid_q", "centroid_k",
        "cell_rowptr", "cell_col", "routed_pairs", "o_sp", "lse", "probe_rows", "probe_tokens",
        "o_probe_dense", "o_probe_sparse", "corr_a", "corr_psi_t", "corr_c", "corr_g", "out")}
    out = {}
    sel = (lambda t: t) if fetch_heads is None else (lambda t: t[list(fetch_heads)])
    for key, t in g.items():
        if t.dtype == torch.bfloat16:
            t = t.float()
        out[key] = sel(t).cpu().numpy()
    out["q_g"] = sel(call.q_g.float() if w.dtype == "bf16" else call.q_g).cpu().numpy()
    out["k_g"] = sel(call.k_g.float() if w.dtype == "bf16" else call.k_g).cpu().numpy()
    out["v_g"] = sel(call.v_g.float()).cpu().numpy()
    out["v_shift"] = sel(call.v_shift).cpu().numpy()
    out["budget"] = call.budget
    out["call"] = call
    return out


def oracle_head(w, hd, budget=None, rank=None, m=None, rows=None, features=None,
                estimator="full", route_rule="global"):
    return oracle.run_head(hd["q"], hd["k"], hd["v"], hd["labels_q"], hd["labels_kv"], w.c_q,
                           w.c_k, w.rho, m=w.m if m is None else m,
                           rank=w.r if rank is None else rank, lam=w.lam, budget=budget,
                           features=features, query_rows=rows, estimator=estimator,
                           route_rule=route_rule)


def cells_from_csr(rowptr, col, c_q, c_k):
    z = np.zeros((c_q, c_k), bool)
    for a in range(c_q):
        z[a, col[rowptr[a]:rowptr[a + 1]]] = True
    return z


def score_gap(scores, z):
    """Smallest |s| distance between a selected and an unselected candidate
    cell score (diagnostic for near-ties at the routing boundary)."""
    sel = scores[z & np.isfinite(scores)]
    uns = scores[~z & np.isfinite(scores)]
    if sel.size == 0 or uns.size == 0:
        return math.inf
    return float(sel.min() - uns.max()) if sel.min() > uns.max() else 0.0


def v_operand(v):
    """The layout's PV operand for one head, from its definition in the C ABI:
    bf16 inputs become fp16(v * 2^-shift), nearest-even, with the shift that
    puts the largest |v| in [2^14, 2^15) (clamped to [-100, 100]; -100 for an
    all-zero head).  Returns (operand as fp32 values, shift)."""
    vmax = float(np.abs(np.asarray(v, np.float32)).max())
    if vmax == 0.0 or vmax < 2.0 ** -126:
        shift = -100
    else:
        shift = max(-100, min(100, math.frexp(vmax)[1] - 1 - 14))
    op = (np.asarray(v, np.float64) * 2.0 ** (-shift)).astype(np.float16).astype(np.float32)
    return op, shift


def row_rel(a, b):
    """Per-row relative L2 error of a against b (rows of b that are zero use
    the absolute error)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    num = np.linalg.norm(a - b, axis=1)
    den = np.linalg.norm(b, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def check_gathered(w, g, h, r, hd):
    """q_g, k_g are bit-exact copies of q, k in group-major order; v_g is the
    fp16 operand of the PV product (fp32 inputs: an fp32 copy, shift 0)."""
    assert np.array_equal(g["q_g"][h], hd["q"][r["perm_q"]].astype(np.float32)), "q_g"
    assert np.array_equal(g["k_g"][h], hd["k"][r["perm_kv"]].astype(np.float32)), "k_g"
    if w.dtype == "bf16":
        op, shift = v_operand(hd["v"])
        assert int(g["v_shift"][h]) == shift, ("v_shift", int(g["v_shift"][h]), shift)
        assert np.array_equal(g["v_g"][h], op[r["perm_kv"]]), "v_g"
    else:
        assert int(g["v_shift"][h]) == 0
        assert np.array_equal(g["v_g"][h], hd["v"][r["perm_kv"]].astype(np.float32)), "v_g"


def compare_head(w, g, h, r, rows_orig=None, check_rows=True, hd=None, fused=False):
    """Asserts parity of head h of GPU results `g` with oracle results `r`
    (and, given the head's inputs `hd`, of the gathered tensors).
    Returns a dict of measured errors."""
    n, c_q, c_k, d = w.n, w.c_q, w.c_k, w.head_dim
    tol = tol_for(w)
    errs = {}
    # layout: bit-exact
    assert np.array_equal(g["perm_q"][h], r["perm_q"]), "perm_q"
    assert np.array_equal(g["perm_kv"][h], r["perm_kv"]), "perm_kv"
    assert np.array_equal(g["offsets_q"][h], r["offsets_q"]), "offsets_q"
    assert np.array_equal(g["offsets_kv"][h], r["offsets_kv"]), "offsets_kv"
    # centroids (fp64 means of the same values; summation order may differ)
    ne = np.diff(r["offsets_q"]) > 0
    cq = g["centroid_q"][h][ne]
    assert np.allclose(cq, r["qbar"][ne], rtol=0, atol=1e-12 * max(1.0, np.abs(cq).max()))
    nek = np.diff(r["offsets_kv"]) > 0
    ck = g["centroid_k"][h][nek]
    assert np.allclose(ck, r["kbar"][nek], rtol=0, atol=1e-12 * max(1.0, np.abs(ck).max()))
    if hd is not None:
        check_gathered(w, g, h, r, hd)
    # routing: bit-exact
    z = cells_from_csr(g["cell_rowptr"][h], g["cell_col"][h], c_q, c_k)
    errs["score_gap"] = score_gap(r["scores"], r["z"])
    assert np.array_equal(z, r["z"]), f"cells differ (boundary score gap {errs['score_gap']:.3e})"
    for a in range(c_q):
        cols = g["cell_col"][h][g["cell_rowptr"][h][a]:g["cell_rowptr"][h][a + 1]]
        assert np.all(np.diff(cols) > 0)
    assert int(g["routed_pairs"][h]) == r["routed_pairs"]
    # probes: bit-exact (selection order); smallest fp64 distance gap at the
    # selection boundaries, a near-tie diagnostic
    errs["probe_gap"] = r.get("probe_gap", math.inf)
    me = min(w.m, n) if "m_override" not in r else r["m_override"]
    probes_tok = g["probe_tokens"][h][:len(r["probes"])]
    assert np.array_equal(probes_tok, r["probes"]), "probe tokens"
    inv = np.empty(n, np.int64)
    inv[r["perm_q"]] = np.arange(n)
    assert np.array_equal(g["probe_rows"][h][:len(r["probes"])], inv[r["probes"]])
    assert np.all(g["probe_tokens"][h][len(r["probes"]):] == -1)
    np_ = len(r["probes"])
    errs["dense_p"] = rel_fro(g["o_probe_dense"][h][:np_], r["dense_p"])
    errs["x_p"] = rel_fro(g["o_probe_sparse"][h][:np_], r["x_p"])
    assert errs["dense_p"] <= tol, errs
    assert errs["x_p"] <= tol, errs
    # fit: compare the unique d x d operator A Psi^T and c
    k = w.r
    T_gpu = g["corr_a"][h][:, :k] @ g["corr_psi_t"][h][:k, :] if k > 0 else np.zeros((d, d))
    errs["T"] = rel_fro(T_gpu, r["T"]) if np.linalg.norm(r["T"]) > 0 else float(np.abs(T_gpu).max())
    errs["c"] = rel_fro(g["corr_c"][h], r["c"])
    # the folded correction is asserted where it is not at the rounding level
    # of the residual (full selection makes R_p ~ 0 and both sides noise)
    row_scale = np.linalg.norm(r["dense_p"]) / math.sqrt(max(len(r["probes"]), 1))
    if np.linalg.norm(r["c"]) > 1e-4 * row_scale:
        assert errs["c"] <= tol, errs
    if r.get("estimator", "full") == "full":
        if np.linalg.norm(r["T"]) > 1e-6:
            assert errs["T"] <= tol, errs
    else:
        # restricted estimators: diagonal gain g = diag(B) / s, no low-rank part
        errs["g"] = (rel_fro(g["corr_g"][h], r["g"]) if np.linalg.norm(r["g"]) > 0
                     else float(np.abs(g["corr_g"][h]).max()))
        if np.linalg.norm(r["g"]) > 1e-6:
            assert errs["g"] <= tol, errs
        # (a rank-0 call has no A or Psi: its one-column buffers are never written)
        rk = g["call"].rank
        assert not np.any(g["corr_a"][h][:, :rk]) and not np.any(g["corr_psi_t"][h][:rk])
    # sparse output rows and final output
    if check_rows:
        rows = r["rows"]
        errs["lse"] = float(np.abs(g["lse"][h][inv[rows]] - r["lse"]).max())
        out_g = g["out"][h][rows]
        errs["out"] = rel_fro(out_g, r["out"])
        errs["out_row_max"] = float(row_rel(out_g, r["out"]).max())
        unprobed = ~np.isin(rows, r["probes"])
        corr_r = r["out"] - r["o_sp"]
        if not fused:
            o_sp_g = g["o_sp"][h][inv[rows]]
            errs["o_sp"] = rel_fro(o_sp_g, r["o_sp"])
            errs["o_sp_row_max"] = float(row_rel(o_sp_g, r["o_sp"]).max())
            corr_g = out_g - o_sp_g
            errs["correction"] = rel_fro(corr_g[unprobed], corr_r[unprobed])
            # the correction term on its own (final-output parity cannot see an error in a
            # correction that is small next to O); looser bound, skipped where it vanishes
            if np.linalg.norm(corr_r[unprobed]) > 1e-3 * np.linalg.norm(r["o_sp"][unprobed]):
                assert errs["correction"] <= (1e-2 if w.dtype == "bf16" else 1e-4), errs
            assert errs["o_sp"] <= tol, errs
            assert errs["o_sp_row_max"] <= 10 * tol, errs
        else:
            # no O_sp is stored: the correction term is the output minus the
            # oracle's hard-drop rows
            corr_g = out_g - r["o_sp"]
            errs["correction"] = rel_fro(corr_g[unprobed], corr_r[unprobed])
            if np.linalg.norm(corr_r[unprobed]) > 1e-3 * np.linalg.norm(r["o_sp"][unprobed]):
                assert errs["correction"] <= (1e-2 if w.dtype == "bf16" else 1e-4), errs
        assert errs["out"] <= tol, errs
        # natural-log normaliser of the kept keys ([paper] §3 hard drop): fp32
        # logits of exact products; with bf16 inputs the row sum adds the fp16
        # values of P, each within 2^-11 relative, so log l moves by at most
        # about 2^-11 = 4.9e-4 (a few kept keys do not average it down)
        assert errs["lse"] <= (5e-4 if w.dtype == "bf16" else 1e-5), errs
        # no single row may be far off while the head-level norm passes
        assert errs["out_row_max"] <= 10 * tol, errs
        probed = np.isin(rows, r["probes"])
        if probed.any():
            dense_rows = {int(t): i for i, t in enumerate(r["probes"])}
            for j in np.nonzero(probed)[0]:
                assert np.array_equal(g["out"][h][rows[j]],
                                      g["o_probe_dense"][h][dense_rows[int(rows[j])]])
    return errs
