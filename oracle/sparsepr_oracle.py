"""Plain CPU reference for one SparsePR attention call (fp64 numpy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only the test suite, the smoke check and the CPU
baseline leg of the benchmark do.  It shares no code with the HIP library.

Source pages (cited by title and section):
  [paper]   "Partition the Support, Reconstruct the Residual: Training-Free
            Sparse Attention for Video Generation and World Models" (SparsePR
            paper body and appendices; its display equations are missing from
            the extracted text, so each formula here is restated from the prose
            around it).
  [review]  The paper.rainbus.top review of the same paper, method summary
            steps (1)-(5) and its hyper-parameter paragraph.
  [project] The SparsePR project page (method cards, Tables 1-2).

Every step works per attention head: the fit is per query head ([paper]
App. A.2, first paragraph).  The section comments below number the steps of
a call: S1 group-major layout (permutation, offsets, gather), S3 group
means, S4 budget and routing, S5 renormalised hard-drop attention, S6 probe
selection, S7 exact probe rows, S8 ridge fit and residual subspace, S9
corrected output.  All floating point is fp64; the inputs are the
exact fp32 values (or the bf16 values widened exactly).

Readings taken where the pages are silent or garbled are marked READING and
listed again in the design notes of the repository.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "group_layout",
    "group_means",
    "routed_pair_budget",
    "route_cells",
    "key_token_budget",
    "route_cells_per_group",
    "sparse_attention",
    "sparse_attention_rows",
    "dense_attention_rows",
    "select_probes",
    "probe_weights",
    "probe_distance_gap",
    "fit_correction",
    "fold_correction",
    "apply_correction",
    "fit_estimator",
    "apply_estimator",
    "ESTIMATORS",
    "run_head",
    "executed_density",
    "evaluation_rows",
    "row_error_stats",
    "correction_report",
]


# ----------------------------------------------------------------------------
# S1: group-major layout
# ----------------------------------------------------------------------------

def group_layout(labels, n_groups):
    """Group-major order of token indices ([paper] §3 problem setup: the query
    and key index sets are partitioned into groups; [review] step (3): Q, K, V
    are permuted to a group-major layout).

    Groups appear in ascending id; inside a group, tokens keep ascending token
    index (READING: the pages do not fix the order inside a group).
    Returns perm (group-major row -> token) and offsets [C+1] (group a holds
    rows offsets[a]:offsets[a+1]; an empty group has equal offsets)."""
    labels = np.asarray(labels)
    perm = np.argsort(labels, kind="stable").astype(np.int64)
    counts = np.bincount(labels, minlength=n_groups).astype(np.int64)
    offsets = np.zeros(n_groups + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return perm, offsets


def group_means(x, labels, n_groups):
    """Centroid of every non-empty group in the original space, fp64
    ([paper] §4.3 routing: query-group centroid and key centroid).  Empty
    groups get a NaN row (they take part in nothing)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.full((n_groups, x.shape[1]), np.nan)
    for a in range(n_groups):
        rows = np.nonzero(labels == a)[0]
        if rows.size:
            out[a] = x[rows].sum(axis=0) / rows.size
    return out


# ----------------------------------------------------------------------------
# S4: budget and routing
# ----------------------------------------------------------------------------

def routed_pair_budget(rho, n_q, n_k, m):
    """Pair budget of the router for an executed-density target rho.

    [paper] §4.3: probes add M/N_q to the executed density, so the router
    targets rho - M/N_q; each selected cell costs |G_a||G_b| pairs.  In pairs
    the routed budget is (rho*N_q - M)*N_k.  READING: "reaches the budget"
    with integer pair counts is the same as reaching its ceiling, computed
    exactly; a negative budget is clamped to 0.  M is the effective probe
    count min(M, N_q)."""
    m_eff = min(m, n_q)
    b = (Fraction(rho) * n_q - m_eff) * n_k
    return max(0, math.ceil(b))


def route_cells(qbar, kbar, n_a, m_b, budget, head_dim):
    """Select cells (a, b) under a routed pair budget.

    Score s_ab = qbar_a . kbar_b / sqrt(d) (centroid logit with the common
    1/sqrt(d) attention scale, [paper] §4.1).  READING (the pages' own
    value-error score is not printed): every non-empty query group first
    keeps its top-scoring cell (ties -> smaller b); then the remaining
    non-empty cells are taken in order (score desc, a asc, b asc) while the
    running pair count is below the budget -- the shortest prefix that
    reaches it ([paper] §4.3).  Forced cells count toward the budget.

    Returns z [Cq, Ck] bool, routed pair count, score matrix."""
    n_a = np.asarray(n_a, dtype=np.int64)
    m_b = np.asarray(m_b, dtype=np.int64)
    Cq, Ck = n_a.size, m_b.size
    qne = n_a > 0
    kne = m_b > 0
    s = np.full((Cq, Ck), -np.inf)
    qa = np.nonzero(qne)[0]
    kb = np.nonzero(kne)[0]
    if qa.size and kb.size:
        s[np.ix_(qa, kb)] = (qbar[qa] @ kbar[kb].T) / math.sqrt(head_dim)
    z = np.zeros((Cq, Ck), dtype=bool)
    pairs = 0
    if kb.size == 0:
        return z, 0, s
    for a in qa:
        row = s[a, kb]
        b = kb[int(np.argmax(row))]          # argmax returns the first maximum
        z[a, b] = True
        pairs += int(n_a[a] * m_b[b])
    # remaining non-empty cells in (score desc, a asc, b asc)
    A, B = np.nonzero(qne[:, None] & kne[None, :] & ~z)
    sc = s[A, B]
    order = np.lexsort((B, A, -sc))
    A, B = A[order], B[order]
    cost = n_a[A] * m_b[B]
    if pairs < budget and A.size:
        cum = pairs + np.cumsum(cost)
        # shortest prefix whose running total reaches the budget
        k = int(np.searchsorted(cum, budget, side="left"))
        take = min(k + 1, A.size)
        z[A[:take], B[:take]] = True
        pairs = int(cum[take - 1])
    return z, pairs, s


def key_token_budget(rho, n_q, n_k, m):
    """Common key-token budget per query of the per-group rule: rho_route * N_k
    with rho_route = rho - M/N_q ([paper] §4.3), i.e. (rho*N_q - M)*N_k/N_q;
    READING: "reaches" the budget is the same as reaching its ceiling,
    computed exactly; clamped at 0."""
    m_eff = min(m, n_q)
    b = (Fraction(rho) * n_q - m_eff) * n_k / n_q
    return max(0, math.ceil(b))


def route_cells_per_group(qbar, kbar, n_a, m_b, key_budget, head_dim):
    """The pages' routing rule ([paper] §4.3): each query group ranks the
    non-empty K/V groups by decreasing score and keeps the shortest prefix
    whose key-token count reaches the common per-query budget; a cell costs
    |G_a||G_b| interactions.  The score is the centroid logit (READING: the
    value-aware score is not printed); ties go to the smaller b.  READING:
    with a budget of 0 a group still keeps its top cell.

    Returns z [Cq, Ck] bool, routed pair count, score matrix."""
    n_a = np.asarray(n_a, dtype=np.int64)
    m_b = np.asarray(m_b, dtype=np.int64)
    Cq, Ck = n_a.size, m_b.size
    s = np.full((Cq, Ck), -np.inf)
    qa = np.nonzero(n_a > 0)[0]
    kb = np.nonzero(m_b > 0)[0]
    z = np.zeros((Cq, Ck), dtype=bool)
    if not (qa.size and kb.size):
        return z, 0, s
    s[np.ix_(qa, kb)] = (qbar[qa] @ kbar[kb].T) / math.sqrt(head_dim)
    pairs = 0
    for a in qa:
        order = kb[np.lexsort((kb, -s[a, kb]))]       # score desc, then b asc
        cum = np.cumsum(m_b[order])
        k = int(np.searchsorted(cum, key_budget, side="left"))   # first prefix reaching it
        take = max(1, min(k + 1, order.size))
        z[a, order[:take]] = True
        pairs += int(n_a[a] * cum[take - 1])
    return z, pairs, s


def executed_density(routed_pairs, n_q, n_k, m):
    """rho_exec = rho_route + M/N_q ([paper] §4.3; [review] step (5))."""
    return Fraction(routed_pairs, n_q * n_k) + Fraction(min(m, n_q), n_q)


# ----------------------------------------------------------------------------
# S5: renormalised hard-drop sparse attention
# ----------------------------------------------------------------------------

def _softmax_rows(logits, vals):
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    den = e.sum(axis=1, keepdims=True)
    return (e @ vals) / den, (mx[:, 0] + np.log(den[:, 0]))


def sparse_attention_rows(q_rows, row_groups, k, v, kv_labels, z, scale, dtype=np.float64):
    """Hard-drop output for selected query rows ([paper] §3: for a query of
    group a only keys of selected groups are kept and the softmax is
    renormalised over them).  q_rows [n, d]; row_groups [n] query group ids;
    k, v, kv_labels in any token order.  Returns (out [n, d], lse [n]).
    dtype: the arithmetic type (fp64 for parity; fp32 is only a timing mode)."""
    q_rows = np.asarray(q_rows, dtype=dtype)
    k = np.asarray(k, dtype=dtype)
    v = np.asarray(v, dtype=dtype)
    out = np.zeros((q_rows.shape[0], k.shape[1]), dtype=dtype)
    lse = np.zeros(q_rows.shape[0], dtype=dtype)
    for a in np.unique(row_groups):
        sel = np.nonzero(row_groups == a)[0]
        keys = np.nonzero(z[a][kv_labels])[0]
        o, l = _softmax_rows((q_rows[sel] @ k[keys].T) * dtype(scale), v[keys])
        out[sel] = o
        lse[sel] = l
    return out, lse


def sparse_attention(q, labels_q, k, v, labels_kv, z, scale):
    """Hard-drop output for every query, in original token order."""
    return sparse_attention_rows(q, np.asarray(labels_q), k, v, np.asarray(labels_kv), z, scale)


def dense_attention_rows(q_rows, k, v, scale, dtype=np.float64):
    """softmax(q K^T * scale) V over all keys ([paper] §3 dense attention; the
    1/sqrt(d) scale is the common attention scale named in §4.1)."""
    q_rows = np.asarray(q_rows, dtype=dtype)
    return _softmax_rows((q_rows @ np.asarray(k, dtype).T) * dtype(scale), np.asarray(v, dtype))


# ----------------------------------------------------------------------------
# S6: probe selection (Algorithm A.1)
# ----------------------------------------------------------------------------

def select_probes(features, labels_q, n_groups, m):
    """Stratified radial round-robin probes ([paper] App. A.2, Algorithm A.1;
    [review] step (4)).

    For every non-empty group, rows are ordered by distance to the group mean
    of the features (READING: Euclidean distance in the features that formed
    the partition), ties by token index.  Non-empty groups are ordered by size
    descending, ties by group id.  Traversal t takes the t-th row of each
    group in that order, skipping exhausted groups, until min(M, N_q) probes.

    Returns (probe tokens in selection order, per-group probe counts m_a)."""
    f = np.asarray(features, dtype=np.float64)
    labels_q = np.asarray(labels_q)
    m_eff = min(m, f.shape[0])
    ranked = {}
    for a in range(n_groups):
        rows = np.nonzero(labels_q == a)[0]
        if rows.size == 0:
            continue
        c = f[rows].sum(axis=0) / rows.size
        dist = np.sqrt(((f[rows] - c) ** 2).sum(axis=1))
        ranked[a] = rows[np.lexsort((rows, dist))]
    groups = sorted(ranked, key=lambda a: (-ranked[a].size, a))
    probes = []
    counts = np.zeros(n_groups, dtype=np.int64)
    t = 0
    while len(probes) < m_eff:
        for a in groups:
            if len(probes) == m_eff:
                break
            if t < ranked[a].size:
                probes.append(int(ranked[a][t]))
                counts[a] += 1
        t += 1
    return np.asarray(probes, dtype=np.int64), counts


def probe_distance_gap(features, labels_q, counts):
    """Smallest fp64 distance gap that Algorithm A.1 decides on: within each
    probed group, between consecutive rows of the (distance, token) order up
    to and including the first row not taken.  A diagnostic of near-ties in
    the probe choice (a zero gap means a tie that the token index breaks)."""
    f = np.asarray(features, dtype=np.float64)
    labels_q = np.asarray(labels_q)
    gap = math.inf
    for a in np.nonzero(np.asarray(counts) > 0)[0]:
        rows = np.nonzero(labels_q == a)[0]
        c = f[rows].sum(axis=0) / rows.size
        dist = np.sort(np.sqrt(((f[rows] - c) ** 2).sum(axis=1)))
        upto = min(int(counts[a]) + 1, dist.size)
        if upto >= 2:
            gap = min(gap, float(np.diff(dist[:upto]).min()))
    return gap


def probe_weights(probe_groups, group_sizes, probe_counts):
    """Coverage weight w_p = |G_a| / m_a for a probe of group a ([review]
    step (4); READING: m_a is the number of probes drawn from group a)."""
    pg = np.asarray(probe_groups)
    return np.asarray(group_sizes, np.float64)[pg] / np.asarray(probe_counts, np.float64)[pg]


# ----------------------------------------------------------------------------
# S8: weighted ridge fit and residual subspace
# ----------------------------------------------------------------------------

def fit_correction(x, R, w, lam, rank, feat_eps=1e-6, sv_tol=1e-10):
    """Coverage-weighted ridge fit of the residual on standardised sparse
    outputs, projected on the leading right singular directions of the
    weighted centred probe residuals.

    [paper] App. A.2: weights normalised to unit sum give the weighted means
    mu_x, mu_R and the feature scale s = sqrt(weighted variance + 1e-6)
    (App. D.3 places the 1e-6 inside the root); features are standardised,
    residuals centred.  Weights normalised to unit mean enter the ridge
    objective sum_p w~_p ||Rbar_p - xbar_p B||^2 + lam ||B||_F^2; the mean is
    not penalised (App. D.4).  [paper] App. D.3 / [review] step (4): the
    centred prediction is projected on the top-r right singular vectors of
    W~^(1/2) Rbar, mu_R is added untruncated; singular values at or below
    1e-10 of the largest are dropped (App. D.5 tolerance).

    Returns dict(mu_x, mu_R, s, B, Psi (d x k), sigma)."""
    x = np.asarray(x, np.float64)
    R = np.asarray(R, np.float64)
    w = np.asarray(w, np.float64)
    M, d = x.shape
    w_hat = w / w.sum()
    w_til = M * w / w.sum()
    mu_x = w_hat @ x
    mu_R = w_hat @ R
    s = np.sqrt(w_hat @ (x - mu_x) ** 2 + feat_eps)
    xb = (x - mu_x) / s
    Rb = R - mu_R
    gram = xb.T @ (w_til[:, None] * xb) + lam * np.eye(d)
    rhs = xb.T @ (w_til[:, None] * Rb)
    B = np.linalg.solve(gram, rhs)
    Y = np.sqrt(w_til)[:, None] * Rb
    _, sig, vt = np.linalg.svd(Y, full_matrices=False)
    if sig.size == 0 or sig[0] <= 0.0:
        k = 0
    else:
        k = int(np.count_nonzero(sig > sv_tol * sig[0]))
    k = min(k, rank)
    Psi = vt[:k].T.copy()
    return {"mu_x": mu_x, "mu_R": mu_R, "s": s, "B": B, "Psi": Psi, "sigma": sig,
            "w_hat": w_hat, "w_til": w_til}


def fold_correction(fit):
    """Fold the fit into out = o + (o A) Psi^T + c:
    A = diag(1/s) B Psi, c = mu_R - (mu_x A) Psi^T.  Returns (A, Psi, c, T)
    with the unique d x d operator T = diag(1/s) B Psi Psi^T."""
    B, Psi, s = fit["B"], fit["Psi"], fit["s"]
    A = (B @ Psi) / s[:, None]
    c = fit["mu_R"] - (fit["mu_x"] @ A) @ Psi.T
    T = A @ Psi.T
    return A, Psi, c, T


def apply_correction(o_sp, fit):
    """Corrected rows mu_R + o + ((o - mu_x) / s) B Psi Psi^T ([paper]
    App. D.3; [review] step (5))."""
    o_sp = np.asarray(o_sp, np.float64)
    xb = (o_sp - fit["mu_x"]) / fit["s"]
    P = fit["Psi"] @ fit["Psi"].T
    return o_sp + fit["mu_R"] + xb @ fit["B"] @ P


# ----------------------------------------------------------------------------
# estimator variants (mean-only, scalar and diagonal affine)
# ----------------------------------------------------------------------------

ESTIMATORS = ("full", "mean", "scalar", "diagonal")


def fit_estimator(x, R, w, lam, kind, feat_eps=1e-6):
    """Restricted estimators compared with the full ridge ([paper] §5 Table 4
    and App. D.4): correction by the weighted mean residual, and affine
    variants mu_R + xbar B with B = a I (scalar) or B = diag(b) (diagonal).
    Each minimises sum_p w~_p ||Rbar_p - xbar_p B||^2 + lam ||B||_F^2 (so the
    scalar penalty is lam d a^2); the mean is not penalised and the output
    is not truncated.  Weights, means and the feature scale are those of the
    full fit.  Returns dict(g, c, ...) with the folded correction
    out = o + g * o + c (g = diag(B) / s, c = mu_R - mu_x * g)."""
    x = np.asarray(x, np.float64)
    R = np.asarray(R, np.float64)
    w = np.asarray(w, np.float64)
    M, d = x.shape
    w_hat = w / w.sum()
    w_til = M * w / w.sum()
    mu_x = w_hat @ x
    mu_R = w_hat @ R
    s = np.sqrt(w_hat @ (x - mu_x) ** 2 + feat_eps)
    xb = (x - mu_x) / s
    Rb = R - mu_R
    if kind == "mean":
        b = np.zeros(d)
    elif kind == "scalar":
        a = float(np.sum(w_til[:, None] * xb * Rb)) / (float(np.sum(w_til[:, None] * xb * xb)) + lam * d)
        b = np.full(d, a)
    elif kind == "diagonal":
        b = (w_til @ (xb * Rb)) / (w_til @ (xb * xb) + lam)
    else:
        raise ValueError(kind)
    g = b / s
    c = mu_R - mu_x * g
    return {"kind": kind, "b": b, "g": g, "c": c, "mu_x": mu_x, "mu_R": mu_R, "s": s,
            "w_til": w_til}


def apply_estimator(o_sp, est):
    """Corrected rows mu_R + o + ((o - mu_x) / s) * b."""
    o_sp = np.asarray(o_sp, np.float64)
    return o_sp + est["mu_R"] + ((o_sp - est["mu_x"]) / est["s"]) * est["b"]


# ----------------------------------------------------------------------------
# quality of the correction (information only)
# ----------------------------------------------------------------------------

def evaluation_rows(n_q, probes, count=2048):
    """`count` evenly spaced rows among the unprobed query tokens (ascending
    token order): the unprobed tokens u_0 < u_1 < ... and rows
    u_floor(i * len(u) / count) for i < count (all of them if fewer).
    READING: the pages' evaluation takes 2048 evenly spaced query rows and
    scores unprobed rows only ([paper] App. D; §5 Table 2)."""
    unprobed = np.setdiff1d(np.arange(n_q, dtype=np.int64), np.asarray(probes, np.int64))
    if unprobed.size <= count:
        return unprobed
    return unprobed[(np.arange(count, dtype=np.int64) * unprobed.size) // count]


def row_error_stats(rows_out, rows_dense):
    """Per-row relative L2 error ||o_i - o_i^dense|| / ||o_i^dense|| over the
    given rows: its mean and 99th percentile (numpy's linear interpolation)."""
    a = np.asarray(rows_out, np.float64)
    b = np.asarray(rows_dense, np.float64)
    e = np.linalg.norm(a - b, axis=1) / np.linalg.norm(b, axis=1)
    return {"mean": float(e.mean()), "p99": float(np.percentile(e, 99)), "rows": int(e.size)}


def correction_report(q, k, v, labels_q, labels_kv, c_q, c_k, rho, m=64, rank=16, lam=0.1,
                      count=2048, **kw):
    """The executed density and the error of the hard-drop output against
    dense attention before and after the fitted correction, on `count`
    evenly spaced unprobed rows ([paper] §4.3: rho_exec = rho_route + M/N_q;
    App. D and §5 Table 2: per-row relative error of unprobed rows, mean and
    p99; [abstract] page: the correction lowers that error).  Information
    only: nothing is asserted on these numbers."""
    r0 = run_head(q, k, v, labels_q, labels_kv, c_q, c_k, rho, m=m, rank=rank, lam=lam,
                  query_rows=np.zeros(0, np.int64), **kw)
    rows = evaluation_rows(len(labels_q), r0["probes"], count)
    r = run_head(q, k, v, labels_q, labels_kv, c_q, c_k, rho, m=m, rank=rank, lam=lam,
                 query_rows=rows, **kw)
    dense, _ = dense_attention_rows(np.asarray(q, np.float64)[rows], k, v, r["scale"])
    return {
        "rows": rows, "dense": dense, "result": r,
        "rho_exec": float(executed_density(r["routed_pairs"], len(labels_q), len(labels_kv), m)),
        "before": row_error_stats(r["o_sp"], dense),
        "after": row_error_stats(r["out"], dense),
    }


# ----------------------------------------------------------------------------
# whole call for one head
# ----------------------------------------------------------------------------

def run_head(q, k, v, labels_q, labels_kv, c_q, c_k, rho, m=64, rank=16, lam=0.1,
             budget=None, features=None, query_rows=None, estimator="full",
             route_rule="global"):
    """Every step of one attention call for one head.

    query_rows: None -> sparse attention and final output for every query;
    otherwise only for the listed token indices (the routing, probes and fit
    always use the whole head).  Returns a dict of intermediates."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    labels_q = np.asarray(labels_q)
    labels_kv = np.asarray(labels_kv)
    n_q, d = q.shape
    n_k = k.shape[0]
    scale = 1.0 / math.sqrt(d)
    perm_q, off_q = group_layout(labels_q, c_q)
    perm_kv, off_kv = group_layout(labels_kv, c_k)
    n_a = np.diff(off_q)
    m_b = np.diff(off_kv)
    qbar = group_means(q, labels_q, c_q)
    kbar = group_means(k, labels_kv, c_k)
    if route_rule == "global":
        if budget is None:
            budget = routed_pair_budget(rho, n_q, n_k, m)
        z, routed, scores = route_cells(qbar, kbar, n_a, m_b, budget, d)
    else:
        if budget is None:
            budget = key_token_budget(rho, n_q, n_k, m)
        z, routed, scores = route_cells_per_group(qbar, kbar, n_a, m_b, budget, d)

    feats = q if features is None else np.asarray(features, np.float64)
    probes, counts = select_probes(feats, labels_q, c_q, m)
    pg = labels_q[probes]
    w = probe_weights(pg, n_a, counts)
    dense_p, _ = dense_attention_rows(q[probes], k, v, scale)
    x_p, _ = sparse_attention_rows(q[probes], pg, k, v, labels_kv, z, scale)
    R_p = dense_p - x_p
    if estimator == "full":
        fit = fit_correction(x_p, R_p, w, lam, rank)
        A, Psi, c, T = fold_correction(fit)
        g = np.zeros(d)
    else:
        fit = fit_estimator(x_p, R_p, w, lam, estimator)
        A, Psi, T = np.zeros((d, 0)), np.zeros((d, 0)), np.zeros((d, d))
        c, g = fit["c"], fit["g"]

    rows = np.arange(n_q) if query_rows is None else np.asarray(query_rows)
    o_sp, lse = sparse_attention_rows(q[rows], labels_q[rows], k, v, labels_kv, z, scale)
    out = apply_correction(o_sp, fit) if estimator == "full" else apply_estimator(o_sp, fit)
    is_probe = np.isin(rows, probes)
    if is_probe.any():
        where = {int(t): i for i, t in enumerate(probes)}
        for j in np.nonzero(is_probe)[0]:
            out[j] = dense_p[where[int(rows[j])]]
    return {
        "perm_q": perm_q, "offsets_q": off_q, "perm_kv": perm_kv, "offsets_kv": off_kv,
        "qbar": qbar, "kbar": kbar, "budget": budget, "z": z, "routed_pairs": routed,
        "scores": scores, "probes": probes, "probe_counts": counts, "probe_weights": w,
        "probe_gap": probe_distance_gap(feats, labels_q, counts),
        "dense_p": dense_p, "x_p": x_p, "R_p": R_p, "fit": fit, "A": A, "Psi": Psi,
        "c": c, "T": T, "g": g, "rows": rows, "o_sp": o_sp, "lse": lse, "out": out,
        "scale": scale, "estimator": estimator,
    }
