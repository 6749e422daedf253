"""Plain CPU reference for Response-Coupled Partitioning (fp64 numpy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only the test suite, the smoke check and the CPU
baseline leg of the benchmark do.  It shares no code with the HIP library.

Source: [paper] "Partition the Support, Reconstruct the Residual" §4.1
(response-coupled partitioning: key-response coordinates for paired K/V
groups, query-response coordinates from K/V groups), App. B.1 (key response
metric), App. B.2 (query response metric, RMS normalisation with floor
1e-6) and App. C.1 (clustering on the GPU, initial centres sampled uniformly
with replacement from the feature rows).  The display equations are missing
from the extracted text; each formula is restated from the prose around it.

Readings (listed again in the design notes):
  * sampled rows: row floor(i * N_q / M_s) for i < M_s, every row when
    N_q <= M_s;
  * key metric M_K = Q_s^T Q_s / M_s; query metric M_Q = K~^T K~ / C_k with
    C_k the number of non-empty K/V groups;
  * eigenvalues are clamped at 0 and normalised to unit mean over the r
    retained; a zero mean gives F = 0;
  * phi_K(k) = k F_K, phi_Q(q) = u / max(RMS(u), 1e-6) with u = q F_Q and
    RMS(u) = sqrt(mean_j u_j^2);
  * one Lloyd iteration assigns every row to its nearest centre (squared
    Euclidean distance, ties to the smaller centre index) and then moves each
    centre to the mean of its rows; an empty cluster keeps its centre; the
    partition is the assignment of the last iteration;
  * initial centre indices are drawn by the caller (the seeded input
    generator) and are inputs here.

Later calls (App. C.1, warm start across calls of the same layer):
  * the factors are updated by two subspace iterations started from the
    previous call's orthonormal basis: Y = M X, then X = Y L^-T with
    Y^T Y = L L^T (Cholesky); a Cholesky pivot at or below 1e-10 of the
    largest diagonal entry of Y^T Y drops its column (X column 0), so a
    rank-deficient metric keeps working;
  * each retained direction is weighted by its Rayleigh quotient x^T M x
    (clamped at 0), normalised to unit mean over the r columns, as the
    eigenvalues are on the first call;
  * k-means starts from the previous call's group centroids in the
    original space, mapped by the current coordinates (phi_K = k F_K for
    keys, phi_Q with its RMS normalisation for queries);
  * the state a call leaves for the next one is the bases and, per group,
    the mean of its members in the original space; a group left empty
    keeps its previous centroid (on the first call, its initial row).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "sample_query_rows",
    "key_response_metric",
    "query_response_metric",
    "response_factor",
    "query_features",
    "sq_distances",
    "kmeans",
    "rcp_partition",
    "response_basis",
    "cholesky_drop",
    "cholesky_orthonormalise",
    "subspace_factor",
    "project_centers",
    "group_means",
]


def sample_query_rows(n_q, m_s):
    """Deterministic evenly spaced query rows ([paper] §4.1 and App. B.1:
    M_s rows at evenly spaced token positions of the current call; App. C.1:
    all rows when fewer are available)."""
    if n_q <= m_s:
        return np.arange(n_q, dtype=np.int64)
    return (np.arange(m_s, dtype=np.int64) * n_q) // m_s


def key_response_metric(q_rows):
    """M_K = Q_s^T Q_s / M_s: (k_j - k_l)^T M_K (k_j - k_l) is the mean over
    the sampled queries of the squared logit difference q_i . (k_j - k_l)
    ([paper] App. B.1)."""
    qs = np.asarray(q_rows, dtype=np.float64)
    return qs.T @ qs / qs.shape[0]


def query_response_metric(k, labels_kv, c_k):
    """M_Q = K~^T K~ / C_k over the non-empty K/V groups: rows of K~ are the
    group centroids in the original key space minus their uniform mean
    ([paper] §4.1 and App. B.2; empty groups take no part).  Returns
    (M_Q, number of non-empty groups)."""
    k = np.asarray(k, dtype=np.float64)
    labels_kv = np.asarray(labels_kv)
    cents = []
    for b in range(c_k):
        rows = np.nonzero(labels_kv == b)[0]
        if rows.size:
            cents.append(k[rows].sum(axis=0) / rows.size)
    cents = np.asarray(cents)
    kt = cents - cents.mean(axis=0)
    return kt.T @ kt / cents.shape[0], cents.shape[0]


def _weighted(basis, lam):
    """basis * sqrt(lam / mean(lam)) column by column; 0 when the mean is 0."""
    mean = lam.mean() if lam.size else 0.0
    if not mean > 0.0:
        return np.zeros_like(basis)
    return basis * np.sqrt(lam / mean)


def response_basis(metric, r):
    """(U, lam, F): the leading r eigenvectors U of the symmetric metric
    (descending eigenvalues), the eigenvalues clamped at 0 and the factor
    F = U diag(sqrt(lam / mean lam)) ([paper] §4.1 and App. B.1)."""
    w, u = np.linalg.eigh(np.asarray(metric, dtype=np.float64))
    order = np.argsort(-w, kind="stable")[:r]
    lam = np.maximum(w[order], 0.0)
    return u[:, order], lam, _weighted(u[:, order], lam)


def response_factor(metric, r):
    """F (d x r): the leading r eigenvectors of the symmetric metric, each
    scaled by the square root of its eigenvalue normalised to unit mean over
    the r retained ([paper] §4.1 and App. B.1)."""
    return response_basis(metric, r)[2]


def cholesky_drop(g, tol=1e-10):
    """Lower-triangular L with G = L L^T, column by column (right-looking).
    A pivot at or below tol * max(diag G) leaves its column of L at 0 (the
    direction is dropped) instead of failing."""
    a = np.array(g, dtype=np.float64)
    r = a.shape[0]
    low = np.zeros_like(a)
    ref = max(float(np.max(np.diag(a))) if r else 0.0, 0.0)
    for j in range(r):
        piv = a[j, j]
        if piv > tol * ref and piv > 0.0:
            low[j, j] = np.sqrt(piv)
            low[j + 1:, j] = a[j + 1:, j] / low[j, j]
            a[j + 1:, j + 1:] -= np.outer(low[j + 1:, j], low[j + 1:, j])
    return low


def cholesky_orthonormalise(y, tol=1e-10):
    """X = Y L^-T with Y^T Y = L L^T: orthonormal columns spanning Y's
    column space (dropped columns are 0).  Solved column by column."""
    y = np.asarray(y, dtype=np.float64)
    low = cholesky_drop(y.T @ y, tol)
    x = np.zeros_like(y)
    for j in range(y.shape[1]):
        if low[j, j] > 0.0:
            x[:, j] = (y[:, j] - x[:, :j] @ low[j, :j]) / low[j, j]
    return x


def subspace_factor(metric, basis_prev, steps=2, tol=1e-10):
    """Factor update of a later call ([paper] App. C.1): `steps` subspace
    iterations X <- orth(M X) from the previous basis, orthonormalised by
    Cholesky; each column weighted by its Rayleigh quotient x^T M x (clamped
    at 0) normalised to unit mean.  Returns (X, lam, F)."""
    m = np.asarray(metric, dtype=np.float64)
    x = np.asarray(basis_prev, dtype=np.float64)
    for _ in range(steps):
        x = cholesky_orthonormalise(m @ x, tol)
    lam = np.maximum(np.sum(x * (m @ x), axis=0), 0.0)
    return x, lam, _weighted(x, lam)


def query_features(q, f_q, eps=1e-6):
    """phi_Q(q) = u / max(RMS(u), eps) with u = q F_Q ([paper] §4.1 and
    App. B.2: RMS normalisation without gain or bias, floor 1e-6)."""
    u = np.asarray(q, dtype=np.float64) @ f_q
    rms = np.sqrt((u * u).mean(axis=1))
    return u / np.maximum(rms, eps)[:, None]


def project_centers(cent, f, rms):
    """Centroids given in the original space, in the current coordinates:
    c F, RMS-normalised (floor 1e-6) for query coordinates ([paper] App. C.1:
    later calls start from the previous centroids projected this way)."""
    u = np.asarray(cent, dtype=np.float64) @ f
    if not rms:
        return u
    return u / np.maximum(np.sqrt((u * u).mean(axis=1)), 1e-6)[:, None]


def group_means(x, labels, c, fallback):
    """Mean of each group's rows of x (original space); a group with no rows
    takes fallback[c]."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(fallback, dtype=np.float64, copy=True)
    counts = np.bincount(labels, minlength=c)
    for j in range(x.shape[1]):
        sums = np.bincount(labels, weights=x[:, j], minlength=c)
        nz = counts > 0
        out[nz, j] = sums[nz] / counts[nz]
    return out


def sq_distances(x, centers):
    """Squared Euclidean distances, rows of x against centres, written as
    |x|^2 + |c|^2 - 2 x.c (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(centers, dtype=np.float64)
    return (x * x).sum(axis=1)[:, None] + (c * c).sum(axis=1)[None, :] - 2.0 * (x @ c.T)


def kmeans(x, init_idx, iters, init_centers=None):
    """Lloyd's k-means from centres x[init_idx] ([paper] App. C.1: initial
    centres sampled from the feature rows), or from init_centers when given
    (later calls).  Returns (labels of the last assignment, centres after the
    last update, objective per iteration)."""
    x = np.asarray(x, dtype=np.float64)
    if init_centers is not None:
        centers = np.array(init_centers, dtype=np.float64, copy=True)
    else:
        centers = x[np.asarray(init_idx)].copy()
    n_c = centers.shape[0]
    labels = np.zeros(x.shape[0], dtype=np.int64)
    objective = []
    xx = (x * x).sum(axis=1)
    for _ in range(iters):
        # nearest centre by |c|^2 - 2 x.c (|x|^2 is the same for every
        # centre of a row); rows in slices only to bound the temporary
        cc = (centers * centers).sum(axis=1)
        best = np.empty(x.shape[0])
        for i0 in range(0, x.shape[0], 8192):
            part = x[i0:i0 + 8192] @ centers.T
            part *= -2.0
            part += cc[None, :]
            lab = np.argmin(part, axis=1)          # first minimum: smaller index on ties
            labels[i0:i0 + 8192] = lab
            best[i0:i0 + 8192] = part[np.arange(lab.size), lab]
        objective.append(float((best + xx).sum()))
        sums = np.stack([np.bincount(labels, weights=x[:, j], minlength=n_c)
                         for j in range(x.shape[1])], axis=1)
        counts = np.bincount(labels, minlength=n_c)
        nz = counts > 0
        centers[nz] = sums[nz] / counts[nz][:, None]
    return labels, centers, objective


def rcp_partition(q, k, m_s, r_k, c_k, r_q, c_q, init_k, init_q, iters, state=None,
                  subspace_steps=2):
    """Response-coupled partition of one head ([paper] §4.1): K/V groups by
    k-means on key-response coordinates, then query groups by k-means on
    RMS-normalised query-response coordinates built from the K/V group
    centroids.  With `state` (the dict a previous call returned under
    "state") the call is a later call of App. C.1: subspace-iteration factors
    and k-means started from the previous centroids; init_k / init_q are
    then unused.  Returns a dict with labels_kv, labels_q, phi_q, the
    intermediate metrics and factors, and the state for the next call."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    rows = sample_query_rows(q.shape[0], m_s)
    m_k = key_response_metric(q[rows])
    if state is None:
        basis_k, _, f_k = response_basis(m_k, r_k)
    else:
        basis_k, _, f_k = subspace_factor(m_k, state["basis_k"], subspace_steps)
    phi_k = k @ f_k
    if state is None:
        labels_kv, _, obj_k = kmeans(phi_k, init_k, iters)
        fb_k = k[np.asarray(init_k)]
    else:
        fb_k = state["cent_k"]
        labels_kv, _, obj_k = kmeans(phi_k, None, iters,
                                     init_centers=project_centers(fb_k, f_k, False))
    m_q, n_nonempty = query_response_metric(k, labels_kv, c_k)
    if state is None:
        basis_q, _, f_q = response_basis(m_q, r_q)
    else:
        basis_q, _, f_q = subspace_factor(m_q, state["basis_q"], subspace_steps)
    phi_q = query_features(q, f_q)
    if state is None:
        labels_q, _, obj_q = kmeans(phi_q, init_q, iters)
        fb_q = q[np.asarray(init_q)]
    else:
        fb_q = state["cent_q"]
        labels_q, _, obj_q = kmeans(phi_q, None, iters,
                                    init_centers=project_centers(fb_q, f_q, True))
    new_state = {"basis_k": basis_k, "basis_q": basis_q,
                 "cent_k": group_means(k, labels_kv, c_k, fb_k),
                 "cent_q": group_means(q, labels_q, c_q, fb_q)}
    return {
        "rows": rows, "m_k": m_k, "f_k": f_k, "phi_k": phi_k, "labels_kv": labels_kv,
        "m_q": m_q, "n_kv_nonempty": n_nonempty, "f_q": f_q, "phi_q": phi_q,
        "labels_q": labels_q, "objective_k": obj_k, "objective_q": obj_q,
        "state": new_state,
    }
