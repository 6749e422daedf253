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


def response_factor(metric, r):
    """F (d x r): the leading r eigenvectors of the symmetric metric, each
    scaled by the square root of its eigenvalue normalised to unit mean over
    the r retained ([paper] §4.1 and App. B.1)."""
    w, u = np.linalg.eigh(np.asarray(metric, dtype=np.float64))
    order = np.argsort(-w, kind="stable")[:r]
    lam = np.maximum(w[order], 0.0)
    mean = lam.mean() if lam.size else 0.0
    if not mean > 0.0:
        return np.zeros((w.size, len(order)))
    return u[:, order] * np.sqrt(lam / mean)


def query_features(q, f_q, eps=1e-6):
    """phi_Q(q) = u / max(RMS(u), eps) with u = q F_Q ([paper] §4.1 and
    App. B.2: RMS normalisation without gain or bias, floor 1e-6)."""
    u = np.asarray(q, dtype=np.float64) @ f_q
    rms = np.sqrt((u * u).mean(axis=1))
    return u / np.maximum(rms, eps)[:, None]


def sq_distances(x, centers):
    """Squared Euclidean distances, rows of x against centres, written as
    |x|^2 + |c|^2 - 2 x.c (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(centers, dtype=np.float64)
    return (x * x).sum(axis=1)[:, None] + (c * c).sum(axis=1)[None, :] - 2.0 * (x @ c.T)


def kmeans(x, init_idx, iters):
    """Lloyd's k-means from centres x[init_idx] ([paper] App. C.1: initial
    centres sampled from the feature rows).  Returns (labels of the last
    assignment, centres after the last update, objective per iteration)."""
    x = np.asarray(x, dtype=np.float64)
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


def rcp_partition(q, k, m_s, r_k, c_k, r_q, c_q, init_k, init_q, iters):
    """Response-coupled partition of one head ([paper] §4.1): K/V groups by
    k-means on key-response coordinates, then query groups by k-means on
    RMS-normalised query-response coordinates built from the K/V group
    centroids.  Returns a dict with labels_kv, labels_q, phi_q and the
    intermediate metrics and factors."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    rows = sample_query_rows(q.shape[0], m_s)
    m_k = key_response_metric(q[rows])
    f_k = response_factor(m_k, r_k)
    phi_k = k @ f_k
    labels_kv, _, obj_k = kmeans(phi_k, init_k, iters)
    m_q, n_nonempty = query_response_metric(k, labels_kv, c_k)
    f_q = response_factor(m_q, r_q)
    phi_q = query_features(q, f_q)
    labels_q, _, obj_q = kmeans(phi_q, init_q, iters)
    return {
        "rows": rows, "m_k": m_k, "f_k": f_k, "phi_k": phi_k, "labels_kv": labels_kv,
        "m_q": m_q, "n_kv_nonempty": n_nonempty, "f_q": f_q, "phi_q": phi_q,
        "labels_q": labels_q, "objective_k": obj_k, "objective_q": obj_q,
    }
