"""Pins of the response-coupled partitioning oracle (oracle.rcp) against facts
that do not come from the oracle: the metric identities the pages state,
closed forms from constructed spectra, brute force on tiny inputs and
invariants of Lloyd's iteration.

[paper] "Partition the Support, Reconstruct the Residual": §4.1
(response-coupled partitioning), App. B.1 (key response metric), App. B.2
(query response metric, RMS normalisation), App. C.1 (GPU clustering)."""
import itertools

import numpy as np
import pytest

from oracle import rcp


def _orthogonal(d, rng):
    q, r = np.linalg.qr(rng.standard_normal((d, d)))
    return q * np.sign(np.diag(r))


def test_sample_rows_evenly_spaced():
    # [paper] App. B.1: deterministic evenly spaced token positions
    assert rcp.sample_query_rows(10, 4).tolist() == [0, 2, 5, 7]
    assert rcp.sample_query_rows(75600, 256)[[0, 1, 255]].tolist() == [0, 295, 75304]
    # App. C.1: every row when fewer than M_s are available
    assert rcp.sample_query_rows(5, 8).tolist() == [0, 1, 2, 3, 4]


def test_key_metric_is_mean_squared_logit_difference():
    # [paper] App. B.1: (dk)^T M_K (dk) is the mean over the sampled queries of
    # the squared difference of their logits against the two keys; with the
    # full-rank factor, squared coordinate distance is that quantity over the
    # mean eigenvalue (a common positive scale, §4.1)
    rng = np.random.default_rng(0)
    d, ms = 6, 11
    qs = rng.standard_normal((ms, d))
    k1, k2 = rng.standard_normal(d), rng.standard_normal(d)
    mk = rcp.key_response_metric(qs)
    brute = np.mean([(qs[i] @ (k1 - k2)) ** 2 for i in range(ms)])
    assert np.isclose((k1 - k2) @ mk @ (k1 - k2), brute, rtol=1e-12)
    f = rcp.response_factor(mk, d)
    lam_mean = np.trace(mk) / d
    dist = np.sum((k1 @ f - k2 @ f) ** 2)
    assert np.isclose(dist, brute / lam_mean, rtol=1e-10)


def test_response_factor_constructed_spectrum():
    # §4.1: leading r eigenvectors, each weighted by the square root of its
    # eigenvalue normalised to unit mean over the r retained
    rng = np.random.default_rng(1)
    d, r = 8, 3
    v = _orthogonal(d, rng)
    lam = np.array([9.0, 7.0, 4.0, 2.0, 1.0, 0.5, 0.25, 0.0])
    m = v @ np.diag(lam) @ v.T
    f = rcp.response_factor(m, r)
    mean = lam[:r].mean()
    expect = v[:, :r] @ np.diag(lam[:r] / mean) @ v[:, :r].T
    assert np.allclose(f @ f.T, expect, atol=1e-12)
    # columns orthogonal, squared norms the normalised eigenvalues (unit mean)
    g = f.T @ f
    assert np.allclose(g, np.diag(np.diag(g)), atol=1e-12)
    assert np.isclose(np.diag(g).mean(), 1.0)
    # a zero metric gives F = 0 (no division by a zero mean)
    assert not np.any(rcp.response_factor(np.zeros((4, 4)), 2))


def test_query_metric_centred_group_logits():
    # [paper] App. B.2: rows of K~ are non-empty group centroids minus their
    # uniform mean; (dq)^T M_Q (dq) is the mean over groups of the squared
    # difference of the centred logit profiles, each group weighted equally
    rng = np.random.default_rng(2)
    d, n, c_k = 5, 40, 6
    k = rng.standard_normal((n, d))
    labels = rng.integers(0, c_k, n)
    labels[labels == 3] = 4                      # group 3 empty
    mq, ne = rcp.query_response_metric(k, labels, c_k)
    assert ne == c_k - 1
    cents = np.array([k[labels == b].mean(axis=0) for b in range(c_k) if np.any(labels == b)])
    q1, q2 = rng.standard_normal(d), rng.standard_normal(d)
    prof1 = cents @ q1 - np.mean(cents @ q1)     # centred logit profiles over groups
    prof2 = cents @ q2 - np.mean(cents @ q2)
    brute = np.mean((prof1 - prof2) ** 2)
    assert np.isclose((q1 - q2) @ mq @ (q1 - q2), brute, rtol=1e-12)
    # centring keeps the softmax over groups: logits shift by one constant
    p1 = np.exp(cents @ q1 - (cents @ q1).max())
    p2 = np.exp(prof1 - prof1.max())
    assert np.allclose(p1 / p1.sum(), p2 / p2.sum(), rtol=1e-12)


def test_query_features_rms_normalised():
    # App. B.2: each projected query divided by its RMS, floor 1e-6
    rng = np.random.default_rng(3)
    f = rng.standard_normal((6, 4))
    q = rng.standard_normal((10, 6))
    phi = rcp.query_features(q, f)
    assert np.allclose((phi ** 2).mean(axis=1), 1.0)
    u = q @ f
    assert np.allclose(phi * np.sqrt((u ** 2).mean(axis=1))[:, None], u)
    tiny = np.full((1, 6), 1e-9)
    assert np.allclose(rcp.query_features(tiny, f), (tiny @ f) / 1e-6)


def test_sq_distances_match_direct_differences():
    rng = np.random.default_rng(4)
    x, c = rng.standard_normal((9, 5)), rng.standard_normal((4, 5))
    direct = np.array([[np.sum((x[i] - c[j]) ** 2) for j in range(4)] for i in range(9)])
    assert np.allclose(rcp.sq_distances(x, c), direct, rtol=1e-12, atol=1e-12)


def _lloyd_brute(x, centers, iters):
    """Lloyd's iteration written with explicit loops (no shared code)."""
    centers = [np.array(c, dtype=np.float64) for c in centers]
    labels = None
    for _ in range(iters):
        labels = []
        for p in x:
            best, best_d = 0, None
            for j, c in enumerate(centers):
                dd = float(np.sum((p - c) ** 2))
                if best_d is None or dd < best_d:
                    best, best_d = j, dd
            labels.append(best)
        for j in range(len(centers)):
            mem = [x[i] for i in range(len(x)) if labels[i] == j]
            if mem:
                centers[j] = np.mean(mem, axis=0)
    return np.array(labels), np.array(centers)


def test_kmeans_brute_force_small():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(m, 0.6, (7, 3)) for m in (-2.0, 0.0, 2.5)])
    for init in ([0, 1, 2], [3, 10, 20], [0, 0, 15], [19, 4, 4]):
        for iters in (1, 2, 5):
            lab, cen, _ = rcp.kmeans(x, init, iters)
            lab_b, cen_b = _lloyd_brute(x, x[init], iters)
            assert np.array_equal(lab, lab_b)
            assert np.allclose(cen, cen_b, atol=1e-12)


def test_kmeans_objective_non_increasing_and_fixed_point():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((200, 4))
    init = rng.integers(0, 200, 12)
    _, _, obj = rcp.kmeans(x, init, 15)
    assert all(b <= a + 1e-9 for a, b in zip(obj, obj[1:]))
    lab, cen, _ = rcp.kmeans(x, init, 60)
    # at a fixed point every row is nearest to its own centre, which is its mean
    d2 = ((x[:, None, :] - cen[None]) ** 2).sum(-1)
    assert np.array_equal(np.argmin(d2, axis=1), lab)
    for j in np.unique(lab):
        assert np.allclose(cen[j], x[lab == j].mean(axis=0))


def test_kmeans_ties_and_empty_cluster():
    x = np.array([[0.0], [1.0], [4.0], [5.0]])
    # duplicate initial centre: ties go to the smaller index, centre 1 stays empty
    lab, cen, _ = rcp.kmeans(x, [0, 0, 3], 1)
    assert lab.tolist() == [0, 0, 2, 2]
    assert cen[1, 0] == 0.0                       # empty cluster keeps its centre
    assert np.allclose(cen[[0, 2], 0], [0.5, 4.5])
    # a row exactly between two centres goes to the smaller index
    lab, _, _ = rcp.kmeans(np.array([[0.0], [1.0], [2.0]]), [0, 2], 1)
    assert lab.tolist() == [0, 0, 1]


def _ari(a, b):
    """Adjusted Rand index (pair counting, written out)."""
    n = len(a)
    cont = {}
    for x, y in zip(a, b):
        cont[(x, y)] = cont.get((x, y), 0) + 1
    comb = lambda m: m * (m - 1) / 2
    sa = {}
    sb = {}
    for (x, y), c in cont.items():
        sa[x] = sa.get(x, 0) + c
        sb[y] = sb.get(y, 0) + c
    idx = sum(comb(c) for c in cont.values())
    ea, eb = sum(comb(c) for c in sa.values()), sum(comb(c) for c in sb.values())
    exp = ea * eb / comb(n)
    return (idx - exp) / (0.5 * (ea + eb) - exp)


def test_rcp_recovers_planted_response_groups():
    # keys from well-separated components whose logits against the sampled
    # queries differ; with one initial centre per component, the K/V groups
    # are the components, and queries built to prefer one key component each
    # are grouped by that preference (§4.1 construction end to end)
    rng = np.random.default_rng(7)
    d, n, comp = 16, 240, 4
    mu_k = rng.normal(0, 3.0, (comp, d))
    lab_true = np.repeat(np.arange(comp), n // comp)
    k = mu_k[lab_true] + rng.normal(0, 0.1, (n, d))
    q_lab = np.tile(np.arange(comp), n // comp)
    q = 2.0 * mu_k[q_lab] + rng.normal(0, 0.1, (n, d))
    init_k = [int(np.nonzero(lab_true == c)[0][0]) for c in range(comp)]
    init_q = [int(np.nonzero(q_lab == c)[0][0]) for c in range(comp)]
    out = rcp.rcp_partition(q, k, m_s=64, r_k=8, c_k=comp, r_q=8, c_q=comp,
                            init_k=init_k, init_q=init_q, iters=5)
    assert _ari(out["labels_kv"], lab_true) == pytest.approx(1.0)
    assert _ari(out["labels_q"], q_lab) == pytest.approx(1.0)
    assert out["n_kv_nonempty"] == comp
    assert np.allclose((out["phi_q"] ** 2).mean(axis=1), 1.0)


def test_ari_helper_against_brute_pairs():
    # the ARI used by the GPU tests, against its pair-counting definition
    from harness import ari
    rng = np.random.default_rng(8)
    a, b = rng.integers(0, 3, 30), rng.integers(0, 4, 30)
    same_a = [a[i] == a[j] for i, j in itertools.combinations(range(30), 2)]
    same_b = [b[i] == b[j] for i, j in itertools.combinations(range(30), 2)]
    n11 = sum(x and y for x, y in zip(same_a, same_b))
    na, nb, npairs = sum(same_a), sum(same_b), len(same_a)
    expect = (n11 - na * nb / npairs) / (0.5 * (na + nb) - na * nb / npairs)
    assert _ari(a, b) == pytest.approx(expect)
    assert _ari(a, a) == pytest.approx(1.0)
    assert ari(a, b) == pytest.approx(expect)
    assert ari(b + 7, (a * 3) % 5) == pytest.approx(_ari(b + 7, (a * 3) % 5))


# ----------------------------------------------------------------------------
# later calls: subspace-iteration factors and warm-started k-means
# ([paper] App. C.1)
# ----------------------------------------------------------------------------

def _spd(d, lam, rng):
    v = _orthogonal(d, rng)
    return v @ np.diag(lam) @ v.T, v


def _projector(x):
    qx, _ = np.linalg.qr(x)
    return qx @ qx.T


def test_cholesky_drop_matches_numpy_and_drops_dependent_columns():
    rng = np.random.default_rng(40)
    y = rng.standard_normal((9, 5))
    g = y.T @ y
    low = rcp.cholesky_drop(g)
    assert np.allclose(low, np.linalg.cholesky(g), atol=1e-12)
    # column 3 a combination of columns 0 and 1: its pivot vanishes
    y[:, 3] = 2.0 * y[:, 0] - y[:, 1]
    low = rcp.cholesky_drop(y.T @ y)
    assert not np.any(low[:, 3])
    x = rcp.cholesky_orthonormalise(y)
    assert not np.any(x[:, 3])
    keep = [0, 1, 2, 4]
    assert np.allclose(x[:, keep].T @ x[:, keep], np.eye(4), atol=1e-12)
    # the kept columns span Y's column space
    assert np.allclose(x @ (x.T @ y), y, atol=1e-10)
    # Gram-Schmidt order: column j lies in the span of Y's first j+1 columns
    for j in keep:
        sub = y[:, :j + 1]
        assert np.allclose(sub @ np.linalg.lstsq(sub, x[:, j], rcond=None)[0], x[:, j], atol=1e-10)


def test_subspace_factor_fixed_point_at_eigenbasis():
    # from the exact leading eigenvectors of an unchanged metric, M U = U Lam,
    # the Cholesky factor is Lam and the basis, weights and factor repeat
    rng = np.random.default_rng(41)
    lam = np.array([9.0, 6.0, 4.0, 2.5, 1.0, 0.5, 0.2, 0.1])
    m, _ = _spd(8, lam, rng)
    u, lam_r, f = rcp.response_basis(m, 3)
    x, lam_x, f_x = rcp.subspace_factor(m, u, steps=2)
    assert np.allclose(x, u, atol=1e-12)
    assert np.allclose(lam_x, lam[:3], rtol=1e-12)
    assert np.allclose(f_x, f, atol=1e-12)


def test_subspace_two_steps_span_m_squared_start():
    # two orthogonal-iteration steps span M^2 X0, with orthonormal columns
    rng = np.random.default_rng(42)
    m, _ = _spd(10, np.linspace(5.0, 0.5, 10), rng)
    x0 = rng.standard_normal((10, 4))
    x, lam_x, _ = rcp.subspace_factor(m, x0, steps=2)
    assert np.allclose(x.T @ x, np.eye(4), atol=1e-12)
    assert np.allclose(_projector(x), _projector(m @ m @ x0), atol=1e-10)
    assert np.allclose(lam_x, [x[:, j] @ m @ x[:, j] for j in range(4)], rtol=1e-12)


def test_subspace_converges_to_eigen_factor_full_and_deficient_rank():
    rng = np.random.default_rng(43)
    # distinct eigenvalues with a gap after the third
    m, _ = _spd(7, np.array([8.0, 5.0, 3.0, 0.4, 0.3, 0.2, 0.1]), rng)
    x, _, f = rcp.subspace_factor(m, rng.standard_normal((7, 3)), steps=300)
    f_ref = rcp.response_factor(m, 3)
    assert np.allclose(f @ f.T, f_ref @ f_ref.T, atol=1e-9)
    # rank 2 metric asked for 4 directions: two columns drop, the weights of
    # the rest are the eigenvalues over the mean of all 4 (zeros included)
    m2, _ = _spd(6, np.array([3.0, 1.0, 0.0, 0.0, 0.0, 0.0]), rng)
    x, lam_x, f = rcp.subspace_factor(m2, rng.standard_normal((6, 4)), steps=300)
    assert int(np.sum(np.any(x != 0.0, axis=0))) == 2
    f_ref = rcp.response_factor(m2, 4)
    assert np.allclose(f @ f.T, f_ref @ f_ref.T, atol=1e-9)
    # a rotated basis of the exact eigenspace: the span and the trace of the
    # Rayleigh quotients are kept after two steps
    u, lam_r, _ = rcp.response_basis(m, 3)
    rot = _orthogonal(3, rng)
    x, lam_x, _ = rcp.subspace_factor(m, u @ rot, steps=2)
    assert np.allclose(_projector(x), u @ u.T, atol=1e-10)
    assert np.isclose(lam_x.sum(), lam_r.sum(), rtol=1e-12)


def test_project_centers_and_group_means_by_loops():
    rng = np.random.default_rng(44)
    c, f = rng.standard_normal((5, 6)), rng.standard_normal((6, 3))
    lin = rcp.project_centers(c, f, False)
    for i in range(5):
        u = [sum(c[i, a] * f[a, j] for a in range(6)) for j in range(3)]
        assert np.allclose(lin[i], u)
        rms = np.sqrt(np.mean(np.square(u)))
        assert np.allclose(rcp.project_centers(c, f, True)[i], np.array(u) / rms)
    x = rng.standard_normal((12, 3))
    labels = np.array([0, 2, 2, 0, 3, 3, 3, 0, 2, 2, 0, 3])       # group 1 empty
    fb = rng.standard_normal((4, 3))
    g = rcp.group_means(x, labels, 4, fb)
    for b in range(4):
        rows = [x[i] for i in range(12) if labels[i] == b]
        assert np.allclose(g[b], np.mean(rows, axis=0) if rows else fb[b])


def _planted(rng, d=16, n=240, comp=4):
    mu_k = rng.normal(0, 3.0, (comp, d))
    lab = np.repeat(np.arange(comp), n // comp)
    k = mu_k[lab] + rng.normal(0, 0.1, (n, d))
    q_lab = np.tile(np.arange(comp), n // comp)
    q = 2.0 * mu_k[q_lab] + rng.normal(0, 0.1, (n, d))
    return q, k, lab, q_lab


def test_warm_call_on_unchanged_inputs_repeats_the_partition():
    # a converged first call leaves bases that are a fixed point of the
    # subspace iteration and key centroids that map to the k-means centres,
    # so one Lloyd iteration of the later call gives the same K/V groups; the
    # query centres differ only by the RMS step (same groups when separated)
    rng = np.random.default_rng(45)
    q, k, lab, q_lab = _planted(rng)
    init_k = [0, 70, 130, 200]
    init_q = [0, 1, 2, 3]
    cold = rcp.rcp_partition(q, k, m_s=64, r_k=6, c_k=4, r_q=3, c_q=4, init_k=init_k,
                             init_q=init_q, iters=30)
    warm = rcp.rcp_partition(q, k, m_s=64, r_k=6, c_k=4, r_q=3, c_q=4, init_k=None, init_q=None,
                             iters=1, state=cold["state"])
    assert np.array_equal(warm["labels_kv"], cold["labels_kv"])
    assert np.allclose(warm["f_k"] @ warm["f_k"].T, cold["f_k"] @ cold["f_k"].T, atol=1e-10)
    assert _ari(warm["labels_q"], cold["labels_q"]) == pytest.approx(1.0)
    # the state's key centroids are the group means in the original space
    for b in range(4):
        assert np.allclose(cold["state"]["cent_k"][b], k[cold["labels_kv"] == b].mean(axis=0))


def test_state_of_an_empty_group_is_its_initial_row_then_kept():
    x = np.array([[0.0], [1.0], [4.0], [5.0]])
    k = np.concatenate([x, 0.5 * x], axis=1)
    q = k.copy()
    # duplicate initial rows: K/V group 1 is empty after one iteration (ties
    # go to the smaller index)
    cold = rcp.rcp_partition(q, k, m_s=4, r_k=1, c_k=3, r_q=1, c_q=2, init_k=[0, 0, 3],
                             init_q=[0, 3], iters=1)
    assert not np.any(cold["labels_kv"] == 1)
    assert np.allclose(cold["state"]["cent_k"][1], k[0])
    warm = rcp.rcp_partition(q, k, m_s=4, r_k=1, c_k=3, r_q=1, c_q=2, init_k=None, init_q=None,
                             iters=2, state=cold["state"])
    # the later call starts group 1 at that row, which then takes row 0
    assert np.array_equal(warm["labels_kv"], [1, 0, 2, 2])
    assert np.allclose(warm["state"]["cent_k"][1], k[0])
    assert np.allclose(warm["state"]["cent_k"][0], k[1])
