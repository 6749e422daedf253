"""Pins of the CPU oracle against facts that do not come from the oracle:
hand-worked examples (tests/golden), closed forms, brute force on tiny
inputs, invariants and library routines used along a different route.

Each test names the passage it follows (page title + section)."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthgen as sg

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_kv(name):
    out, cases = {}, []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("case"):
                cases.append([p.strip() for p in line[4:].split("|")])
            else:
                k, v = line.split("=", 1)
                out[k.strip()] = v.split()
    return out, cases


# ----------------------------------------------------------------------------
# F1 layout and centroids
# ----------------------------------------------------------------------------

def _brute_layout(labels, C):
    perm, offs = [], [0]
    for a in range(C):
        for i, l in enumerate(labels):
            if l == a:
                perm.append(i)
        offs.append(len(perm))
    return perm, offs


@pytest.mark.parametrize("seed", range(6))
def test_layout_brute_force(seed):
    """SparsePR paper §3 problem setup / rainbus review step (3): group-major
    permutation with per-group offsets; empty groups keep equal offsets."""
    rng = np.random.default_rng(seed)
    C = int(rng.integers(1, 9))
    n = int(rng.integers(1, 60))
    labels = rng.integers(0, C, size=n)
    if seed % 2:   # force some empty groups
        labels = labels % max(1, C // 2)
    perm, offs = oracle.group_layout(labels, C)
    bp, bo = _brute_layout(labels.tolist(), C)
    assert perm.tolist() == bp
    assert offs.tolist() == bo
    assert sorted(perm.tolist()) == list(range(n))


def test_group_means_brute_force():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, 5))
    labels = rng.integers(0, 6, size=40)
    labels[labels == 4] = 0          # group 4 empty
    mu = oracle.group_means(x, labels, 6)
    for a in range(6):
        rows = [i for i in range(40) if labels[i] == a]
        if not rows:
            assert np.isnan(mu[a]).all()
            continue
        for j in range(5):
            acc = 0.0
            for i in rows:
                acc += x[i, j]
            assert abs(mu[a, j] - acc / len(rows)) < 1e-12


# ----------------------------------------------------------------------------
# budgets and density (closed forms worked by hand)
# ----------------------------------------------------------------------------

def test_budgets_closed_form():
    """SparsePR paper §4.3: routed budget = (rho - M/N_q) * N_q * N_k.  Values
    worked by hand: (0.26*4096-64)*4096 = 4099932.16 -> 4099933;
    (0.26*17550-64)*17550 = 4499*17550; (0.22*75600-64)*75600 = 16568*75600;
    (0.26*118800-64)*118800 = 30824*118800."""
    assert oracle.routed_pair_budget("0.26", 4096, 4096, 64) == 4099933
    assert oracle.routed_pair_budget("0.26", 17550, 17550, 64) == 4499 * 17550
    assert oracle.routed_pair_budget("0.22", 75600, 75600, 64) == 16568 * 75600
    assert oracle.routed_pair_budget("0.26", 118800, 118800, 64) == 30824 * 118800
    # reserve + routed budget reaches the executed target
    assert 4099933 + 64 * 4096 == math.ceil(Fraction("0.26") * 4096 * 4096)
    # fewer tokens than probes: budget clamps at zero
    assert oracle.routed_pair_budget("0.01", 50, 50, 64) == 0


def test_probe_fraction_golden():
    """SparsePR paper App. A.2: probes add M/N_q, 0.054% at the longest
    evaluated sequence."""
    kv, _ = _read_kv("probe_fraction.txt")
    m, n = int(kv["m"][0]), int(kv["n_q"][0])
    frac = oracle.executed_density(0, n, n, m)
    assert round(float(frac) * 100, 3) == float(kv["percent_rounded_3dp"][0])


def test_executed_density_identity():
    """SparsePR paper §4.3: rho_exec = rho_route + M/N_q."""
    rho = oracle.executed_density(123456, 700, 900, 64)
    assert rho == Fraction(123456, 700 * 900) + Fraction(64, 700)
    assert oracle.executed_density(10, 30, 40, 64) == Fraction(10, 1200) + 1


# ----------------------------------------------------------------------------
# F2 routing
# ----------------------------------------------------------------------------

def test_route_golden():
    kv, cases = _read_kv("route_example.txt")
    qbar = np.array([[float(t) for t in kv[f"qbar{a}"]] for a in range(3)])
    kbar = np.array([[float(t) for t in kv[f"kbar{b}"]] for b in range(3)])
    n_a = [int(t) for t in kv["n_a"]]
    m_b = [int(t) for t in kv["m_b"]]
    forced = {(0, 0), (1, 1), (2, 2)}
    for budget, extra, routed in cases:
        z, pairs, _ = oracle.route_cells(qbar, kbar, n_a, m_b, int(budget), 4)
        want = set(forced)
        if extra != "-":
            want |= {tuple(int(t) for t in c.split(",")) for c in extra.split()}
        got = {(int(a), int(b)) for a, b in zip(*np.nonzero(z))}
        assert got == want, budget
        assert pairs == int(routed)


def _brute_route(qbar, kbar, n_a, m_b, budget, d):
    Cq, Ck = len(n_a), len(m_b)
    s = {}
    for a in range(Cq):
        for b in range(Ck):
            if n_a[a] and m_b[b]:
                s[(a, b)] = sum(qbar[a][j] * kbar[b][j] for j in range(d)) / math.sqrt(d)
    sel, pairs = set(), 0
    for a in range(Cq):
        if not n_a[a]:
            continue
        best = None
        for b in range(Ck):
            if (a, b) in s and (best is None or s[(a, b)] > s[(a, best)]):
                best = b
        if best is not None:
            sel.add((a, best))
            pairs += n_a[a] * m_b[best]
    rest = sorted((c for c in s if c not in sel), key=lambda c: (-s[c], c[0], c[1]))
    for c in rest:
        if pairs >= budget:
            break
        sel.add(c)
        pairs += n_a[c[0]] * m_b[c[1]]
    return sel, pairs


@pytest.mark.parametrize("seed", range(12))
def test_route_brute_force_with_ties(seed):
    """Brute-force walk of the rule on tiny inputs.  Integer centroids make
    many scores tie exactly, exercising the (a, b) tie order."""
    rng = np.random.default_rng(100 + seed)
    Cq, Ck, d = int(rng.integers(1, 6)), int(rng.integers(1, 7)), 4
    qbar = rng.integers(-2, 3, size=(Cq, d)).astype(float)
    kbar = rng.integers(-2, 3, size=(Ck, d)).astype(float)
    n_a = rng.integers(0, 5, size=Cq)
    m_b = rng.integers(0, 5, size=Ck)
    if n_a.sum() == 0:
        n_a[0] = 1
    if m_b.sum() == 0:
        m_b[-1] = 2
    total = int(n_a.sum() * m_b.sum())
    for budget in sorted({0, 1, total // 3, total // 2, total - 1, total, total + 5}):
        z, pairs, _ = oracle.route_cells(qbar, kbar, n_a, m_b, budget, d)
        sel, bp = _brute_route(qbar.tolist(), kbar.tolist(), n_a.tolist(), m_b.tolist(), budget, d)
        got = {(int(a), int(b)) for a, b in zip(*np.nonzero(z))}
        assert got == sel
        assert pairs == bp


@pytest.mark.parametrize("seed", range(5))
def test_route_invariants(seed):
    """Invariants of the greedy rule: every non-empty query group keeps a
    cell; no empty group is touched; the budget is reached unless every
    cell is taken; dropping the last greedy cell falls short (minimality)."""
    rng = np.random.default_rng(seed)
    Cq, Ck, d = 7, 9, 8
    qbar = rng.standard_normal((Cq, d))
    kbar = rng.standard_normal((Ck, d))
    n_a = rng.integers(0, 20, size=Cq)
    m_b = rng.integers(0, 20, size=Ck)
    n_a[0] = 0
    m_b[1] = 0
    total = int(n_a.sum() * m_b.sum())
    for frac in (0.0, 0.1, 0.3, 0.6, 1.0, 1.2):
        budget = int(frac * total)
        z, pairs, s = oracle.route_cells(qbar, kbar, n_a, m_b, budget, d)
        assert not z[n_a == 0].any() and not z[:, m_b == 0].any()
        for a in np.nonzero(n_a)[0]:
            assert z[a].any()
        assert pairs == int((z * np.outer(n_a, m_b)).sum())
        if pairs < budget:
            assert z[np.ix_(n_a > 0, m_b > 0)].all()
        # minimality: the lowest-ranked greedy cell was needed
        forced = set()
        for a in np.nonzero(n_a)[0]:
            cand = [b for b in range(Ck) if m_b[b]]
            forced.add((a, max(cand, key=lambda b: (s[a, b], -b))))
        greedy = [(a, b) for a, b in zip(*np.nonzero(z)) if (a, b) not in forced]
        if greedy:
            last = min(greedy, key=lambda c: (s[c], -c[0], -c[1]))
            assert pairs - n_a[last[0]] * m_b[last[1]] < budget


# ----------------------------------------------------------------------------
# F3 sparse attention
# ----------------------------------------------------------------------------

def _brute_row(q, keys, vals, scale):
    logits = [sum(q[j] * k[j] for j in range(len(q))) * scale for k in keys]
    mx = max(logits)
    e = [math.exp(x - mx) for x in logits]
    den = sum(e)
    return [sum(e[i] * vals[i][j] for i in range(len(keys))) / den for j in range(len(vals[0]))]


@pytest.mark.parametrize("seed", range(4))
def test_sparse_attention_brute_force(seed):
    """SparsePR paper §3: renormalised hard drop over the keys of selected
    groups, written out with explicit loops."""
    rng = np.random.default_rng(seed)
    n, d, Cq, Ck = 14, 4, 3, 4
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    lq = rng.integers(0, Cq, size=n)
    lk = rng.integers(0, Ck, size=n)
    z = rng.random((Cq, Ck)) < 0.5
    for a in range(Cq):
        z[a, lk[a % n]] = True       # at least one non-empty selected group
    out, _ = oracle.sparse_attention(q, lq, k, v, lk, z, 0.5)
    for i in range(n):
        keys = [j for j in range(n) if z[lq[i], lk[j]]]
        want = _brute_row(q[i], k[keys], v[keys], 0.5)
        assert np.allclose(out[i], want, rtol=1e-12, atol=1e-12)


def test_full_selection_is_dense():
    """SparsePR paper §3: selecting every cell recovers dense attention."""
    rng = np.random.default_rng(7)
    n, d = 50, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    lq = rng.integers(0, 5, size=n)
    lk = rng.integers(0, 6, size=n)
    z = np.ones((5, 6), bool)
    out, lse = oracle.sparse_attention(q, lq, k, v, lk, z, 1 / math.sqrt(d))
    dense, dlse = oracle.dense_attention_rows(q, k, v, 1 / math.sqrt(d))
    assert np.allclose(out, dense, atol=1e-13)
    assert np.allclose(lse, dlse, atol=1e-13)


def test_single_key_cell_returns_value():
    rng = np.random.default_rng(8)
    n, d = 9, 4
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    lq = np.zeros(n, int)
    lk = np.arange(n) % 3
    lk[5] = 3                        # group 3 holds only key 5
    z = np.zeros((1, 4), bool)
    z[0, 3] = True
    out, lse = oracle.sparse_attention(q, lq, k, v, lk, z, 0.5)
    assert np.allclose(out, v[5][None, :], atol=1e-15)
    assert np.allclose(lse, q @ k[5] * 0.5, atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_hard_drop_residual_identity(seed):
    """SparsePR paper App. A.1: with omitted mass p_U and the output O_U
    renormalised over the omitted keys, O_dense = (1 - p_U) O_sp + p_U O_U,
    so R = p_U (O_U - O_sp).  p_U and O_U are computed here by loops."""
    rng = np.random.default_rng(seed)
    n, d = 30, 6
    q, k, v = (rng.standard_normal((n, d)) * 1.5 for _ in range(3))
    lq = rng.integers(0, 3, size=n)
    lk = rng.integers(0, 5, size=n)
    z = rng.random((3, 5)) < 0.4
    for a in range(3):
        z[a, lk[a]] = True
    sc = 1 / math.sqrt(d)
    o_sp, _ = oracle.sparse_attention(q, lq, k, v, lk, z, sc)
    dense, _ = oracle.dense_attention_rows(q, k, v, sc)
    for i in range(n):
        omitted = [j for j in range(n) if not z[lq[i], lk[j]]]
        if not omitted:
            assert np.allclose(dense[i], o_sp[i], atol=1e-13)
            continue
        logit = [float(q[i] @ k[j]) * sc for j in range(n)]
        e = [math.exp(x) for x in logit]
        p_u = sum(e[j] for j in omitted) / sum(e)
        o_u = sum(e[j] * v[j] for j in omitted) / sum(e[j] for j in omitted)
        assert np.allclose(dense[i], (1 - p_u) * o_sp[i] + p_u * o_u, atol=1e-12)
        assert np.allclose(dense[i] - o_sp[i], p_u * (o_u - o_sp[i]), atol=1e-12)


def test_dense_rows_match_torch_sdpa():
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((17, 64)) for _ in range(3))
    out, _ = oracle.dense_attention_rows(q, k, v, 1 / 8)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0]
    assert np.allclose(out, ref.numpy(), atol=1e-12)


# ----------------------------------------------------------------------------
# F5 probes (Algorithm A.1)
# ----------------------------------------------------------------------------

def test_probes_golden():
    kv, cases = _read_kv("probe_example.txt")
    labels = np.array([int(t) for t in kv["labels"]])
    feats = np.array([[float(t)] for t in kv["features"]])
    sizes = np.bincount(labels, minlength=4)
    for m, probes, counts, weights in cases:
        p, c = oracle.select_probes(feats, labels, 4, int(m))
        assert p.tolist() == [int(t) for t in probes.split()]
        assert c.tolist() == [int(t) for t in counts.split()]
        w = oracle.probe_weights(labels[p], sizes, c)
        assert np.allclose(w, [float(t) for t in weights.split()], rtol=0, atol=1e-15)


def test_probe_distance_gap_hand_values():
    # the golden example above: group 2's two rows tie at distance 2 -> gap 0
    kv, _ = _read_kv("probe_example.txt")
    labels = np.array([int(t) for t in kv["labels"]])
    feats = np.array([[float(t)] for t in kv["features"]])
    for m in (5, 8, 20):
        _, c = oracle.select_probes(feats, labels, 4, m)
        assert oracle.probe_distance_gap(feats, labels, c) == 0.0
    # groups 0 and 1 only (distances 0,1,2,3 and 1,2,3), M = 3 takes two rows of
    # group 0 and one of group 1: the decided gaps are all 1
    keep = labels <= 1
    _, c = oracle.select_probes(feats[keep], labels[keep], 2, 3)
    assert c.tolist() == [2, 1]
    assert oracle.probe_distance_gap(feats[keep], labels[keep], c) == 1.0
    # one row per group: nothing to decide
    assert oracle.probe_distance_gap(np.zeros((2, 1)), np.array([0, 1]), np.array([1, 1])) == math.inf


def _brute_probes(f, labels, C, M):
    n = len(labels)
    order = {}
    for a in range(C):
        rows = [i for i in range(n) if labels[i] == a]
        if not rows:
            continue
        c = [sum(f[i][j] for i in rows) / len(rows) for j in range(len(f[0]))]
        dist = {i: math.sqrt(sum((f[i][j] - c[j]) ** 2 for j in range(len(c)))) for i in rows}
        order[a] = sorted(rows, key=lambda i: (dist[i], i))
    groups = sorted(order, key=lambda a: (-len(order[a]), a))
    out, t = [], 0
    while len(out) < min(M, n):
        for a in groups:
            if t < len(order[a]) and len(out) < min(M, n):
                out.append(order[a][t])
        t += 1
    return out


@pytest.mark.parametrize("seed", range(8))
def test_probes_brute_force(seed):
    rng = np.random.default_rng(seed)
    n, d, C = int(rng.integers(3, 40)), 3, int(rng.integers(1, 9))
    f = rng.integers(-3, 4, size=(n, d)).astype(float)   # integer features: ties
    labels = rng.integers(0, C, size=n)
    for M in (1, 4, 7, 64):
        p, c = oracle.select_probes(f, labels, C, M)
        assert p.tolist() == _brute_probes(f.tolist(), labels.tolist(), C, M)
        assert c.sum() == min(M, n)
        assert len(set(p.tolist())) == len(p)


def test_probes_many_groups_take_nearest_of_largest():
    """SparsePR paper App. A.2: with at least M non-empty groups, the probes
    are the row nearest the centroid in each of the M largest groups."""
    rng = np.random.default_rng(4)
    n, d, C, M = 2000, 6, 100, 64
    f = rng.standard_normal((n, d))
    labels = rng.integers(0, C, size=n)
    p, c = oracle.select_probes(f, labels, C, M)
    sizes = np.bincount(labels, minlength=C)
    largest = sorted(range(C), key=lambda a: (-sizes[a], a))[:M]
    assert [int(labels[i]) for i in p] == largest
    for i in p:
        rows = np.nonzero(labels == labels[i])[0]
        cen = f[rows].mean(axis=0)
        dist = np.linalg.norm(f[rows] - cen, axis=1)
        assert i == rows[np.argmin(dist)]


def test_probes_tiny_and_cogvideox_workloads():
    """32 groups and M = 64 -> two full traversals (2 per group); 64 groups
    -> one probe per group."""
    w = sg.workload("tiny_fp32")
    hd = sg.make_head(w, 0)
    _, c = oracle.select_probes(hd["q"], hd["labels_q"], w.c_q, w.m)
    assert c.tolist() == [2] * 32
    w2 = sg.workload("cogvideox")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w2.seed, 0])))
    labels = rng.integers(0, w2.components, size=w2.n)
    f = np.random.default_rng(0).standard_normal((w2.n, 4))
    _, c2 = oracle.select_probes(f, labels, w2.c_q, w2.m)
    assert c2.tolist() == [1] * 64


# ----------------------------------------------------------------------------
# F4 fit
# ----------------------------------------------------------------------------

def _rand_fit_case(seed, M=64, d=16):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, d)) * rng.uniform(0.2, 3.0, size=d) + rng.standard_normal(d)
    R = x @ rng.standard_normal((d, d)) * 0.1 + rng.standard_normal((M, d)) * 0.05
    w = rng.uniform(0.5, 4.0, size=M)
    return x, R, w


def _standardise(x, R, w):
    """Weighted statistics written from the definitions (unit-sum weights)."""
    wh = w / w.sum()
    mu_x = (wh[:, None] * x).sum(0)
    mu_r = (wh[:, None] * R).sum(0)
    var = (wh[:, None] * (x - mu_x) ** 2).sum(0)
    return (x - mu_x) / np.sqrt(var + 1e-6), R - mu_r, len(w) * w / w.sum()


def test_fit_d1_golden():
    kv, _ = _read_kv("fit_d1_example.txt")
    x = np.array([[float(t)] for t in kv["x"]])
    R = np.array([[float(t)] for t in kv["R"]])
    w = np.array([float(t) for t in kv["w"]])
    lam = float(kv["lam"][0])
    fit = oracle.fit_correction(x, R, w, lam, rank=1)
    s = math.sqrt(1.000001)
    B = (2 / s) / (2 / s ** 2 + lam)
    assert abs(fit["mu_x"][0] - 1) < 1e-15 and abs(fit["mu_R"][0] - 2) < 1e-15
    assert abs(fit["s"][0] - s) < 1e-15
    assert abs(fit["B"][0, 0] - B) < 1e-14
    o = np.array([[0.5], [3.0]])
    corr = oracle.apply_correction(o, fit)
    assert np.allclose(corr - o, 2 + (o - 1) / s * B, atol=1e-14)


@pytest.mark.parametrize("seed", range(3))
def test_fit_augmented_least_squares(seed):
    """SparsePR paper App. A.2: the ridge objective with unit-mean weights is
    an ordinary least-squares problem on [sqrt(W~) Xbar; sqrt(lam) I] B =
    [sqrt(W~) Rbar; 0]; solved by lstsq (not the normal equations)."""
    x, R, w = _rand_fit_case(seed)
    fit = oracle.fit_correction(x, R, w, 0.1, rank=16)
    xb, rb, wt = _standardise(x, R, w)
    d = x.shape[1]
    A = np.vstack([np.sqrt(wt)[:, None] * xb, math.sqrt(0.1) * np.eye(d)])
    Y = np.vstack([np.sqrt(wt)[:, None] * rb, np.zeros((d, d))])
    B = np.linalg.lstsq(A, Y, rcond=None)[0]
    assert np.allclose(fit["B"], B, atol=1e-10)


def test_fit_dual_form_and_normal_equations():
    x, R, w = _rand_fit_case(11, M=20, d=30)   # d > M: rank-deficient Gram
    lam = 0.1
    fit = oracle.fit_correction(x, R, w, lam, rank=16)
    xb, rb, wt = _standardise(x, R, w)
    Xw = np.sqrt(wt)[:, None] * xb
    Rw = np.sqrt(wt)[:, None] * rb
    B_dual = Xw.T @ np.linalg.solve(Xw @ Xw.T + lam * np.eye(len(w)), Rw)
    assert np.allclose(fit["B"], B_dual, atol=1e-10)
    resid = (Xw.T @ Xw + lam * np.eye(x.shape[1])) @ fit["B"] - Xw.T @ Rw
    assert np.abs(resid).max() < 1e-10


def test_fit_subspace_properties():
    """Psi orthonormal; Psi Psi^T equals the projector on the top eigenvectors
    of Y^T Y (eigh, a different routine from the SVD used inside); rows of B
    lie in the row space of Rbar, so rank >= rank(Rbar) reproduces the
    unprojected estimator (SparsePR paper App. D.3 reference estimator)."""
    x, R, w = _rand_fit_case(5, M=64, d=32)
    fit = oracle.fit_correction(x, R, w, 0.1, rank=8)
    Psi = fit["Psi"]
    assert np.allclose(Psi.T @ Psi, np.eye(8), atol=1e-12)
    _, rb, wt = _standardise(x, R, w)
    Y = np.sqrt(wt)[:, None] * rb
    evals, evecs = np.linalg.eigh(Y.T @ Y)
    top = evecs[:, ::-1][:, :8]
    assert np.allclose(Psi @ Psi.T, top @ top.T, atol=1e-9)
    # rowspace property
    P_row = np.linalg.pinv(rb) @ rb
    assert np.allclose(fit["B"] @ P_row, fit["B"], atol=1e-9)
    full = oracle.fit_correction(x, R, w, 0.1, rank=64)
    o = np.random.default_rng(1).standard_normal((10, 32))
    xb = (o - full["mu_x"]) / full["s"]
    unprojected = o + full["mu_R"] + xb @ full["B"]
    assert np.allclose(oracle.apply_correction(o, full), unprojected, atol=1e-10)


def test_fit_limits():
    """lambda -> infinity: B -> 0, the mean-only correction (SparsePR paper
    App. D.4).  Constant residual: Rbar = 0, no direction kept, correction
    = mu_R, no NaN.  Weight normalisations: unit sum and unit mean."""
    x, R, w = _rand_fit_case(2)
    fit = oracle.fit_correction(x, R, w, 1e12, rank=16)
    assert np.abs(fit["B"]).max() < 1e-9
    assert abs(fit["w_hat"].sum() - 1) < 1e-14 and abs(fit["w_til"].mean() - 1) < 1e-14
    fit_z = oracle.fit_correction(x, np.zeros((64, 16)), w, 0.1, rank=16)
    assert fit_z["Psi"].shape[1] == 0 and np.all(fit_z["B"] == 0)
    Rc = np.tile(np.arange(16.0), (64, 1))
    fit0 = oracle.fit_correction(x, Rc, w, 0.1, rank=16)
    o = np.random.default_rng(0).standard_normal((5, 16))
    out = oracle.apply_correction(o, fit0)
    assert np.all(np.isfinite(out)) and np.allclose(out, o + np.arange(16.0), atol=1e-12)


def test_fold_matches_apply():
    x, R, w = _rand_fit_case(3)
    fit = oracle.fit_correction(x, R, w, 0.1, rank=5)
    A, Psi, c, T = oracle.fold_correction(fit)
    o = np.random.default_rng(5).standard_normal((7, 16))
    assert np.allclose(o + (o @ A) @ Psi.T + c, oracle.apply_correction(o, fit), atol=1e-12)
    assert np.allclose(o @ T, (o @ A) @ Psi.T, atol=1e-12)


# ----------------------------------------------------------------------------
# F6 whole call
# ----------------------------------------------------------------------------

def test_whole_call_closed_forms():
    """Probe rows output their dense rows exactly (rainbus review step (5));
    at full density the call equals dense attention (R = 0 -> mu_R = 0,
    B = 0); executed density = routed + M/N_q."""
    w = sg.small_workload(heads=1, n=300, head_dim=16, components=6, kv_split=2,
                          dtype="f32", rho="0.4", m=16, r=4)
    hd = sg.make_head(w, 0)
    r = oracle.run_head(hd["q"], hd["k"], hd["v"], hd["labels_q"], hd["labels_kv"],
                        w.c_q, w.c_k, w.rho, m=w.m, rank=w.r)
    dense, _ = oracle.dense_attention_rows(hd["q"], hd["k"], hd["v"], r["scale"])
    assert np.array_equal(r["out"][r["probes"]], r["dense_p"])
    assert np.allclose(r["dense_p"], dense[r["probes"]], atol=1e-13)
    assert r["routed_pairs"] >= r["budget"]
    rho = oracle.executed_density(r["routed_pairs"], w.n, w.n, w.m)
    assert rho == Fraction(r["routed_pairs"], w.n ** 2) + Fraction(w.m, w.n)
    full = oracle.run_head(hd["q"], hd["k"], hd["v"], hd["labels_q"], hd["labels_kv"],
                           w.c_q, w.c_k, w.rho, m=w.m, rank=w.r, budget=w.n * w.n)
    assert full["z"].all() and full["routed_pairs"] == w.n * w.n
    assert np.allclose(full["out"], dense, atol=1e-12)
    assert np.abs(full["R_p"]).max() < 1e-13


def test_generator_shapes_and_labels():
    w = sg.small_workload(heads=1, n=333, components=5, kv_split=4, grid=(3, 3, 37))
    hd = sg.make_head(w, 0)
    assert hd["q"].shape == (333, 64) and hd["q_bits"].dtype == np.uint16
    assert np.array_equal(sg.bf16_bits_to_f32(hd["q_bits"]), hd["q"])
    lq, lk = hd["labels_q"], hd["labels_kv"]
    assert np.array_equal(lk // 4, lq)
    for c in range(5):
        idx = np.nonzero(lq == c)[0]
        sub = lk[idx] % 4
        assert np.all(np.diff(sub) >= 0)       # consecutive runs in token order
        n = idx.size
        for j in range(4):
            assert np.count_nonzero(sub == j) == (j + 1) * n // 4 - j * n // 4
    # bf16 rounding is nearest-even
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5e-5], dtype=np.float32)
    b = sg.f32_to_bf16_bits(x)
    assert sg.bf16_bits_to_f32(b).tolist()[:3] == [1.0, 1.0, 1.015625]


# ----------------------------------------------------------------------------
# estimator variants ([paper] §5 Table 4, App. D.4)
# ----------------------------------------------------------------------------

def _est_case(seed=21, M=12, d=5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, d))
    R = 0.3 * x @ rng.standard_normal((d, d)) + 0.1 * rng.standard_normal((M, d))
    w = rng.uniform(0.5, 3.0, M)
    return x, R, w


def _objective(xb, Rb, w_til, B, lam):
    res = Rb - xb @ B
    return float(np.sum(w_til[:, None] * res * res) + lam * np.sum(B * B))


def test_scalar_estimator_minimises_penalised_objective():
    # the scalar variant minimises the common objective over B = a I, so the
    # penalty is lam * d * a^2 (Table 4 note); brute check of the minimum
    x, R, w = _est_case()
    lam = 0.7
    e = oracle.fit_estimator(x, R, w, lam, "scalar")
    xb = (x - e["mu_x"]) / e["s"]
    Rb = R - e["mu_R"]
    a = e["b"][0]
    d = x.shape[1]
    f = lambda t: _objective(xb, Rb, e["w_til"], t * np.eye(d), lam)
    grid = np.linspace(a - 1.0, a + 1.0, 2001)
    vals = np.array([f(t) for t in grid])
    assert abs(grid[np.argmin(vals)] - a) <= 1e-3
    h = 1e-5
    assert abs((f(a + h) - f(a - h)) / (2 * h)) < 1e-6 * max(1.0, abs(f(a)))


def test_diagonal_estimator_is_per_dimension_ridge():
    # diagonal variant: dimension j solves an independent ridge; checked with
    # lstsq on the augmented system [sqrt(w~) xbar_j; sqrt(lam)] b = [sqrt(w~) Rbar_j; 0]
    x, R, w = _est_case(22)
    lam = 0.4
    e = oracle.fit_estimator(x, R, w, lam, "diagonal")
    xb = (x - e["mu_x"]) / e["s"]
    Rb = R - e["mu_R"]
    sw = np.sqrt(e["w_til"])
    for j in range(x.shape[1]):
        A = np.concatenate([sw * xb[:, j], [math.sqrt(lam)]])[:, None]
        y = np.concatenate([sw * Rb[:, j], [0.0]])
        bj = np.linalg.lstsq(A, y, rcond=None)[0][0]
        assert np.isclose(e["b"][j], bj, rtol=1e-12, atol=1e-14)


def test_estimators_coincide_in_one_dimension_and_limits():
    # d = 1: scalar, diagonal and the full (unprojected) ridge are one model
    x, R, w = _est_case(23, M=9, d=1)
    lam = 0.3
    full = oracle.fit_correction(x, R, w, lam, rank=1)
    A, Psi, c, T = oracle.fold_correction(full)
    for kind in ("scalar", "diagonal"):
        e = oracle.fit_estimator(x, R, w, lam, kind)
        assert np.allclose(e["g"], np.diag(T), rtol=1e-10)
        assert np.allclose(e["c"], c, rtol=1e-10, atol=1e-14)
    # mean-only: the weighted mean residual, no gain
    x, R, w = _est_case(24)
    e = oracle.fit_estimator(x, R, w, 0.1, "mean")
    assert not np.any(e["g"])
    assert np.allclose(e["c"], (w / w.sum()) @ R)
    # lam -> infinity: every affine variant tends to the mean-only correction
    for kind in ("scalar", "diagonal"):
        e = oracle.fit_estimator(x, R, w, 1e12, kind)
        assert np.abs(e["g"]).max() < 1e-9
    # the folded form reproduces mu_R + xbar B
    e = oracle.fit_estimator(x, R, w, 0.2, "diagonal")
    o = np.random.default_rng(25).standard_normal((4, x.shape[1]))
    assert np.allclose(oracle.apply_estimator(o, e), o + e["g"] * o + e["c"])


# ----------------------------------------------------------------------------
# per-group routing rule ([paper] §4.3)
# ----------------------------------------------------------------------------

def test_key_token_budget_hand_values():
    # (rho*N_q - M) * N_k / N_q, ceiling: 0.22 at the Wan shape
    # (0.22*75600 - 64) * 75600 / 75600 = 16568 exactly
    assert oracle.key_token_budget("0.22", 75600, 75600, 64) == 16568
    # 0.26 at 4096 tokens: (1064.96 - 64) = 1000.96 -> 1001
    assert oracle.key_token_budget("0.26", 4096, 4096, 64) == 1001
    assert oracle.key_token_budget("0.01", 4096, 4096, 64) == 0


def _brute_per_group(qbar, kbar, n_a, m_b, budget, d):
    """Written out with plain loops: for every non-empty query group, every
    prefix of the (score desc, b asc) order is tried from the shortest."""
    Cq, Ck = len(n_a), len(m_b)
    z = np.zeros((Cq, Ck), bool)
    pairs = 0
    for a in range(Cq):
        if n_a[a] == 0:
            continue
        cand = [(-float(np.dot(qbar[a], kbar[b]) / math.sqrt(d)), b) for b in range(Ck) if m_b[b] > 0]
        cand.sort()
        chosen = []
        total = 0
        for _, b in cand:
            chosen.append(b)
            total += m_b[b]
            if total >= budget:
                break
        for b in chosen:
            z[a, b] = True
        pairs += n_a[a] * total
    return z, pairs


def test_per_group_routing_brute_force_with_ties():
    rng = np.random.default_rng(31)
    d = 4
    for trial in range(30):
        Cq, Ck = 5, 7
        qbar = rng.integers(-2, 3, (Cq, d)).astype(float)     # integer data: exact ties
        kbar = rng.integers(-2, 3, (Ck, d)).astype(float)
        n_a = rng.integers(0, 4, Cq)
        m_b = rng.integers(0, 5, Ck)
        if m_b.sum() == 0:
            m_b[0] = 1
        for budget in (0, 1, 3, 6, 50):
            z, pairs, _ = oracle.route_cells_per_group(qbar, kbar, n_a, m_b, budget, d)
            zb, pb = _brute_per_group(qbar, kbar, n_a, m_b, budget, d)
            assert np.array_equal(z, zb) and pairs == pb, (trial, budget)
            # invariants: every non-empty group keeps a cell, reaches the budget
            # unless it holds every non-empty K/V group, and is minimal
            for a in np.nonzero(n_a)[0]:
                keys = int(m_b[z[a]].sum())
                assert z[a].any()
                assert keys >= budget or z[a].sum() == (m_b > 0).sum()
            assert not z[:, m_b == 0].any() and not z[n_a == 0].any()


def test_per_group_full_budget_selects_everything():
    rng = np.random.default_rng(32)
    qbar, kbar = rng.standard_normal((3, 5)), rng.standard_normal((6, 5))
    n_a, m_b = np.array([2, 0, 3]), np.array([1, 4, 0, 2, 2, 1])
    z, pairs, _ = oracle.route_cells_per_group(qbar, kbar, n_a, m_b, int(m_b.sum()), 5)
    assert np.array_equal(z, np.outer(n_a > 0, m_b > 0))
    assert pairs == int(n_a.sum() * m_b.sum())


# ----------------------------------------------------------------------------
# O-13: error of the hard-drop output before / after the correction
# ----------------------------------------------------------------------------

def test_evaluation_rows_hand_values():
    # unprobed tokens of 10 with probes {2, 5}: 0 1 3 4 6 7 8 9; four evenly
    # spaced ones sit at positions 0, 2, 4, 6
    assert oracle.evaluation_rows(10, [2, 5], 4).tolist() == [0, 3, 6, 8]
    assert oracle.evaluation_rows(10, [2, 5], 8).tolist() == [0, 1, 3, 4, 6, 7, 8, 9]
    assert oracle.evaluation_rows(10, [2, 5], 50).tolist() == [0, 1, 3, 4, 6, 7, 8, 9]
    rows = oracle.evaluation_rows(75600, np.arange(64) * 1000, 2048)
    assert rows.size == 2048 and np.all(np.diff(rows) > 0)
    assert not np.isin(rows, np.arange(64) * 1000).any()


def test_row_error_stats_hand_values():
    st = oracle.row_error_stats([[1.0, 0.0], [0.0, 2.0]], [[1.0, 1.0], [0.0, 1.0]])
    # errors 1/sqrt(2) and 1
    assert abs(st["mean"] - (2 ** -0.5 + 1.0) / 2) < 1e-15
    assert abs(st["p99"] - (2 ** -0.5 + 0.99 * (1.0 - 2 ** -0.5))) < 1e-15
    assert st["rows"] == 2


def test_correction_report_full_density_is_exact():
    # one query group, one K/V group: the single cell is kept, the hard-drop
    # output is dense attention and the residual is 0, so both errors vanish
    rng = np.random.default_rng(7)
    n, d = 300, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    lab = np.zeros(n, np.int64)
    rep = oracle.correction_report(q, k, v, lab, lab, 1, 1, "1", m=16, rank=4, count=100)
    assert rep["rows"].size == 100
    assert rep["before"]["mean"] < 1e-13 and rep["after"]["p99"] < 1e-13
    assert abs(rep["rho_exec"] - 1.0) < 1e-12 or rep["rho_exec"] >= 1.0


def test_correction_report_matches_its_parts():
    # the report's numbers are the per-row errors of the call's own outputs
    w = sg.small_workload(heads=1, n=700, head_dim=32, components=6, kv_split=2, rho="0.3",
                          seed=17)
    hd = sg.make_call(w)[0]
    rep = oracle.correction_report(hd["q"], hd["k"], hd["v"], hd["labels_q"], hd["labels_kv"],
                                   w.c_q, w.c_k, w.rho, m=w.m, rank=w.r, lam=w.lam, count=256)
    r = rep["result"]
    assert not np.isin(rep["rows"], r["probes"]).any()
    e_b = [np.linalg.norm(r["o_sp"][i] - rep["dense"][i]) / np.linalg.norm(rep["dense"][i])
           for i in range(len(rep["rows"]))]
    e_a = [np.linalg.norm(r["out"][i] - rep["dense"][i]) / np.linalg.norm(rep["dense"][i])
           for i in range(len(rep["rows"]))]
    assert abs(rep["before"]["mean"] - sum(e_b) / len(e_b)) < 1e-12
    assert abs(rep["after"]["mean"] - sum(e_a) / len(e_a)) < 1e-12
    assert rep["rho_exec"] == float(oracle.executed_density(r["routed_pairs"], w.n, w.n, w.m))


def test_fp32_timing_mode_tracks_fp64():
    # the fp32 arithmetic mode (used only to time the oracle) stays within
    # fp32 rounding of the fp64 result
    w = sg.small_workload(heads=1, n=600, head_dim=64, components=5, rho="0.4", seed=18)
    hd = sg.make_call(w)[0]
    r = oracle.run_head(hd["q"], hd["k"], hd["v"], hd["labels_q"], hd["labels_kv"], w.c_q, w.c_k,
                        w.rho, m=w.m, rank=w.r, lam=w.lam, query_rows=np.zeros(0, np.int64))
    o64, _ = oracle.sparse_attention_rows(hd["q"], hd["labels_q"], hd["k"], hd["v"],
                                          hd["labels_kv"], r["z"], r["scale"])
    o32, _ = oracle.sparse_attention_rows(hd["q"], hd["labels_q"], hd["k"], hd["v"],
                                          hd["labels_kv"], r["z"], r["scale"], dtype=np.float32)
    assert o32.dtype == np.float32
    assert np.linalg.norm(o32 - o64) / np.linalg.norm(o64) < 1e-5
