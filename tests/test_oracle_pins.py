"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against a closed form, an identity stated on the pages,
a reduction to an independent definition, brute force, or a hand-worked fixture under
tests/golden/.  Page references: PARK, paperpeel.com/paper/2609.38978 (sections and
equations as printed there); SCOPE, paperpeel.com/paper/2608.12780.
"""
import itertools
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rand_qk(L, d, seed=0, centres=4):
    rng = np.random.default_rng(seed)
    mu = rng.normal(0, 2, (centres, d))
    z = rng.integers(0, centres, L)
    Q = (mu[z] + rng.normal(0, 0.5, (L, d))).astype(np.float32)
    K = (mu[z] + rng.normal(0, 0.5, (L, d))).astype(np.float32)
    V = rng.normal(0, 1, (L, d)).astype(np.float32)
    return Q, K, V


# ---------------------------------------------------------------- metric (a1-a3)

def test_gram_quadratic_form(orc):
    """App. D.2 'Euclidean realization': x^T G_Q x = ||Q x||^2 / L >= 0."""
    Q, K, _ = _rand_qk(300, 16, 1)
    G, _, _, ok = orc.query_metric(Q)
    assert ok
    rng = np.random.default_rng(5)
    Q64 = Q.astype(np.float64)
    for _ in range(5):
        x = rng.normal(size=16)
        lhs = x @ G @ x
        rhs = np.sum((Q64 @ x) ** 2) / Q.shape[0]
        assert lhs >= 0
        assert abs(lhs - rhs) <= 1e-12 * rhs


def test_cholesky_factor(orc):
    """App. D.2: Gs = R R^T with R lower triangular, positive diagonal (unique factor)."""
    Q, _, _ = _rand_qk(200, 24, 2)
    G, Gs, R, ok = orc.query_metric(Q)
    assert ok
    assert np.all(np.triu(R, 1) == 0)
    assert np.all(np.diag(R) > 0)
    assert np.abs(R @ R.T - Gs).max() <= 1e-12 * np.abs(Gs).max()


def test_shrinkage_limits(orc):
    """App. D.2 last paragraph: alpha = 1 is isotropic up to scale; alpha = 0 is the query
    metric up to the stability term.  s_Q = tr(G_Q)/d = ||Q||_F^2 / (L d)."""
    Q, _, _ = _rand_qk(150, 12, 3)
    L, d = Q.shape
    s = np.sum(Q.astype(np.float64) ** 2) / (L * d)
    _, Gs1, R1, ok = orc.query_metric(Q, alpha=1.0)
    assert ok
    np.testing.assert_allclose(R1, np.sqrt((1 + orc.EPS) * s) * np.eye(d), rtol=1e-12, atol=0)
    G0, Gs0, _, ok = orc.query_metric(Q, alpha=0.0)
    assert ok
    np.testing.assert_allclose(Gs0 - G0, orc.EPS * s * np.eye(d), rtol=1e-9, atol=1e-18)


def test_euclidean_metric_is_identity(orc):
    Q, _, _ = _rand_qk(50, 8, 4)
    _, _, R, ok = orc.query_metric(Q, metric="euclidean")
    assert ok and np.array_equal(R, np.eye(8))


def test_metric_failure_reported(orc):
    """A factorisation that cannot succeed (non-finite queries) is reported, not hidden
    (App. D.2 "Numerically stable Cholesky factorization" plans a per-head flag), and the
    head falls back to R = I, so its keys are clustered with the Euclidean metric: the
    transform is then the identity and the clustering equals the Euclidean one."""
    Q, K, _ = _rand_qk(40, 8, 5)
    Q[3, 2] = np.nan
    *_, R, ok = orc.query_metric(Q)
    assert not ok
    assert np.array_equal(R, np.eye(8))
    assert np.array_equal(orc.transform(K, R), K)
    a = orc.cluster_keys(Q, K, 5, 3)
    b = orc.cluster_keys(Q, K, 5, 3, metric="euclidean")
    assert not a["ok"] and b["ok"]
    assert np.array_equal(a["labels"], b["labels"])
    # the flag needs a non-finite input: an all-zero head still factors (s_Q = s_min)
    *_, R0, ok0 = orc.query_metric(np.zeros((10, 8), np.float32))
    assert ok0 and np.all(np.diag(R0) > 0)


def test_qrkc_objective_identity(orc):
    """Section 5.2, the J_QRKC identity: with k~ = R^T k,
    sum_j ||k~_j - c~_{a_j}||^2 = (1-alpha) (1/L) sum_i sum_j [q_i^T (k_j - c_{a_j})]^2
                                  + (alpha+eps) s_Q sum_j ||k_j - c_{a_j}||^2."""
    Q, K, _ = _rand_qk(120, 10, 6)
    L, d = Q.shape
    rng = np.random.default_rng(7)
    labels = rng.integers(0, 5, L)
    C = rng.normal(0, 2, (5, d))
    _, _, R, ok = orc.query_metric(Q)
    assert ok
    Kt = orc.transform(K, R).astype(np.float64)
    Ct = orc.transform(C.astype(np.float32), R).astype(np.float64)
    lhs = np.sum((Kt - Ct[labels]) ** 2)
    Dlt = K.astype(np.float64) - C.astype(np.float32).astype(np.float64)[labels]
    jq = 0.0
    for i in range(L):
        for j in range(L):
            jq += float(Q[i].astype(np.float64) @ Dlt[j]) ** 2
    jq /= L
    je = np.sum(Dlt ** 2)
    s = np.sum(Q.astype(np.float64) ** 2) / (L * d)
    rhs = (1 - orc.ALPHA) * jq + (orc.ALPHA + orc.EPS) * s * je
    assert abs(lhs - rhs) <= 1e-5 * rhs   # float rounding of the transformed keys


# ---------------------------------------------------------------- k-means (a4-a6)

def test_kmeans_golden_line(orc):
    g = _gold("kmeans_line.json")
    Kt = np.array(g["Kt"], np.float32)
    km = orc.kmeans(Kt, 2, 2, init_idx=g["init_idx"])
    assert km["labels_hist"][0].tolist() == g["labels"]
    np.testing.assert_array_equal(km["C_hist"][1], np.array(g["centroids"], np.float32))
    assert km["J_assign"][0] == g["J_assign_1"]
    assert km["J_update"][0] == g["J_update_1"]
    assert abs(km["margins"][0][1] - g["margin_key1_step1"]) < 1e-15


def test_kmeans_tie_rule_golden(orc):
    """Reading of the silent argmin tie rule: exact ties go to the lowest cluster index
    (hand-worked in golden/kmeans_ties_empty.json)."""
    g = _gold("kmeans_ties_empty.json")["ties"]
    Kt = np.array(g["Kt"], np.float32)
    C = np.array(g["C"], np.float32)
    lab, _, dist, J = orc.assign(Kt, C)
    assert lab.tolist() == g["labels"]
    assert dist.tolist() == g["dist"]
    # the same keys against the centroids in reverse order: still the lowest index of a tie
    lab_r, *_ = orc.assign(Kt, C[::-1].copy())
    assert lab_r.tolist() == [0, 1, 0]


def test_kmeans_empty_cluster_keeps_centroid(orc):
    """Reading of the silent empty-cluster rule: a cluster without keys keeps its centroid
    through the update (hand-worked in golden/kmeans_ties_empty.json); the final outputs
    give it count 0 and a zero centroid."""
    g = _gold("kmeans_ties_empty.json")["empty"]
    Kt = np.array(g["Kt"], np.float32)
    C0 = np.array(g["C0"], np.float32)
    lab1, *_ = orc.assign(Kt, C0)
    assert lab1.tolist() == g["labels_1"]
    C1 = orc.update(Kt, lab1, C0)
    np.testing.assert_array_equal(C1, np.array(g["C1"], np.float32))
    lab2, *_ = orc.assign(Kt, C1)
    assert lab2.tolist() == g["labels_2"]
    km = orc.kmeans(Kt, 3, 2, init_idx=[0, 2, 2])
    # init (0,0), (10,0), (10,0): cluster 2 ties with cluster 1 for key 2 and loses, so it
    # is empty after every step and keeps its anchor
    assert km["labels"].tolist() == [0, 0, 1]
    np.testing.assert_array_equal(km["centroids"][2], np.array([10.0, 0.0], np.float32))
    cent, counts, perm, offsets = orc.finalize(Kt, km["labels"], 3)
    assert counts.tolist() == [2, 1, 0] and offsets.tolist() == [0, 2, 3, 3]
    assert np.array_equal(cent[2], np.zeros(2, np.float32))


def test_kmeans_objective_non_increasing(orc):
    """Lloyd steps never increase the objective (k-means, App. D.2 'K-means optimizes the
    specified objective iteratively')."""
    import park_synth
    Q, K, _ = park_synth.generate(park_synth.TINY)
    cl = orc.cluster_keys(Q[0, 0], K[0, 0], 32, 10)
    ja, ju = cl["km"]["J_assign"], cl["km"]["J_update"]
    for t in range(len(ja)):
        assert ju[t] <= ja[t] * (1 + 1e-9)
        if t + 1 < len(ja):
            assert ja[t + 1] <= ju[t] * (1 + 1e-9)


def test_kmeans_singletons_identity(orc):
    """N_K = L with strided anchors: every key is its own cluster."""
    Q, K, _ = _rand_qk(64, 8, 8)
    cl = orc.cluster_keys(Q, K, 64, 3)
    assert cl["labels"].tolist() == list(range(64))
    assert cl["counts"].tolist() == [1] * 64


def test_alpha_one_matches_euclidean(orc):
    """alpha = 1 makes the metric isotropic, so labels equal plain Euclidean k-means on
    the raw keys up to near-ties."""
    Q, K, _ = _rand_qk(400, 16, 9, centres=6)
    a = orc.cluster_keys(Q, K, 12, 4, alpha=1.0)
    b = orc.cluster_keys(Q, K, 12, 4, metric="euclidean")
    ok = (a["labels"] == b["labels"]) | (b["km"]["margins"][-1] < 1e-5)
    assert ok.all()


def test_finalize_invariants(orc):
    Q, K, _ = _rand_qk(333, 8, 10)
    cl = orc.cluster_keys(Q, K, 7, 3)
    off, perm, lab, cnt = cl["offsets"], cl["perm"], cl["labels"], cl["counts"]
    assert off[0] == 0 and off[-1] == 333
    assert sorted(perm.tolist()) == list(range(333))
    keys = [(lab[p], p) for p in perm]
    assert keys == sorted(keys)
    assert np.array_equal(np.diff(off), cnt)


# ---------------------------------------------------------------- PAMA (a8)

def test_pama_golden(orc):
    g = _gold("pama_closed_form.json")
    for case in ("case_a", "case_b"):
        c = g[case]
        Q = np.array(c["Q"], np.float32)
        W = orc.pama(Q, np.array(c["C"], np.float32), np.array(c["counts"]), len(Q), 1.0)
        np.testing.assert_allclose(W[0], c["W"], rtol=1e-7, atol=0)


def test_pama_rows_sum_to_one(orc):
    """E8: each query's distribution over key blocks sums to 1, so each W_u sums to 1."""
    Q, K, _ = _rand_qk(300, 16, 11)
    cl = orc.cluster_keys(Q, K, 9, 3)
    W = orc.pama(Q, cl["centroids"], cl["counts"], 64, 0.25)
    np.testing.assert_allclose(W.sum(1), 1.0, rtol=0, atol=1e-12)


def test_pama_singletons_equal_exact_importance(orc):
    """With one key per block, c_v = k_v and log n_v = 0, so PAMA is the exact block
    importance of section 3.2 Eq. (3) (computed by an independent dense routine)."""
    Q, K, _ = _rand_qk(96, 8, 12)
    labels = np.arange(96, dtype=np.int32)
    cent, counts, _, _ = orc.finalize(K, labels, 96)
    W = orc.pama(Q, cent, counts, 32, 0.3)
    Wx = orc.exact_block_importance(Q, K, labels, 96, 32, 0.3)
    np.testing.assert_allclose(W, Wx, rtol=1e-10, atol=1e-15)


def test_pama_identical_keys_equal_exact_importance(orc):
    """App. D.2 exact decomposition: S*_iv = log n_v + q_i^T c_v scale + Delta^K_iv, and
    Delta^K vanishes when a block's keys are identical; PAMA then equals Eq. (3)."""
    rng = np.random.default_rng(13)
    base = rng.normal(0, 1, (6, 8)).astype(np.float32)
    labels = rng.integers(0, 6, 150).astype(np.int32)
    labels[:6] = np.arange(6)
    K = base[labels]
    Q = rng.normal(0, 1, (150, 8)).astype(np.float32)
    cent, counts, _, _ = orc.finalize(K, labels, 6)
    W = orc.pama(Q, cent, counts, 50, 0.7)
    Wx = orc.exact_block_importance(Q, K, labels, 6, 50, 0.7)
    np.testing.assert_allclose(W, Wx, rtol=1e-9, atol=1e-15)


def test_pooled_identical_queries_equal_pama(orc):
    """App. D.1: if all queries in a block are identical the query-centroid estimate is
    exact, i.e. the pooled scores equal PAMA."""
    rng = np.random.default_rng(14)
    q = rng.normal(0, 1, (4, 8)).astype(np.float32)
    Q = np.repeat(q, 16, axis=0)
    _, K, _ = _rand_qk(64, 8, 15)
    cl = orc.cluster_keys(Q, K, 5, 2)
    Wp = orc.pooled_scores(Q, cl["centroids"], cl["counts"], 16, 0.5)
    Wa = orc.pama(Q, cl["centroids"], cl["counts"], 16, 0.5)
    np.testing.assert_allclose(Wp, Wa, rtol=1e-10, atol=1e-15)


# ---------------------------------------------------------------- selection (a9)

def test_select_golden(orc):
    for c in _gold("select_rows.json")["cases"]:
        W = np.array([c["W"]])
        mask, lst, cnt, _, _ = orc.select(W, np.array(c["counts"]), c["p"], c["k"])
        assert cnt[0] == c["count"], c["why"]
        assert lst[0, :cnt[0]].tolist() == c["list"], c["why"]
        assert np.all(lst[0, cnt[0]:] == -1)
        assert mask[0].nonzero()[0].tolist() == c["list"]


def _brute_force_select(w, counts, p, k):
    """Smallest set of non-empty blocks holding at least p of the mass; among those the
    larger mass, then the lexicographically smallest id list; then grown to k blocks by
    the largest remaining masses (ids ascending on ties)."""
    ne = [v for v in range(len(w)) if counts[v] > 0]
    total = float(sum(w[v] for v in ne))
    best = None
    if p > 0:
        for r in range(1, len(ne) + 1):
            for sub in itertools.combinations(ne, r):
                m = float(np.sum(w[list(sub)]))
                if m >= p * total:
                    key = (-m, list(sub))
                    if best is None or key < best[0]:
                        best = (key, list(sub))
            if best is not None:
                break
    chosen = [] if best is None else best[1]
    rest = sorted([v for v in ne if v not in chosen], key=lambda v: (-w[v], v))
    while len(chosen) < min(k, len(ne)):
        chosen.append(rest.pop(0))
    return sorted(chosen)


def test_select_brute_force(orc):
    rng = np.random.default_rng(16)
    for trial in range(300):
        nk = int(rng.integers(1, 10))
        counts = rng.integers(0, 3, nk)
        if counts.sum() == 0:
            counts[0] = 1
        # small integer masses: every subset sum is exact, and ties are frequent
        w = (rng.integers(0, 9, nk) ** 2 * (counts > 0)).astype(np.float64)
        p = float(rng.choice([0.0, 0.3, 0.5, 0.9, 1.0]))
        k = int(rng.integers(0, nk + 2))
        _, lst, cnt, _, _ = orc.select(w[None, :], counts, p, k)
        bf = _brute_force_select(w, counts, p, k)
        assert lst[0, :cnt[0]].tolist() == bf, (w, counts, p, k)


# ---------------------------------------------------------------- attention (a10)

def test_attention_golden(orc):
    g = _gold("attention_closed_form.json")
    Q, K, V = (np.array(g[x], np.float32) for x in "QKV")
    perm = np.array([0, 1]); off = np.array([0, 2]); lst = np.array([[0]]); cnt = np.array([1])
    O, lse = orc.block_sparse_attn(Q, K, V, perm, off, lst, cnt, 1, 1.0)
    np.testing.assert_allclose(O[0], g["O"], rtol=1e-7)
    assert abs(lse[0] - g["lse"]) < 1e-7
    Q2 = np.concatenate([Q, np.zeros_like(Q)])          # the dense routine takes L queries and L keys
    Od, lsed = orc.dense_attn(Q2, K, V, 1.0, rows=[0])
    np.testing.assert_allclose(Od[0], g["O"], rtol=1e-7)
    assert abs(lsed[0] - g["lse"]) < 1e-7


def test_density_one_equals_dense(orc):
    """Section 3.1: with every block selected, sparse attention is dense attention
    (the dense routine is an independent textbook triple loop)."""
    Q, K, V = _rand_qk(200, 16, 17)
    cl = orc.cluster_keys(Q, K, 6, 2)
    nq = (200 + 63) // 64
    lst = np.tile(np.arange(6, dtype=np.int32), (nq, 1))
    cnt = np.full(nq, 6, np.int32)
    O, lse = orc.block_sparse_attn(Q, K, V, cl["perm"], cl["offsets"], lst, cnt, 64, 0.25)
    Od, lsed = orc.dense_attn(Q, K, V, 0.25)
    np.testing.assert_allclose(O, Od, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, rtol=1e-12, atol=1e-12)


def test_singleton_selection_returns_value(orc):
    """A single selected one-key block: the softmax has one term, O_i = v_j."""
    Q, K, V = _rand_qk(10, 4, 18)
    perm = np.array([3, 0, 1, 2, 4, 5, 6, 7, 8, 9], np.int32)
    off = np.array([0, 1, 10], np.int32)
    lst = np.array([[0, -1]], np.int32); cnt = np.array([1], np.int32)
    O, lse = orc.block_sparse_attn(Q, K, V, perm, off, lst, cnt, 10, 0.5)
    np.testing.assert_allclose(O, np.repeat(V[3:4].astype(np.float64), 10, 0), rtol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * (Q.astype(np.float64) @ K[3].astype(np.float64)), rtol=1e-12)


def test_empty_selection(orc):
    Q, K, V = _rand_qk(8, 4, 19)
    O, lse = orc.block_sparse_attn(Q, K, V, np.arange(8), np.array([0, 8]), np.array([[-1]]),
                                   np.array([0]), 8, 0.5)
    assert np.all(O == 0) and np.all(np.isneginf(lse))


def test_top_p_on_exact_importance_gives_recall(orc):
    """Table 1 'Full/Full' rows: top-p over the exact block importance keeps at least p of
    each query block's attention mass.  Recall per block is the mean over its queries of
    exp(lse_sparse - lse_dense) (section 3.2, Recall), and it equals the kept mass."""
    Q, K, V = _rand_qk(256, 16, 20, centres=8)
    cl = orc.cluster_keys(Q, K, 10, 3)
    scale = 0.25
    Wx = orc.exact_block_importance(Q, K, cl["labels"], 10, 64, scale)
    _, lst, cnt, _, _ = orc.select(Wx, cl["counts"], 0.9, 0)
    O, lse = orc.block_sparse_attn(Q, K, V, cl["perm"], cl["offsets"], lst, cnt, 64, scale)
    _, lsed = orc.dense_attn(Q, K, V, scale)
    rec = np.exp(lse - lsed)
    for u in range(4):
        r = rec[64 * u:64 * u + 64].mean()
        kept = Wx[u, lst[u, :cnt[u]]].sum()
        assert r >= 0.9 - 1e-12
        assert abs(r - kept) < 1e-10


def test_literal_masked_attention_is_recall_times_output(orc):
    """Section 3.1: the literal O^sp = (A .* M) V equals recall_i times the renormalised
    sparse output (A from the dense definition, written out here for a tiny case)."""
    Q, K, V = _rand_qk(40, 6, 21)
    cl = orc.cluster_keys(Q, K, 4, 2)
    lst = np.array([[0, 2, -1, -1]], np.int32); cnt = np.array([2], np.int32)
    O, lse = orc.block_sparse_attn(Q, K, V, cl["perm"], cl["offsets"], lst, cnt, 40, 0.3)
    _, lsed = orc.dense_attn(Q, K, V, 0.3)
    sel = np.isin(cl["labels"], [0, 2])
    Z = 0.3 * Q.astype(np.float64) @ K.astype(np.float64).T
    A = np.exp(Z - Z.max(1, keepdims=True)); A /= A.sum(1, keepdims=True)
    lit = (A * sel[None, :]) @ V.astype(np.float64)
    np.testing.assert_allclose(lit, np.exp(lse - lsed)[:, None] * O, rtol=1e-9, atol=1e-12)


# ------------------------------------------------- clustered query blocks (next row 1)

def _consecutive_blocks(L, qb):
    """The 64-token layout written as a query permutation: identity order, blocks of qb."""
    return np.arange(L, dtype=np.int32), np.minimum(np.arange(0, L + qb, qb), L).astype(np.int32)[: (L + qb - 1) // qb + 1]


def test_pama_blocks_reduces_to_consecutive_blocks(orc):
    """With the identity permutation and 64-token boundaries the clustered-block PAMA is the
    64-token PAMA (a separately pinned routine), to the last bit: same sums in the same order."""
    Q, K, _ = _rand_qk(300, 16, 31)
    cl = orc.cluster_keys(Q, K, 9, 3)
    qperm, qoff = _consecutive_blocks(300, 64)
    W = orc.pama_blocks(Q, cl["centroids"], cl["counts"], qperm, qoff, 0.25)
    np.testing.assert_array_equal(W, orc.pama(Q, cl["centroids"], cl["counts"], 64, 0.25))


def test_pama_blocks_rows_sum_to_one_and_order_free(orc):
    """E8 with clustered blocks: each non-empty row sums to 1, an empty block gives a zero row,
    and the order of a block's queries in the permutation changes W only by rounding."""
    Q, K, _ = _rand_qk(240, 12, 32, centres=6)
    cl = orc.cluster_keys(Q, K, 7, 3)
    qc = orc.cluster_queries(Q, 5, 4)
    qoff = np.concatenate([qc["offsets"][:3], qc["offsets"][2:]]).astype(np.int32)  # block 2 empty
    W = orc.pama_blocks(Q, cl["centroids"], cl["counts"], qc["perm"], qoff, 0.3)
    sizes = np.diff(qoff)
    assert sizes[2] == 0 and np.all(W[2] == 0)
    np.testing.assert_allclose(W[sizes > 0].sum(1), 1.0, rtol=0, atol=1e-12)
    rng = np.random.default_rng(33)
    shuf = qc["perm"].copy()
    for u in range(len(qoff) - 1):
        seg = shuf[qoff[u]:qoff[u + 1]]
        shuf[qoff[u]:qoff[u + 1]] = seg[rng.permutation(len(seg))]
    W2 = orc.pama_blocks(Q, cl["centroids"], cl["counts"], shuf, qoff, 0.3)
    np.testing.assert_allclose(W2, W, rtol=1e-12, atol=1e-15)


def test_pama_blocks_brute_force(orc):
    """Tiny case against a per-query softmax written out in numpy: block u's row is the mean
    of its members' distributions, whatever their positions in the sequence."""
    rng = np.random.default_rng(34)
    Q = rng.normal(0, 1, (12, 4)).astype(np.float32)
    C = rng.normal(0, 1, (3, 4)).astype(np.float32)
    counts = np.array([2, 5, 1], np.int32)
    qperm = np.array([5, 0, 11, 3, 7, 1, 2, 4, 6, 8, 9, 10], np.int32)
    qoff = np.array([0, 3, 4, 12], np.int32)
    W = orc.pama_blocks(Q, C, counts, qperm, qoff, 0.5)
    S = 0.5 * Q.astype(np.float64) @ C.astype(np.float64).T + np.log(counts)
    P = np.exp(S - S.max(1, keepdims=True)); P /= P.sum(1, keepdims=True)
    for u in range(3):
        np.testing.assert_allclose(W[u], P[qperm[qoff[u]:qoff[u + 1]]].mean(0), rtol=1e-13)


def test_attention_blocks_reduces_to_consecutive_blocks(orc):
    """Identity permutation with 64-token boundaries: the clustered-block attention is the
    64-token routine exactly (same keys, same order, same arithmetic per query)."""
    Q, K, V = _rand_qk(200, 16, 35)
    cl = orc.cluster_keys(Q, K, 6, 2)
    W = orc.pama(Q, cl["centroids"], cl["counts"], 64, 0.25)
    _, lst, cnt, _, _ = orc.select(W, cl["counts"], 0.8, 2)
    qperm, qoff = _consecutive_blocks(200, 64)
    O, lse = orc.block_sparse_attn_blocks(Q, K, V, cl["perm"], cl["offsets"], qperm, qoff, lst, cnt, 0.25)
    O2, lse2 = orc.block_sparse_attn(Q, K, V, cl["perm"], cl["offsets"], lst, cnt, 64, 0.25)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(lse, lse2)


def test_attention_blocks_density_one_equals_dense(orc):
    """Every key cluster selected for every clustered query block: dense attention (the
    independent textbook routine), for queries scattered across the blocks."""
    Q, K, V = _rand_qk(180, 8, 36, centres=5)
    cl = orc.cluster_keys(Q, K, 5, 2)
    qc = orc.cluster_queries(Q, 4, 3)
    lst = np.tile(np.arange(5, dtype=np.int32), (4, 1)); cnt = np.full(4, 5, np.int32)
    O, lse = orc.block_sparse_attn_blocks(Q, K, V, cl["perm"], cl["offsets"], qc["perm"], qc["offsets"], lst,
                                          cnt, 0.4)
    Od, lsed = orc.dense_attn(Q, K, V, 0.4)
    np.testing.assert_allclose(O, Od, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, rtol=1e-12, atol=1e-12)


def test_attention_blocks_follow_each_query_block(orc):
    """Each query gets its own block's selection: with one cluster selected per block, query i
    of block u attends exactly to the keys of that cluster (checked against the 64-token routine
    run on that query alone as a one-query block)."""
    Q, K, V = _rand_qk(90, 6, 37, centres=3)
    cl = orc.cluster_keys(Q, K, 3, 2)
    qc = orc.cluster_queries(Q, 3, 3)
    lst = np.array([[2, -1, -1], [0, -1, -1], [1, -1, -1]], np.int32); cnt = np.ones(3, np.int32)
    O, lse = orc.block_sparse_attn_blocks(Q, K, V, cl["perm"], cl["offsets"], qc["perm"], qc["offsets"], lst,
                                          cnt, 0.5)
    for u in range(3):
        for i in qc["perm"][qc["offsets"][u]:qc["offsets"][u + 1]][:4]:
            o1, l1 = orc.block_sparse_attn(Q[i:i + 1], K, V, cl["perm"], cl["offsets"], lst[u:u + 1],
                                           cnt[u:u + 1], 1, 0.5)
            np.testing.assert_array_equal(O[i], o1[0])
            assert lse[i] == l1[0]


def test_query_clustering_blocks_hold_their_members(orc):
    """Query blocks from Euclidean k-means of the queries: block u's queries all carry label u,
    the permutation covers every query once, and the blocks partition the sequence."""
    Q, _, _ = _rand_qk(256, 16, 38, centres=6)
    qc = orc.cluster_queries(Q, 8, 4)
    assert np.array_equal(np.sort(qc["perm"]), np.arange(256))
    assert qc["offsets"][0] == 0 and qc["offsets"][-1] == 256
    for u in range(8):
        assert np.all(qc["labels"][qc["perm"][qc["offsets"][u]:qc["offsets"][u + 1]]] == u)


# ------------------------------------------------- retrieval-accuracy diagnostics (next row 3)

def test_tv_hand_example_and_limits(orc):
    """Appendix A, M1: block-size weighted half-L1 distance.  Hand example: blocks of 64 and 36
    queries, TV 0.5 each -> 0.5; identical maps -> 0; disjoint one-hot rows -> 1; symmetric."""
    We = np.array([[0.5, 0.5], [1.0, 0.0]]); Wx = np.array([[1.0, 0.0], [0.5, 0.5]])
    assert abs(orc.tv(We, Wx, [64, 36]) - 0.5) < 1e-15
    assert orc.tv(We, We, [64, 36]) == 0.0
    assert orc.tv(np.eye(3), np.roll(np.eye(3), 1, 1), [10, 10, 5]) == 1.0
    assert orc.tv(We, Wx, [64, 36]) == orc.tv(Wx, We, [64, 36])
    assert list(orc.block_sizes(130)) == [64, 64, 2]


def test_tv_of_pama_on_singleton_clusters_is_zero(orc):
    """With one key per cluster PAMA is the exact importance (pinned above), so its M1 error
    against the independent exact routine vanishes; pooled queries do not (App. D.1)."""
    Q, K, _ = _rand_qk(96, 8, 39)
    labels = np.arange(96, dtype=np.int32)
    cent, counts, _, _ = orc.finalize(K, labels, 96)
    Wx = orc.exact_block_importance(Q, K, labels, 96, 32, 0.3)
    Wp = orc.pama(Q, cent, counts, 32, 0.3)
    Wc = orc.pooled_scores(Q, cent, counts, 32, 0.3)
    sizes = orc.block_sizes(96, 32)
    assert orc.tv(Wp, Wx, sizes) < 1e-12
    assert orc.tv(Wc, Wx, sizes) > 1e-3


def test_logmass_rmse_exact_cases(orc):
    """M2 (section 4.2 quantities): one key per cluster, or identical keys within a cluster,
    make the centroid log-mass exact (App. D.2 exact decomposition), so the RMSE vanishes."""
    Q, K, _ = _rand_qk(80, 8, 40)
    labels = np.arange(80, dtype=np.int32)
    cent, counts, _, _ = orc.finalize(K, labels, 80)
    assert orc.logmass_rmse(Q, K, labels, cent, counts, 0.4) < 1e-12
    rng = np.random.default_rng(41)
    base = rng.normal(0, 1, (5, 8)).astype(np.float32)
    lab = rng.integers(0, 5, 120).astype(np.int32); lab[:5] = np.arange(5)
    cent, counts, _, _ = orc.finalize(base[lab], lab, 5)
    assert orc.logmass_rmse(Q[:60].repeat(2, 0), base[lab], lab, cent, counts, 0.4) < 1e-12


def test_logmass_rmse_closed_form_and_translation(orc):
    """Two keys c_v +- e_v per cluster: S* - S = log cosh(scale q.e_v) exactly, so the centred
    RMSE has a closed form; moving every key by one vector leaves it unchanged."""
    rng = np.random.default_rng(42)
    nk, d, s = 6, 4, 0.7
    c = rng.normal(0, 1, (nk, d)); e = rng.normal(0, 0.6, (nk, d))
    K = np.concatenate([c + e, c - e]).astype(np.float32)
    lab = np.concatenate([np.arange(nk), np.arange(nk)]).astype(np.int32)
    Q = rng.normal(0, 1, (2 * nk, d)).astype(np.float32)
    cent, counts, _, _ = orc.finalize(K, lab, nk)
    Kd = K.astype(np.float64)
    ed = (Kd[:nk] - Kd[nk:]) / 2
    D = np.log(np.cosh(s * Q.astype(np.float64) @ ed.T))
    Dc = D - D.mean(1, keepdims=True)
    ref = np.sqrt((Dc ** 2).mean())
    got = orc.logmass_rmse(Q, K, lab, cent, counts, s)
    assert abs(got - ref) < 1e-6 * max(ref, 1e-3), (got, ref)
    K2 = (K + np.float32(0.5)).astype(np.float32)
    cent2, _, _, _ = orc.finalize(K2, lab, nk)
    assert abs(orc.logmass_rmse(Q, K2, lab, cent2, counts, s) - got) < 1e-6



@pytest.mark.parametrize("seed", range(4))
def test_qrkc_lowers_logmass_error_for_anisotropic_queries(orc, seed):
    """PARK section 5.2 and appendix B (M2): within a cluster, the log-mass error of a query
    grows with the variance of q . (k - c_v), whose mean over the queries is the query-metric
    norm (k - c_v)^T G (k - c_v) that QRKC minimises; Euclidean k-means minimises |k - c_v|^2.
    With class-centred keys and queries whose spread is concentrated on a few coordinates, the
    QRKC clustering must give a clearly lower centred log-mass RMSE than the Euclidean one (the
    ratio is 0.61-0.81 on these seeds)."""
    rng = np.random.default_rng(seed)
    N, d, M, nk, iters = 2000, 32, 8, 32, 8
    mu = rng.normal(0, 2, (M, d))
    z = rng.integers(0, M, N)
    s = np.r_[np.full(4, 4.0), np.full(d - 4, 0.25)]
    Q = ((mu[z] + rng.normal(0, 0.5, (N, d))) * s).astype(np.float32)
    K = (mu[z] + rng.normal(0, 0.5, (N, d))).astype(np.float32)
    rows = np.arange(0, N, 4)
    err = {}
    for metric in ("qrkc", "euclidean"):
        cl = orc.cluster_keys(Q, K, nk, iters, metric=metric)
        err[metric] = orc.logmass_rmse(Q, K, cl["labels"], cl["centroids"], cl["counts"], 1 / np.sqrt(d), rows=rows)
    assert err["qrkc"] < 0.9 * err["euclidean"], err

# ---------------------------------------------------------------- SCOPE online per-head top-k

def test_select_online_hand_example(orc):
    """SCOPE, section 3 "Online Per-Head Top-k Estimation": base counts b = (1, 6, 1) of
    query blocks of sizes (64, 64, 1) give the weighted minimum ceil(449 / 129) = 4 (the
    unweighted mean, its floor or its rounding would give 3); blocks 0 and 2 are extended
    along their rankings to 4 clusters, block 1 keeps its 6.  Cluster 7 is empty."""
    W = np.array([[0.9, 0.012, 0.05, 0.004, 0.02, 0.008, 0.006, 0.0],
                  [0.16, 0.155, 0.15, 0.145, 0.14, 0.135, 0.115, 0.0],
                  [0.002, 0.003, 0.005, 0.87, 0.05, 0.04, 0.03, 0.0]])
    counts = np.array([5, 5, 5, 5, 5, 5, 5, 0], np.int32)
    mask, lst, cnt, base, k_on = orc.select_online(W, counts, 0.8, 1, orc.block_sizes(129))
    assert base.tolist() == [1, 6, 1] and k_on == 4
    assert cnt.tolist() == [4, 6, 4]
    assert lst[0, :4].tolist() == [0, 1, 2, 4]
    assert lst[1, :6].tolist() == [0, 1, 2, 3, 4, 5]
    assert lst[2, :4].tolist() == [3, 4, 5, 6]
    for u in range(3):
        assert np.all(lst[u, cnt[u]:] == -1) and mask[u].nonzero()[0].tolist() == lst[u, :cnt[u]].tolist()


def test_select_online_invariants(orc):
    """On random rows: counts never drop, rows at or above the minimum are untouched, the
    others hold exactly min(k_on, non-empty) clusters, and every selection is a prefix of its
    row's ranking (W descending, index ascending)."""
    rng = np.random.default_rng(41)
    nq, nk = 37, 50
    counts = rng.integers(0, 4, nk).astype(np.int32)
    ne = int((counts > 0).sum())
    W = rng.dirichlet(np.full(nk, 0.3), nq) * (counts > 0)
    sizes = rng.integers(1, 65, nq)
    m0, l0, c0, _, _ = orc.select(W, counts, 0.7, 2)
    mask, lst, cnt, base, k_on = orc.select_online(W, counts, 0.7, 2, sizes)
    assert np.array_equal(base, c0)
    assert k_on >= (sizes * base).sum() / sizes.sum() > k_on - 1
    assert np.all(cnt >= base)
    keep = base >= k_on
    assert np.array_equal(cnt[keep], c0[keep]) and np.array_equal(lst[keep], l0[keep])
    assert np.all(cnt[~keep] == min(k_on, ne)) and (~keep).any() and keep.any()
    for u in range(nq):
        order = sorted((v for v in range(nk) if counts[v] > 0), key=lambda v: (-W[u, v], v))
        assert sorted(order[:cnt[u]]) == lst[u, :cnt[u]].tolist()


def test_select_online_fixed_k_is_unchanged(orc):
    """Pure top-k (p = 0): every base count is k, so the minimum is k and nothing changes;
    equal base counts with any block sizes leave the selection as it was."""
    rng = np.random.default_rng(42)
    W = rng.dirichlet(np.ones(20), 9)
    counts = np.ones(20, np.int32)
    m0, l0, c0, _, _ = orc.select(W, counts, 0.0, 6)
    mask, lst, cnt, base, k_on = orc.select_online(W, counts, 0.0, 6, rng.integers(1, 65, 9))
    assert k_on == 6 and np.array_equal(cnt, c0) and np.array_equal(lst, l0) and np.array_equal(mask, m0)
