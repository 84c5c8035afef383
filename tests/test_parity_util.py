"""Host-side checks of the GPU parity comparators (no GPU): the selection comparison implements
the "bit-exact except where the margin is below 1e-5" rule, and the teacher-forced k-means
chain follows the oracle's own update rule.  The "GPU" side here is the oracle's output on
slightly moved scores, or a hand-made wrong selection."""
import numpy as np
import pytest

from parity_util import MARGIN, compare_selection, near_prefix, teacher_forced_chain


def _rows(nq=40, nk=24, seed=0):
    rng = np.random.default_rng(seed)
    W = rng.dirichlet(np.full(nk, 0.3), size=nq)
    counts = rng.integers(1, 9, nk).astype(np.int32)
    counts[3] = 0
    W[:, 3] = 0.0
    W /= W.sum(axis=1, keepdims=True)
    return W, counts


def test_identical_selection_passes(orc):
    W, counts = _rows()
    m, l, c, _, _ = orc.select(W, counts, 0.9, 2)
    n, ex, nd = compare_selection(W.astype(np.float32), W, counts, 0.9, 2, m, l, c, orc)
    assert n == W.shape[0] and nd == 0


def test_difference_in_a_decided_row_fails(orc):
    W, counts = _rows(seed=1)
    m, l, c, cm, gm = orc.select(W, counts, 0.9, 2)
    u = int(np.nonzero((cm >= 1e-3) & (gm >= 1e-3))[0][0])
    m2, l2, c2 = m.copy(), l.copy(), c.copy()
    # drop the last kept cluster of a row whose cut and gap are far from any tie
    keep = l[u, :c[u]].tolist()
    order = sorted(keep, key=lambda v: (-W[u, v], v))
    drop = order[-1]
    keep.remove(drop)
    m2[u, drop] = 0
    l2[u, :] = -1
    l2[u, :len(keep)] = sorted(keep)
    c2[u] = len(keep)
    with pytest.raises(AssertionError):
        compare_selection(W.astype(np.float32), W, counts, 0.9, 2, m2, l2, c2, orc)


def test_near_tie_swap_is_exempt(orc):
    """Two clusters within 1e-5 at the boundary of the kept prefix: either may be kept."""
    nk = 6
    W = np.array([[0.40, 0.30, 0.149996, 0.150004, 0.0, 0.0]])
    counts = np.array([5, 5, 5, 5, 5, 5], np.int32)
    m, l, c, cm, gm = orc.select(W, counts, 0.5, 3)
    assert c[0] == 3 and gm[0] < MARGIN
    assert l[0, :3].tolist() == [0, 1, 3]
    # the other member of the near tie
    m2 = np.zeros_like(m); m2[0, [0, 1, 2]] = 1
    l2 = np.full_like(l, -1); l2[0, :3] = [0, 1, 2]
    _, ex, nd = compare_selection(W.astype(np.float32), W, counts, 0.5, 3, m2, l2, c, orc)
    assert ex == 1 and nd == 1
    # a cluster far below the boundary is not a near tie
    m3 = np.zeros_like(m); m3[0, [0, 1, 4]] = 1
    l3 = np.full_like(l, -1); l3[0, :3] = [0, 1, 4]
    with pytest.raises(AssertionError):
        compare_selection(W.astype(np.float32), W, counts, 0.5, 3, m3, l3, c, orc)


def test_near_prefix():
    W = np.array([0.5, 0.2, 0.2 - 5e-6, 0.1, 0.0])
    counts = np.array([1, 1, 1, 1, 0], np.int32)
    assert near_prefix(W, counts, [0, 1]) and near_prefix(W, counts, [0, 2])
    assert not near_prefix(W, counts, [0, 3])
    assert not near_prefix(W, counts, [0, 4])          # an empty cluster is never selected


def test_teacher_forced_chain_accepts_the_oracle_and_rejects_a_moved_label(orc):
    rng = np.random.default_rng(4)
    mu = rng.normal(0, 2, (5, 8))
    z = rng.integers(0, 5, 300)
    Q = (mu[z] + rng.normal(0, 0.5, (300, 8))).astype(np.float32)
    K = (mu[z] + rng.normal(0, 0.5, (300, 8))).astype(np.float32)
    km = orc.cluster_keys(Q, K, 7, 4)["km"]
    hist = [x.copy() for x in km["labels_hist"]]
    n_diff, n_keys, _ = teacher_forced_chain(orc, Q, K, 7, hist)
    assert n_diff == 0 and n_keys == 4 * 300
    # move one key of step 3 to a cluster it is far from
    mar = km["margins"][2]
    j = int(np.argmax(mar))
    hist[2][j] = (hist[2][j] + 1) % 7
    with pytest.raises(AssertionError):
        teacher_forced_chain(orc, Q, K, 7, hist)
