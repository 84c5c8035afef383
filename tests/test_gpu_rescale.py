"""The attention kernel's moves of its softmax reference, GPU against the oracle.

An item's reference m starts at its first tile's row maximum.  Here the clustering and the
selection are given by hand so that one key range holds two clusters in order: a first one whose
scores are 0 and a second one whose scores lie a chosen number of log2 units above them.  At 80
units a tile's probability sums leave [0, 2^60] but stay finite, so the reference moves with a
rescale.  At 200 units the probabilities overflow float, so the scores are recomputed.  Both must
give the exact softmax over the selected keys (PARK section 3.1, E1/E2) that the oracle computes.

Cluster sizes and the range placement: every block selects all five clusters.  The ranges are
dealt by work (selections x 8-key groups), largest first, serpentine over the four ranges, ties
to the lower id.  So clusters 0-2 (64 keys, 8 groups each) take ranges 0-2, and clusters 3 (32
keys, one full tile) and 4 (8 keys) both land in range 3, in that order.
"""
import numpy as np
import pytest

from parity_util import host, to_dev

pytestmark = pytest.mark.gpu

SIZES = [64, 64, 64, 32, 8]   # keys per cluster, in permutation order
D = 128


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_response_amd as park
    park.lib()
    return park


def _inputs(gap_log2, seed):
    """Q, K, V (bf16-exact) and the clustering: every query (32, 0, ..., 0) plus noise in the
    other coordinates; keys of clusters 0-3 orthogonal to it (score 0); keys of cluster 4 along
    it, so that their scores exceed the others' by gap_log2 log2 units."""
    rng = np.random.default_rng(seed)
    N = sum(SIZES)
    scale = 1.0 / np.sqrt(D)
    Q = np.zeros((N, D), np.float32)
    Q[:, 0] = 32.0
    Q[:, 2:] = rng.integers(-2, 3, (N, D - 2))
    K = np.zeros((N, D), np.float32)
    K[:, 1] = rng.integers(-4, 5, N)          # clusters 0-3: orthogonal to every query
    k4 = gap_log2 / (np.log2(np.e) * scale * 32.0)
    start = sum(SIZES[:4])
    K[start:, 0] = np.round(k4)               # cluster 4 (the last 8 positions): along the queries
    K[start:, 1] = 0.0
    V = rng.integers(-8, 9, (N, D)).astype(np.float32) / 8.0
    perm = np.arange(N, dtype=np.int32)
    offsets = np.concatenate([[0], np.cumsum(SIZES)]).astype(np.int32)
    NQ = (N + 63) // 64
    nk = len(SIZES)
    lst = np.tile(np.arange(nk, dtype=np.int32), (NQ, 1))
    cnt = np.full(NQ, nk, np.int32)
    return Q, K, V, perm, offsets, lst, cnt, scale


@pytest.mark.parametrize("gap", [80.0, 200.0])
def test_reference_moves(dev, gap):
    import oracle
    Q, K, V, perm, offsets, lst, cnt, scale = _inputs(gap, seed=int(gap))
    N = Q.shape[0]
    as_bf16 = lambda x: to_dev(x[None, None], "bf16")
    as_i32 = lambda x: to_dev(x[None, None], "i32")
    O, lse = dev.park_block_sparse_attn(as_bf16(Q), as_bf16(K), as_bf16(V), as_i32(perm), as_i32(offsets),
                                        as_i32(lst), as_i32(cnt))
    Oo, lo = oracle.block_sparse_attn(Q, K, V, perm, offsets, lst, cnt, 64, scale)
    Og = host(O)[0, 0].astype(np.float64)
    lg = host(lse)[0, 0].astype(np.float64)
    assert np.all(np.isfinite(Og)) and np.all(np.isfinite(lg))
    assert np.abs(Og - Oo).max() <= 2e-2
    assert np.abs(lg - lo).max() <= 1e-3
    # the softmax is carried by cluster 4 alone: O is close to the mean of its values
    assert np.abs(Oo - V[N - SIZES[-1]:].mean(axis=0)).max() < 1e-6
