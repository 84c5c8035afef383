"""Degenerate and maximum sizes through the whole path, GPU against the oracle: a single
token, one cluster, every key its own cluster, sizes just below, at and above one query block,
and the largest cluster and query-block counts the library takes, for both dtypes and head
sizes, with 64-token and clustered query blocks."""
import numpy as np
import pytest

from parity_util import check_scores, compare_selection, host, teacher_forced_chain, to_dev

pytestmark = pytest.mark.gpu

# (N, d, dtype, key clusters, query blocks for the clustered path)
SHAPES = [(1, 64, "f32", 1, 1), (1, 128, "bf16", 1, 1), (5, 64, "bf16", 5, 2), (63, 128, "f32", 1, 3),
          (64, 64, "bf16", 3, 1), (65, 128, "bf16", 65, 4), (129, 64, "f32", 7, 5), (200, 128, "bf16", 200, 8),
          # the library's maxima: PARK_MAX_CLUSTERS key clusters and PARK_MAX_QUERY_BLOCKS query blocks
          (4000, 128, "bf16", 1536, 1536), (3001, 64, "f32", 1536, 1536)]


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_response_amd as park
    park.lib()
    return park


def _inputs(N, d, dtype, seed):
    import torch
    rng = np.random.default_rng(seed)
    mu = rng.normal(0, 2, (3, d))
    z = rng.integers(0, 3, N)
    Q = (mu[z] + rng.normal(0, 0.5, (N, d)))[None, None].astype(np.float32)
    K = (mu[z] + rng.normal(0, 0.5, (N, d)))[None, None].astype(np.float32)
    V = rng.normal(0, 1, (1, 1, N, d)).astype(np.float32)
    if dtype == "bf16":   # values exactly representable in bf16, as the path reads them
        Q, K, V = (torch.from_numpy(x).to(torch.bfloat16).float().numpy() for x in (Q, K, V))
    return Q, K, V


@pytest.mark.parametrize("N,d,dtype,nk,nq", SHAPES)
def test_degenerate_sizes(dev, orc, N, d, dtype, nk, nq):
    import torch
    Q, K, V = _inputs(N, d, dtype, N * 7 + d)
    iters, top_p, top_k = 3, 0.9, 1
    scale = 1.0 / np.sqrt(d)
    q, k, v = (to_dev(x, dtype) for x in (Q, K, V))
    # clustering: from the GPU's labels the oracle's finalisation must match bit for bit, and
    # the labels must be the oracle's assignment from the GPU's previous step (teacher forced)
    runs = [{kk: host(vv) for kk, vv in dev.park_cluster_keys(q, k, nk, t).items()} for t in range(1, iters + 1)]
    cl = runs[-1]
    lab = cl["labels"][0, 0]
    assert lab.min() >= 0 and lab.max() < nk
    assert all(r["status"][0, 0] == 0 for r in runs)
    n_diff, n_keys, n_empty = teacher_forced_chain(orc, Q[0, 0], K[0, 0], nk, [r["labels"][0, 0] for r in runs])
    print(f"N={N} nk={nk}: {n_diff} near-tie label differences over {n_keys} keys, {n_empty} empty clusters")
    cent, counts, perm, offsets = orc.finalize(K[0, 0], lab, nk)
    assert np.array_equal(cl["counts"][0, 0], counts) and np.array_equal(cl["perm"][0, 0], perm)
    assert np.array_equal(cl["offsets"][0, 0], offsets)
    # retrieval and attention on the GPU's clustering
    rb = dev.park_retrieve_blocks(q, to_dev(cent[None, None], "f32"), to_dev(counts[None, None], "f32"), top_p, top_k)
    torch.cuda.synchronize()
    g = {kk: host(vv) for kk, vv in rb.items()}
    W = orc.pama(Q[0, 0], cent, counts, 64, scale)
    check_scores(g["scores"][0, 0], W)
    compare_selection(g["scores"][0, 0], W, counts, top_p, top_k, g["mask"][0, 0], g["block_list"][0, 0],
                      g["block_count"][0, 0], orc)
    O, lse = dev.park_block_sparse_attn(q, k, v, to_dev(perm[None, None], "f32"), to_dev(offsets[None, None], "f32"),
                                        rb["block_list"], rb["block_count"])
    torch.cuda.synchronize()
    Oo, lo = orc.block_sparse_attn(Q[0, 0], K[0, 0], V[0, 0], perm, offsets, g["block_list"][0, 0],
                                   g["block_count"][0, 0], 64, scale)
    tol = 2e-2 if dtype == "bf16" else 1e-4
    assert np.abs(host(O)[0, 0] - Oo).max() <= tol
    assert np.abs(host(lse)[0, 0] - lo).max() <= 1e-3
    # clustered query blocks on the oracle's query clustering
    qc = orc.cluster_queries(Q[0, 0], nq, iters)
    qp, qo = to_dev(qc["perm"][None, None], "f32"), to_dev(qc["offsets"][None, None], "f32")
    rc = dev.park_retrieve_blocks_clustered(q, to_dev(cent[None, None], "f32"), to_dev(counts[None, None], "f32"), qp, qo,
                                            top_p, top_k)
    torch.cuda.synchronize()
    gc = {kk: host(vv) for kk, vv in rc.items()}
    Wc = orc.pama_blocks(Q[0, 0], cent, counts, qc["perm"], qc["offsets"], scale)
    check_scores(gc["scores"][0, 0], Wc)
    compare_selection(gc["scores"][0, 0], Wc, counts, top_p, top_k, gc["mask"][0, 0], gc["block_list"][0, 0],
                      gc["block_count"][0, 0], orc)
    O2, lse2 = dev.park_block_sparse_attn_clustered(q, k, v, to_dev(perm[None, None], "f32"),
                                                    to_dev(offsets[None, None], "f32"), qp, qo, rc["block_list"],
                                                    rc["block_count"])
    torch.cuda.synchronize()
    Oo2, lo2 = orc.block_sparse_attn_blocks(Q[0, 0], K[0, 0], V[0, 0], perm, offsets, qc["perm"], qc["offsets"],
                                            gc["block_list"][0, 0], gc["block_count"][0, 0], scale)
    assert np.abs(host(O2)[0, 0] - Oo2).max() <= tol
    assert np.abs(host(lse2)[0, 0] - lo2).max() <= 1e-3


# The assignment screens in fp16.  A key with a component beyond the fp16 range has no finite
# screening bound, and a head whose |R c~| reaches 2^14 could overflow the screen operand: such
# keys compare every cluster exactly.  Queries scaled down keep R small, so the first two cases
# reach only the key condition (the first half of the keys scaled past the range, beside keys
# screened as usual, then every key); the third reaches only the head condition.  12 clusters
# fit a key's candidate lists, 40 do not.  (query scale, key scale, keys scaled)
RANGE_CASES = [(2.0 ** -10, 2.0 ** 15, 300), (2.0 ** -10, 2.0 ** 15, 600), (1.0, 2.0 ** 12, 600)]


@pytest.mark.parametrize("qscale,kscale,nscaled", RANGE_CASES)
@pytest.mark.parametrize("nk", [12, 40])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_screen_beyond_fp16_range(dev, orc, qscale, kscale, nscaled, nk, dtype):
    N, d, iters = 600, 128, 3
    Q, K, _ = _inputs(N, d, dtype, 11 * nk + nscaled)
    Q = Q * np.float32(qscale)
    K[0, 0, :nscaled] *= np.float32(kscale)   # powers of two: still exact in bf16
    _, _, R, ok = orc.query_metric(Q[0, 0])
    C0 = orc.init_centroids(orc.transform(K[0, 0], R), nk)
    beyond = int((np.abs(K[0, 0]) > 65504.0).any(axis=1).sum())
    G = float(np.linalg.norm(C0 @ R.T, axis=1).max())
    if qscale < 1.0:
        assert beyond == nscaled and G < 2.0 ** 14
    else:
        assert beyond == 0 and G >= 2.0 ** 14
    q, k = to_dev(Q, dtype), to_dev(K, dtype)
    runs = [{kk: host(vv) for kk, vv in dev.park_cluster_keys(q, k, nk, t).items()} for t in range(1, iters + 1)]
    assert all(r["status"][0, 0] == 0 for r in runs)
    n_diff, n_keys, _ = teacher_forced_chain(orc, Q[0, 0], K[0, 0], nk, [r["labels"][0, 0] for r in runs])
    print(f"keys beyond fp16 {beyond}/{N}, max |R c~| {G:.3g}: {n_diff} near-tie label differences over {n_keys} keys")
    lab = runs[-1]["labels"][0, 0]
    cent, counts, perm, offsets = orc.finalize(K[0, 0], lab, nk)
    assert np.array_equal(runs[-1]["counts"][0, 0], counts) and np.array_equal(runs[-1]["perm"][0, 0], perm)
    assert np.array_equal(runs[-1]["offsets"][0, 0], offsets)
