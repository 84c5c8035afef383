"""Clustered query blocks (PARK's own setting: Euclidean k-means of the queries into N_Q
blocks, Figure 2 and section 6 "Implementations"), GPU against the CPU oracle through the
C ABI on seeded synthetic inputs, with the bars of the 64-token path:
  * query-cluster labels bit-exact (teacher-forced) except where the oracle's margin < 1e-5,
    counts / offsets / perm bit-exact;
  * W relative error <= 1e-3; the selection equals the oracle's on the oracle's own W except
    in rows whose cut or gap margin lies within the score error;
  * attention max abs error <= 2e-2 for bf16 against the double oracle, 1e-4 for float,
    lse within 1e-3.
Retrieval and attention take the oracle's query and key clusterings as inputs."""
import numpy as np
import pytest

import park_synth
from park_synth import Config
from parity_util import check_scores, compare_selection, host, to_dev

pytestmark = pytest.mark.gpu

# (config, heads, query blocks)
CASES = {
    "cfg0-f32-d64-q16": (park_synth.TINY, None, 16),
    "ragged-bf16-d128-q8": (Config("ragged-bf16-d128", 1, 2, (3, 10, 33), 0, 128, "bf16", 8, (44, 42, 42), 24, 4,
                                   0.9, 3), None, 8),
    "ragged-bf16-d64-text-q5": (Config("ragged-bf16-d64", 1, 2, (2, 17, 29), 37, 64, "bf16", 6, (22, 21, 21), 20, 3,
                                       0.8, 2), None, 5),
    "cfg1-2heads-q128": (park_synth.WAN13B_480P, [0, 7], 128),
}


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_response_amd as park
    park.lib()
    return park


_cache = {}


def _case(orc, name):
    """Inputs plus the oracle's query and key clusterings of every (b, h)."""
    if name not in _cache:
        cfg, heads, nq = CASES[name]
        Q, K, V = park_synth.generate(cfg, seed=0, heads=heads)
        B, H = Q.shape[:2]
        qc = [[orc.cluster_queries(Q[b, h], nq, cfg.iters) for h in range(H)] for b in range(B)]
        kc = [[orc.cluster_keys(Q[b, h], K[b, h], cfg.n_clusters, cfg.iters) for h in range(H)] for b in range(B)]
        _cache[name] = (cfg, nq, Q, K, V, qc, kc)
    return _cache[name]


def _stack(cl, key, dtype=None):
    a = np.stack([np.stack([c[key] for c in row]) for row in cl])
    return a.astype(dtype) if dtype is not None else a


def test_cluster_queries_stagewise(dev, orc):
    """Teacher-forced chain, as for the keys, on the raw queries (R = I): labels after step t
    equal the oracle's assignment from the centroids it rebuilds from the GPU's step t-1."""
    import torch
    for name in ("ragged-bf16-d128-q8", "cfg0-f32-d64-q16"):
        cfg, nq, Q, K, V, qc, kc = _case(orc, name)
        B, H = Q.shape[:2]
        runs = [None]
        for t in range(1, cfg.iters + 1):
            o = dev.park_cluster_queries(to_dev(Q, cfg.dtype), nq, t)
            torch.cuda.synchronize()
            runs.append({k: host(v) for k, v in o.items()})
        diff_total = 0
        for b in range(B):
            for h in range(H):
                Xt = orc.transform(Q[b, h], np.eye(cfg.d))
                C = orc.init_centroids(Xt, nq)
                for t in range(1, cfg.iters + 1):
                    if t >= 2:
                        C = orc.update(Xt, runs[t - 1]["labels"][b, h], C)
                    lab_o, mar, _, _ = orc.assign(Xt, C)
                    diff = lab_o != runs[t]["labels"][b, h]
                    assert np.all(mar[diff] < 1e-5), f"{name} b{b} h{h} step {t}: {diff.sum()} labels differ"
                    diff_total += int(diff.sum())
                g = runs[cfg.iters]
                cent, counts, perm, offsets = orc.finalize(Q[b, h], g["labels"][b, h], nq)
                assert np.array_equal(g["counts"][b, h], counts)
                assert np.array_equal(g["offsets"][b, h], offsets)
                assert np.array_equal(g["perm"][b, h], perm)
                assert np.abs(g["centroids"][b, h] - cent).max() <= 1e-6 * max(1e-30, np.abs(cent).max())
        print(f"{name}: {diff_total} near-tie label differences")


@pytest.mark.parametrize("name", list(CASES))
def test_retrieve_clustered(dev, orc, name):
    import torch
    cfg, nq, Q, K, V, qc, kc = _case(orc, name)
    B, H = Q.shape[:2]
    cent = _stack(kc, "centroids"); counts = _stack(kc, "counts", np.int32)
    qperm = _stack(qc, "perm", np.int32); qoff = _stack(qc, "offsets", np.int32)
    out = dev.park_retrieve_blocks_clustered(to_dev(Q, cfg.dtype), to_dev(cent, "f32"), to_dev(counts, "f32"),
                                             to_dev(qperm, "f32"), to_dev(qoff, "f32"), cfg.top_p, cfg.top_k)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in out.items()}
    assert g["scores"].shape == (B, H, nq, cfg.n_clusters)
    scale = 1.0 / np.sqrt(cfg.d)
    rows = ex = 0
    for b in range(B):
        for h in range(H):
            W = orc.pama_blocks(Q[b, h], cent[b, h], counts[b, h], qperm[b, h], qoff[b, h], scale)
            check_scores(g["scores"][b, h], W)
            n, e, _ = compare_selection(g["scores"][b, h], W, counts[b, h], cfg.top_p, cfg.top_k, g["mask"][b, h],
                                     g["block_list"][b, h], g["block_count"][b, h], orc)
            rows += n; ex += e
    print(f"{name}: {ex} of {rows} rows exempt by margin")


def _attn(dev, orc, name, lists=None, qperm=None, qoff=None):
    import torch
    cfg, nq, Q, K, V, qc, kc = _case(orc, name)
    B, H, N, d = Q.shape
    nk = cfg.n_clusters
    scale = 1.0 / np.sqrt(d)
    perm = _stack(kc, "perm", np.int32); off = _stack(kc, "offsets", np.int32)
    if qperm is None:
        qperm = _stack(qc, "perm", np.int32); qoff = _stack(qc, "offsets", np.int32)
    nqb = qoff.shape[-1] - 1
    lst = np.zeros((B, H, nqb, nk), np.int32); cnt = np.zeros((B, H, nqb), np.int32)
    for b in range(B):
        for h in range(H):
            if lists is None:
                W = orc.pama_blocks(Q[b, h], kc[b][h]["centroids"], kc[b][h]["counts"], qperm[b, h], qoff[b, h], scale)
                _, l, c, _, _ = orc.select(W, kc[b][h]["counts"], cfg.top_p, cfg.top_k)
            else:
                l, c = lists(nqb, nk)
            lst[b, h], cnt[b, h] = l, c
    O, lse = dev.park_block_sparse_attn_clustered(to_dev(Q, cfg.dtype), to_dev(K, cfg.dtype), to_dev(V, cfg.dtype),
                                                  to_dev(perm, "f32"), to_dev(off, "f32"), to_dev(qperm, "f32"),
                                                  to_dev(qoff, "f32"), to_dev(lst, "f32"), to_dev(cnt, "f32"))
    torch.cuda.synchronize()
    return cfg, Q, K, V, perm, off, qperm, qoff, lst, cnt, host(O), host(lse), scale


def _check_attn(orc, name, res, ub=None):
    cfg, Q, K, V, perm, off, qperm, qoff, lst, cnt, Og, lseg, scale = res
    tol = 2e-2 if cfg.dtype == "bf16" else 1e-4
    B, H = Q.shape[:2]
    worst = 0.0
    for b in range(B):
        for h in range(H):
            Oo, lo = orc.block_sparse_attn_blocks(Q[b, h], K[b, h], V[b, h], perm[b, h], off[b, h], qperm[b, h],
                                                  qoff[b, h], lst[b, h], cnt[b, h], scale, ub)
            rows = ~np.isnan(lo)
            fin = rows & np.isfinite(lo)
            assert np.all(np.isneginf(lseg[b, h][rows & ~fin])) and np.all(Og[b, h][rows & ~fin] == 0)
            if fin.any():
                err = np.abs(Og[b, h][fin] - Oo[fin]).max()
                worst = max(worst, err)
                assert err <= tol, f"{name} b{b} h{h}: max abs err {err:.3e}"
                assert np.abs(lseg[b, h][fin] - lo[fin]).max() <= 1e-3
    return worst


@pytest.mark.parametrize("name", list(CASES))
def test_attention_clustered(dev, orc, name):
    res = _attn(dev, orc, name)
    nq = CASES[name][2]
    ub = None if nq <= 16 else np.unique(np.r_[np.arange(0, nq, 9), nq - 1])
    print(f"{name}: attention max abs err {_check_attn(orc, name, res, ub):.3e}")


@pytest.mark.parametrize("name", ["cfg0-f32-d64-q16", "ragged-bf16-d128-q8", "ragged-bf16-d64-text-q5"])
def test_attention_clustered_density_one(dev, orc, name):
    """Every key cluster for every query block: dense attention for every query."""
    def all_blocks(nqb, nk):
        return np.tile(np.arange(nk, dtype=np.int32), (nqb, 1)), np.full(nqb, nk, np.int32)
    cfg, Q, K, V, perm, off, qperm, qoff, lst, cnt, Og, lseg, scale = _attn(dev, orc, name, all_blocks)
    tol = 2e-2 if cfg.dtype == "bf16" else 1e-4
    for b in range(Q.shape[0]):
        for h in range(Q.shape[1]):
            Od, ld = orc.dense_attn(Q[b, h], K[b, h], V[b, h], scale)
            assert np.abs(Og[b, h] - Od).max() <= tol
            assert np.abs(lseg[b, h] - ld).max() <= 1e-3


def test_ragged_and_empty_query_blocks(dev, orc):
    """Blocks of 0, 1, 63, 64, 65 and the remaining queries of a random permutation, with a
    selection that leaves one block without clusters: retrieval and attention against the
    oracle (an empty block has a zero W row; queries with no keys get O = 0, lse = -inf)."""
    import torch
    name = "ragged-bf16-d128-q8"
    cfg, nq, Q, K, V, qc, kc = _case(orc, name)
    B, H, N, d = Q.shape
    rng = np.random.default_rng(5)
    sizes = [0, 1, 63, 64, 65]
    sizes.append(N - sum(sizes))
    qperm = np.stack([np.stack([rng.permutation(N).astype(np.int32) for _ in range(H)]) for _ in range(B)])
    qoff = np.broadcast_to(np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32), (B, H, len(sizes) + 1)).copy()
    cent = _stack(kc, "centroids"); counts = _stack(kc, "counts", np.int32)
    out = dev.park_retrieve_blocks_clustered(to_dev(Q, cfg.dtype), to_dev(cent, "f32"), to_dev(counts, "f32"),
                                             to_dev(qperm, "f32"), to_dev(qoff, "f32"), cfg.top_p, cfg.top_k)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in out.items()}
    scale = 1.0 / np.sqrt(d)
    for b in range(B):
        for h in range(H):
            W = orc.pama_blocks(Q[b, h], cent[b, h], counts[b, h], qperm[b, h], qoff[b, h], scale)
            assert np.all(g["scores"][b, h][0] == 0) and np.all(W[0] == 0)
            check_scores(g["scores"][b, h], W)

    def lists(nqb, nk):
        l = np.full((nqb, nk), -1, np.int32); c = np.zeros(nqb, np.int32)
        for u in range(nqb):
            if u != 2:
                c[u] = min(nk, u + 1); l[u, :c[u]] = np.arange(0, nk, max(1, nk // (u + 1)))[:c[u]]
        return l, c
    res = _attn(dev, orc, name, lists, qperm, qoff)
    print(f"ragged blocks: attention max abs err {_check_attn(orc, name, res):.3e}")


def test_consecutive_blocks_match_64_token_path(dev, orc):
    """The identity permutation with 64-token offsets makes the clustered entry points compute
    the 64-token ones: W differs at most by the final division's rounding; attention sees the
    same queries and tiles, but the clustered call takes a block's tiles in one pass where the
    64-token call splits them into key ranges and merges the partial states, so O agrees to two
    bf16 units in the last place and lse to float rounding."""
    import torch
    name = "ragged-bf16-d128-q8"
    cfg, nq, Q, K, V, qc, kc = _case(orc, name)
    B, H, N, d = Q.shape
    NQ = (N + 63) // 64
    qperm = np.broadcast_to(np.arange(N, dtype=np.int32), (B, H, N)).copy()
    qoff = np.broadcast_to(np.minimum(np.arange(NQ + 1) * 64, N).astype(np.int32), (B, H, NQ + 1)).copy()
    cent = _stack(kc, "centroids"); counts = _stack(kc, "counts", np.int32)
    perm = _stack(kc, "perm", np.int32); off = _stack(kc, "offsets", np.int32)
    args = (to_dev(Q, cfg.dtype), to_dev(cent, "f32"), to_dev(counts, "f32"))
    a = dev.park_retrieve_blocks(*args, cfg.top_p, cfg.top_k)
    c = dev.park_retrieve_blocks_clustered(*args, to_dev(qperm, "f32"), to_dev(qoff, "f32"), cfg.top_p, cfg.top_k)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(c["scores"]), host(a["scores"]), rtol=1e-6, atol=1e-12)
    lst, cnt = a["block_list"], a["block_count"]
    dv = [to_dev(x, cfg.dtype) for x in (Q, K, V)]
    O1, l1 = dev.park_block_sparse_attn(*dv, to_dev(perm, "f32"), to_dev(off, "f32"), lst, cnt)
    O2, l2 = dev.park_block_sparse_attn_clustered(*dv, to_dev(perm, "f32"), to_dev(off, "f32"), to_dev(qperm, "f32"),
                                                  to_dev(qoff, "f32"), lst, cnt)
    torch.cuda.synchronize()
    o1, o2 = host(O1).astype(np.float64), host(O2).astype(np.float64)
    assert np.all(np.abs(o2 - o1) <= 2.0 ** -6 * np.maximum(1.0, np.abs(o1)))
    lse1, lse2 = host(l1).astype(np.float64), host(l2).astype(np.float64)
    assert np.all(np.abs(lse2 - lse1) <= 1e-5 * np.maximum(1.0, np.abs(lse1)))
