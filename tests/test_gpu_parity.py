"""GPU (HIP, gfx950) against the CPU oracle, through the C ABI, on seeded synthetic inputs.

Bars:
  * cluster assignments bit-exact except where the oracle's margin < 1e-5;
  * masks: the oracle's selection on its own W, bit-exact except in rows whose cut or gap
    margin lies within the score error;
  * retrieval scores W: relative error <= 1e-3 (absolute <= 1e-9 where W < 1e-6);
  * attention output: max abs error <= 2e-2 for bf16 (against the double oracle),
    1e-4 for float inputs.
k-means is checked stage by stage (teacher-forced): the labels after step t must equal
the oracle's assignment from the centroids the oracle computes from the GPU's labels of
step t-1.  Retrieval and attention get the oracle's clustering as input.
"""
import numpy as np
import pytest

import park_synth
from park_synth import Config
from parity_util import check_scores, compare_selection, host, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "cfg0-f32-d64": (park_synth.TINY, None),
    "ragged-bf16-d128": (Config("ragged-bf16-d128", 1, 2, (3, 10, 33), 0, 128, "bf16", 8, (44, 42, 42), 24, 4,
                                0.9, 3), None),
    "ragged-bf16-d64-text": (Config("ragged-bf16-d64", 1, 2, (2, 17, 29), 37, 64, "bf16", 6, (22, 21, 21), 20, 3,
                                    0.8, 2), None),
    "ragged-f32-d128": (Config("ragged-f32-d128", 2, 1, (1, 20, 35), 0, 128, "f32", 5, (44, 42, 42), 16, 3,
                               0.9, 4), None),
    "cfg1-2heads": (park_synth.WAN13B_480P, [0, 7]),
}


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_response_amd as park
    park.lib()
    return park


_data_cache = {}


def _data(name):
    if name not in _data_cache:
        cfg, heads = CASES[name]
        Q, K, V = park_synth.generate(cfg, seed=0, heads=heads)
        _data_cache[name] = (cfg, Q, K, V)
    return _data_cache[name]


_orc_cache = {}


def _oracle_clusters(orc, name):
    """Oracle clustering of every (b, h) of a case."""
    if name not in _orc_cache:
        cfg, Q, K, V = _data(name)
        B, H = Q.shape[:2]
        _orc_cache[name] = [[orc.cluster_keys(Q[b, h], K[b, h], cfg.n_clusters, cfg.iters) for h in range(H)]
                            for b in range(B)]
    return _orc_cache[name]


def _gpu_cluster(park, cfg, Q, K, iters, **kw):
    import torch
    out = park.park_cluster_keys(to_dev(Q, cfg.dtype), to_dev(K, cfg.dtype), cfg.n_clusters, iters, **kw)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


@pytest.mark.parametrize("name", list(CASES))
def test_cluster_stagewise(dev, orc, name):
    """Teacher-forced chain: GPU runs with 1..T steps give labels_t; the oracle rebuilds the
    centroids of step t-1 from the GPU's labels_{t-1} (its own update rule, empty clusters
    keeping their previous centroid) and its assignment must reproduce labels_t except at
    keys whose oracle margin is below 1e-5."""
    cfg, Q, K, V = _data(name)
    B, H = Q.shape[:2]
    runs = [None] + [_gpu_cluster(dev, cfg, Q, K, t) for t in range(1, cfg.iters + 1)]
    n_exempt = n_keys = 0
    for b in range(B):
        for h in range(H):
            _, _, R, ok = orc.query_metric(Q[b, h])
            assert ok
            Kt = orc.transform(K[b, h], R)
            C = orc.init_centroids(Kt, cfg.n_clusters)
            for t in range(1, cfg.iters + 1):
                assert runs[t]["status"][b, h] == 0
                if t >= 2:
                    C = orc.update(Kt, runs[t - 1]["labels"][b, h], C)
                lab_o, mar, _, _ = orc.assign(Kt, C)
                lab_g = runs[t]["labels"][b, h]
                diff = lab_o != lab_g
                assert np.all(mar[diff] < 1e-5), f"{name} b{b} h{h} step {t}: {diff.sum()} labels differ"
                n_exempt += int(diff.sum())
                n_keys += lab_o.size
    print(f"{name}: {n_exempt} near-tie label differences over {n_keys} checked keys")


@pytest.mark.parametrize("name", list(CASES))
def test_cluster_outputs(dev, orc, name):
    """counts / offsets / perm bit-exact and centroids equal to the oracle's finalisation of
    the GPU's own final labels.  With bf16 keys the GPU carries each cluster's member sum
    from step to step (adding the keys that joined, subtracting those that left) while the
    oracle sums the final members afresh; both double sums of bf16 values are exact (keys of
    magnitude 2^-24 and up), so the float means agree bit for bit but for a rare tiny key."""
    cfg, Q, K, V = _data(name)
    g = _gpu_cluster(dev, cfg, Q, K, cfg.iters)
    B, H = Q.shape[:2]
    n_diff = n_all = 0
    for b in range(B):
        for h in range(H):
            lab = g["labels"][b, h]
            assert lab.min() >= 0 and lab.max() < cfg.n_clusters
            cent, counts, perm, offsets = orc.finalize(K[b, h], lab, cfg.n_clusters)
            assert np.array_equal(g["counts"][b, h], counts)
            assert np.array_equal(g["offsets"][b, h], offsets)
            assert np.array_equal(g["perm"][b, h], perm)
            err = np.abs(g["centroids"][b, h] - cent).max() / max(1e-30, np.abs(cent).max())
            assert err <= 1e-6, err
            n_diff += int((g["centroids"][b, h] != cent).sum())
            n_all += cent.size
    print(f"{name}: {n_diff} of {n_all} centroid values not bit-equal to the oracle's")
    if cfg.dtype == "bf16":
        assert n_diff <= 1e-4 * n_all


@pytest.mark.parametrize("name", list(CASES))
def test_cluster_end_to_end_agreement(dev, orc, name):
    """Full runs on both sides: near-ties may cascade through later steps, so this reports
    the agreement and bounds the objective ratio instead of requiring equality."""
    cfg, Q, K, V = _data(name)
    g = _gpu_cluster(dev, cfg, Q, K, cfg.iters)
    ocl = _oracle_clusters(orc, name)
    B, H = Q.shape[:2]
    agree = []
    for b in range(B):
        for h in range(H):
            o = ocl[b][h]
            agree.append(np.mean(o["labels"] == g["labels"][b, h]))
            Jo = orc.objective(o["Kt"], orc.update(o["Kt"], o["labels"], o["km"]["centroids"]), o["labels"])
            Jg = orc.objective(o["Kt"], orc.update(o["Kt"], g["labels"][b, h], o["km"]["centroids"]),
                               g["labels"][b, h])
            assert Jg <= Jo * 1.01
    print(f"{name}: end-to-end label agreement min {min(agree):.5f} mean {np.mean(agree):.5f}")
    assert min(agree) >= 0.9


@pytest.mark.parametrize("pooled", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_retrieve(dev, orc, name, pooled):
    import torch
    cfg, Q, K, V = _data(name)
    ocl = _oracle_clusters(orc, name)
    B, H = Q.shape[:2]
    cent = np.stack([np.stack([ocl[b][h]["centroids"] for h in range(H)]) for b in range(B)])
    counts = np.stack([np.stack([ocl[b][h]["counts"] for h in range(H)]) for b in range(B)]).astype(np.int32)
    scale = 1.0 / np.sqrt(cfg.d)
    f = dev.park_retrieve_blocks_pooled if pooled else dev.park_retrieve_blocks
    out = f(to_dev(Q, cfg.dtype), to_dev(cent, "f32"), to_dev(counts, "f32"), cfg.top_p, cfg.top_k)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in out.items()}
    ref = orc.pooled_scores if pooled else orc.pama
    ex = rows = 0
    for b in range(B):
        for h in range(H):
            W_ref = ref(Q[b, h], cent[b, h], counts[b, h], 64, scale)
            check_scores(g["scores"][b, h], W_ref)
            n, e, _ = compare_selection(g["scores"][b, h], W_ref, counts[b, h], cfg.top_p, cfg.top_k, g["mask"][b, h],
                                     g["block_list"][b, h], g["block_count"][b, h], orc)
            rows += n; ex += e
    print(f"{name} pooled={pooled}: {ex} of {rows} rows exempt by margin")


@pytest.mark.parametrize("name", list(CASES))
def test_retrieve_unfused(dev, orc, name):
    """The unfused ablation (PARK section 5.1): the materialised probabilities P equal the
    oracle's per-query softmax (PAMA over one-query blocks), and its W and selection meet the
    same bars as the fused call's."""
    import torch
    cfg, Q, K, V = _data(name)
    ocl = _oracle_clusters(orc, name)
    B, H = Q.shape[:2]
    cent = np.stack([np.stack([ocl[b][h]["centroids"] for h in range(H)]) for b in range(B)])
    counts = np.stack([np.stack([ocl[b][h]["counts"] for h in range(H)]) for b in range(B)]).astype(np.int32)
    scale = 1.0 / np.sqrt(cfg.d)
    out = dev.park_retrieve_blocks_unfused(to_dev(Q, cfg.dtype), to_dev(cent, "f32"), to_dev(counts, "f32"),
                                           cfg.top_p, cfg.top_k)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in out.items()}
    assert g["probs"].shape == Q.shape[:3] + (cfg.n_clusters,)
    for b in range(B):
        for h in range(H):
            P_ref = orc.pama(Q[b, h], cent[b, h], counts[b, h], 1, scale)
            check_scores(g["probs"][b, h], P_ref)
            assert np.all(g["probs"][b, h][:, counts[b, h] == 0] == 0.0)
            W_ref = orc.pama(Q[b, h], cent[b, h], counts[b, h], 64, scale)
            check_scores(g["scores"][b, h], W_ref)
            compare_selection(g["scores"][b, h], W_ref, counts[b, h], cfg.top_p, cfg.top_k, g["mask"][b, h],
                              g["block_list"][b, h], g["block_count"][b, h], orc)


@pytest.mark.parametrize("p,k", [(0.0, 5), (1.0, 0), (0.5, 10 ** 6), (0.0, 0)])
def test_retrieve_edge_parameters(dev, orc, p, k):
    import torch
    name = "ragged-bf16-d128"
    cfg, Q, K, V = _data(name)
    ocl = _oracle_clusters(orc, name)
    cent = np.stack([o["centroids"] for o in ocl[0]])[None]
    counts = np.stack([o["counts"] for o in ocl[0]])[None].astype(np.int32)
    out = dev.park_retrieve_blocks(to_dev(Q, cfg.dtype), to_dev(cent, "f32"), to_dev(counts, "f32"), p, k)
    torch.cuda.synchronize()
    g = {kk: host(v) for kk, v in out.items()}
    for h in range(Q.shape[1]):
        W_ref = orc.pama(Q[0, h], cent[0, h], counts[0, h], 64, 1.0 / np.sqrt(cfg.d))
        compare_selection(g["scores"][0, h], W_ref, counts[0, h], p, k, g["mask"][0, h], g["block_list"][0, h],
                          g["block_count"][0, h], orc)


@pytest.mark.parametrize("nk", [288, 544, 1312])
def test_pama_spare_cluster_tiles(dev, orc, nk):
    """Cluster counts whose 32-cluster tiles do not fill the fused kernel's waves evenly (288:
    5 waves of two tiles for 9; 544: 6 of three for 17; 1312: 7 of six for 41): the spare
    tiles' logits start at -inf, as an empty cluster's do, and stay there.  W and the selection
    against the oracle, with some empty clusters."""
    import torch
    cfg = Config("spare", 1, 2, (2, 24, 30), 5, 128, "bf16", 8, (44, 42, 42), nk, 1, 0.9, 3)
    Q, _, _ = park_synth.generate(cfg, seed=11)
    rng = np.random.default_rng(nk)
    cent = rng.normal(0, 0.7, (1, 2, nk, 128)).astype(np.float32)
    counts = rng.integers(0, 40, (1, 2, nk)).astype(np.int32)
    counts[0, :, rng.integers(0, nk, 7)] = 0
    out = dev.park_retrieve_blocks(to_dev(Q, "bf16"), to_dev(cent, "f32"), to_dev(counts, "f32"), 0.9, 3)
    torch.cuda.synchronize()
    g = {kk: host(v) for kk, v in out.items()}
    for h in range(2):
        W_ref = orc.pama(Q[0, h], cent[0, h], counts[0, h], 64, 1.0 / np.sqrt(128))
        check_scores(g["scores"][0, h], W_ref)
        compare_selection(g["scores"][0, h], W_ref, counts[0, h], 0.9, 3, g["mask"][0, h], g["block_list"][0, h],
                          g["block_count"][0, h], orc)


def _attn_case(dev, orc, name, lists=None):
    import torch
    cfg, Q, K, V = _data(name)
    ocl = _oracle_clusters(orc, name)
    B, H, N, d = Q.shape
    scale = 1.0 / np.sqrt(d)
    NQ = (N + 63) // 64
    nk = cfg.n_clusters
    perm = np.zeros((B, H, N), np.int32); off = np.zeros((B, H, nk + 1), np.int32)
    lst = np.zeros((B, H, NQ, nk), np.int32); cnt = np.zeros((B, H, NQ), np.int32)
    for b in range(B):
        for h in range(H):
            o = ocl[b][h]
            perm[b, h], off[b, h] = o["perm"], o["offsets"]
            if lists is None:
                W = orc.pama(Q[b, h], o["centroids"], o["counts"], 64, scale)
                _, l, c, _, _ = orc.select(W, o["counts"], cfg.top_p, cfg.top_k)
            else:
                l, c = lists(NQ, nk)
            lst[b, h], cnt[b, h] = l, c
    O, lse = dev.park_block_sparse_attn(to_dev(Q, cfg.dtype), to_dev(K, cfg.dtype), to_dev(V, cfg.dtype),
                                        to_dev(perm, "f32"), to_dev(off, "f32"), to_dev(lst, "f32"),
                                        to_dev(cnt, "f32"))
    torch.cuda.synchronize()
    return cfg, Q, K, V, perm, off, lst, cnt, host(O), host(lse), scale


@pytest.mark.parametrize("name", list(CASES))
def test_attention_selected(dev, orc, name):
    cfg, Q, K, V, perm, off, lst, cnt, Og, lseg, scale = _attn_case(dev, orc, name)
    tol = 2e-2 if cfg.dtype == "bf16" else 1e-4
    B, H, N, d = Q.shape
    NQ = (N + 63) // 64
    ub = None if NQ <= 64 else np.unique(np.r_[np.arange(0, NQ, 7), NQ - 1])
    worst = 0.0
    for b in range(B):
        for h in range(H):
            Oo, lo = orc.block_sparse_attn(Q[b, h], K[b, h], V[b, h], perm[b, h], off[b, h], lst[b, h], cnt[b, h],
                                           64, scale, ub)
            rows = ~np.isnan(lo)
            err = np.abs(Og[b, h][rows] - Oo[rows]).max()
            worst = max(worst, err)
            assert err <= tol, f"{name} b{b} h{h}: max abs err {err:.3e}"
            assert np.abs(lseg[b, h][rows] - lo[rows]).max() <= 1e-3
    print(f"{name}: attention max abs err {worst:.3e}")


@pytest.mark.parametrize("name", ["cfg0-f32-d64", "ragged-bf16-d128", "ragged-bf16-d64-text", "ragged-f32-d128"])
def test_density_one_is_dense(dev, orc, name):
    """Listing every cluster gives dense attention (section 3.1)."""
    def all_blocks(NQ, nk):
        return np.tile(np.arange(nk, dtype=np.int32), (NQ, 1)), np.full(NQ, nk, np.int32)
    cfg, Q, K, V, perm, off, lst, cnt, Og, lseg, scale = _attn_case(dev, orc, name, all_blocks)
    tol = 2e-2 if cfg.dtype == "bf16" else 1e-4
    B, H, N, d = Q.shape
    for b in range(B):
        for h in range(H):
            Od, ld = orc.dense_attn(Q[b, h], K[b, h], V[b, h], scale)
            assert np.abs(Og[b, h] - Od).max() <= tol
            assert np.abs(lseg[b, h] - ld).max() <= 1e-3


def test_empty_and_partial_selection(dev, orc):
    """count 0 gives O = 0 and lse = -inf; a list with empty clusters and ids of one block."""
    def lists(NQ, nk):
        l = np.full((NQ, nk), -1, np.int32)
        c = np.zeros(NQ, np.int32)
        for u in range(NQ):
            if u % 3 == 1:
                c[u] = 1; l[u, 0] = u % nk
            elif u % 3 == 2:
                c[u] = 3; l[u, :3] = [0, nk // 2, nk - 1]
        return l, c
    name = "ragged-bf16-d128"
    cfg, Q, K, V, perm, off, lst, cnt, Og, lseg, scale = _attn_case(dev, orc, name, lists)
    for h in range(Q.shape[1]):
        Oo, lo = orc.block_sparse_attn(Q[0, h], K[0, h], V[0, h], perm[0, h], off[0, h], lst[0, h], cnt[0, h], 64, scale)
        z = np.isneginf(lo)
        assert np.all(np.isneginf(lseg[0, h][z])) and np.all(Og[0, h][z] == 0)
        assert np.abs(Og[0, h][~z] - Oo[~z]).max() <= 2e-2


@pytest.mark.parametrize("name", ["cfg0-f32-d64", "ragged-bf16-d128", "ragged-bf16-d64-text", "ragged-f32-d128"])
def test_exact_block_importance(dev, orc, name):
    """Retrieval-accuracy diagnostic (section 3.2, Eq. (3); appendix A, M1): the GPU's exact
    block importance against the oracle's, and the M1 error of the GPU's PAMA map measured
    with either one."""
    import torch
    cfg, Q, K, V = _data(name)
    ocl = _oracle_clusters(orc, name)
    B, H, N, d = Q.shape
    perm = np.stack([np.stack([o["perm"] for o in row]) for row in ocl]).astype(np.int32)
    off = np.stack([np.stack([o["offsets"] for o in row]) for row in ocl]).astype(np.int32)
    cent = np.stack([np.stack([o["centroids"] for o in row]) for row in ocl])
    counts = np.stack([np.stack([o["counts"] for o in row]) for row in ocl]).astype(np.int32)
    Wg = dev.park_block_importance_exact(to_dev(Q, cfg.dtype), to_dev(K, cfg.dtype), to_dev(perm, "f32"),
                                         to_dev(off, "f32"))
    rb = dev.park_retrieve_blocks(to_dev(Q, cfg.dtype), to_dev(cent, "f32"), to_dev(counts, "f32"), cfg.top_p,
                                  cfg.top_k)
    torch.cuda.synchronize()
    Wg, Wp = host(Wg), host(rb["scores"])
    tol = 2e-3 if cfg.dtype == "bf16" else 1e-5
    sizes = orc.block_sizes(N)
    for b in range(B):
        for h in range(H):
            Wx = orc.exact_block_importance(Q[b, h], K[b, h], ocl[b][h]["labels"], cfg.n_clusters, 64,
                                            1.0 / np.sqrt(d))
            assert np.abs(Wg[b, h] - Wx).max() <= tol
            assert abs(orc.tv(Wp[b, h], Wg[b, h], sizes) - orc.tv(Wp[b, h], Wx, sizes)) <= tol


@pytest.mark.parametrize("name", ["ragged-bf16-d128", "ragged-bf16-d64-text"])
def test_logmass_rmse(dev, orc, name):
    """Retrieval-accuracy diagnostic M2 (appendix B): the GPU's centred log-mass RMSE per head
    against the oracle's, for the oracle's QRKC clusters and for Euclidean ones."""
    import torch
    cfg, Q, K, V = _data(name)
    B, H, N, d = Q.shape
    for metric in ("qrkc", "euclidean"):
        cl = [[orc.cluster_keys(Q[b, h], K[b, h], cfg.n_clusters, cfg.iters, metric) for h in range(H)]
              for b in range(B)]
        st = {k: np.stack([np.stack([c[k] for c in row]) for row in cl]) for k in
              ("perm", "offsets", "centroids", "counts", "labels")}
        r = dev.park_logmass_rmse(to_dev(Q, cfg.dtype), to_dev(K, cfg.dtype), to_dev(st["perm"].astype(np.int32), "f32"),
                                  to_dev(st["offsets"].astype(np.int32), "f32"), to_dev(st["centroids"], "f32"),
                                  to_dev(st["counts"].astype(np.int32), "f32"))
        torch.cuda.synchronize()
        r = host(r)
        for b in range(B):
            for h in range(H):
                ref = orc.logmass_rmse(Q[b, h], K[b, h], st["labels"][b, h], st["centroids"][b, h],
                                       st["counts"][b, h], 1.0 / np.sqrt(d))
                assert abs(r[b, h] - ref) <= 1e-3 * ref, (metric, b, h, r[b, h], ref)
