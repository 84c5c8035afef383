"""Full-size parity at the benchmark shapes (all heads on the GPU, in the launch
configuration bench.py times), checked on sampled heads and sampled query blocks that the
CPU oracle can afford:
  * k-means: the first step from the anchors, and the last step teacher-forced (the oracle's
    centroids rebuilt from the GPU's labels of every earlier step; margin < 1e-5 exempt);
  * clustering outputs (counts, offsets, perm, centroids) against the oracle's finalisation
    of the GPU labels, for every head;
  * PAMA scores (rel 1e-3) and the selection (the oracle's on its own scores, bit-exact
    except where a cut or gap margin lies within the score error), teacher-forced on the
    GPU's own clustering;
  * attention on sampled query blocks (max abs 2e-2 against the double oracle);
  * and, with no oracle input from the GPU, one head clustered by the oracle from scratch: label
    agreement and objective against the GPU's full run, then retrieval and attention on the
    oracle's clustering and selection.
"""
import numpy as np
import pytest

import park_synth
from parity_util import check_scores, compare_selection, host, teacher_forced_chain, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_response_amd as park
    park.lib()
    return park


def _run(park, cfg, Q, K, V, iters, top_p, top_k, metric="qrkc", pooled=False):
    import torch
    q, k, v = (to_dev(x, cfg.dtype) for x in (Q, K, V))
    cl = park.park_cluster_keys(q, k, cfg.n_clusters, iters, metric=metric)
    f = park.park_retrieve_blocks_pooled if pooled else park.park_retrieve_blocks
    rb = f(q, cl["centroids"], cl["counts"], top_p, top_k)
    O, lse = park.park_block_sparse_attn(q, k, v, cl["perm"], cl["offsets"], rb["block_list"], rb["block_count"])
    torch.cuda.synchronize()
    out = {kk: host(vv) for kk, vv in cl.items()}
    out.update({kk: host(vv) for kk, vv in rb.items()})
    out["O"], out["lse"] = host(O), host(lse)
    del q, k, v, O, lse
    return out


def _cluster_labels(park, cfg, Q, K, iters):
    """The GPU's labels after 1 .. iters - 1 Lloyd steps (clustering only, every head)."""
    import torch
    q, k = (to_dev(x, cfg.dtype) for x in (Q, K))
    out = []
    for t in range(1, iters):
        cl = park.park_cluster_keys(q, k, cfg.n_clusters, t)
        torch.cuda.synchronize()
        out.append(host(cl["labels"]))
        assert np.all(host(cl["status"]) == 0)
        del cl
    del q, k
    torch.cuda.empty_cache()
    return out


def _check_head(orc, cfg, Q, K, V, labels_hist, gT, b, h, top_p, top_k, metric="qrkc", pooled=False, ub_step=37):
    q, k, v = Q[b, h], K[b, h], V[b, h]
    nk = cfg.n_clusters
    _, _, R, ok = orc.query_metric(q, metric=metric)
    assert ok
    # the first and the last step, teacher-forced: the oracle's centroid chain follows the
    # GPU's labels of every step (empty clusters keep their centroid), and its assignment
    # must give the GPU's labels after step 1 and after step T
    chain = [lh[b, h] for lh in labels_hist] + [gT["labels"][b, h]]
    n_diff, n_keys, n_empty = teacher_forced_chain(orc, q, k, nk, chain, metric=metric, steps=(1, len(chain)))
    print(f"head {h}: {n_diff} near-tie label differences over {n_keys} keys (steps 1 and {len(chain)}), "
          f"{n_empty} empty clusters along the chain")
    # outputs of the final clustering
    cent, counts, perm, offsets = orc.finalize(k, gT["labels"][b, h], nk)
    assert np.array_equal(gT["counts"][b, h], counts)
    assert np.array_equal(gT["offsets"][b, h], offsets)
    assert np.array_equal(gT["perm"][b, h], perm)
    assert np.abs(gT["centroids"][b, h] - cent).max() <= 1e-6 * max(1.0, np.abs(cent).max())
    # retrieval on the GPU's clustering
    scale = 1.0 / np.sqrt(q.shape[1])
    ref = orc.pooled_scores if pooled else orc.pama
    W = ref(q, cent, counts, 64, scale)
    check_scores(gT["scores"][b, h], W)
    _, ex, _ = compare_selection(gT["scores"][b, h], W, counts, top_p, top_k, gT["mask"][b, h], gT["block_list"][b, h],
                              gT["block_count"][b, h], orc)
    # attention on sampled query blocks
    NQ = W.shape[0]
    ub = np.unique(np.r_[np.arange(0, NQ, ub_step), NQ - 1])
    Oo, lo = orc.block_sparse_attn(q, k, v, perm, offsets, gT["block_list"][b, h], gT["block_count"][b, h], 64,
                                   scale, ub)
    rows = ~np.isnan(lo)
    err = np.abs(gT["O"][b, h][rows] - Oo[rows]).max()
    assert err <= 2e-2, f"attention max abs err {err}"
    assert np.abs(gT["lse"][b, h][rows] - lo[rows]).max() <= 1e-3
    return ex, err


@pytest.mark.parametrize("cid,heads", [("wan1.3b-480p-21x30x52", (0, 11)), ("wan2.1-14b-720p-21x45x80", (0, 39)),
                                       ("hunyuan-720p-33x45x80+256text", (5, 23))])
def test_fullsize_workload(dev, orc, cid, heads):
    cfg = park_synth.WORKLOADS[cid]
    Q, K, V = park_synth.generate(cfg, seed=0, workers=16)
    labels_hist = _cluster_labels(dev, cfg, Q, K, cfg.iters)
    gT = _run(dev, cfg, Q, K, V, cfg.iters, cfg.top_p, cfg.top_k)
    B, H = Q.shape[:2]
    for b in range(B):
        for h in range(H):   # every head: output invariants
            off = gT["offsets"][b, h]
            assert off[0] == 0 and off[-1] == cfg.N
            assert np.array_equal(np.sort(gT["perm"][b, h]), np.arange(cfg.N))
            assert np.array_equal(np.diff(off), gT["counts"][b, h])
            assert np.all(gT["block_count"][b, h] >= np.minimum(cfg.top_k, (gT["counts"][b, h] > 0).sum()))
    for h in heads:
        ex, err = _check_head(orc, cfg, Q, K, V, labels_hist, gT, 0, h, cfg.top_p, cfg.top_k)
        print(f"{cid} head {h}: {ex} selection rows exempt by margin, attention err {err:.2e}")


@pytest.mark.parametrize("pooled", [False, True])
def test_density_sweep_config4(dev, orc, pooled):
    """The density sweep: forced top-k (top_p = 0) at the 75.6k-token shape; PARK and the pooled-query /
    Euclidean-key baseline.  k = 1024 (every cluster) must reproduce dense attention."""
    cfg = park_synth.DENSITY_SWEEP
    Q, K, V = park_synth.generate(cfg, seed=0, heads=[0, 1, 2, 3], workers=4)
    metric = "euclidean" if pooled else "qrkc"
    import torch
    ref = orc.pooled_scores if pooled else orc.pama
    W_ref = cl_ref = None
    for kk in cfg.forced_k:
        g = _run(dev, cfg, Q, K, V, cfg.iters, 0.0, kk, metric=metric, pooled=pooled)
        h = 1
        counts = g["counts"][0, h]
        nne = int((counts > 0).sum())
        assert np.all(g["block_count"][0, h] == min(kk, nne))
        # the clustering does not depend on k: the oracle's scores on it are computed once
        if W_ref is None:
            cl_ref = (g["centroids"][0, h].copy(), counts.copy())
            W_ref = ref(Q[0, h], cl_ref[0], cl_ref[1], 64, 1.0 / np.sqrt(cfg.d))
        assert np.array_equal(counts, cl_ref[1]) and np.array_equal(g["centroids"][0, h], cl_ref[0])
        compare_selection(g["scores"][0, h], W_ref, counts, 0.0, kk, g["mask"][0, h], g["block_list"][0, h],
                          g["block_count"][0, h], orc)
        if kk == 1024:
            rows = np.r_[np.arange(0, cfg.N, 997), cfg.N - 1]
            Od, ld = orc.dense_attn(Q[0, h], K[0, h], V[0, h], 1.0 / np.sqrt(cfg.d), rows)
            assert np.abs(g["O"][0, h][rows] - Od).max() <= 2e-2
            assert np.abs(g["lse"][0, h][rows] - ld).max() <= 1e-3
        torch.cuda.empty_cache()


@pytest.mark.parametrize("cid,h", [("wan2.1-14b-720p-21x45x80", 17), ("hunyuan-720p-33x45x80+256text", 9)])
def test_fullsize_from_oracle_clustering(dev, orc, cid, h):
    """A full-size head with no oracle input taken from the GPU.  The oracle clusters head h
    from scratch: the GPU's own full run must agree on >= 99% of the labels with an objective
    within 1% (near-ties may cascade through the steps).  Then the GPU retrieval and attention,
    launched on every head as the benchmark does, take the oracle's clustering (and, for the
    attention, the oracle's selection) for head h, and head h's scores, selection and sampled
    query blocks meet the usual bars against the oracle on those same inputs."""
    import torch
    cfg = park_synth.WORKLOADS[cid]
    Q, K, V = park_synth.generate(cfg, seed=0, workers=16)
    g = _run(dev, cfg, Q, K, V, cfg.iters, cfg.top_p, cfg.top_k)
    nk, scale = cfg.n_clusters, 1.0 / np.sqrt(cfg.d)
    o = orc.cluster_keys(Q[0, h], K[0, h], nk, cfg.iters)
    agree = float(np.mean(o["labels"] == g["labels"][0, h]))
    Jo = orc.objective(o["Kt"], orc.update(o["Kt"], o["labels"], o["km"]["centroids"]), o["labels"])
    Jg = orc.objective(o["Kt"], orc.update(o["Kt"], g["labels"][0, h], o["km"]["centroids"]), g["labels"][0, h])
    print(f"{cid} head {h}: label agreement {agree:.5f}, objective ratio {Jg / Jo:.6f}")
    assert agree >= 0.99 and Jg <= Jo * 1.01
    # retrieval on the oracle's clustering of head h
    cent, counts = g["centroids"].copy(), g["counts"].copy()
    perm, offsets = g["perm"].copy(), g["offsets"].copy()
    cent[0, h], counts[0, h], perm[0, h], offsets[0, h] = o["centroids"], o["counts"], o["perm"], o["offsets"]
    q, k, v = (to_dev(x, cfg.dtype) for x in (Q, K, V))
    rb = dev.park_retrieve_blocks(q, to_dev(cent, "f32"), to_dev(counts, "f32"), cfg.top_p, cfg.top_k)
    torch.cuda.synchronize()
    W = orc.pama(Q[0, h], o["centroids"], o["counts"], 64, scale)
    sc = host(rb["scores"][0, h])
    check_scores(sc, W)
    _, ex, _ = compare_selection(sc, W, o["counts"], cfg.top_p, cfg.top_k, host(rb["mask"][0, h]),
                              host(rb["block_list"][0, h]), host(rb["block_count"][0, h]), orc)
    # attention with the oracle's selection for head h
    _, lst_o, cnt_o, _, _ = orc.select(W, o["counts"], cfg.top_p, cfg.top_k)
    lst, cnt = rb["block_list"].clone(), rb["block_count"].clone()
    lst[0, h] = torch.from_numpy(lst_o).to(lst.device)
    cnt[0, h] = torch.from_numpy(cnt_o).to(cnt.device)
    O, lse = dev.park_block_sparse_attn(q, k, v, to_dev(perm, "f32"), to_dev(offsets, "f32"), lst, cnt)
    torch.cuda.synchronize()
    NQ = W.shape[0]
    ub = np.unique(np.r_[np.arange(0, NQ, 37), NQ - 1])
    Oo, lo = orc.block_sparse_attn(Q[0, h], K[0, h], V[0, h], o["perm"], o["offsets"], lst_o, cnt_o, 64, scale, ub)
    rows = np.concatenate([np.arange(64 * u, min(64 * u + 64, cfg.N)) for u in ub])
    err = np.abs(host(O[0, h])[rows] - Oo[rows]).max()
    print(f"{cid} head {h}: {ex} selection rows exempt, attention err {err:.2e}")
    assert err <= 2e-2
    assert np.abs(host(lse[0, h])[rows] - lo[rows]).max() <= 1e-3
    del q, k, v, O, lse
    torch.cuda.empty_cache()
