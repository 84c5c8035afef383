"""The step schedule on the GPU: dense steps are dense attention, reuse steps compute the
current Q, K, V with the kept clustering and selection (checked against the oracle given
that clustering), and reusing on unchanged inputs reproduces the recompute step exactly."""
import numpy as np
import pytest

import park_synth
from park_synth import Config
from parity_util import host, to_dev

pytestmark = pytest.mark.gpu

CFG = Config("ragged-bf16-d128", 1, 2, (3, 10, 33), 0, 128, "bf16", 8, (44, 42, 42), 24, 4, 0.9, 3)


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_response_amd as park
    park.lib()
    return park


def _inputs():
    Q, K, V = park_synth.generate(CFG, seed=0)
    rng = np.random.default_rng(1)
    # the next step's activations: a small drift, rounded to bf16 like the inputs
    import torch
    drift = [torch.from_numpy(x + rng.normal(0, 0.05, x.shape).astype(np.float32)).to(torch.bfloat16).float().numpy()
             for x in (Q, K, V)]
    return (Q, K, V), tuple(drift)


def test_dense_step_is_dense_attention(dev, orc):
    from block_sparse_attention_response_amd.schedule import ParkSchedule
    import torch
    (Q, K, V), _ = _inputs()
    s = ParkSchedule(CFG.n_clusters, CFG.iters, CFG.top_p, CFG.top_k, total_steps=10, dense_fraction=0.2)
    O, lse = s.attention(0, *(to_dev(x, "bf16") for x in (Q, K, V)))
    torch.cuda.synchronize()
    for h in range(Q.shape[1]):
        Od, ld = orc.dense_attn(Q[0, h], K[0, h], V[0, h], 1.0 / np.sqrt(CFG.d))
        assert np.abs(host(O)[0, h] - Od).max() <= 2e-2
        assert np.abs(host(lse)[0, h] - ld).max() <= 1e-3


@pytest.mark.parametrize("query_blocks", [None, 6])
def test_reuse_step_uses_kept_clustering(dev, orc, query_blocks):
    from block_sparse_attention_response_amd.schedule import ParkSchedule
    import torch
    (Q, K, V), (Q2, K2, V2) = _inputs()
    s = ParkSchedule(CFG.n_clusters, CFG.iters, CFG.top_p, CFG.top_k, total_steps=3, dense_fraction=0.0,
                     recompute_every=10, query_blocks=query_blocks)
    first = [to_dev(x, "bf16") for x in (Q, K, V)]
    O0, l0 = s.attention(0, *first)
    O0, l0 = host(O0), host(l0)
    st = {k: {kk: host(vv) for kk, vv in v.items()} if v is not None else None for k, v in s.state.items()}
    # unchanged inputs: the reuse step repeats the recompute step bit for bit
    O1, l1 = s.attention(1, *first)
    torch.cuda.synchronize()
    assert np.array_equal(host(O1), O0) and np.array_equal(host(l1), l0)
    # drifted inputs: attention of the new Q, K, V over the kept clusters and selection
    O2, l2 = s.attention(2, *(to_dev(x, "bf16") for x in (Q2, K2, V2)))
    torch.cuda.synchronize()
    O2, l2 = host(O2), host(l2)
    cl, qc, rb = st["cl"], st["qc"], st["rb"]
    scale = 1.0 / np.sqrt(CFG.d)
    for h in range(Q.shape[1]):
        if qc is None:
            Oo, lo = orc.block_sparse_attn(Q2[0, h], K2[0, h], V2[0, h], cl["perm"][0, h], cl["offsets"][0, h],
                                           rb["block_list"][0, h], rb["block_count"][0, h], 64, scale)
        else:
            Oo, lo = orc.block_sparse_attn_blocks(Q2[0, h], K2[0, h], V2[0, h], cl["perm"][0, h], cl["offsets"][0, h],
                                                  qc["perm"][0, h], qc["offsets"][0, h], rb["block_list"][0, h],
                                                  rb["block_count"][0, h], scale)
        fin = np.isfinite(lo)
        assert np.abs(O2[0, h][fin] - Oo[fin]).max() <= 2e-2
        assert np.abs(l2[0, h][fin] - lo[fin]).max() <= 1e-3
