"""The no-allocation retrieval entry point (for callers that cannot call hipMalloc) against
park_retrieve_blocks, through the C ABI: two calls in a row, the second on a smaller input,
each equal to the workspace entry point's outputs (the same kernels: scores, masks, lists and
counts bit for bit), and the scores within the usual bar of the oracle."""
import numpy as np
import pytest

import park_synth
from park_synth import Config
from parity_util import check_scores, host, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_response_amd as park
    park.lib()
    return park


def _case(park, cfg):
    import torch
    Q, K, _ = park_synth.generate(cfg, seed=1)
    q, k = to_dev(Q, cfg.dtype), to_dev(K, cfg.dtype)
    cl = park.park_cluster_keys(q, k, cfg.n_clusters, cfg.iters)
    torch.cuda.synchronize()
    return Q, q, cl


def _same(a, b):
    import torch
    for key in ("scores", "mask", "block_list", "block_count"):
        x, y = a[key], b[key]
        if x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), key


def test_noalloc_matches_workspace_entry_point(dev, orc):
    import torch
    big = Config("noalloc-big", 1, 3, (3, 20, 40), 0, 128, "bf16", 12, (44, 42, 42), 96, 3, 0.9, 4)
    small = Config("noalloc-small", 1, 1, (1, 13, 31), 0, 64, "bf16", 5, (22, 21, 21), 20, 2, 0.8, 2)
    outs = []
    for cfg in (big, small):   # the second call reuses the same scratch for a smaller shape
        Q, q, cl = _case(dev, cfg)
        na = dev.park_retrieve_blocks_noalloc(q, cl["centroids"], cl["counts"], cfg.top_p, cfg.top_k)
        torch.cuda.synchronize()
        ref = dev.park_retrieve_blocks(q, cl["centroids"], cl["counts"], cfg.top_p, cfg.top_k)
        torch.cuda.synchronize()
        _same(na, ref)
        scale = 1.0 / np.sqrt(cfg.d)
        for h in range(cfg.H):
            W = orc.pama(Q[0, h], host(cl["centroids"][0, h]), host(cl["counts"][0, h]), 64, scale)
            check_scores(host(na["scores"][0, h]), W)
        outs.append(na)
    # the first call's outputs are untouched by the second (they live in caller memory)
    assert outs[0]["scores"].shape[1] == 3
