"""PARK's schedule over the denoising steps of one attention layer (host logic; every
step of attention runs in libpark).

The page ("PARK: Accurate Block Retrieval for Sparse Attention in Video Diffusion
Transformers", section 5 on query and key clustering, and section 6, "Implementations")
reuses the clustering results and the sparse masks across diffusion steps and recomputes
them every R steps (R = 10), runs dense attention during the first 20% of the steps (of 50)
and clusters the queries into N_Q = 128 blocks.  Here:

  * step s < floor(dense_fraction * total_steps) is dense: the keys split into up to 64
    runs of consecutive keys, every run selected for every query block, which the
    block-sparse kernel computes as dense attention (with work for every key range);
  * the first sparse step and every `recompute_every`-th step after it cluster the keys
    (and, with query blocks, the queries), score and select the blocks;
  * the other sparse steps reuse the last clustering and selection with the CURRENT Q, K
    and V: keys and values are gathered through the kept key permutation, queries through
    the kept query permutation.
"""
from __future__ import annotations

from . import (park_block_sparse_attn, park_block_sparse_attn_clustered, park_cluster_keys, park_cluster_queries,
               park_retrieve_blocks, park_retrieve_blocks_clustered)


class ParkSchedule:
    def __init__(self, n_clusters: int, iters: int, top_p: float, top_k: int, total_steps: int = 50,
                 dense_fraction: float = 0.2, recompute_every: int = 10, query_blocks: int | None = None):
        if total_steps < 1 or recompute_every < 1 or not 0.0 <= dense_fraction <= 1.0:
            raise ValueError("total_steps and recompute_every must be >= 1 and dense_fraction in [0, 1]")
        self.n_clusters, self.iters, self.top_p, self.top_k = n_clusters, iters, top_p, top_k
        self.total_steps, self.recompute_every, self.query_blocks = total_steps, recompute_every, query_blocks
        self.dense_steps = int(dense_fraction * total_steps)
        self.state = None          # clustering and selection of the last recompute step

    def is_dense(self, step: int) -> bool:
        return step < self.dense_steps

    def recomputes(self, step: int) -> bool:
        return not self.is_dense(step) and (step - self.dense_steps) % self.recompute_every == 0

    def kind(self, step: int) -> str:
        return "dense" if self.is_dense(step) else "recompute" if self.recomputes(step) else "reuse"

    @staticmethod
    def dense(Q, K, V):
        """Dense attention through the block-sparse kernel: the keys as nk <= 64 runs of
        consecutive keys, all of them selected for every query block."""
        import torch
        B, H, N, d = Q.shape
        dev = Q.device
        nk = min(64, N)
        perm = torch.arange(N, dtype=torch.int32, device=dev).expand(B, H, N).contiguous()
        bounds = [(v * N) // nk for v in range(nk + 1)]
        offsets = torch.tensor(bounds, dtype=torch.int32, device=dev).expand(B, H, nk + 1).contiguous()
        NQ = (N + 63) // 64
        block_list = torch.arange(nk, dtype=torch.int32, device=dev).expand(B, H, NQ, nk).contiguous()
        block_count = torch.full((B, H, NQ), nk, dtype=torch.int32, device=dev)
        return park_block_sparse_attn(Q, K, V, perm, offsets, block_list, block_count)

    def refresh(self, Q, K):
        """Cluster and select on the current Q and K; kept for the following reuse steps."""
        cl = park_cluster_keys(Q, K, self.n_clusters, self.iters)
        if self.query_blocks:
            qc = park_cluster_queries(Q, self.query_blocks, self.iters)
            rb = park_retrieve_blocks_clustered(Q, cl["centroids"], cl["counts"], qc["perm"], qc["offsets"], self.top_p,
                                                self.top_k, scores=False)
        else:
            qc = None
            rb = park_retrieve_blocks(Q, cl["centroids"], cl["counts"], self.top_p, self.top_k, scores=False)
        self.state = dict(cl=cl, qc=qc, rb=rb)
        return self.state

    def sparse(self, Q, K, V):
        """Attention with the kept clustering and selection on the current Q, K, V."""
        s = self.state
        cl, qc, rb = s["cl"], s["qc"], s["rb"]
        if qc is None:
            return park_block_sparse_attn(Q, K, V, cl["perm"], cl["offsets"], rb["block_list"], rb["block_count"])
        return park_block_sparse_attn_clustered(Q, K, V, cl["perm"], cl["offsets"], qc["perm"], qc["offsets"],
                                                rb["block_list"], rb["block_count"])

    def attention(self, step: int, Q, K, V):
        """(O, lse) of this layer at denoising step `step` (0-based)."""
        if not 0 <= step < self.total_steps:
            raise ValueError(f"step {step} outside [0, {self.total_steps})")
        if self.is_dense(step):
            return self.dense(Q, K, V)
        if self.recomputes(step) or self.state is None:
            self.refresh(Q, K)
        return self.sparse(Q, K, V)
