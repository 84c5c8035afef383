"""Seeded synthetic Q/K/V shaped like one attention layer of a video DiT.

This module holds only input preparation: Gaussian class centres, per-token noise,
3D rotary position embedding and bf16 rounding. None of the retrieval or attention
arithmetic lives here; it is shared by the GPU tests, the CPU oracle tests and the
benchmark so that both sides see identical inputs.

Why the inputs look like this (PARK, paperpeel.com/paper/2609.38978):
  * section 6.1 names the workloads: Wan2.1 at 720p with 21 latent frames and
    HunyuanVideo, 3,600 tokens per frame; the trained activations are not available,
    so clustered Gaussian tokens stand in for them;
  * SCOPE (paperpeel.com/paper/2608.12780), section 1, notes that 3D RoPE acts on
    disjoint temporal / height / width channel ranges; the rotary step below applies a
    separate 1D rotary embedding to each of the three channel segments.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = ["Config", "WORKLOADS", "TINY", "WAN13B_480P", "WAN14B_720P", "HUNYUAN_720P", "DENSITY_SWEEP", "generate",
           "round_bf16", "rope_3d"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    grid: tuple          # (T, Hh, Ww) latent grid of video tokens
    n_text: int          # text tokens appended after the video tokens (no RoPE)
    d: int
    dtype: str           # "f32" or "bf16"
    n_centres: int
    split: tuple         # RoPE channel split t:h:w (channels)
    n_clusters: int
    iters: int
    top_p: float
    top_k: int
    q_block: int = 64
    forced_k: tuple = ()  # density sweep: forced top-k values (top_p = 0)

    @property
    def N(self) -> int:
        t, h, w = self.grid
        return t * h * w + self.n_text

    @property
    def n_qblocks(self) -> int:
        return (self.N + self.q_block - 1) // self.q_block


TINY = Config("tiny-fp32-2x32x32", 1, 1, (2, 32, 32), 0, 64, "f32", 16, (22, 21, 21), 32, 5, 0.9, 2)
WAN13B_480P = Config("wan1.3b-480p-21x30x52", 1, 12, (21, 30, 52), 0, 128, "bf16", 64, (44, 42, 42), 512, 10, 0.9, 8)
WAN14B_720P = Config("wan2.1-14b-720p-21x45x80", 1, 40, (21, 45, 80), 0, 128, "bf16", 128, (44, 42, 42), 1024, 10,
                     0.9, 8)
HUNYUAN_720P = Config("hunyuan-720p-33x45x80+256text", 1, 24, (33, 45, 80), 256, 128, "bf16", 128, (16, 56, 56), 1536,
                      10, 0.9, 8)
DENSITY_SWEEP = Config("density-sweep-wan2.1-14b-720p", 1, 40, (21, 45, 80), 0, 128, "bf16", 128, (44, 42, 42), 1024,
                       10, 0.0, 0, forced_k=(51, 102, 205, 410, 1024))
# every workload by its name
WORKLOADS = {c.name: c for c in (TINY, WAN13B_480P, WAN14B_720P, HUNYUAN_720P, DENSITY_SWEEP)}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _rope_tables(grid: tuple, split: tuple, theta: float):
    T, Hh, Ww = grid
    n = T * Hh * Ww
    idx = np.arange(n)
    pos = (idx // (Hh * Ww), (idx // Ww) % Hh, idx % Ww)
    tabs = []
    c0 = 0
    for seg, p in zip(split, pos):
        half = seg // 2
        if half:
            k = np.arange(half)
            ang = p[:, None].astype(np.float64) * theta ** (-2.0 * k.astype(np.float64) / seg)[None, :]
            tabs.append((c0 + 2 * k, np.cos(ang), np.sin(ang)))
        c0 += seg
    return tabs


def rope_3d(x: np.ndarray, grid: tuple, split: tuple, theta: float = 10000.0, tables=None) -> np.ndarray:
    """Rotate channel pairs of each of the t / h / w segments by the token's coordinate.

    x: [n_video, d], tokens in t-major raster order over ``grid``.  Within a segment of
    n_a channels, the pair (2k, 2k+1), k < n_a // 2, turns by pos_a * theta**(-2k / n_a);
    an odd leftover channel stays as it is.
    """
    T, Hh, Ww = grid
    assert x.shape[0] == T * Hh * Ww and sum(split) == x.shape[1]
    if tables is None:
        tables = _rope_tables(grid, split, theta)
    x = x.astype(np.float64)
    out = x.copy()
    for ch, cs, sn in tables:
        a = x[:, ch]
        b = x[:, ch + 1]
        out[:, ch] = a * cs - b * sn
        out[:, ch + 1] = a * sn + b * cs
    return out


def head_rng(seed: int, b: int, h: int) -> np.random.Generator:
    """Independent PCG64 stream for (batch b, head h) of a given seed."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(b, h))))


def _one_head(cfg: Config, seed: int, b: int, h: int, tabs):
    T, Hh, Ww = cfg.grid
    nv = T * Hh * Ww
    N, d, M = cfg.N, cfg.d, cfg.n_centres
    rng = head_rng(seed, b, h)
    mu = 2.0 * rng.standard_normal((M, d), dtype=np.float32)
    z = rng.integers(0, M, size=nv)
    q = mu[z] + 0.5 * rng.standard_normal((nv, d), dtype=np.float32)
    k = mu[z] + 0.5 * rng.standard_normal((nv, d), dtype=np.float32)
    v = rng.standard_normal((N, d), dtype=np.float32)
    Q = np.empty((N, d), np.float32)
    K = np.empty((N, d), np.float32)
    Q[:nv] = rope_3d(q, cfg.grid, cfg.split, tables=tabs)
    K[:nv] = rope_3d(k, cfg.grid, cfg.split, tables=tabs)
    if cfg.n_text:
        Q[nv:] = rng.standard_normal((cfg.n_text, d), dtype=np.float32)
        K[nv:] = rng.standard_normal((cfg.n_text, d), dtype=np.float32)
    if cfg.dtype == "bf16":
        Q, K, v = round_bf16(Q), round_bf16(K), round_bf16(v)
    return Q, K, v


def generate(cfg: Config, seed: int = 0, heads=None, workers: int = 0):
    """Q, K, V as float32 arrays [B, H', N, d] (bf16-exact values for bf16 configs).

    Each (batch b, head h) draws from its own PCG64 stream ``head_rng(seed, b, h)``:
      centres mu [M, d] ~ N(0, 2^2); class z_n ~ U{0..M-1} shared by q_n and k_n;
      q_n = mu_z + N(0, 0.5^2); k_n = mu_z + N(0, 0.5^2); V ~ N(0, 1) for all N tokens;
      then (only with text tokens) Q and K of the text tokens ~ N(0, 1).
    Normal draws are float32.  3D RoPE is applied to the video part of Q and K, then
    everything is rounded to bf16 for bf16 configs.  ``heads`` (head indices) restricts
    the output to those heads (H' = len(heads)); each head's values do not depend on
    which other heads are generated.  ``workers`` > 1 generates heads on that many threads.
    """
    keep = list(range(cfg.H)) if heads is None else sorted(set(int(h) for h in heads))
    tabs = _rope_tables(cfg.grid, cfg.split, 10000.0)
    N, d = cfg.N, cfg.d
    Q = np.empty((cfg.B, len(keep), N, d), np.float32)
    K = np.empty_like(Q)
    V = np.empty_like(Q)
    jobs = [(b, hi, h) for b in range(cfg.B) for hi, h in enumerate(keep)]

    def run(job):
        b, hi, h = job
        Q[b, hi], K[b, hi], V[b, hi] = _one_head(cfg, seed, b, h, tabs)

    if workers and workers > 1 and len(jobs) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(min(workers, len(jobs))) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)
    return Q, K, V
