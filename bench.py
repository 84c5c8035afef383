#!/usr/bin/env python3
"""Benchmark of the PARK hot path on one MI355X.

One step = park_cluster_keys (query-response key clustering, 10 k-means steps) +
park_retrieve_blocks (PAMA scores + top-p / top-k selection) + park_block_sparse_attn
for one attention layer of the Wan2.1-14B-720p shape (40 heads, 75,600 tokens as a
21x45x80 latent grid, d = 128, bf16, 1024 key clusters, top-p 0.9, top-k floor 8) on
seeded synthetic Q/K/V.  Inputs are resident on the GPU before timing starts.

Prints one JSON line.  `value` is the whole-step throughput expressed as effective
sparse-attention TFLOP/s: 4 d x (selected query-key pairs) per step divided by the
whole step time (clustering + retrieval + attention).  Per-entry-point times, the
attention kernel's own TFLOP/s against the bf16 MFMA peak, recall against dense
attention and the CPU oracle's time on a bounded sample are reported beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (fp16 is the same)
PEAK_HBM_GBS = 8000.0
EXP_PER_S = 9.8e12          # v_exp_f32 throughput of the chip (256 CUs), estimated


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def effective_pairs(torch, counts, block_list, block_count, N, qcounts=None):
    """Sum over (b, h, query block u) of n_u * sum_{v selected} n_v; n_u = 64 (the last
    block ragged) or the clustered blocks' sizes qcounts [B, H, NQ]."""
    B, H, NQ, nk = block_list.shape
    valid = block_list >= 0
    idx = block_list.clamp(min=0).long()
    sizes = torch.gather(counts.long().unsqueeze(2).expand(B, H, NQ, nk), 3, idx) * valid
    keys_per_block = sizes.sum(-1)                               # [B, H, NQ]
    if qcounts is None:
        nu = torch.full((NQ,), 64, dtype=torch.long, device=counts.device)
        nu[-1] = N - 64 * (NQ - 1)
    else:
        nu = qcounts.long()
    return int((keys_per_block * nu).sum().item()), keys_per_block


def cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.strip().startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, Q, K, V, budget_heads=1):
    """The oracle on head 0 of batch 0, attention on every 16th query block (plus the last);
    per-layer time extrapolated to all heads and blocks."""
    import numpy as np
    import oracle
    oracle.lib()
    d = cfg.d
    scale = 1.0 / np.sqrt(d)
    q, k, v = Q[0, 0], K[0, 0], V[0, 0]
    t0 = time.perf_counter()
    cl = oracle.cluster_keys(q, k, cfg.n_clusters, cfg.iters)
    t1 = time.perf_counter()
    W = oracle.pama(q, cl["centroids"], cl["counts"], 64, scale)
    _, lst, cnt, _, _ = oracle.select(W, cl["counts"], cfg.top_p, cfg.top_k)
    t2 = time.perf_counter()
    NQ = cfg.n_qblocks
    ub = np.unique(np.r_[np.arange(0, NQ, 16), NQ - 1])
    oracle.block_sparse_attn(q, k, v, cl["perm"], cl["offsets"], lst, cnt, 64, scale, ub)
    t3 = time.perf_counter()
    sizes = np.diff(cl["offsets"])
    nu = np.full(NQ, 64); nu[-1] = cfg.N - 64 * (NQ - 1)
    pairs_head = float(sum(nu[u] * sizes[lst[u, :cnt[u]]].sum() for u in range(NQ)))
    heads = cfg.B * cfg.H
    layer_s = heads * ((t1 - t0) + (t2 - t1) + (t3 - t2) * NQ / len(ub))
    flops = 4.0 * d * pairs_head * heads
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {
        "value": flops / layer_s / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "cpu_model": cpu_model(), "nproc": os.cpu_count(),
        "sample": (f"batch 0 head 0 of {heads}: full clustering ({cfg.iters} k-means steps) and retrieval, "
                   f"attention on {len(ub)} of {NQ} query blocks; per-layer time extrapolated x{heads} heads "
                   f"(attention x{NQ / len(ub):.1f})"),
        "sample_s": round(t3 - t0, 2),
        "layer_s_extrapolated": round(layer_s, 1),
        "cluster_s_per_head": round(t1 - t0, 2), "retrieve_s_per_head": round(t2 - t1, 2),
        "attn_s_per_head_extrapolated": round((t3 - t2) * NQ / len(ub), 2),
    }


CSRC = os.path.join(ROOT, "block_sparse_attention_response_amd", "csrc")


def traffic_bytes(tag, source, workload):
    """HBM bytes per launch of a kernel, from the committed rocprofv3 counter summary
    profiles/<tag>_<workload>_traffic.txt (FETCH_SIZE and WRITE_SIZE scaled by a plain copy of
    known size); None when there is none or the kernel's source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{tag}_{workload}_traffic.txt")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    sha = hashlib.sha256(open(os.path.join(CSRC, source), "rb").read()).hexdigest()
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("traffic_bytes_per_launch")


def streaming_rooflines(workload, BH, N, d, nk, NQ, esz, ranges=4, attn_passes=1):
    """HBM roofline entries of the step's streaming kernels, from the committed kernel trace and
    counters (profiles/streaming_kernels_<workload>_traffic.txt): profiled, not timed in this
    run.  Algorithmic bytes are each kernel's minimum reads and writes per launch at these sizes
    (the attention call's kernels run once per pass over the heads, attn_passes launches of
    BH / attn_passes heads each); an entry whose kernel source changed since the profile was
    taken carries no measured figures."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", f"streaming_kernels_{workload}_traffic.txt")))
    except (OSError, ValueError):
        return []
    nkp = (nk + 31) // 32 * 32
    alg = {
        "park::k_km_sums<128, bf16>": ("the keys once (by perm), perm once, the means and sums (double) once "
                                       "(the first k-means step)",
                                       BH * N * d * esz + BH * N * 4 + 2 * BH * nkp * d * 8),
        "park::k_km_sums_delta<128>": ("the later k-means steps: both steps' perm and labels once (16 bytes per key), "
                                       "the carried sums read and written, the means written; the rows of the keys "
                                       "that changed cluster come on top (data-dependent, not counted)",
                                       BH * N * 16 + 3 * BH * nkp * d * 8),
        "park::k_km_ctx<128>": ("the means (double) and R, R^T once; c~ (float), the fp16 screen operand and "
                                "the per-cluster figures once", BH * nkp * d * 8 + 2 * BH * d * d * 8 + BH * nkp * (d * 6 + 20)),
        "park::k_transform_bf16<128>": ("the keys once; K~ (float) and the key norms once",
                                        BH * N * d * esz + BH * N * d * 4 + BH * N * 16),
        "park::k_gram_bf16<128>": ("the queries once", BH * N * d * esz),
        "park::k_sort_scatter": ("the labels once, perm once", 2 * BH * N * 4),
        "park::k_select<16>": ("W once; mask, list and count once", BH * NQ * nk * (4 + 1 + 4) + BH * NQ * 4),
        "park::k_pack_kv<128>": ("K, V and perm once; the packed groups once (one pass's heads)",
                                 (2 * BH * N * d * esz + BH * N * 4 + 2 * BH * (N + 8 * nk) * d * esz) / attn_passes),
        "park::k_attn_merge<128>": ("every range's (m, l) and one range's partial output per query (the ranges "
                                    "below 2^-20 of a row's weight are skipped, so the reads lie between this and "
                                    "all ranges' outputs); O and lse once (one pass's heads)",
                                    (BH * N * (ranges * 8 + d * 2) + BH * N * (d * esz + 4)) / attn_passes),
    }
    out = []
    for k in rec.get("kernels", []):
        if k["kernel"] not in alg:
            continue
        desc, nbytes = alg[k["kernel"]]
        e = {"kernel": k["kernel"].replace("park::", ""), "bound": "hbm", "algorithmic": desc,
             "dispatches_per_step": k["dispatches_per_step"],
             "over": "profiled: kernel trace average and FETCH_SIZE + WRITE_SIZE per dispatch (profiles/)"}
        sha = hashlib.sha256(open(os.path.join(ROOT, k["source"]), "rb").read()).hexdigest()
        if sha != k["source_sha256"]:
            e["stale"] = "the kernel's source changed since the profile was taken"
        else:
            sec = k["average_us"] * 1e-6
            meas = k["fetch_bytes_per_dispatch"] + k["write_bytes_per_dispatch"]
            e.update({"kernel_ms": round(k["average_us"] / 1e3, 4),
                      "hbm_algorithmic": {"bytes": int(nbytes), "GBps": round(nbytes / sec / 1e9, 1),
                                          "frac": round(nbytes / sec / 1e9 / PEAK_HBM_GBS, 4)},
                      "traffic": int(meas),
                      "hbm_measured": {"GBps": round(meas / sec / 1e9, 1), "frac": round(meas / sec / 1e9 / PEAK_HBM_GBS, 4)}})
        out.append(e)
    return out


def kernel_roofline(name, bound, flops, kernel_ms, algorithmic, alg_bytes, traffic, extra=None):
    """One kernel's roofline entry from its launch's algorithmic work and live duration."""
    sec = kernel_ms * 1e-3
    r = {"kernel": name, "bound": bound, "kernel_ms": round(kernel_ms, 3)}
    if bound == "mfma":
        ach = flops / sec / 1e12
        r.update({"achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                  "frac": round(ach / PEAK_BF16_TFLOPS, 4)})
    r["algorithmic"] = algorithmic
    gbs = alg_bytes / sec / 1e9
    r["hbm_algorithmic"] = {"bytes": int(alg_bytes), "GBps": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
    r["traffic"] = traffic
    if traffic:
        tg = traffic / sec / 1e9
        r["hbm_measured"] = {"GBps": round(tg, 1), "frac": round(tg / PEAK_HBM_GBS, 4),
                             "over": "FETCH_SIZE + WRITE_SIZE per launch (profiles/) / live duration"}
    if extra:
        r.update(extra)
    return r


def copy_calibration(gib):
    """A plain device-to-device copy of `gib` GiB (5 launches), for scaling the FETCH_SIZE /
    WRITE_SIZE counters: each launch reads and writes exactly that many bytes."""
    import torch
    n = int(gib * (1 << 30))
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t) / 5
    print(json.dumps({"copy_bytes": n, "launches": 5, "ms_per_copy": round(dt * 1e3, 3),
                      "GBps": round(2 * n / dt / 1e9, 1)}), flush=True)


def attn_clocks(args):
    """The attention kernel's per-item clock stamps (libpark_clocks.so, the build compiled with
    PARK_ATTN_CLOCKS; record layout in include/park_clocks.h) on the workload's inputs: where an
    item's time goes (prologue, tiles, epilogue, the gap to the workgroup's next item) and the
    cycles per 32-key tile.  Every call runs through the clocked build; prints one JSON line."""
    import ctypes
    import numpy as np
    import park_synth
    import torch
    import block_sparse_attention_response_amd as park
    clocked = os.path.join(os.path.dirname(park.LIB_PATH), "libpark_clocks.so")
    if not os.path.exists(clocked):
        raise SystemExit(f"{clocked} is missing: build it with __graft_entry__.build()")
    park.LIB_PATH, park._lib = clocked, None
    L = park.lib()
    cfg = park_synth.WORKLOADS[args.workload]
    log(f"clock stamps: generating {cfg.name}")
    Q, K, V = park_synth.generate(cfg, seed=0, workers=16)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x).to(dt).cuda() for x in (Q, K, V))
    del Q, K, V
    B, H, N, d = q.shape
    cl = park.park_cluster_keys(q, k, cfg.n_clusters, cfg.iters)
    rb = park.park_retrieve_blocks(q, cl["centroids"], cl["counts"], cfg.top_p, cfg.top_k, scores=False)
    passes = park.attn_passes(B, H, N, d, cfg.n_clusters)
    hpp = -(-B * H // passes)              # heads per pass
    ev = park.HipEvents(passes)
    times = []
    for _ in range(3):
        park.park_block_sparse_attn(q, k, v, cl["perm"], cl["offsets"], rb["block_list"], rb["block_count"],
                                    events=ev)
        times.append(ev.elapsed_ms())
    torch.cuda.synchronize()
    NQ = (N + 63) // 64
    items = B * H * NQ * 4
    L.park_attn_clock_words.restype = ctypes.c_size_t
    words = min(5 * items, int(L.park_attn_clock_words()))
    buf = np.zeros(words, np.uint64)
    L.park_attn_clock_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    if L.park_attn_clock_read(buf.ctypes.data, words) != 0:
        raise RuntimeError("park_attn_clock_read failed")
    c = buf.reshape(-1, 5).astype(np.int64)
    idx = np.nonzero(c[:, 0] > 0)[0]       # items with tiles (the last call's stamps)
    c = c[idx]
    wg, nt = c[:, 4] >> 32, c[:, 4] & 0xFFFFFFFF
    wg = wg + (idx // (4 * NQ) // hpp) * (1 << 20)   # the workgroups of each pass apart
    pro, til, epi = c[:, 1] - c[:, 0], c[:, 2] - c[:, 1], c[:, 3] - c[:, 2]
    o = np.lexsort((c[:, 0], wg))          # a workgroup's items in time order (one XCD's clock)
    same = wg[o][1:] == wg[o][:-1]
    gap = (c[o, 0][1:] - c[o, 3][:-1])[same]
    total = pro.sum() + til.sum() + epi.sum() + gap.sum()
    many = nt >= 8
    out = {"mode": "attn_clocks", "workload": cfg.name, "library": os.path.basename(clocked),
           "kernel_ms": round(float(np.median(times)), 3), "items": int(len(c)), "tiles": int(nt.sum()),
           "share": {"prologue": round(float(pro.sum() / total), 4), "tiles": round(float(til.sum() / total), 4),
                     "epilogue": round(float(epi.sum() / total), 4), "gap": round(float(gap.sum() / total), 4)},
           "cycles_median": {"prologue": float(np.median(pro)), "epilogue": float(np.median(epi)),
                             "gap": float(np.median(gap)) if len(gap) else None},
           "cycles_per_tile": {"median": round(float(np.median(til[many] / nt[many])), 1),
                               "mean": round(float(til[many].sum() / nt[many].sum()), 1)}}
    print(json.dumps(out), flush=True)


def clustered_leg(args, park, torch, np, cfg, q, k, v, top_p, top_k, stream, lse_dense):
    """PARK's own configuration: query blocks by Euclidean k-means of the queries (NQ blocks,
    the same k-means steps as the keys), timed like the main leg on the same inputs."""
    B, H, N, d = q.shape
    nk, nq = cfg.n_clusters, args.query_blocks
    ws_q = torch.empty(park.workspace_bytes_clustered(park.OP_CLUSTER_KEYS, B, H, N, d, nq, nq), dtype=torch.uint8,
                       device="cuda")
    ws_c = torch.empty(park.workspace_bytes(park.OP_CLUSTER_KEYS, B, H, N, d, nk), dtype=torch.uint8, device="cuda")
    ws_r = torch.empty(park.workspace_bytes_clustered(park.OP_RETRIEVE_BLOCKS, B, H, N, d, nk, nq),
                       dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(park.workspace_bytes_clustered(park.OP_BLOCK_SPARSE_ATTN, B, H, N, d, nk, nq),
                       dtype=torch.uint8, device="cuda")

    def step(ev=None):
        if ev: ev[0].record(stream)
        qc = park.park_cluster_queries(q, nq, cfg.iters, workspace=ws_q)
        if ev: ev[1].record(stream)
        cl = park.park_cluster_keys(q, k, nk, cfg.iters, workspace=ws_c)
        if ev: ev[2].record(stream)
        rb = park.park_retrieve_blocks_clustered(q, cl["centroids"], cl["counts"], qc["perm"], qc["offsets"], top_p,
                                                 top_k, workspace=ws_r)
        if ev: ev[3].record(stream)
        O, lse = park.park_block_sparse_attn_clustered(q, k, v, cl["perm"], cl["offsets"], qc["perm"], qc["offsets"],
                                                       rb["block_list"], rb["block_count"], workspace=ws_a)
        if ev: ev[4].record(stream)
        return qc, cl, rb, O, lse

    log(f"clustered query blocks ({nq}): warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        out = step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    qc, cl, rb, O, lse = out
    ms = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(4)] for i in range(args.steps)]).mean(0)
    ms_per_step = wall * 1e3 / args.steps
    pairs, _ = effective_pairs(torch, cl["counts"], rb["block_list"], rb["block_count"], N, qc["counts"])
    flops = 4.0 * d * pairs
    log(f"clustered step {ms_per_step:.2f} ms: query clusters {ms[0]:.2f} key clusters {ms[1]:.2f} "
        f"retrieve {ms[2]:.2f} attention {ms[3]:.2f}")
    res = {"query_blocks": nq, "ms_per_step": round(ms_per_step, 3),
           "effective_tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
           "query_cluster_ms_per_layer": round(float(ms[0]), 3), "cluster_ms_per_layer": round(float(ms[1]), 3),
           "retrieval_ms_per_layer": round(float(ms[2]), 3), "attn_ms_per_layer": round(float(ms[3]), 3),
           "attn_effective_tflops": round(flops / (ms[3] * 1e-3) / 1e12, 2),
           "block_density": round(float(rb["block_count"].float().mean().item()) / nk, 4),
           "pair_density": round(pairs / (B * H * float(N) * N), 4)}
    if lse_dense is not None:
        rec = torch.exp((lse - lse_dense).double()).mean(-1).flatten().cpu().numpy()
        res["recall"] = {"mean": round(float(rec.mean()), 4), "p05": round(float(np.percentile(rec, 5)), 4),
                         "worst": round(float(rec.min()), 4), "over": "heads (mean over queries)"}
    return res


def online_leg(args, park, torch, np, cfg, q, k, v, cl, top_p, top_k, stream, lse_dense, ws_r, ws_a):
    """SCOPE's online per-head top-k floor (its section 3, "Online Per-Head Top-k Estimation")
    on 64-token query blocks, timed on the main leg's key clustering: the two-pass selection
    and the attention over its larger selections, with the densities and recall beside the
    fixed-floor selection's."""
    B, H, N, d = q.shape
    nk = cfg.n_clusters

    def step(ev=None):
        if ev: ev[0].record(stream)
        rb = park.park_retrieve_blocks_online(q, cl["centroids"], cl["counts"], top_p, top_k, workspace=ws_r)
        if ev: ev[1].record(stream)
        O, lse = park.park_block_sparse_attn(q, k, v, cl["perm"], cl["offsets"], rb["block_list"], rb["block_count"],
                                             workspace=ws_a)
        if ev: ev[2].record(stream)
        return rb, O, lse

    log("online per-head top-k: warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        rb, O, lse = step(evs[i])
    torch.cuda.synchronize()
    ms = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(2)] for i in range(args.steps)]).mean(0)
    pairs, _ = effective_pairs(torch, cl["counts"], rb["block_list"], rb["block_count"], N)
    flops = 4.0 * d * pairs
    log(f"online: retrieve {ms[0]:.2f} ms, attention {ms[1]:.2f} ms")
    res = {"retrieval_ms_per_layer": round(float(ms[0]), 3), "attn_ms_per_layer": round(float(ms[1]), 3),
           "attn_effective_tflops": round(flops / (ms[1] * 1e-3) / 1e12, 2),
           "block_density": round(float(rb["block_count"].float().mean().item()) / nk, 4),
           "pair_density": round(pairs / (B * H * float(N) * N), 4)}
    if lse_dense is not None:
        rec = torch.exp((lse - lse_dense).double()).mean(-1).flatten().cpu().numpy()
        res["recall"] = {"mean": round(float(rec.mean()), 4), "p05": round(float(np.percentile(rec, 5)), 4),
                         "worst": round(float(rec.min()), 4), "over": "heads (mean over queries)"}
    return res


def sweep_leg(args, park, torch, np, cfg, q, k, v, cl, lse_dense, ws_c, ws_r, ws_a):
    """The density sweep (forced top-k with top-p = 0, the k values of the density-sweep
    workload) for PARK (QRKC clusters, PAMA scores) and for the baseline (Euclidean clusters,
    pooled-query scores), on the main leg's inputs: retrieval and attention times, densities
    and recall against dense attention for every k."""
    import park_synth
    B, H, N, d = q.shape
    nk = cfg.n_clusters
    ks = park_synth.DENSITY_SWEEP.forced_k
    ce = park.park_cluster_keys(q, k, nk, cfg.iters, metric="euclidean", workspace=ws_c)

    def timed(fn):
        out = fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return out, e0.elapsed_time(e1) / args.steps

    res = {"k": list(ks), "top_p": 0.0}
    for name, c, f in (("park", cl, park.park_retrieve_blocks),
                       ("pooled_euclidean", ce, park.park_retrieve_blocks_pooled)):
        rows = []
        for kk in ks:
            log(f"sweep {name} k={kk}")
            rb, t_r = timed(lambda: f(q, c["centroids"], c["counts"], 0.0, kk, scores=False, workspace=ws_r))
            (O, lse), t_a = timed(lambda: park.park_block_sparse_attn(q, k, v, c["perm"], c["offsets"], rb["block_list"],
                                                                     rb["block_count"], workspace=ws_a))
            pairs, _ = effective_pairs(torch, c["counts"], rb["block_list"], rb["block_count"], N)
            row = {"k": kk, "retrieval_ms": round(t_r, 3), "attn_ms": round(t_a, 3),
                   "attn_effective_tflops": round(4.0 * d * pairs / (t_a * 1e-3) / 1e12, 2),
                   "block_density": round(float(rb["block_count"].float().mean().item()) / nk, 4),
                   "pair_density": round(pairs / (B * H * float(N) * N), 4)}
            if lse_dense is not None:
                rec = torch.exp((lse - lse_dense).double()).mean(-1).flatten().cpu().numpy()
                row["recall"] = {"mean": round(float(rec.mean()), 4), "p05": round(float(np.percentile(rec, 5)), 4),
                                 "worst": round(float(rec.min()), 4)}
            rows.append(row)
            del rb, O, lse
        res[name] = rows
    return res


def unfused_ablation(args, park, torch, np, cfg, q, cl, top_p, top_k, ws_r):
    """The ablation of PARK's fused retrieval kernel (section 5.1): the same retrieval with the
    per-query probabilities P [B,H,N,N_K] float32 written to HBM and averaged by a second
    kernel, timed against the fused call on the same clustering."""
    B, H, N, d = q.shape
    nk = cfg.n_clusters
    probs = torch.empty(B, H, N, nk, dtype=torch.float32, device="cuda")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    fused = timed(lambda: park.park_retrieve_blocks(q, cl["centroids"], cl["counts"], top_p, top_k, workspace=ws_r))
    unfused = timed(lambda: park.park_retrieve_blocks_unfused(q, cl["centroids"], cl["counts"], top_p, top_k,
                                                              probs=probs, workspace=ws_r))
    nbytes = probs.numel() * 4
    del probs
    return {"fused_ms": round(fused, 3), "unfused_ms": round(unfused, 3),
            "probs_bytes": nbytes, "extra_ms": round(unfused - fused, 3),
            "extra_hbm_GBps": round(2 * nbytes / ((unfused - fused) * 1e-3) / 1e9, 1) if unfused > fused else None,
            "note": "P written once and read once: 2 x probs_bytes of extra HBM traffic"}


def diagnostics_leg(park, torch, cfg, q, k, cl, W_pama):
    """Retrieval accuracy (PARK appendix A, M1): the total-variation error, weighted by block
    size and averaged over heads, of the PAMA map and of the pooled-query map (same key
    clusters) against the exact block importance of Eq. (3), computed on the GPU."""
    B, H, N, d = q.shape
    t0 = time.perf_counter()
    Wx = park.park_block_importance_exact(q, k, cl["perm"], cl["offsets"])
    Wc = park.park_retrieve_blocks_pooled(q, cl["centroids"], cl["counts"], cfg.top_p, cfg.top_k)["scores"]
    torch.cuda.synchronize()
    secs = time.perf_counter() - t0
    nq = Wx.shape[2]
    nu = torch.clamp(N - 64 * torch.arange(nq, device=Wx.device), max=64).double()

    def tv(We):
        return float(((We.double() - Wx.double()).abs().sum(-1) * 0.5 * nu / N).sum(-1).mean().item())
    res = {"tv_pama": round(tv(W_pama), 4), "tv_pooled": round(tv(Wc), 4),
           "over": "heads (block-size weighted TV per head against the exact Eq. (3) map)",
           "exact_map_s": round(secs, 2)}
    if q.dtype == torch.bfloat16:
        # M2 (appendix B): centred log-mass RMSE of the QRKC key centroids and of Euclidean ones
        t0 = time.perf_counter()
        ce = park.park_cluster_keys(q, k, cfg.n_clusters, cfg.iters, metric="euclidean")
        r_q = park.park_logmass_rmse(q, k, cl["perm"], cl["offsets"], cl["centroids"], cl["counts"])
        r_e = park.park_logmass_rmse(q, k, ce["perm"], ce["offsets"], ce["centroids"], ce["counts"])
        torch.cuda.synchronize()
        res["logmass_rmse"] = {"qrkc": round(float(r_q.mean().item()), 4), "euclidean": round(float(r_e.mean().item()), 4),
                               "over": "heads", "s": round(time.perf_counter() - t0, 2)}
    return res


def schedule_leg(args, torch, np, cfg, q, k, v, top_p, top_k):
    """PARK's step schedule (section 6: 50 steps, dense for the first 20%, clustering and
    masks recomputed every R = 10 steps): the three kinds of step timed on the same inputs
    and combined into the mean time per layer-step over the schedule."""
    from block_sparse_attention_response_amd.schedule import ParkSchedule
    s = ParkSchedule(cfg.n_clusters, cfg.iters, top_p, top_k, query_blocks=args.query_blocks or None)
    kinds = [s.kind(t) for t in range(s.total_steps)]

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    log("schedule: dense, recompute and reuse steps")
    t = {"dense": timed(lambda: s.dense(q, k, v)),
         "recompute": timed(lambda: (s.refresh(q, k), s.sparse(q, k, v))),
         "reuse": timed(lambda: s.sparse(q, k, v))}
    mean = sum(t[x] for x in kinds) / len(kinds)
    return {"total_steps": s.total_steps, "dense_steps": kinds.count("dense"),
            "recompute_steps": kinds.count("recompute"), "reuse_steps": kinds.count("reuse"),
            "recompute_every": s.recompute_every, "query_blocks": args.query_blocks or 64,
            "dense_step_ms": round(t["dense"], 3), "recompute_step_ms": round(t["recompute"], 3),
            "reuse_step_ms": round(t["reuse"], 3), "mean_step_ms": round(mean, 3),
            "speedup_vs_dense": round(t["dense"] / mean, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan2.1-14b-720p-21x45x80",
                    help="synthetic workload by name (park_synth.WORKLOADS)")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--recall", choices=["on", "off"], default="on")
    ap.add_argument("--query-blocks", type=int, default=128, metavar="NQ",
                    help="also time the clustered-query-block path with NQ query clusters (0: skip)")
    ap.add_argument("--schedule", choices=["on", "off"], default="on",
                    help="also time the 50-step schedule (dense prefix, recompute every 10 steps)")
    ap.add_argument("--online", choices=["on", "off"], default="on",
                    help="also time SCOPE's online per-head top-k selection on 64-token blocks")
    ap.add_argument("--diagnostics", choices=["on", "off"], default="on",
                    help="also measure the retrieval TV and log-mass errors and time the unfused retrieval")
    ap.add_argument("--sweep", choices=["on", "off"], default="on",
                    help="also time the forced top-k density sweep for PARK and the pooled/Euclidean baseline")
    ap.add_argument("--leg", choices=["all", "clustered"], default="all",
                    help="clustered: time only the clustered-query-block step (for kernel traces of it)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="only run a plain device copy of this many GiB (counter calibration) and exit")
    ap.add_argument("--attn-clocks", action="store_true",
                    help="only run the attention kernel's clock-stamped build (libpark_clocks.so) and "
                         "print where its items' time goes, then exit")
    args = ap.parse_args()
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    if args.attn_clocks:
        attn_clocks(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (heads would be "
              "sharded across GPUs with no exchange inside the layer).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import park_synth
    cfg = park_synth.WORKLOADS[args.workload]
    log(f"generating {cfg.name}: B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} {cfg.dtype}")
    t = time.perf_counter()
    Q, K, V = park_synth.generate(cfg, seed=0, workers=16)
    log(f"inputs ready in {time.perf_counter() - t:.1f}s")

    import torch
    import block_sparse_attention_response_amd as park
    park.lib()
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q = torch.from_numpy(Q).to(dt).cuda()
    k = torch.from_numpy(K).to(dt).cuda()
    v = torch.from_numpy(V).to(dt).cuda()
    B, H, N, d = q.shape
    nk = cfg.n_clusters
    top_p, top_k = cfg.top_p, (cfg.top_k if not cfg.forced_k else cfg.forced_k[1])
    stream = torch.cuda.current_stream()
    if args.leg == "clustered":
        if args.query_blocks <= 0:
            print("--leg clustered needs --query-blocks > 0", file=sys.stderr)
            sys.exit(2)
        res = clustered_leg(args, park, torch, np, cfg, q, k, v, top_p, top_k, stream, None)
        print(json.dumps({"leg": "query_clustered", "workload": cfg.name, "steps": args.steps,
                          "warmup": args.warmup, **res}), flush=True)
        return
    ws_c = torch.empty(park.workspace_bytes(park.OP_CLUSTER_KEYS, B, H, N, d, nk), dtype=torch.uint8, device="cuda")
    ws_r = torch.empty(park.workspace_bytes(park.OP_RETRIEVE_BLOCKS, B, H, N, d, nk), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(park.workspace_bytes(park.OP_BLOCK_SPARSE_ATTN, B, H, N, d, nk), dtype=torch.uint8, device="cuda")

    def step(ev=None, kev=None, cev=None, rev=None):
        if ev: ev[0].record(stream)
        cl = park.park_cluster_keys(q, k, nk, cfg.iters, workspace=ws_c, events=cev.handles if cev else None)
        if ev: ev[1].record(stream)
        rb = park.park_retrieve_blocks(q, cl["centroids"], cl["counts"], top_p, top_k, workspace=ws_r,
                                       events=rev.handles if rev else None)
        if ev: ev[2].record(stream)
        O, lse = park.park_block_sparse_attn(q, k, v, cl["perm"], cl["offsets"], rb["block_list"], rb["block_count"],
                                             workspace=ws_a, events=kev)
        if ev: ev[3].record(stream)
        return cl, rb, O, lse

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    passes = park.attn_passes(B, H, N, d, nk)
    kevs = [park.HipEvents(passes) for _ in range(args.steps)]   # around the attention kernel of each pass
    cevs = [park.HipEvents() for _ in range(args.steps)]   # around the last k-means assignment kernel
    revs = [park.HipEvents() for _ in range(args.steps)]   # around the fused PAMA kernel
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        out = step(evs[i], kevs[i], cevs[i], revs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cl, rb, O, lse = out
    ms = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(3)] for i in range(args.steps)])
    cluster_ms, retrieve_ms, attn_ms = ms.mean(0)
    kernel_ms = float(np.mean([e.elapsed_ms() for e in kevs]))
    assign_ms = float(np.mean([e.elapsed_ms() for e in cevs]))
    pama_ms = float(np.mean([e.elapsed_ms() for e in revs]))
    ms_per_step = wall * 1e3 / args.steps
    log(f"step {ms_per_step:.2f} ms: cluster {cluster_ms:.2f} retrieve {retrieve_ms:.2f} attention {attn_ms:.2f}")
    log(f"kernels: attention {kernel_ms:.3f} ms, PAMA {pama_ms:.3f} ms, last k-means assignment {assign_ms:.3f} ms")

    pairs, keys_per_block = effective_pairs(torch, cl["counts"], rb["block_list"], rb["block_count"], N)
    attn_flops = 4.0 * d * pairs
    attn_tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    kernel_tflops = attn_flops / (kernel_ms * 1e-3) / 1e12
    value = attn_flops / (ms_per_step * 1e-3) / 1e12
    block_density = float(rb["block_count"].float().mean().item()) / nk
    pair_density = pairs / (B * H * float(N) * N)

    result = {
        "metric": "retrieval ms/layer + sparse-attn effective TFLOP/s (75.6k tok, 40 heads)",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded clustered Gaussian Q/K with 3D RoPE, V ~ N(0,1)); no trained weights",
        "config": {"workload": cfg.name, "batch": B, "heads": H, "tokens": N, "head_dim": d,
                   "key_clusters": nk, "kmeans_iters": cfg.iters, "top_p": top_p, "top_k_floor": top_k,
                   "query_block": 64, "parallelism": "single GPU"},
        "retrieval_ms_per_layer": round(float(retrieve_ms), 3),
        "median_ms": {"cluster": round(float(np.median(ms[:, 0])), 3), "retrieval": round(float(np.median(ms[:, 1])), 3),
                      "attention": round(float(np.median(ms[:, 2])), 3),
                      "attention_kernel": round(float(np.median([e.elapsed_ms() for e in kevs])), 3),
                      "over": "timed steps"},
        "cluster_ms_per_layer": round(float(cluster_ms), 3),
        "attn_ms_per_layer": round(float(attn_ms), 3),
        "attn_effective_tflops": round(attn_tflops, 2),
        "block_density": round(block_density, 4),
        "pair_density": round(pair_density, 4),
        "roofline": {"bound": "mfma", "kernel": "k_attn_items<128, false>", "achieved": round(kernel_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(kernel_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_bytes("k_attn_items", "k_attn.hip", cfg.name),
                     "kernel_ms": round(kernel_ms / passes, 3), "launches_per_call": passes,
                     "algorithmic": "4 d FLOP per selected (query, key) pair, %.4g TFLOP per launch (the call's "
                                    "%.4g TFLOP over its %d passes of %d heads or fewer)"
                                    % (attn_flops / passes / 1e12, attn_flops / 1e12, passes, -(-B * H // passes))},
    }
    result["workspace_bytes"] = {"cluster": int(ws_c.numel()), "retrieval": int(ws_r.numel()),
                                 "attention": int(ws_a.numel()), "attention_passes": passes}
    # the three heavy kernels of the step, each timed live (HIP events around one launch)
    BH, NQ = B * H, (N + 63) // 64
    esz = 2 if cfg.dtype == "bf16" else 4
    kv_bytes = 4.0 * d * float(keys_per_block.sum().item())      # K and V of every selected key, once per block
    pama_flops = 2.0 * BH * N * nk * d
    assign_flops = 2.0 * BH * N * nk * d
    result["kernels"] = [
        kernel_roofline("k_attn_items<128, false>", "mfma", attn_flops / passes, kernel_ms / passes,
                        "4 d FLOP per selected (query, key) pair; bytes: Q and O once, K and V once per "
                        "(query block, selected key); per launch: the call's work over its %d passes" % passes,
                        (BH * N * d * esz * 2 + kv_bytes) / passes,
                        traffic_bytes("k_attn_items", "k_attn.hip", cfg.name)),
        kernel_roofline("k_pama<128, 4, false, false>", "mfma", pama_flops, pama_ms,
                        "2 N_K d FLOP per query (the score product; the kernel runs it twice on the matrix unit, "
                        "hi and lo halves of the centroids) and N_K exponentials; bytes: Q once, the centroids once "
                        "per head, W once", BH * N * d * esz + BH * nk * d * 4 + BH * NQ * nk * 4,
                        traffic_bytes("k_pama", "k_retrieve.hip", cfg.name),
                        {"mfma_issued_frac": round(2 * pama_flops / (pama_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "exp_floor_ms": round(BH * N * nk / EXP_PER_S * 1e3, 3)}),
        kernel_roofline("k_km_assign<128, false>", "mfma", assign_flops, assign_ms,
                        "2 N_K d FLOP per key (the fp16 distance screen of one k-means step, against the fp16 peak, which equals "
                        "the bf16 one; the last step's "
                        "launch); bytes: the keys once, the screen operand once per head, the labels once",
                        BH * N * d * esz + BH * nk * d * 2 + BH * N * 4,
                        traffic_bytes("k_km_assign", "k_cluster.hip", cfg.name)),
    ]
    # the streaming kernels of the step against the HBM roofline (from the committed profiles)
    result["streaming_kernels"] = streaming_rooflines(cfg.name, BH, N, d, nk, NQ, esz, attn_passes=passes)

    if args.recall == "on":
        allb = torch.arange(nk, dtype=torch.int32, device="cuda").expand(B, H, rb["block_list"].shape[2], nk).contiguous()
        allc = torch.full_like(rb["block_count"], nk)
        _, lse_dense = park.park_block_sparse_attn(q, k, v, cl["perm"], cl["offsets"], allb, allc, workspace=ws_a)
        del allb, allc
        torch.cuda.synchronize()
        rec = torch.exp((lse - lse_dense).double()).mean(-1).flatten().cpu().numpy()
        result["recall"] = {"mean": round(float(rec.mean()), 4), "p05": round(float(np.percentile(rec, 5)), 4),
                            "worst": round(float(rec.min()), 4), "over": "heads (mean over queries)"}

    if args.sweep == "on":
        result["density_sweep"] = sweep_leg(args, park, torch, np, cfg, q, k, v, cl,
                                            lse_dense if args.recall == "on" else None, ws_c, ws_r, ws_a)

    if args.online == "on":
        result["online_topk"] = online_leg(args, park, torch, np, cfg, q, k, v, cl, top_p, top_k, stream,
                                           lse_dense if args.recall == "on" else None, ws_r, ws_a)

    if args.query_blocks > 0:
        result["query_clustered"] = clustered_leg(args, park, torch, np, cfg, q, k, v, top_p, top_k, stream,
                                                  lse_dense if args.recall == "on" else None)

    if args.schedule == "on":
        result["schedule"] = schedule_leg(args, torch, np, cfg, q, k, v, top_p, top_k)

    if args.diagnostics == "on":
        log("diagnostics: exact block importance and TV errors")
        W_pama = park.park_retrieve_blocks(q, cl["centroids"], cl["counts"], top_p, top_k, workspace=ws_r)["scores"]
        result["retrieval_tv"] = diagnostics_leg(park, torch, cfg, q, k, cl, W_pama)
        log("diagnostics: unfused retrieval ablation")
        result["pama_unfused"] = unfused_ablation(args, park, torch, np, cfg, q, cl, top_p, top_k, ws_r)

    if args.cpu_baseline == "on":
        log("CPU oracle baseline on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(cfg, Q, K, V)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
