"""Host-side pieces of bench.py that need no GPU: the refusal of more than one GPU, the count
of selected (query, key) pairs that the throughput is computed from, and the streaming
kernels' HBM entries taken from the committed profile."""
import importlib.util
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_effective_pairs_brute_force():
    """sum over (b, h, u) of n_u * sum of the selected clusters' sizes, against explicit loops,
    for 64-token blocks (ragged last block) and for given block sizes."""
    import torch
    bench = _bench()
    rng = np.random.default_rng(3)
    B, H, N, nk = 2, 3, 200, 7
    NQ = (N + 63) // 64
    counts = rng.integers(0, 40, (B, H, nk)).astype(np.int32)
    lst = np.full((B, H, NQ, nk), -1, np.int32)
    cnt = rng.integers(0, nk + 1, (B, H, NQ)).astype(np.int32)
    for b in range(B):
        for h in range(H):
            for u in range(NQ):
                lst[b, h, u, :cnt[b, h, u]] = np.sort(rng.choice(nk, cnt[b, h, u], replace=False))
    qsizes = rng.integers(0, 90, (B, H, NQ))
    for qc in (None, qsizes):
        want = 0
        for b in range(B):
            for h in range(H):
                for u in range(NQ):
                    nu = (64 if u < NQ - 1 else N - 64 * (NQ - 1)) if qc is None else int(qc[b, h, u])
                    want += nu * sum(int(counts[b, h, v]) for v in lst[b, h, u, :cnt[b, h, u]])
        got, kpb = bench.effective_pairs(torch, torch.from_numpy(counts), torch.from_numpy(lst),
                                         torch.from_numpy(cnt), N, None if qc is None else torch.from_numpy(qc))
        assert got == want
        assert kpb.shape == (B, H, NQ)


def test_streaming_rooflines_follow_the_committed_profile(tmp_path, monkeypatch):
    """The streaming kernels' HBM entries come from the committed profile record; an entry
    whose kernel source no longer matches the recorded SHA-256 carries no measured figures."""
    bench = _bench()
    wl = "wan2.1-14b-720p-21x45x80"
    rec_path = os.path.join(bench.ROOT, "profiles", f"streaming_kernels_{wl}_traffic.txt")
    if not os.path.exists(rec_path):
        import pytest
        pytest.skip("no streaming-kernel profile for this workload")
    BH, N, d, nk = 40, 75600, 128, 1024
    entries = bench.streaming_rooflines(wl, BH, N, d, nk, (N + 63) // 64, 2)
    assert entries and all(e["bound"] == "hbm" for e in entries)
    sums = next(e for e in entries if e["kernel"].startswith("k_km_sums"))
    if "stale" not in sums:
        # the sums read every key once: at least B H N d bf16 bytes
        assert sums["hbm_algorithmic"]["bytes"] >= BH * N * d * 2
        # kernel_ms is rounded to 1 us, so the rate recomputed from it agrees to that rounding
        rate = sums["traffic"] / (sums["kernel_ms"] * 1e-3) / 1e9
        assert abs(sums["hbm_measured"]["GBps"] - rate) <= rate * 0.0006 / sums["kernel_ms"] + 0.1
    # a record whose hashes do not match the sources gives stale entries only
    import json
    rec = json.load(open(rec_path))
    for k in rec["kernels"]:
        k["source_sha256"] = "0" * 64
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / f"streaming_kernels_{wl}_traffic.txt").write_text(json.dumps(rec))
    real_root = bench.ROOT
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for k in rec["kernels"]:   # the sources are read relative to ROOT as well
        src = tmp_path / k["source"]
        src.parent.mkdir(parents=True, exist_ok=True)
        src.write_bytes(open(os.path.join(real_root, k["source"]), "rb").read())
    stale = bench.streaming_rooflines(wl, BH, N, d, nk, (N + 63) // 64, 2)
    assert stale and all("stale" in e and "kernel_ms" not in e for e in stale)
