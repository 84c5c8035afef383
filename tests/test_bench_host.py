"""Host-side pieces of bench.py that need no GPU: the refusal of more than one GPU and the
count of selected (query, key) pairs that the throughput is computed from."""
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
