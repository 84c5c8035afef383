"""Helpers shared by the GPU parity tests (host-side comparison logic only)."""
from __future__ import annotations

import numpy as np


def to_dev(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)   # values are already bf16-exact
    return t.to("cuda")


def host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def prefix_of_ranking(W_row: np.ndarray, counts: np.ndarray, sel: list) -> bool:
    """True if `sel` (ids) is a prefix of the ranking (W desc, id asc; empty last) of some
    length, allowing any order among exactly tied W values."""
    ne = counts > 0
    key = sorted(range(len(W_row)), key=lambda v: (not ne[v], -W_row[v], v))
    n = len(sel)
    if n == 0:
        return True
    top = set(key[:n])
    if set(sel) == top:
        return True
    # ties at the boundary: the n-th value may be shared by several ids
    wn = W_row[key[n - 1]]
    strictly = {v for v in key[:n] if W_row[v] > wn}
    tied = {v for v in range(len(W_row)) if ne[v] and W_row[v] == wn}
    s = set(sel)
    return strictly <= s and s <= strictly | tied


def compare_selection(W_gpu: np.ndarray, W_ref: np.ndarray, counts: np.ndarray, p: float, k: int, mask_g, list_g,
                      count_g, orc):
    """The GPU's selection against the oracle's selection on the oracle's own scores W_ref.

    A row may differ only where the decision lies within the score error: its cut margin
    (distance of the crossing prefix sum from p * total) below (1 + p) * sum_v |dW_v|, the
    bound on how far any top-t prefix sum and the target can move, or its gap margin (W of
    the last kept minus the first dropped cluster) below 2 max_v |dW_v|.  Such rows must
    still keep a prefix of the GPU's own ranking, with a count within one of the oracle's.
    Returns (n_rows, n_exempt)."""
    NQ, nk = W_gpu.shape
    W_ref = np.asarray(W_ref, np.float64)
    mask_o, list_o, cnt_o, cm, gm = orc.select(W_ref, counts, p, k)
    dW = np.abs(W_gpu.astype(np.float64) - W_ref)
    exempt = (cm <= (1.0 + p) * dW.sum(axis=1) + 1e-15) | (gm <= 2.0 * dW.max(axis=1) + 1e-15)
    ok = exempt | ((cnt_o == count_g) & np.all(mask_o == mask_g, axis=1) & np.all(list_o == list_g, axis=1))
    bad = np.nonzero(~ok)[0]
    assert bad.size == 0, f"selection differs on rows {bad[:10]} (count gpu {count_g[bad[:5]]} oracle {cnt_o[bad[:5]]})"
    for u in np.nonzero(exempt)[0]:
        sel = list(list_g[u, :count_g[u]])
        assert abs(int(count_g[u]) - int(cnt_o[u])) <= 1
        assert prefix_of_ranking(W_gpu[u].astype(np.float64), counts, sel)
        assert sorted(sel) == sel and np.all(list_g[u, count_g[u]:] == -1)
        assert mask_g[u].nonzero()[0].tolist() == sel
    return NQ, int(exempt.sum())


def check_scores(W_gpu: np.ndarray, W_ref: np.ndarray, rel: float = 1e-3, abs_small: float = 1e-9):
    big = W_ref >= 1e-6
    err_big = np.abs(W_gpu[big] - W_ref[big]) / W_ref[big] if big.any() else np.zeros(1)
    err_small = np.abs(W_gpu[~big] - W_ref[~big]) if (~big).any() else np.zeros(1)
    assert err_big.max() <= rel, f"max rel err {err_big.max():.3e}"
    assert err_small.max() <= abs_small, f"max abs err (W < 1e-6) {err_small.max():.3e}"
    return float(err_big.max()), float(err_small.max())
