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


def teacher_forced_chain(orc, Q, K, nk, labels_by_step, metric="qrkc", steps=None, init_idx=None):
    """Stage-by-stage k-means parity for one head.  labels_by_step[t - 1] holds the GPU's
    labels after t Lloyd steps (t = 1 .. T).  The oracle rebuilds the centroids of every
    step from the GPU's labels of the step before (its own update rule: an empty cluster
    keeps its previous centroid), starting from its own anchors, and its assignment from
    them must reproduce the GPU's labels of the next step except at keys whose oracle margin
    is below 1e-5.  `steps` (default: all) are the steps whose assignment is compared; the
    centroid chain always runs through every step.  Returns (differing keys, checked keys,
    clusters empty at some step)."""
    _, _, R, _ = orc.query_metric(Q, metric=metric)
    Kt = orc.transform(K, R)
    C = orc.init_centroids(Kt, nk, init_idx)
    T = len(labels_by_step)
    steps = range(1, T + 1) if steps is None else steps
    n_diff = n_keys = n_empty = 0
    for t in range(1, T + 1):
        if t >= 2:
            prev = labels_by_step[t - 2]
            n_empty += int((np.bincount(prev, minlength=nk) == 0).sum())
            C = orc.update(Kt, prev, C)
        if t in steps:
            lab_o, mar, _, _ = orc.assign(Kt, C)
            diff = lab_o != labels_by_step[t - 1]
            assert np.all(mar[diff] < MARGIN), f"step {t}: {int(diff.sum())} labels differ, " \
                f"max margin {mar[diff].max() if diff.any() else 0:.3e}"
            n_diff += int(diff.sum())
            n_keys += lab_o.size
    return n_diff, n_keys, n_empty


MARGIN = 1e-5   # "bit-exact except where the score margin is below 1e-5"


def near_prefix(W_row: np.ndarray, counts: np.ndarray, sel, tol: float = MARGIN) -> bool:
    """True if `sel` is a prefix of the ranking of W_row (W descending, empty clusters last)
    up to near-ties: no non-empty cluster left out has W more than `tol` above a kept one."""
    sel = np.asarray(sel, np.int64)
    ne = counts > 0
    if sel.size == 0:
        return True
    if not np.all(ne[sel]):
        return False
    out = np.ones(len(W_row), bool)
    out[sel] = False
    out &= ne
    if not out.any():
        return True
    return float(W_row[out].max()) <= float(W_row[sel].min()) + tol


def compare_selection(W_gpu: np.ndarray, W_ref: np.ndarray, counts: np.ndarray, p: float, k: int, mask_g, list_g,
                      count_g, orc):
    """The GPU's selection against the oracle's selection on the oracle's own scores W_ref,
    bit-exact except in rows whose decision the oracle finds within 1e-5 (reading R20):
      cut margin: |prefix sum at the top-p crossing - p * row total| < 1e-5 (either side of
                  the crossing), or
      gap margin: W of the last kept minus W of the first dropped cluster < 1e-5.
    An exempt row must still keep ids in ascending order with -1 after them, a mask equal to
    the list, a count within one of the oracle's, and a prefix of the ORACLE's ranking up to
    near-ties (no dropped cluster more than 1e-5 above a kept one).  Every row that differs
    from the oracle must be exempt.  Returns (n_rows, n_exempt, n_differ)."""
    NQ, nk = W_gpu.shape
    W_ref = np.asarray(W_ref, np.float64)
    mask_o, list_o, cnt_o, cm, gm = orc.select(W_ref, counts, p, k)
    exempt = (cm < MARGIN) | (gm < MARGIN)
    same = (cnt_o == count_g) & np.all(mask_o == mask_g, axis=1) & np.all(list_o == list_g, axis=1)
    bad = np.nonzero(~(same | exempt))[0]
    assert bad.size == 0, f"selection differs on rows {bad[:10]} (count gpu {count_g[bad[:5]]} oracle {cnt_o[bad[:5]]})"
    for u in np.nonzero(exempt & ~same)[0]:
        sel = list(list_g[u, :count_g[u]])
        assert abs(int(count_g[u]) - int(cnt_o[u])) <= 1, f"row {u}: count {count_g[u]} vs oracle {cnt_o[u]}"
        assert near_prefix(W_ref[u], counts, sel), f"row {u}: not a prefix of the oracle's ranking"
        assert sorted(sel) == sel and np.all(list_g[u, count_g[u]:] == -1)
        assert mask_g[u].nonzero()[0].tolist() == sel
    n_differ = int((~same).sum())
    assert n_differ <= int(exempt.sum())
    return NQ, int(exempt.sum()), n_differ


def check_scores(W_gpu: np.ndarray, W_ref: np.ndarray, rel: float = 1e-3, abs_small: float = 1e-9):
    big = W_ref >= 1e-6
    err_big = np.abs(W_gpu[big] - W_ref[big]) / W_ref[big] if big.any() else np.zeros(1)
    err_small = np.abs(W_gpu[~big] - W_ref[~big]) if (~big).any() else np.zeros(1)
    assert err_big.max() <= rel, f"max rel err {err_big.max():.3e}"
    assert err_small.max() <= abs_small, f"max abs err (W < 1e-6) {err_small.max():.3e}"
    return float(err_big.max()), float(err_small.max())
