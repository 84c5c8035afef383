"""The premise of the carried k-means member sums, checked on the CPU.

With bf16 keys the library keeps each cluster's member sum in double from one Lloyd step to
the next, adding the rows of the keys that joined the cluster and subtracting those that left
it, instead of summing the members afresh.  That gives the fresh sum bit for bit when every
partial sum is exact in double: bf16 values carry 8 significant bits, so any sum of them is a
multiple of the smallest term's last place, and it is exact while it stays below 2^53 such
units.  Here: sums of bf16-rounded keys of the synthetic workloads, fresh in member order
against carried through several relabellings in arbitrary order, are bitwise equal; and the
condition (every non-zero key value at least 2^-24 in magnitude, with |sum| < 2^22 for the
largest clusters) holds for the generator's keys.
"""
import numpy as np

import park_synth


def _bf16(x):
    return park_synth.round_bf16(np.asarray(x, np.float32)).astype(np.float64)


def _fresh(K, labels, nk):
    S = np.zeros((nk, K.shape[1]))
    for v in range(nk):
        for row in K[labels == v]:      # member order
            S[v] += row
    return S


def test_carried_sums_equal_fresh_sums():
    rng = np.random.default_rng(5)
    cfg = park_synth.Config("carry", 1, 1, (2, 12, 16), 0, 64, "bf16", 8, (22, 21, 21), 24, 3, 0.9, 2)
    _, K, _ = park_synth.generate(cfg, seed=1)
    K = _bf16(K[0, 0])
    N, nk = K.shape[0], 24
    lab = rng.integers(0, nk, N)
    S = _fresh(K, lab, nk)
    for step in range(6):
        new = lab.copy()
        move = rng.random(N) < [0.3, 0.2, 0.1, 0.05, 0.02, 0.01][step]
        new[move] = rng.integers(0, nk, int(move.sum()))
        changed = np.nonzero(new != lab)[0]
        for j in rng.permutation(changed):   # any order
            S[new[j]] += K[j]
            S[lab[j]] -= K[j]
        lab = new
        F = _fresh(K, lab, nk)
        assert np.array_equal(S, F), f"step {step}: carried sums differ from fresh ones"
        counts = np.bincount(lab, minlength=nk)
        live = counts > 0
        assert np.array_equal((S[live] / counts[live, None]).astype(np.float32),
                              (F[live] / counts[live, None]).astype(np.float32))


def test_tiny_terms_break_exactness_only_below_the_bound():
    # the condition matters: a term far below the others' last place is rounded away
    big = _bf16([3.0])[0]
    tiny = 2.0 ** -60
    assert (big + tiny) - big == 0.0                    # not exact
    a = _bf16([2.0 ** -24, 1.5, -7.0, 2.0 ** 20])
    assert np.sum(a) == a[3] + a[2] + a[1] + a[0] == a[0] + a[1] + a[2] + a[3]


def test_synthetic_keys_meet_the_exactness_condition():
    cfg = park_synth.WORKLOADS["wan1.3b-480p-21x30x52"]
    _, K, _ = park_synth.generate(cfg, seed=0, heads=[0])
    K = _bf16(K[0, 0])
    nz = np.abs(K[K != 0])
    frac_tiny = float(np.mean(nz < 2.0 ** -24))
    # every cluster sum stays below 2^22 in magnitude: at most N rows of the largest |value|
    assert K.shape[0] * np.abs(K).max() < 2.0 ** 22
    assert frac_tiny < 1e-6, frac_tiny
