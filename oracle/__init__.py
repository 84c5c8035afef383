"""CPU oracle for PARK block retrieval + block-sparse attention (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU
baseline may import this package; the GPU library and its Python binding never do.

The per-head pipeline `run_head` takes the steps in the order of PARK
(paperpeel.com/paper/2609.38978): query-response metric and key transform
(section 5.2, App. D.2), k-means on the transformed keys, key reorder, per-query
attention-mass aggregation (section 5.1), top-p selection with a top-k floor
(section 6.1; SCOPE appendix for the floor), then attention over the selected blocks
(section 3.1).  Each step is one function of oracle.c, whose comments state the reading
taken where the page is garbled or silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ALPHA = 0.05      # shrinkage weight (App. D.2, last paragraph)
EPS = 1e-6        # stability term (value not given on the page)
S_MIN = 1e-6      # floor of s_Q (value not given on the page)


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so next to it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_L = ctypes.c_long
_I = ctypes.c_int
_D = ctypes.c_double


def _declare(L):
    L.orc_query_metric.argtypes = [_P, _L, _I, _I, _D, _D, _D, _P, _P, _P]
    L.orc_query_metric.restype = _I
    L.orc_transform.argtypes = [_P, _L, _I, _P, _P]
    L.orc_init_centroids.argtypes = [_P, _L, _I, _I, _P, _P]
    L.orc_assign.argtypes = [_P, _L, _I, _P, _I, _P, _P, _P]
    L.orc_assign.restype = _D
    L.orc_update.argtypes = [_P, _L, _I, _P, _I, _P]
    L.orc_objective.argtypes = [_P, _L, _I, _P, _P]
    L.orc_objective.restype = _D
    L.orc_finalize.argtypes = [_P, _L, _I, _P, _I, _P, _P, _P, _P]
    L.orc_pama.argtypes = [_P, _L, _I, _P, _P, _I, _I, _D, _P]
    L.orc_pooled_scores.argtypes = [_P, _L, _I, _P, _P, _I, _I, _D, _P]
    L.orc_select.argtypes = [_P, _L, _I, _P, _D, _I, _P, _P, _P, _P, _P]
    L.orc_block_sparse_attn.argtypes = [_P, _P, _P, _L, _I, _P, _P, _I, _P, _P, _I, _D, _P, _L, _P, _P]
    L.orc_dense_attn.argtypes = [_P, _P, _P, _L, _I, _D, _P, _L, _P, _P]
    L.orc_pama_blocks.argtypes = [_P, _L, _I, _P, _P, _I, _P, _P, _L, _D, _P]
    L.orc_tv.argtypes = [_P, _P, _P, _L, _I, _L]
    L.orc_tv.restype = _D
    L.orc_logmass_rmse.argtypes = [_P, _P, _L, _I, _P, _P, _P, _I, _D, _P, _L]
    L.orc_logmass_rmse.restype = _D
    L.orc_block_sparse_attn_blocks.argtypes = [_P, _P, _P, _L, _I, _P, _P, _I, _P, _P, _L, _P, _P, _D, _P, _L,
                                               _P, _P]
    L.orc_exact_block_importance.argtypes = [_P, _P, _L, _I, _P, _I, _I, _D, _P]


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _i32(x):
    return np.ascontiguousarray(x, dtype=np.int32)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


# ----------------------------------------------------------------------------- steps

def query_metric(Q, metric: str = "qrkc", alpha: float = ALPHA, eps: float = EPS, s_min: float = S_MIN):
    """(G, Gs, R, ok) for one head; Q: [L, d]."""
    Q = _f32(Q)
    L_, d = Q.shape
    G = np.zeros((d, d)); Gs = np.zeros((d, d)); R = np.zeros((d, d))
    fail = lib().orc_query_metric(_p(Q), L_, d, 1 if metric == "euclidean" else 0, alpha, eps, s_min,
                                  _p(G), _p(Gs), _p(R))
    return G, Gs, R, fail == 0


def transform(K, R):
    K = _f32(K); R = _f64(R)
    out = np.empty_like(K)
    lib().orc_transform(_p(K), K.shape[0], K.shape[1], _p(R), _p(out))
    return out


def init_centroids(Kt, nk: int, init_idx=None):
    Kt = _f32(Kt)
    C = np.empty((nk, Kt.shape[1]), np.float32)
    idx = _i32(init_idx) if init_idx is not None else None
    lib().orc_init_centroids(_p(Kt), Kt.shape[0], Kt.shape[1], nk, _p(idx), _p(C))
    return C


def assign(Kt, C):
    """(labels, margin, dist, J) of one Lloyd assignment step."""
    Kt = _f32(Kt); C = _f32(C)
    L_, d = Kt.shape
    lab = np.empty(L_, np.int32); mar = np.empty(L_); dist = np.empty(L_)
    J = lib().orc_assign(_p(Kt), L_, d, _p(C), C.shape[0], _p(lab), _p(mar), _p(dist))
    return lab, mar, dist, J


def update(Kt, labels, C):
    """New centroids (copy of C updated); empty clusters keep their row of C."""
    Kt = _f32(Kt); C = _f32(C).copy(); labels = _i32(labels)
    lib().orc_update(_p(Kt), Kt.shape[0], Kt.shape[1], _p(labels), C.shape[0], _p(C))
    return C


def objective(Kt, C, labels):
    Kt = _f32(Kt); C = _f32(C); labels = _i32(labels)
    return lib().orc_objective(_p(Kt), Kt.shape[0], Kt.shape[1], _p(C), _p(labels))


def kmeans(Kt, nk: int, iters: int, init_idx=None):
    """Exactly `iters` Lloyd steps from the strided (or given) anchors.

    Returns dict(labels, centroids (transformed space), J_assign[t], J_update[t],
    margins[t] (per-key assignment margins of step t), labels_hist[t])."""
    C = init_centroids(Kt, nk, init_idx)
    hist = dict(J_assign=[], J_update=[], margins=[], labels_hist=[], C_hist=[C.copy()])
    labels = None
    for _ in range(iters):
        labels, mar, _, J = assign(Kt, C)
        C = update(Kt, labels, C)
        hist["J_assign"].append(J)
        hist["J_update"].append(objective(Kt, C, labels))
        hist["margins"].append(mar)
        hist["labels_hist"].append(labels.copy())
        hist["C_hist"].append(C.copy())
    hist["labels"] = labels
    hist["centroids"] = C
    return hist


def finalize(K, labels, nk: int):
    """(centroids [N_K, d] original space, counts, perm, offsets)."""
    K = _f32(K); labels = _i32(labels)
    L_, d = K.shape
    cent = np.empty((nk, d), np.float32); counts = np.empty(nk, np.int32)
    perm = np.empty(L_, np.int32); offsets = np.empty(nk + 1, np.int32)
    lib().orc_finalize(_p(K), L_, d, _p(labels), nk, _p(cent), _p(counts), _p(perm), _p(offsets))
    return cent, counts, perm, offsets


def pama(Q, cent, counts, q_block: int, scale: float):
    Q = _f32(Q); cent = _f32(cent); counts = _i32(counts)
    L_, d = Q.shape
    nq = (L_ + q_block - 1) // q_block
    W = np.empty((nq, cent.shape[0]))
    lib().orc_pama(_p(Q), L_, d, _p(cent), _p(counts), cent.shape[0], q_block, scale, _p(W))
    return W


def pooled_scores(Q, cent, counts, q_block: int, scale: float):
    Q = _f32(Q); cent = _f32(cent); counts = _i32(counts)
    L_, d = Q.shape
    nq = (L_ + q_block - 1) // q_block
    W = np.empty((nq, cent.shape[0]))
    lib().orc_pooled_scores(_p(Q), L_, d, _p(cent), _p(counts), cent.shape[0], q_block, scale, _p(W))
    return W


def select(W, counts, top_p: float, top_k: int):
    """(mask u8 [NQ,N_K], list int32 [NQ,N_K], count int32 [NQ], cut_margin, gap_margin)."""
    W = _f64(W); counts = _i32(counts)
    nq, nk = W.shape
    mask = np.empty((nq, nk), np.uint8); lst = np.empty((nq, nk), np.int32)
    cnt = np.empty(nq, np.int32); cm = np.empty(nq); gm = np.empty(nq)
    lib().orc_select(_p(W), nq, nk, _p(counts), top_p, top_k, _p(mask), _p(lst), _p(cnt), _p(cm), _p(gm))
    return mask, lst, cnt, cm, gm


def select_online(W, counts, top_p: float, top_k: int, sizes):
    """SCOPE's online per-head top-k (SCOPE, paperpeel.com/paper/2608.12780, section 3 "Online
    Per-Head Top-k Estimation" and the appendix "Online Per-Head Top-k Selection"), over the
    rows of one head:
      1. base counts b_u of the hybrid top-p / fixed top-k selection (`select`);
      2. the head's online minimum k_on, the query-size-weighted average of the b_u, rounded
         up to a whole count: ceil(sum_u n_u b_u / sum_u n_u), in exact integer arithmetic;
      3. each row below k_on is extended along its own ranking to k_on keys (at most the
         non-empty clusters); the other rows keep their selection.
    Returns (mask, list, count, base_count, k_on)."""
    mask, lst, cnt, _, _ = select(W, counts, top_p, top_k)
    base = cnt.copy()
    n = np.asarray(sizes, dtype=np.int64)
    tot = int(n.sum())
    k_on = -(-int((n * base.astype(np.int64)).sum()) // tot) if tot > 0 else 0
    W = _f64(W)
    for u in np.nonzero(base < k_on)[0]:
        m1, l1, c1, _, _ = select(W[u:u + 1], counts, top_p, k_on)
        mask[u], lst[u], cnt[u] = m1[0], l1[0], c1[0]
    return mask, lst, cnt, base, k_on


def block_sparse_attn(Q, K, V, perm, offsets, block_list, block_count, q_block: int, scale: float,
                      ublocks=None):
    """(O [L,d] float64, lse [L]); rows of blocks not in `ublocks` are NaN."""
    Q = _f32(Q); K = _f32(K); V = _f32(V)
    perm = _i32(perm); offsets = _i32(offsets); block_list = _i32(block_list); block_count = _i32(block_count)
    L_, d = Q.shape
    O = np.full((L_, d), np.nan); lse = np.full(L_, np.nan)
    ub = np.ascontiguousarray(ublocks, dtype=np.int64) if ublocks is not None else None
    lib().orc_block_sparse_attn(_p(Q), _p(K), _p(V), L_, d, _p(perm), _p(offsets), offsets.shape[0] - 1,
                                _p(block_list), _p(block_count), q_block, scale, _p(ub),
                                0 if ub is None else ub.shape[0], _p(O), _p(lse))
    return O, lse


def pama_blocks(Q, cent, counts, qperm, qoffsets, scale: float):
    """W [N_Q, N_K] over clustered query blocks (block u = queries qperm[qoffsets[u]:qoffsets[u+1]])."""
    Q = _f32(Q); cent = _f32(cent); counts = _i32(counts); qperm = _i32(qperm); qoffsets = _i32(qoffsets)
    L_, d = Q.shape
    nq = qoffsets.shape[0] - 1
    W = np.empty((nq, cent.shape[0]))
    lib().orc_pama_blocks(_p(Q), L_, d, _p(cent), _p(counts), cent.shape[0], _p(qperm), _p(qoffsets), nq, scale,
                          _p(W))
    return W


def block_sparse_attn_blocks(Q, K, V, perm, offsets, qperm, qoffsets, block_list, block_count, scale: float,
                             ublocks=None):
    """(O [L,d] float64, lse [L]) over clustered query blocks; rows of blocks not in `ublocks` are NaN."""
    Q = _f32(Q); K = _f32(K); V = _f32(V)
    perm = _i32(perm); offsets = _i32(offsets); qperm = _i32(qperm); qoffsets = _i32(qoffsets)
    block_list = _i32(block_list); block_count = _i32(block_count)
    L_, d = Q.shape
    O = np.full((L_, d), np.nan); lse = np.full(L_, np.nan)
    ub = np.ascontiguousarray(ublocks, dtype=np.int64) if ublocks is not None else None
    lib().orc_block_sparse_attn_blocks(_p(Q), _p(K), _p(V), L_, d, _p(perm), _p(offsets), offsets.shape[0] - 1,
                                       _p(qperm), _p(qoffsets), qoffsets.shape[0] - 1, _p(block_list),
                                       _p(block_count), scale, _p(ub), 0 if ub is None else ub.shape[0], _p(O),
                                       _p(lse))
    return O, lse


def tv(W_est, W_exact, block_sizes):
    """M1 total-variation error of an estimated map against the exact one (block-size weighted)."""
    W_est = _f64(W_est); W_exact = _f64(W_exact)
    nu = np.ascontiguousarray(block_sizes, dtype=np.int64)
    nq, nk = W_est.shape
    return lib().orc_tv(_p(W_est), _p(W_exact), _p(nu), nq, nk, int(nu.sum()))


def logmass_rmse(Q, K, labels, cent, counts, scale: float, rows=None):
    """M2 centred log-mass RMSE of the key centroids over the given query rows (all if None)."""
    Q = _f32(Q); K = _f32(K); labels = _i32(labels); cent = _f32(cent); counts = _i32(counts)
    L_, d = Q.shape
    r = np.ascontiguousarray(rows, dtype=np.int64) if rows is not None else None
    return lib().orc_logmass_rmse(_p(Q), _p(K), L_, d, _p(labels), _p(cent), _p(counts), cent.shape[0], scale,
                                  _p(r), 0 if r is None else r.shape[0])


def block_sizes(L: int, q_block: int = 64):
    """n_u of the q_block-token query blocks (the last one ragged)."""
    return np.minimum(q_block, L - q_block * np.arange((L + q_block - 1) // q_block))


def dense_attn(Q, K, V, scale: float, rows=None):
    """(O [R,d], lse [R]) for the given query rows (all rows if None)."""
    Q = _f32(Q); K = _f32(K); V = _f32(V)
    L_, d = Q.shape
    r = np.ascontiguousarray(rows, dtype=np.int64) if rows is not None else None
    nr = L_ if r is None else r.shape[0]
    O = np.empty((nr, d)); lse = np.empty(nr)
    lib().orc_dense_attn(_p(Q), _p(K), _p(V), L_, d, scale, _p(r), nr, _p(O), _p(lse))
    return O, lse


def exact_block_importance(Q, K, labels, nk: int, q_block: int, scale: float):
    Q = _f32(Q); K = _f32(K); labels = _i32(labels)
    L_, d = Q.shape
    nq = (L_ + q_block - 1) // q_block
    W = np.empty((nq, nk))
    lib().orc_exact_block_importance(_p(Q), _p(K), L_, d, _p(labels), nk, q_block, scale, _p(W))
    return W


# ------------------------------------------------------------------------- pipeline

def cluster_keys(Q, K, nk: int, iters: int, metric: str = "qrkc", alpha: float = ALPHA, init_idx=None):
    """Query-response key clustering for one head (section 5.2): returns a dict with the
    metric, the k-means history and the final outputs (centroids in the original space,
    counts, labels, perm, offsets)."""
    G, Gs, R, ok = query_metric(Q, metric, alpha)
    Kt = transform(K, R)
    km = kmeans(Kt, nk, iters, init_idx)
    cent, counts, perm, offsets = finalize(K, km["labels"], nk)
    return dict(G=G, Gs=Gs, R=R, ok=ok, Kt=Kt, km=km, labels=km["labels"], centroids=cent,
                counts=counts, perm=perm, offsets=offsets)


def cluster_queries(Q, nq: int, iters: int, init_idx=None):
    """Query blocks by plain Euclidean k-means of the queries (Figure 2; N_Q = 128 in section
    6): the key-clustering routine with R = I applied to the queries."""
    return cluster_keys(Q, Q, nq, iters, "euclidean", init_idx=init_idx)


def run_head_clustered(Q, K, V, nk: int, nq: int, iters: int, top_p: float, top_k: int, scale=None, ublocks=None):
    """Whole path for one head with clustered query blocks (PARK's own configuration)."""
    d = Q.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    qc = cluster_queries(Q, nq, iters)
    cl = cluster_keys(Q, K, nk, iters)
    W = pama_blocks(Q, cl["centroids"], cl["counts"], qc["perm"], qc["offsets"], scale)
    mask, lst, cnt, cm, gm = select(W, cl["counts"], top_p, top_k)
    O, lse = block_sparse_attn_blocks(Q, K, V, cl["perm"], cl["offsets"], qc["perm"], qc["offsets"], lst, cnt,
                                      scale, ublocks)
    return dict(qc=qc, cl=cl, W=W, mask=mask, list=lst, count=cnt, cut_margin=cm, gap_margin=gm, O=O, lse=lse)


def run_head(Q, K, V, nk: int, iters: int, top_p: float, top_k: int, q_block: int = 64, scale=None,
             metric: str = "qrkc", pooled: bool = False, ublocks=None):
    """Whole path for one head.  pooled=True is the query-centroid / Euclidean baseline."""
    d = Q.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    cl = cluster_keys(Q, K, nk, iters, "euclidean" if pooled else metric)
    f = pooled_scores if pooled else pama
    W = f(Q, cl["centroids"], cl["counts"], q_block, scale)
    mask, lst, cnt, cm, gm = select(W, cl["counts"], top_p, top_k)
    O, lse = block_sparse_attn(Q, K, V, cl["perm"], cl["offsets"], lst, cnt, q_block, scale, ublocks)
    return dict(cl=cl, W=W, mask=mask, list=lst, count=cnt, cut_margin=cm, gap_margin=gm, O=O, lse=lse)
