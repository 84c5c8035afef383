"""Python binding of libpark (ctypes): argument marshalling only.

Every step of the path runs in the HIP kernels of libpark.so; PyTorch supplies device
memory and the current stream.  The functions carry the names of the C entry points
declared in include/park.h:

  park_cluster_keys        query-response key clustering (PARK, section 5.2)
  park_retrieve_blocks     PAMA block scores + top-p / top-k selection (section 5.1, 6.1)
  park_retrieve_blocks_pooled  the pooled-query baseline (section 4.1)
  park_retrieve_blocks_unfused the same retrieval with P materialised in HBM (the ablation of
                               the fused kernel, section 5.1)
  park_block_sparse_attn   attention over the selected blocks (section 3.1)

and, for query blocks formed by Euclidean k-means of the queries (PARK's own setting,
Figure 2 and section 6):

  park_cluster_queries             the query blocks
  park_retrieve_blocks_clustered   PAMA + selection over them
  park_block_sparse_attn_clustered attention over them

and SCOPE's online per-head top-k floor over either kind of query block:

  park_retrieve_blocks_online      PAMA + the two-pass selection

There is no fallback: if libpark.so is missing or was built for another GPU the calls
raise.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "ParkError", "lib", "workspace_bytes", "park_abi_version", "park_cluster_keys",
    "park_retrieve_blocks", "park_retrieve_blocks_pooled", "park_retrieve_blocks_unfused", "park_block_sparse_attn", "HipEvents", "attn_passes",
    "workspace_bytes_clustered", "park_cluster_queries", "park_retrieve_blocks_clustered",
    "park_block_sparse_attn_clustered", "park_retrieve_blocks_online", "park_block_importance_exact", "OP_BLOCK_IMPORTANCE", "park_logmass_rmse",
    "PARK_OK", "PARK_ERR_INVALID", "PARK_ERR_UNSUPPORTED", "PARK_ERR_WORKSPACE", "PARK_ERR_HIP",
    "PARK_ERR_NUMERIC", "numeric_status", "park_retrieve_blocks_noalloc", "OP_CLUSTER_KEYS", "OP_RETRIEVE_BLOCKS", "OP_BLOCK_SPARSE_ATTN",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpark.so")

PARK_OK, PARK_ERR_INVALID, PARK_ERR_UNSUPPORTED, PARK_ERR_WORKSPACE, PARK_ERR_HIP, PARK_ERR_NUMERIC = range(6)
OP_CLUSTER_KEYS, OP_RETRIEVE_BLOCKS, OP_BLOCK_SPARSE_ATTN, OP_BLOCK_IMPORTANCE = range(4)
_METRIC = {"qrkc": 0, "euclidean": 1}


class ParkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} returned {_lib_status_string(status)} ({status})")


_lib = None
_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


def lib():
    """The loaded libpark.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_response_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.park_abi_version.restype = _I
        L.park_status_string.argtypes = [_I]
        L.park_status_string.restype = ctypes.c_char_p
        L.park_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I]
        L.park_workspace_bytes.restype = _S
        L.park_cluster_keys.argtypes = [_P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _P,
                                        _P, _S, _P]
        L.park_cluster_keys.restype = _I
        L.park_cluster_keys_timed.argtypes = L.park_cluster_keys.argtypes + [_P, _P]
        L.park_cluster_keys_timed.restype = _I
        L.park_retrieve_blocks_timed.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P, _I, _I, _F, _I, _F, _P, _P, _P, _P,
                                                 _P, _S, _P, _P, _P]
        L.park_retrieve_blocks_timed.restype = _I
        for name in ("park_retrieve_blocks", "park_retrieve_blocks_pooled"):
            f = getattr(L, name)
            f.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P, _I, _I, _F, _I, _F, _P, _P, _P, _P, _P, _S, _P]
            f.restype = _I
        L.park_retrieve_blocks_unfused.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P, _I, _I, _F, _I, _F, _P, _P, _P,
                                                   _P, _P, _P, _S, _P]
        L.park_retrieve_blocks_unfused.restype = _I
        L.park_block_sparse_attn.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _I, _F, _P, _P,
                                             _P, _S, _P]
        L.park_block_sparse_attn.restype = _I
        L.park_block_sparse_attn_timed.argtypes = L.park_block_sparse_attn.argtypes + [_P, _P, _I]
        L.park_block_sparse_attn_timed.restype = _I
        L.park_attn_passes.argtypes = [_I, _I, _I, _I, _I, _I]
        L.park_attn_passes.restype = _I
        L.park_workspace_bytes_clustered.argtypes = [_I, _I, _I, _I, _I, _I, _I]
        L.park_workspace_bytes_clustered.restype = _S
        L.park_cluster_queries.argtypes = [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _S, _P]
        L.park_cluster_queries.restype = _I
        L.park_retrieve_blocks_clustered.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _I, _F, _I, _F,
                                                     _P, _P, _P, _P, _P, _S, _P]
        L.park_retrieve_blocks_clustered.restype = _I
        L.park_retrieve_blocks_online.argtypes = L.park_retrieve_blocks_clustered.argtypes
        L.park_retrieve_blocks_online.restype = _I
        L.park_block_sparse_attn_clustered.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _I, _P,
                                                       _P, _F, _P, _P, _P, _S, _P]
        L.park_block_sparse_attn_clustered.restype = _I
        L.park_block_importance_exact.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _F, _P, _P, _S, _P]
        L.park_block_importance_exact.restype = _I
        L.park_logmass_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
        L.park_logmass_workspace_bytes.restype = _S
        L.park_logmass_rmse.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _F, _P, _P, _S, _P]
        L.park_logmass_rmse.restype = _I
        L.park_noalloc_scratch_bytes.argtypes = [_I, _I, _I, _I, _I]
        L.park_noalloc_scratch_bytes.restype = _S
        L.park_retrieve_blocks_noalloc.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P, _I, _I, _F, _I, _F, _P, _P, _P,
                                                   _P, _P]
        L.park_retrieve_blocks_noalloc.restype = _I
        _lib = L
    return _lib


def _lib_status_string(status: int) -> str:
    try:
        return lib().park_status_string(status).decode()
    except Exception:  # pragma: no cover - only while the library is unusable
        return f"status {status}"


def park_abi_version() -> int:
    return lib().park_abi_version()


def workspace_bytes(op: int, B: int, H: int, N: int, d: int, n_clusters: int) -> int:
    return int(lib().park_workspace_bytes(op, B, H, N, d, n_clusters))


def workspace_bytes_clustered(op: int, B: int, H: int, N: int, d: int, n_clusters: int, n_qblocks: int) -> int:
    return int(lib().park_workspace_bytes_clustered(op, B, H, N, d, n_clusters, n_qblocks))


# ----------------------------------------------------------------------------- helpers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return 1
    if t.dtype == torch.float32:
        return 0
    raise ValueError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _workspace(nbytes: int, device, given=None):
    torch = _torch()
    if nbytes == 0:
        return None, 0
    if given is not None:
        return given, given.numel() * given.element_size()
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + nbytes], nbytes


def _bhnd(x, name):
    if x.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d]")
    return x.shape


def _check(st: int, where: str):
    if st != PARK_OK:
        raise ParkError(st, where)


# ------------------------------------------------------------------------- entry points

def park_cluster_keys(Q, K, n_clusters: int, iters: int, metric: str = "qrkc", alpha: float = 0.05,
                      init_idx=None, workspace=None, events=None):
    """Cluster the keys of every (b, h).  Returns a dict of GPU tensors:
    centroids [B,H,nk,d] float32, counts [B,H,nk], labels [B,H,N], perm [B,H,N],
    offsets [B,H,nk+1], status [B,H] (int32).  `events` = (begin, end) raw hipEvent_t
    handles selects park_cluster_keys_timed (events around the last step's assignment kernel)."""
    torch = _torch()
    _dev(Q, "Q"); _dev(K, "K")
    B, H, N, d = _bhnd(Q, "Q")
    if K.shape != Q.shape or K.dtype != Q.dtype:
        raise ValueError("K must match Q in shape and dtype")
    dev = Q.device
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(centroids=torch.empty(B, H, n_clusters, d, dtype=torch.float32, device=dev),
               counts=torch.empty(B, H, n_clusters, **i32), labels=torch.empty(B, H, N, **i32),
               perm=torch.empty(B, H, N, **i32), offsets=torch.empty(B, H, n_clusters + 1, **i32),
               status=torch.empty(B, H, **i32))
    if init_idx is not None:
        _dev(init_idx, "init_idx")
        if init_idx.dtype != torch.int32 or init_idx.numel() != n_clusters:
            raise ValueError("init_idx must be int32 [n_clusters]")
    ws, wsb = _workspace(workspace_bytes(OP_CLUSTER_KEYS, B, H, N, d, n_clusters), dev, workspace)
    args = (_ptr(Q), _ptr(K), _dtype_code(Q), B, H, N, d, n_clusters, iters, _METRIC[metric], alpha, _ptr(init_idx),
            _ptr(out["centroids"]), _ptr(out["counts"]), _ptr(out["labels"]), _ptr(out["perm"]), _ptr(out["offsets"]),
            _ptr(out["status"]), _ptr(ws), wsb, _stream(Q))
    if events is None:
        _check(lib().park_cluster_keys(*args), "park_cluster_keys")
    else:
        _check(lib().park_cluster_keys_timed(*args, events[0], events[1]), "park_cluster_keys_timed")
    return out


def numeric_status(status) -> int:
    """PARK_ERR_NUMERIC if any head of a park_cluster_keys `status` tensor is flagged (its
    query metric could not be factored and the head was clustered with R = I), else PARK_OK.
    Reads the tensor on the host, so it waits for the clustering to finish."""
    return PARK_ERR_NUMERIC if bool((status != 0).any().item()) else PARK_OK


def _retrieve(fn, where, Q, centroids, counts, top_p, top_k, scale, scores, workspace, probs=None, events=None):
    torch = _torch()
    _dev(Q, "Q"); _dev(centroids, "centroids"); _dev(counts, "counts")
    B, H, N, d = _bhnd(Q, "Q")
    nk = centroids.shape[2]
    if centroids.shape != (B, H, nk, d) or centroids.dtype != torch.float32:
        raise ValueError("centroids must be float32 [B, H, n_clusters, d]")
    if counts.shape != (B, H, nk) or counts.dtype != torch.int32:
        raise ValueError("counts must be int32 [B, H, n_clusters]")
    NQ = (N + 63) // 64
    dev = Q.device
    out = dict(mask=torch.empty(B, H, NQ, nk, dtype=torch.uint8, device=dev),
               block_list=torch.empty(B, H, NQ, nk, dtype=torch.int32, device=dev),
               block_count=torch.empty(B, H, NQ, dtype=torch.int32, device=dev))
    if scores:
        out["scores"] = torch.empty(B, H, NQ, nk, dtype=torch.float32, device=dev)
    need = workspace_bytes(OP_RETRIEVE_BLOCKS, B, H, N, d, nk)
    ws, wsb = _workspace(need, dev, workspace)
    sc = -1.0 if scale is None else float(scale)
    extra = ()
    if probs is not None:
        if probs is True:
            probs = torch.empty(B, H, N, nk, dtype=torch.float32, device=dev)
        elif probs.shape != (B, H, N, nk) or probs.dtype != torch.float32 or not probs.is_contiguous():
            raise ValueError("probs must be contiguous float32 [B, H, N, n_clusters]")
        out["probs"] = probs
        extra = (_ptr(probs),)
    st = fn(_ptr(Q), _dtype_code(Q), B, H, N, d, _ptr(centroids), _ptr(counts), nk, 64, float(top_p),
            int(top_k), sc, *extra, _ptr(out.get("scores")), _ptr(out["mask"]), _ptr(out["block_list"]),
            _ptr(out["block_count"]), _ptr(ws), wsb, _stream(Q), *(events or ()))
    _check(st, where)
    return out


def park_retrieve_blocks_noalloc(Q, centroids, counts, top_p: float, top_k: int, scale=None, out=None):
    """park_retrieve_blocks through the entry point that allocates nothing (its scratch is the
    library's static per-GPU array).  `out` may hold preallocated outputs (scores, mask,
    block_list, block_count); missing ones are allocated here, by the caller's side, before
    the call.  Calls on one GPU share the scratch: overlapping calls race."""
    torch = _torch()
    _dev(Q, "Q"); _dev(centroids, "centroids"); _dev(counts, "counts")
    B, H, N, d = _bhnd(Q, "Q")
    nk = centroids.shape[2]
    if centroids.shape != (B, H, nk, d) or centroids.dtype != torch.float32:
        raise ValueError("centroids must be float32 [B, H, n_clusters, d]")
    if counts.shape != (B, H, nk) or counts.dtype != torch.int32:
        raise ValueError("counts must be int32 [B, H, n_clusters]")
    NQ = (N + 63) // 64
    dev = Q.device
    want = dict(scores=((B, H, NQ, nk), torch.float32), mask=((B, H, NQ, nk), torch.uint8),
                block_list=((B, H, NQ, nk), torch.int32), block_count=((B, H, NQ), torch.int32))
    out = dict(out or {})
    for k, (shape, dt) in want.items():
        if k not in out:
            out[k] = torch.empty(shape, dtype=dt, device=dev)
        elif tuple(out[k].shape) != shape or out[k].dtype != dt or not out[k].is_contiguous():
            raise ValueError(f"out[{k!r}] must be contiguous {dt} {list(shape)}")
    sc = -1.0 if scale is None else float(scale)
    st = lib().park_retrieve_blocks_noalloc(_ptr(Q), _dtype_code(Q), B, H, N, d, _ptr(centroids), _ptr(counts), nk, 64,
                                            float(top_p), int(top_k), sc, _ptr(out["scores"]), _ptr(out["mask"]),
                                            _ptr(out["block_list"]), _ptr(out["block_count"]), _stream(Q))
    _check(st, "park_retrieve_blocks_noalloc")
    return out


def park_retrieve_blocks(Q, centroids, counts, top_p: float, top_k: int, scale=None, scores: bool = True,
                         workspace=None, events=None):
    """PAMA scores and top-p / top-k selection.  Returns dict(scores?, mask, block_list,
    block_count).  `events` = (begin, end) raw hipEvent_t handles selects
    park_retrieve_blocks_timed (events around the fused PAMA kernel)."""
    if events is not None:
        return _retrieve(lib().park_retrieve_blocks_timed, "park_retrieve_blocks_timed", Q, centroids, counts, top_p,
                         top_k, scale, scores, workspace, events=events)
    return _retrieve(lib().park_retrieve_blocks, "park_retrieve_blocks", Q, centroids, counts, top_p, top_k,
                     scale, scores, workspace)


def park_retrieve_blocks_unfused(Q, centroids, counts, top_p: float, top_k: int, scale=None, scores: bool = True,
                                 probs=None, workspace=None):
    """park_retrieve_blocks without the fusion: the probabilities P [B,H,N,n_clusters] float32
    go to HBM (`probs`, allocated when None) and a second kernel averages them into W.
    Returns dict(probs, scores?, mask, block_list, block_count)."""
    return _retrieve(lib().park_retrieve_blocks_unfused, "park_retrieve_blocks_unfused", Q, centroids, counts,
                     top_p, top_k, scale, scores, workspace, probs=True if probs is None else probs)


def park_retrieve_blocks_pooled(Q, centroids, counts, top_p: float, top_k: int, scale=None,
                                scores: bool = True, workspace=None):
    """Pooled-query baseline scores and the same selection."""
    return _retrieve(lib().park_retrieve_blocks_pooled, "park_retrieve_blocks_pooled", Q, centroids, counts,
                     top_p, top_k, scale, scores, workspace)


def park_block_sparse_attn(Q, K, V, perm, offsets, block_list, block_count, scale=None, want_lse: bool = True,
                           out=None, lse=None, workspace=None, events=None):
    """Attention over the selected blocks.  Returns (O [B,H,N,d] in Q's dtype, lse [B,H,N]
    float32 or None).  `events` = a HipEvents with one pair per pass (attn_passes()) selects
    park_block_sparse_attn_timed, which records pair p around pass p's attention kernel."""
    torch = _torch()
    for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (perm, "perm"), (offsets, "offsets"),
                 (block_list, "block_list"), (block_count, "block_count")):
        _dev(t, n)
    B, H, N, d = _bhnd(Q, "Q")
    if K.shape != Q.shape or V.shape != Q.shape or K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise ValueError("K and V must match Q in shape and dtype")
    nk = offsets.shape[-1] - 1
    NQ = (N + 63) // 64
    if block_list.shape != (B, H, NQ, nk) or block_count.shape != (B, H, NQ):
        raise ValueError("block_list must be [B, H, NQ, n_clusters] and block_count [B, H, NQ]")
    if perm.shape != (B, H, N) or offsets.shape != (B, H, nk + 1):
        raise ValueError("perm must be [B, H, N] and offsets [B, H, n_clusters + 1]")
    O = torch.empty_like(Q) if out is None else out
    if want_lse and lse is None:
        lse = torch.empty(B, H, N, dtype=torch.float32, device=Q.device)
    sc = -1.0 if scale is None else float(scale)
    ws, wsb = _workspace(workspace_bytes(OP_BLOCK_SPARSE_ATTN, B, H, N, d, nk), Q.device, workspace)
    args = (_ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), B, H, N, d, _ptr(perm), _ptr(offsets), nk, _ptr(block_list),
            _ptr(block_count), 64, sc, _ptr(O), _ptr(lse if want_lse else None), _ptr(ws), wsb, _stream(Q))
    if events is None:
        _check(lib().park_block_sparse_attn(*args), "park_block_sparse_attn")
    else:
        begins, ends, n = events.arrays
        _check(lib().park_block_sparse_attn_timed(*args, begins, ends, n), "park_block_sparse_attn_timed")
    return O, (lse if want_lse else None)


def park_cluster_queries(Q, n_qblocks: int, iters: int, init_idx=None, workspace=None):
    """Query blocks by Euclidean k-means of the queries.  Returns a dict of GPU tensors:
    centroids [B,H,n_qblocks,d] float32, counts [B,H,n_qblocks], labels [B,H,N],
    perm [B,H,N] (the q_perm of the clustered calls), offsets [B,H,n_qblocks+1] (q_offsets)."""
    torch = _torch()
    _dev(Q, "Q")
    B, H, N, d = _bhnd(Q, "Q")
    dev = Q.device
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(centroids=torch.empty(B, H, n_qblocks, d, dtype=torch.float32, device=dev),
               counts=torch.empty(B, H, n_qblocks, **i32), labels=torch.empty(B, H, N, **i32),
               perm=torch.empty(B, H, N, **i32), offsets=torch.empty(B, H, n_qblocks + 1, **i32))
    if init_idx is not None:
        _dev(init_idx, "init_idx")
        if init_idx.dtype != torch.int32 or init_idx.numel() != n_qblocks:
            raise ValueError("init_idx must be int32 [n_qblocks]")
    ws, wsb = _workspace(workspace_bytes(OP_CLUSTER_KEYS, B, H, N, d, n_qblocks), dev, workspace)
    st = lib().park_cluster_queries(_ptr(Q), _dtype_code(Q), B, H, N, d, n_qblocks, iters, _ptr(init_idx),
                                    _ptr(out["centroids"]), _ptr(out["counts"]), _ptr(out["labels"]),
                                    _ptr(out["perm"]), _ptr(out["offsets"]), _ptr(ws), wsb, _stream(Q))
    _check(st, "park_cluster_queries")
    return out


def _qblocks(q_perm, q_offsets, B, H, N):
    _dev(q_perm, "q_perm"); _dev(q_offsets, "q_offsets")
    nq = q_offsets.shape[-1] - 1
    if q_perm.shape != (B, H, N) or q_offsets.shape != (B, H, nq + 1):
        raise ValueError("q_perm must be [B, H, N] and q_offsets [B, H, n_qblocks + 1]")
    return nq


def park_retrieve_blocks_clustered(Q, centroids, counts, q_perm, q_offsets, top_p: float, top_k: int, scale=None,
                                   scores: bool = True, workspace=None):
    """PAMA and the top-p / top-k selection over clustered query blocks (q_perm / q_offsets as
    park_cluster_queries returns them).  Returns dict(scores?, mask, block_list, block_count)
    with n_qblocks rows per head."""
    torch = _torch()
    _dev(Q, "Q"); _dev(centroids, "centroids"); _dev(counts, "counts")
    B, H, N, d = _bhnd(Q, "Q")
    nk = centroids.shape[2]
    if centroids.shape != (B, H, nk, d) or centroids.dtype != torch.float32:
        raise ValueError("centroids must be float32 [B, H, n_clusters, d]")
    if counts.shape != (B, H, nk) or counts.dtype != torch.int32:
        raise ValueError("counts must be int32 [B, H, n_clusters]")
    nq = _qblocks(q_perm, q_offsets, B, H, N)
    dev = Q.device
    out = dict(mask=torch.empty(B, H, nq, nk, dtype=torch.uint8, device=dev),
               block_list=torch.empty(B, H, nq, nk, dtype=torch.int32, device=dev),
               block_count=torch.empty(B, H, nq, dtype=torch.int32, device=dev))
    if scores:
        out["scores"] = torch.empty(B, H, nq, nk, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(workspace_bytes_clustered(OP_RETRIEVE_BLOCKS, B, H, N, d, nk, nq), dev, workspace)
    sc = -1.0 if scale is None else float(scale)
    st = lib().park_retrieve_blocks_clustered(_ptr(Q), _dtype_code(Q), B, H, N, d, _ptr(centroids), _ptr(counts),
                                              nk, _ptr(q_perm), _ptr(q_offsets), nq, float(top_p), int(top_k), sc,
                                              _ptr(out.get("scores")), _ptr(out["mask"]), _ptr(out["block_list"]),
                                              _ptr(out["block_count"]), _ptr(ws), wsb, _stream(Q))
    _check(st, "park_retrieve_blocks_clustered")
    return out


def park_retrieve_blocks_online(Q, centroids, counts, top_p: float, top_k: int, q_perm=None, q_offsets=None,
                                scale=None, scores: bool = True, workspace=None):
    """PAMA scores and SCOPE's online per-head top-k selection: 64-token query blocks when
    q_perm / q_offsets are None, else the clustered blocks they describe.  Returns
    dict(scores?, mask, block_list, block_count)."""
    torch = _torch()
    _dev(Q, "Q"); _dev(centroids, "centroids"); _dev(counts, "counts")
    B, H, N, d = _bhnd(Q, "Q")
    nk = centroids.shape[2]
    if centroids.shape != (B, H, nk, d) or centroids.dtype != torch.float32:
        raise ValueError("centroids must be float32 [B, H, n_clusters, d]")
    if counts.shape != (B, H, nk) or counts.dtype != torch.int32:
        raise ValueError("counts must be int32 [B, H, n_clusters]")
    clustered = q_perm is not None or q_offsets is not None
    if clustered:
        nq = _qblocks(q_perm, q_offsets, B, H, N)
        need = workspace_bytes_clustered(OP_RETRIEVE_BLOCKS, B, H, N, d, nk, nq)
    else:
        nq = (N + 63) // 64
        need = workspace_bytes(OP_RETRIEVE_BLOCKS, B, H, N, d, nk)
    dev = Q.device
    out = dict(mask=torch.empty(B, H, nq, nk, dtype=torch.uint8, device=dev),
               block_list=torch.empty(B, H, nq, nk, dtype=torch.int32, device=dev),
               block_count=torch.empty(B, H, nq, dtype=torch.int32, device=dev))
    if scores:
        out["scores"] = torch.empty(B, H, nq, nk, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(need, dev, workspace)
    sc = -1.0 if scale is None else float(scale)
    st = lib().park_retrieve_blocks_online(_ptr(Q), _dtype_code(Q), B, H, N, d, _ptr(centroids), _ptr(counts), nk,
                                           _ptr(q_perm), _ptr(q_offsets), nq, float(top_p), int(top_k), sc,
                                           _ptr(out.get("scores")), _ptr(out["mask"]), _ptr(out["block_list"]),
                                           _ptr(out["block_count"]), _ptr(ws), wsb, _stream(Q))
    _check(st, "park_retrieve_blocks_online")
    return out


def park_block_sparse_attn_clustered(Q, K, V, perm, offsets, q_perm, q_offsets, block_list, block_count, scale=None,
                                     want_lse: bool = True, out=None, lse=None, workspace=None):
    """Attention over the clusters selected for each clustered query block.  Returns
    (O [B,H,N,d] in Q's dtype, lse [B,H,N] float32 or None), in the original query order."""
    torch = _torch()
    for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (perm, "perm"), (offsets, "offsets"),
                 (block_list, "block_list"), (block_count, "block_count")):
        _dev(t, n)
    B, H, N, d = _bhnd(Q, "Q")
    if K.shape != Q.shape or V.shape != Q.shape or K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise ValueError("K and V must match Q in shape and dtype")
    nk = offsets.shape[-1] - 1
    nq = _qblocks(q_perm, q_offsets, B, H, N)
    if block_list.shape != (B, H, nq, nk) or block_count.shape != (B, H, nq):
        raise ValueError("block_list must be [B, H, n_qblocks, n_clusters] and block_count [B, H, n_qblocks]")
    if perm.shape != (B, H, N) or offsets.shape != (B, H, nk + 1):
        raise ValueError("perm must be [B, H, N] and offsets [B, H, n_clusters + 1]")
    O = torch.empty_like(Q) if out is None else out
    if want_lse and lse is None:
        lse = torch.empty(B, H, N, dtype=torch.float32, device=Q.device)
    sc = -1.0 if scale is None else float(scale)
    ws, wsb = _workspace(workspace_bytes_clustered(OP_BLOCK_SPARSE_ATTN, B, H, N, d, nk, nq), Q.device, workspace)
    st = lib().park_block_sparse_attn_clustered(_ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), B, H, N, d, _ptr(perm),
                                                _ptr(offsets), nk, _ptr(q_perm), _ptr(q_offsets), nq,
                                                _ptr(block_list), _ptr(block_count), sc, _ptr(O),
                                                _ptr(lse if want_lse else None), _ptr(ws), wsb, _stream(Q))
    _check(st, "park_block_sparse_attn_clustered")
    return O, (lse if want_lse else None)


def park_block_importance_exact(Q, K, perm, offsets, scale=None, workspace=None):
    """Exact block importance (section 3.2, Eq. (3)) of every 64-token query block over the
    key clusters: W [B,H,NQ,n_clusters] float32 (a retrieval-accuracy diagnostic)."""
    torch = _torch()
    for t, n in ((Q, "Q"), (K, "K"), (perm, "perm"), (offsets, "offsets")):
        _dev(t, n)
    B, H, N, d = _bhnd(Q, "Q")
    if K.shape != Q.shape or K.dtype != Q.dtype:
        raise ValueError("K must match Q in shape and dtype")
    nk = offsets.shape[-1] - 1
    if perm.shape != (B, H, N) or offsets.shape != (B, H, nk + 1):
        raise ValueError("perm must be [B, H, N] and offsets [B, H, n_clusters + 1]")
    W = torch.empty(B, H, (N + 63) // 64, nk, dtype=torch.float32, device=Q.device)
    ws, wsb = _workspace(workspace_bytes(OP_BLOCK_IMPORTANCE, B, H, N, d, nk), Q.device, workspace)
    sc = -1.0 if scale is None else float(scale)
    st = lib().park_block_importance_exact(_ptr(Q), _ptr(K), _dtype_code(Q), B, H, N, d, _ptr(perm), _ptr(offsets),
                                           nk, sc, _ptr(W), _ptr(ws), wsb, _stream(Q))
    _check(st, "park_block_importance_exact")
    return W


def park_logmass_rmse(Q, K, perm, offsets, centroids, counts, scale=None, workspace=None):
    """Centred log-mass RMSE of the key centroids (PARK appendix B, M2) per head: [B, H] float32."""
    torch = _torch()
    for t, n in ((Q, "Q"), (K, "K"), (perm, "perm"), (offsets, "offsets"), (centroids, "centroids"),
                 (counts, "counts")):
        _dev(t, n)
    B, H, N, d = _bhnd(Q, "Q")
    nk = offsets.shape[-1] - 1
    if K.shape != Q.shape or K.dtype != Q.dtype:
        raise ValueError("K must match Q in shape and dtype")
    if centroids.shape != (B, H, nk, d) or counts.shape != (B, H, nk):
        raise ValueError("centroids must be [B, H, n_clusters, d] and counts [B, H, n_clusters]")
    out = torch.empty(B, H, dtype=torch.float32, device=Q.device)
    ws, wsb = _workspace(int(lib().park_logmass_workspace_bytes(B, H, N, d, nk)), Q.device, workspace)
    sc = -1.0 if scale is None else float(scale)
    st = lib().park_logmass_rmse(_ptr(Q), _ptr(K), _dtype_code(Q), B, H, N, d, _ptr(perm), _ptr(offsets), nk,
                                 _ptr(centroids), _ptr(counts), sc, _ptr(out), _ptr(ws), wsb, _stream(Q))
    _check(st, "park_logmass_rmse")
    return out


def attn_passes(B: int, H: int, N: int, d: int, n_clusters: int, dtype: str = "bf16") -> int:
    """Passes over the heads that park_block_sparse_attn makes for these sizes."""
    return lib().park_attn_passes(1 if dtype == "bf16" else 0, B, H, N, d, n_clusters)


class HipEvents:
    """`n` pairs of HIP events for timing one kernel through the *_timed entry points (one pair
    for park_cluster_keys and park_retrieve_blocks, one per pass for park_block_sparse_attn):
    created and read through libamdhip64 directly (torch's events only see its own calls)."""

    def __init__(self, n: int = 1):
        import ctypes.util
        name = ctypes.util.find_library("amdhip64") or "libamdhip64.so"
        self._hip = ctypes.CDLL(name)
        self.begins = (ctypes.c_void_p * n)()
        self.ends = (ctypes.c_void_p * n)()
        self.n = n
        for arr in (self.begins, self.ends):
            for i in range(n):
                ev = ctypes.c_void_p()
                if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                arr[i] = ev.value

    @property
    def handles(self):
        """(begin, end) of the first pair."""
        return (ctypes.c_void_p(self.begins[0]), ctypes.c_void_p(self.ends[0]))

    @property
    def arrays(self):
        """(begin handles, end handles, n) as host arrays."""
        return (self.begins, self.ends, self.n)

    def elapsed_ms(self) -> float:
        """Sum over the pairs of the time between begin and end."""
        total = 0.0
        for i in range(self.n):
            ms = ctypes.c_float()
            b, e = ctypes.c_void_p(self.begins[i]), ctypes.c_void_p(self.ends[i])
            if self._hip.hipEventSynchronize(e) != 0 or \
                    self._hip.hipEventElapsedTime(ctypes.byref(ms), b, e) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            total += ms.value
        return total

    def __del__(self):
        try:
            for arr in (self.begins, self.ends):
                for i in range(self.n):
                    self._hip.hipEventDestroy(ctypes.c_void_p(arr[i]))
        except Exception:  # pragma: no cover - interpreter shutdown
            pass


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
