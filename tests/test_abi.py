"""C ABI checks that need no GPU: the library loads, exports every entry point declared in
include/park.h, and rejects invalid arguments on the host before anything is launched.
(The pointers passed here are never dereferenced: every call fails a host-side check.)"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "park.h")
LIB = os.path.join(ROOT, "block_sparse_attention_response_amd", "libpark.so")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)   # a non-null address; never used by a rejected call


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libpark.so is not built (run __graft_entry__.build())")
    import block_sparse_attention_response_amd as park
    return park.lib()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"PARK_API\s+[\w\s\*]+?\b(park_\w+)\s*\(", text)


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("park_cluster_keys", "park_retrieve_blocks", "park_retrieve_blocks_pooled",
              "park_block_sparse_attn", "park_block_sparse_attn_timed", "park_workspace_bytes", "park_abi_version",
              "park_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_clock_build_exports_only_its_declared_symbols(lib):
    """libpark_clocks.so exports the measurement entry points of include/park_clocks.h beside
    every entry point of park.h; the product library exports none of them."""
    clocks = os.path.join(ROOT, "block_sparse_attention_response_amd", "libpark_clocks.so")
    if not os.path.exists(clocks):
        pytest.fail("libpark_clocks.so is not built (run __graft_entry__.build())")
    text = open(os.path.join(ROOT, "include", "park_clocks.h")).read()
    names = re.findall(r"PARK_CLOCKS_API\s+[\w\s\*]+?\b(park_\w+)\s*\(", text)
    assert sorted(names) == ["park_attn_clock_read", "park_attn_clock_words"]
    L = ctypes.CDLL(clocks)
    for n in names + declared_functions():
        assert hasattr(L, n), n
    for n in names:
        assert not hasattr(lib, n), n
    L.park_attn_clock_words.restype = ctypes.c_size_t
    assert L.park_attn_clock_words() == 1 << 21
    L.park_attn_clock_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    assert L.park_attn_clock_read(None, 5) == INVALID                      # no host buffer
    assert L.park_attn_clock_read(FAKE, (1 << 21) + 1) == INVALID          # beyond the record


def test_version_and_status_strings(lib):
    assert lib.park_abi_version() == 2
    names = [lib.park_status_string(i).decode() for i in range(6)]
    assert names == ["PARK_OK", "PARK_ERR_INVALID", "PARK_ERR_UNSUPPORTED", "PARK_ERR_WORKSPACE", "PARK_ERR_HIP",
                     "PARK_ERR_NUMERIC"]
    assert lib.park_status_string(99).decode() == "PARK_ERR_UNKNOWN"


def test_workspace_sizes(lib):
    for op in range(3):
        assert lib.park_workspace_bytes(op, 1, 2, 1000, 128, 24) > 0
    assert lib.park_workspace_bytes(0, 1, 2, 1000, 96, 24) == 0      # unsupported d
    assert lib.park_workspace_bytes(0, 1, 2, 10, 128, 24) == 0       # more clusters than tokens
    assert lib.park_workspace_bytes(7, 1, 2, 1000, 128, 24) == 0     # unknown op
    a = lib.park_workspace_bytes(0, 1, 40, 75600, 128, 1024)
    b = lib.park_workspace_bytes(0, 1, 40, 75600, 128, 1536)
    assert b > a > 0


def test_clustered_attention_workspace_has_no_partial_states(lib):
    """Clustered query blocks: whole-row attention items write O and lse themselves, so the
    workspace holds no per-range partial states (fp16 O and float (m, l) per query and key
    range), only the chunk tables that the 64-token path does not need."""
    a256 = lambda x: (x + 255) // 256 * 256
    B, H, N, d, nk = 1, 4, 75600, 128, 1024    # four heads: one pass on both paths
    NQ = (N + 63) // 64          # as many clustered blocks as 64-token blocks: same plan size
    BH, maxc = B * H, (N + 63) // 64 + NQ
    w64 = lib.park_workspace_bytes(2, B, H, N, d, nk)
    wcl = lib.park_workspace_bytes_clustered(2, B, H, N, d, nk, NQ)
    R = 4                        # key ranges of the 64-token path
    partial = a256(BH * N * R * d * 2) + a256(BH * N * R * 8)
    tables = a256(BH * maxc * 16) + a256(BH * (NQ + 1) * 4) + a256(BH * 4)
    assert lib.park_attn_passes(1, B, H, N, d, nk) == 1
    assert w64 - wcl == partial - tables


@pytest.mark.parametrize("B,H,N,nk", [(1, 40, 75600, 1024), (1, 24, 119056, 1536), (2, 12, 32760, 512)])
def test_attention_workspace_holds_one_pass_of_heads(lib, B, H, N, nk):
    """The attention call walks the heads in passes whose packed keys and values, tile plan and
    partial states fit in 2.5 GiB; the workspace is that of one pass of ceil(B H / passes)
    heads plus a few small per-head tables of all heads, so the 75.6k-token, 40-head layer
    needs under 3 GB."""
    d = 128
    a256 = lambda x: (x + 255) // 256 * 256
    # per-head tables of all heads (first packed group and key range of each cluster, |V| max)
    tabs = lambda bh: a256(bh * (nk + 1) * 4) + a256(bh * nk * 4) + a256(bh * 4)
    passes = lib.park_attn_passes(1, B, H, N, d, nk)
    assert passes >= 1
    hpp = -(-B * H // passes)
    assert -(-B * H // hpp) == passes                       # balanced passes
    ws = lib.park_workspace_bytes(2, B, H, N, d, nk)
    one_pass = lib.park_workspace_bytes(2, 1, hpp, N, d, nk) - tabs(hpp)
    assert ws == tabs(B * H) + one_pass
    assert lib.park_attn_passes(1, 1, hpp, N, d, nk) == 1
    assert one_pass <= 5 << 29
    if hpp > 1:   # one more head would not fit in 2.5 GiB... or the passes would not be balanced
        assert lib.park_workspace_bytes(2, 1, hpp + 1, N, d, nk) - tabs(hpp + 1) > 5 << 29 or \
            -(-B * H // (hpp + 1)) == passes
    if (B, H, N, nk) == (1, 40, 75600, 1024):
        assert passes > 1 and ws < 3e9
    assert lib.park_attn_passes(1, 0, H, N, d, nk) == 0      # invalid sizes
    assert lib.park_attn_passes(0, B, H, N, d, nk) == 1      # float inputs keep no per-head buffers


def test_noalloc_retrieve_rejects(lib):
    """The no-allocation retrieval: host-side rejections, including sizes whose scratch would
    exceed the library's fixed per-GPU array (nothing is launched or looked up for them)."""
    limit = 32 << 20
    def call(**kw):
        a = dict(Q=FAKE, dtype=1, B=1, H=2, N=256, d=128, cent=FAKE, counts=FAKE, nk=8, qb=64, p=0.9, k=2,
                 scale=-1.0, scores=FAKE, mask=FAKE, lst=FAKE, cnt=FAKE)
        a.update(kw)
        return lib.park_retrieve_blocks_noalloc(a["Q"], a["dtype"], a["B"], a["H"], a["N"], a["d"], a["cent"],
                                                a["counts"], a["nk"], a["qb"], a["p"], a["k"], a["scale"],
                                                a["scores"], a["mask"], a["lst"], a["cnt"], None)
    assert call(scores=None) == INVALID            # W is an output here, never scratch
    assert call(mask=None) == INVALID
    assert call(p=1.5) == INVALID
    assert call(k=-1) == INVALID
    assert call(nk=300) == INVALID
    assert call(qb=32) == UNSUPPORTED
    assert call(d=96) == UNSUPPORTED
    assert lib.park_noalloc_scratch_bytes(1, 40, 75600, 128, 1024) <= limit
    assert lib.park_noalloc_scratch_bytes(1, 24, 119056, 128, 1536) <= limit
    assert lib.park_noalloc_scratch_bytes(1, 40, 75600, 96, 1024) == 0
    assert lib.park_noalloc_scratch_bytes(1, 160, 75600, 128, 1536) > limit
    assert call(H=160, N=75600, nk=1536) == WORKSPACE


def _cluster(lib, **kw):
    a = dict(Q=FAKE, K=FAKE, dtype=1, B=1, H=1, N=256, d=128, nk=8, iters=2, metric=0, alpha=0.05, init=None,
             cent=FAKE, counts=FAKE, labels=FAKE, perm=FAKE, offsets=FAKE, status=None, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return lib.park_cluster_keys(a["Q"], a["K"], a["dtype"], a["B"], a["H"], a["N"], a["d"], a["nk"], a["iters"],
                                 a["metric"], a["alpha"], a["init"], a["cent"], a["counts"], a["labels"], a["perm"],
                                 a["offsets"], a["status"], a["ws"], a["wsb"], None)


def test_cluster_keys_rejects(lib):
    assert _cluster(lib, Q=None) == INVALID
    assert _cluster(lib, perm=None) == INVALID
    assert _cluster(lib, N=0) == INVALID
    assert _cluster(lib, nk=300) == INVALID
    assert _cluster(lib, nk=0) == INVALID
    assert _cluster(lib, iters=0) == INVALID
    assert _cluster(lib, alpha=1.5) == INVALID
    assert _cluster(lib, alpha=float("nan")) == INVALID
    assert _cluster(lib, metric=5) == INVALID
    assert _cluster(lib, dtype=7) == INVALID
    assert _cluster(lib, d=96) == UNSUPPORTED
    assert _cluster(lib, N=4000, nk=2000) == UNSUPPORTED
    assert _cluster(lib, ws=None) == WORKSPACE
    assert _cluster(lib, wsb=1024) == WORKSPACE
    assert _cluster(lib, ws=ctypes.c_void_p(0x10008)) == WORKSPACE   # not 256-byte aligned


def _retrieve(lib, fn="park_retrieve_blocks", **kw):
    a = dict(Q=FAKE, dtype=1, B=1, H=1, N=256, d=128, cent=FAKE, counts=FAKE, nk=8, qb=64, p=0.9, k=2, scale=-1.0,
             scores=FAKE, mask=FAKE, lst=FAKE, cnt=FAKE, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return getattr(lib, fn)(a["Q"], a["dtype"], a["B"], a["H"], a["N"], a["d"], a["cent"], a["counts"], a["nk"],
                            a["qb"], a["p"], a["k"], a["scale"], a["scores"], a["mask"], a["lst"], a["cnt"], a["ws"],
                            a["wsb"], None)


@pytest.mark.parametrize("fn", ["park_retrieve_blocks", "park_retrieve_blocks_pooled"])
def test_retrieve_rejects(lib, fn):
    assert _retrieve(lib, fn, mask=None) == INVALID
    assert _retrieve(lib, fn, p=1.5) == INVALID
    assert _retrieve(lib, fn, p=-0.1) == INVALID
    assert _retrieve(lib, fn, k=-1) == INVALID
    assert _retrieve(lib, fn, scale=float("inf")) == INVALID
    assert _retrieve(lib, fn, qb=32) == UNSUPPORTED
    assert _retrieve(lib, fn, d=80) == UNSUPPORTED
    assert _retrieve(lib, fn, ws=None) == WORKSPACE
    assert _retrieve(lib, fn, wsb=16) == WORKSPACE


def test_unfused_retrieve_rejects(lib):
    def call(**kw):
        a = dict(Q=FAKE, dtype=1, B=1, H=1, N=256, d=128, cent=FAKE, counts=FAKE, nk=8, qb=64, p=0.9, k=2,
                 scale=-1.0, probs=FAKE, scores=FAKE, mask=FAKE, lst=FAKE, cnt=FAKE, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return lib.park_retrieve_blocks_unfused(a["Q"], a["dtype"], a["B"], a["H"], a["N"], a["d"], a["cent"],
                                                a["counts"], a["nk"], a["qb"], a["p"], a["k"], a["scale"], a["probs"],
                                                a["scores"], a["mask"], a["lst"], a["cnt"], a["ws"], a["wsb"], None)
    assert call(probs=None) == INVALID
    assert call(mask=None) == INVALID
    assert call(p=2.0) == INVALID
    assert call(qb=16) == UNSUPPORTED
    assert call(ws=None) == WORKSPACE


def test_online_retrieve_rejects(lib):
    def call(**kw):
        a = dict(Q=FAKE, dtype=1, B=1, H=1, N=256, d=128, cent=FAKE, counts=FAKE, nk=8, qperm=None, qoff=None, nq=0,
                 p=0.9, k=2, scale=-1.0, scores=FAKE, mask=FAKE, lst=FAKE, cnt=FAKE, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return lib.park_retrieve_blocks_online(a["Q"], a["dtype"], a["B"], a["H"], a["N"], a["d"], a["cent"],
                                               a["counts"], a["nk"], a["qperm"], a["qoff"], a["nq"], a["p"], a["k"],
                                               a["scale"], a["scores"], a["mask"], a["lst"], a["cnt"], a["ws"],
                                               a["wsb"], None)
    assert call(nq=3) == INVALID                       # 64-token blocks: 0 or ceil(N / 64) = 4
    assert call(qperm=FAKE) == INVALID                 # one table without the other
    assert call(qperm=FAKE, qoff=FAKE, nq=0) == INVALID
    assert call(qperm=FAKE, qoff=FAKE, nq=257) == INVALID
    assert call(k=-1) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(ws=None) == WORKSPACE
    assert call(nq=4, ws=None) == WORKSPACE            # valid sizes reach the workspace check
    assert call(qperm=FAKE, qoff=FAKE, nq=8, wsb=64) == WORKSPACE


def _attn(lib, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, dtype=1, B=1, H=1, N=256, d=128, perm=FAKE, off=FAKE, nk=8, lst=FAKE, cnt=FAKE,
             qb=64, scale=-1.0, O=FAKE, lse=None, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return lib.park_block_sparse_attn(a["Q"], a["K"], a["V"], a["dtype"], a["B"], a["H"], a["N"], a["d"], a["perm"],
                                      a["off"], a["nk"], a["lst"], a["cnt"], a["qb"], a["scale"], a["O"], a["lse"],
                                      a["ws"], a["wsb"], None)


def test_attention_rejects(lib):
    assert _attn(lib, V=None) == INVALID
    assert _attn(lib, O=None) == INVALID
    assert _attn(lib, B=0) == INVALID
    assert _attn(lib, scale=float("nan")) == INVALID
    assert _attn(lib, qb=128) == UNSUPPORTED
    assert _attn(lib, d=32) == UNSUPPORTED
    assert _attn(lib, ws=None) == WORKSPACE
    assert _attn(lib, wsb=100) == WORKSPACE


def test_timed_cluster_and_retrieve_reject_like_the_plain_calls(lib):
    # the measurement variants run the same host checks before they record any event
    for over, want in ((dict(Q=None), INVALID), (dict(d=96), UNSUPPORTED), (dict(ws=None), WORKSPACE)):
        a = dict(Q=FAKE, K=FAKE, dtype=1, B=1, H=1, N=256, d=128, nk=8, iters=2, metric=0, alpha=0.05, init=None,
                 cent=FAKE, counts=FAKE, labels=FAKE, perm=FAKE, offsets=FAKE, status=None, ws=FAKE, wsb=1 << 40)
        a.update(over)
        st = lib.park_cluster_keys_timed(a["Q"], a["K"], a["dtype"], a["B"], a["H"], a["N"], a["d"], a["nk"],
                                         a["iters"], a["metric"], a["alpha"], a["init"], a["cent"], a["counts"],
                                         a["labels"], a["perm"], a["offsets"], a["status"], a["ws"], a["wsb"], None,
                                         FAKE, FAKE)
        assert st == want, (over, st)
    for over, want in ((dict(mask=None), INVALID), (dict(qb=32), UNSUPPORTED), (dict(ws=None), WORKSPACE)):
        a = dict(Q=FAKE, dtype=1, B=1, H=1, N=256, d=128, cent=FAKE, counts=FAKE, nk=8, qb=64, p=0.9, k=2,
                 scale=-1.0, scores=FAKE, mask=FAKE, lst=FAKE, cnt=FAKE, ws=FAKE, wsb=1 << 40)
        a.update(over)
        st = lib.park_retrieve_blocks_timed(a["Q"], a["dtype"], a["B"], a["H"], a["N"], a["d"], a["cent"],
                                            a["counts"], a["nk"], a["qb"], a["p"], a["k"], a["scale"], a["scores"],
                                            a["mask"], a["lst"], a["cnt"], a["ws"], a["wsb"], None, FAKE, FAKE)
        assert st == want, (over, st)


def test_timed_attention_rejects_like_attention(lib):
    # the measurement variant runs the same host checks before it records any event
    base = dict(Q=FAKE, K=FAKE, V=FAKE, dtype=1, B=1, H=1, N=128, d=128, perm=FAKE, off=FAKE, nk=2, lst=FAKE,
                cnt=FAKE, qb=64, scale=0.0, O=FAKE, lse=None, ws=None, wsb=0)
    for over, want in ((dict(V=None), INVALID), (dict(qb=128), UNSUPPORTED), (dict(d=32), UNSUPPORTED),
                       (dict(), WORKSPACE)):
        a = dict(base, **over)
        st = lib.park_block_sparse_attn_timed(a["Q"], a["K"], a["V"], a["dtype"], a["B"], a["H"], a["N"], a["d"],
                                              a["perm"], a["off"], a["nk"], a["lst"], a["cnt"], a["qb"], a["scale"],
                                              a["O"], a["lse"], a["ws"], a["wsb"], None, FAKE, FAKE, 1)
        assert st == want, (over, st)
    # the event arrays: n_events >= 0, and both arrays given when n_events > 0
    a = dict(base, ws=FAKE, wsb=1 << 40, V=FAKE)
    for evb, eve, n in ((FAKE, FAKE, -1), (None, FAKE, 1), (FAKE, None, 2)):
        st = lib.park_block_sparse_attn_timed(a["Q"], a["K"], a["V"], a["dtype"], a["B"], a["H"], a["N"], a["d"],
                                              a["perm"], a["off"], a["nk"], a["lst"], a["cnt"], a["qb"], a["scale"],
                                              a["O"], a["lse"], a["ws"], a["wsb"], None, evb, eve, n)
        assert st == INVALID, (evb, eve, n, st)
