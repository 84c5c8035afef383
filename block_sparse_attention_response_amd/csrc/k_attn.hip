// Block-sparse attention (PARK section 3.1, E1/E2 with the softmax renormalised over the
// selected keys): every query block attends to the union of its selected key clusters.  The
// bf16 path packs the clusters' keys and values, splits each head's clusters into four key
// ranges (each computed on two XCDs), computes a partial softmax state per (query block, key
// range) and merges them; the float path walks the selected clusters through the cluster
// permutation.
#include <algorithm>
#include <atomic>
#include <climits>
#include <type_traits>

#include "park_device.h"
#include "park_internal.h"
#include "../../include/park.h"

namespace park {

// Size of cluster v; ids outside [0, nk) count as empty clusters.
__device__ __forceinline__ int cluster_size(int v, const int32_t* __restrict__ off, int nk) {
  return (v >= 0 && v < nk) ? off[v + 1] - off[v] : 0;
}

// Exclusive prefix sums of the selected clusters' sizes for one query block:
// pre[r] = number of keys in clusters list[0..r-1], pre[cnt] = total.  128 threads.
__device__ __forceinline__ int selected_prefix(const int32_t* __restrict__ lst, const int32_t* __restrict__ off,
                                               int cnt, int nk, int* pre, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (cnt + 127) / 128;
  const int b0 = min(tid * per, cnt), b1 = min(b0 + per, cnt);
  int s = 0;
  for (int i = b0; i < b1; ++i) s += cluster_size(lst[i], off, nk);
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int ex = incl - s + (w == 1 ? wsum[0] : 0);
  for (int i = b0; i < b1; ++i) {
    pre[i] = ex;
    ex += cluster_size(lst[i], off, nk);
  }
  const int T = wsum[0] + wsum[1];
  if (tid == 0) pre[cnt] = T;
  __syncthreads();
  return T;
}

// Key index at position p (< T) of the concatenated selection.
__device__ __forceinline__ int selected_key(int p, const int* pre, int cnt, const int32_t* __restrict__ lst,
                                            const int32_t* __restrict__ off, const int32_t* __restrict__ pm) {
  // largest r with pre[r] <= p; empty clusters give equal neighbours, so take the last
  int lo = 0, hi = cnt - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= p) lo = mid; else hi = mid - 1;
  }
  const int v = lst[lo];
  return pm[off[v] + (p - pre[lo])];
}

// ---------------------------------------------------------------------------------------
// bf16 path.  Three kernels prepare the work:
//  * the keys and values of every cluster are packed, in cluster order, into 8-key groups
//    in the operand layouts of the two MFMA products;
//  * the clusters of every head are dealt to kRanges key ranges of about equal work;
//    range r of every head is computed on XCDs r and r + 4 (the dispatcher deals consecutive
//    workgroups to the 8 XCDs in turn), so each XCD's L2 serves a quarter of a head's keys
//    and values to the query blocks of that head it runs.  Four ranges rather than eight:
//    the partial states (written once, read once by the merge) halve, which outweighs the
//    L2 holding a larger share of the keys (measured at 75.6k tokens x 40 heads: attention
//    call 15.5 ms with eight ranges, 14.6 ms with four, 16.5 ms with two);
//  * every (query block, range) pair is a work item: the groups of its selected clusters in
//    that range, in list order, cut into 32-key tiles of 4 groups.
// One wave per item computes a partial softmax state over its tiles (k_attn_items) and a last
// kernel merges the kRanges partial states of every query (k_attn_merge).
constexpr int kRanges = 4;

// Clock-stamped measurement build (compiled with PARK_ATTN_CLOCKS into a separate library; the
// product build has none of it): per 64-token-block item, the shader clock (s_memtime) at the
// item's start, before its tile loop, after it and after its stores, and (wave, tiles), five
// words per item, written by lane 0.  The stamps add four scalar reads and one store per item
// and change no other instruction.
#ifdef PARK_ATTN_CLOCKS
constexpr size_t kAttnClockWords = size_t(1) << 21;
__device__ unsigned long long attn_clock[kAttnClockWords];
#define PARK_ATTN_STAMP(x) const unsigned long long x = __builtin_amdgcn_s_memtime()
#else
#define PARK_ATTN_STAMP(x) do { } while (0)
#endif
static_assert(8 % kRanges == 0, "range r runs on the XCDs x with x % kRanges == r");

// Step 1: gstart[v] = first group of cluster v (exclusive scan of ceil(n_v / 8)); a cluster
// of n keys takes ceil(n / 8) groups and the tail of its last group is zero padding.
__global__ __launch_bounds__(256) void k_group_scan(const int32_t* __restrict__ offsets, int nk,
                                                    int32_t* __restrict__ gstart, float* __restrict__ vmax) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, bh = blockIdx.x;
  if (tid == 0) vmax[bh] = 0.0f;
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  const int per = (nk + 255) / 256;
  const int b0 = min(tid * per, nk), b1 = min(b0 + per, nk);
  int s = 0;
  for (int v = b0; v < b1; ++v) s += (off[v + 1] - off[v] + 7) >> 3;
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int ex = incl - s;
  for (int i = 0; i < w; ++i) ex += wsum[i];
  int32_t* gs = gstart + (size_t)bh * (nk + 1);
  for (int v = b0; v < b1; ++v) {
    gs[v] = ex;
    ex += (off[v + 1] - off[v] + 7) >> 3;
  }
  if (tid == 255) gs[nk] = ex;
}

// Per-head unit of the fp16 partial outputs: the smallest power of two >= the largest |value|
// of the head (1 for an all-zero head); a partial output is a convex combination of values,
// so in this unit its entries lie in [-1, 1].
__device__ __forceinline__ float value_unit(float vmax) {
  if (!(vmax > 0.0f)) return 1.0f;
  int ex;
  frexpf(vmax, &ex);   // vmax = f 2^ex, f in [0.5, 1)
  return ldexpf(1.0f, ex);
}

// Packed group layouts (8 keys, D columns):
//   Kp[g] (bf16): D/16 column chunks, each 8 keys x 16 values (chunk c of key slot s at
//          128 c + 16 s), so the A operand of S^T = K Q^T (16 columns of one key per lane)
//          is one 16-byte load and the four groups of a tile give 1 KB per chunk;
//   Vp[g] (bf16): D rows of 8 keys (V^T), the A operand of O^T += V^T P^T.
// Group Gcap of every head is all zeros: the filler of partial tiles.  vmax[bh] (zeroed by
// k_group_scan) becomes the largest |value| of the head.
template <int D>
__global__ __launch_bounds__(128) void k_pack_kv(const bf16* __restrict__ K, const bf16* __restrict__ V,
                                                 const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ gstart, int N, int nk, int Gcap,
                                                 bf16* __restrict__ Kp, bf16* __restrict__ Vp, float* __restrict__ vmax) {
  constexpr int NS = D / 8;
  const int v = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  const int a = off[v], n = off[v + 1] - a;
  const int ng = (n + 7) >> 3;
  const int g0 = gstart[(size_t)bh * (nk + 1) + v];
  const int32_t* pm = perm + (size_t)bh * N + a;
  const bf16* Kh = K + (size_t)bh * N * D;
  const bf16* Vh = V + (size_t)bh * N * D;
  bf16* Kph = Kp + (size_t)bh * (Gcap + 1) * 8 * D;
  bf16* Vph = Vp + (size_t)bh * (Gcap + 1) * 8 * D;
  if (v == 0) {
    for (int e = tid; e < D; e += 128) {
      bf16x8 z;
#pragma unroll
      for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
      *reinterpret_cast<bf16x8*>(Kph + (size_t)Gcap * 8 * D + e * 8) = z;
      *reinterpret_cast<bf16x8*>(Vph + (size_t)Gcap * 8 * D + e * 8) = z;
    }
  }
  // Branch-free copies (a branch around each access makes the compiler wait for every
  // earlier load and store before the next one): member indices are clamped to the cluster,
  // padding slots are zeroed by a select, and the stores of slots past the cluster's groups
  // go to the head's all-zero filler group (writing zeros there changes nothing).
  const bf16* Kz = Kph + (size_t)Gcap * 8 * D;
  Kph += (size_t)g0 * 8 * D;
  Vph += (size_t)g0 * 8 * D;
  bf16x8 zero8;
#pragma unroll
  for (int i = 0; i < 8; ++i) zero8[i] = (bf16)0.0f;
  // keys: thread t copies the 16-byte piece sg = t % NS of key slots t / NS + SPI u, U slots in
  // flight (their member indices, then their rows, then the stores)
  {
    constexpr int SPI = 128 / NS, U = 8;
    const int sg = tid % NS, s0 = tid / NS;
    const uint32_t in_group = (uint32_t)((sg >> 1) * 128 + (sg & 1) * 8);
    for (int base = 0; base < ng * 8; base += SPI * U) {
      int src[U];
#pragma unroll
      for (int u = 0; u < U; ++u) src[u] = pm[min(base + s0 + SPI * u, n - 1)];
      bf16x8 val[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bf16x8 x = load_bf16x8(Kh + (size_t)src[u] * D + sg * 8);
        val[u] = base + s0 + SPI * u < n ? x : zero8;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int slot = base + s0 + SPI * u, j = slot >> 3, sl = slot & 7;
        bf16* dst = slot < ng * 8 ? Kph + (size_t)j * 8 * D : const_cast<bf16*>(Kz);
        *reinterpret_cast<bf16x8*>(dst + in_group + sl * 16) = val[u];
      }
    }
  }
  // values: thread t transposes the 8 x 8 block (group j, columns 8 sg .. + 7): 8 member rows
  // in, 8 rows of V^T out
  float amax = 0.0f;
  for (int e = tid; e < ng * NS; e += 128) {
    const int j = e / NS, sg = e % NS;
    int src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) src[i] = pm[min(8 * j + i, n - 1)];
    bf16x8 rows[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x8 x = load_bf16x8(Vh + (size_t)src[i] * D + sg * 8);
      rows[i] = 8 * j + i < n ? x : zero8;
    }
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      bf16x8 col;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        col[i] = rows[i][dd];
        amax = fmaxf(amax, fabsf((float)col[i]));
      }
      *reinterpret_cast<bf16x8*>(Vph + (size_t)j * 8 * D + (size_t)(sg * 8 + dd) * 8) = col;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  // non-negative floats order like their bit patterns
  if ((tid & 63) == 0 && amax > 0.0f) atomicMax(reinterpret_cast<int*>(vmax) + bh, __float_as_int(amax));
}

// Step 2: the range of every cluster.  work(v) = (query blocks selecting v) x (groups of v);
// clusters sorted by work (ties by id) are dealt to the ranges in serpentine order
// 0..7, 7..0, 0..7, ..., so every range gets about the same work and every query block's
// selection spreads about evenly over the ranges.  One workgroup per head.
__global__ __launch_bounds__(1024) void k_range_assign(const int32_t* __restrict__ list,
                                                       const int32_t* __restrict__ count,
                                                       const int32_t* __restrict__ offsets, int nk, int NQ,
                                                       int32_t* __restrict__ rng) {
  constexpr int P = 2048;   // power of two >= PARK_MAX_CLUSTERS
  static_assert(P >= PARK_MAX_CLUSTERS, "sort size");
  __shared__ unsigned long long key[P];
  __shared__ int freq[PARK_MAX_CLUSTERS];
  const int tid = threadIdx.x, bh = blockIdx.x;
  for (int v = tid; v < nk; v += 1024) freq[v] = 0;
  __syncthreads();
  const int32_t* L = list + (size_t)bh * NQ * nk;
  const int32_t* C = count + (size_t)bh * NQ;
  // wave w counts blocks w, w + 16, ...: kB blocks at a time, their counts and the first 128
  // entries of each loaded together (entries past a block's count are masked, not skipped);
  // the rare blocks with more than 128 entries finish in a second loop
  {
    constexpr int kB = 8, W = 1024 / 64;
    const int lane = tid & 63, wv = tid >> 6;
    for (int u0 = wv; u0 < NQ; u0 += W * kB) {
      int cnt[kB], v0[kB], v1[kB];
      // lane b loads the count of block u0 + W b (one load for the wave)
      const int cl = C[min(u0 + W * (lane & (kB - 1)), NQ - 1)];
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        const int u = min(u0 + W * b, NQ - 1);
        const int cu = __builtin_amdgcn_readlane(cl, b);
        cnt[b] = u0 + W * b < NQ ? min(max(cu, 0), nk) : 0;
        v0[b] = L[(size_t)u * nk + min(lane, nk - 1)];
        v1[b] = L[(size_t)u * nk + min(64 + lane, nk - 1)];
      }
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        if (lane < cnt[b] && v0[b] >= 0 && v0[b] < nk) atomicAdd(&freq[v0[b]], 1);
        if (64 + lane < cnt[b] && v1[b] >= 0 && v1[b] < nk) atomicAdd(&freq[v1[b]], 1);
        const int u = u0 + W * b;
        for (int i = 128 + lane; i < cnt[b]; i += 64) {
          const int v = L[(size_t)u * nk + i];
          if (v >= 0 && v < nk) atomicAdd(&freq[v], 1);
        }
      }
    }
  }
  __syncthreads();
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  for (int p = tid; p < P; p += 1024) {
    unsigned long long w = 0;
    if (p < nk) w = (unsigned long long)freq[p] * (unsigned long long)((off[p + 1] - off[p] + 7) >> 3);
    key[p] = (w << 32) | (unsigned)(P - 1 - p);   // larger work first; equal work: lower id first
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += 1024) {
        const int l = i ^ j;
        if (l > i) {
          const unsigned long long x = key[i], y = key[l];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) { key[i] = y; key[l] = x; }
        }
      }
      __syncthreads();
    }
  }
  for (int p = tid; p < P; p += 1024) {
    const int v = P - 1 - (int)(key[p] & 0xffffffffu);
    const int blk = p / kRanges, pos = p % kRanges;
    if (v < nk) rng[(size_t)bh * nk + v] = (blk & 1) ? kRanges - 1 - pos : pos;
  }
}

// Step 3: the tile plan.  Items are numbered ((b h) NQ + u) kRanges + r.  Plan entry
// (g << 4) | nv names a packed group g and its number of real keys nv (0..8); 4 entries make
// a 32-key tile and the last tile of an item is filled with the all-zero group Gcap.
// tbase is the exclusive scan of tiles per item.
__global__ __launch_bounds__(256) void k_plan_count(const int32_t* __restrict__ list, const int32_t* __restrict__ count,
                                                    const int32_t* __restrict__ offsets, const int32_t* __restrict__ rng,
                                                    int nk, int NQ, int rows, int32_t* __restrict__ ntiles) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int bh = row / NQ;
  const int cnt = min(max(count[row], 0), nk);
  const int32_t* lst = list + (size_t)row * nk;
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  const int32_t* rg = rng + (size_t)bh * nk;
  int s[kRanges];
#pragma unroll
  for (int j = 0; j < kRanges; ++j) s[j] = 0;
  for (int i = lane; i < cnt; i += 64) {
    const int v = lst[i];
    if (v >= 0 && v < nk) {
      const int ng = (off[v + 1] - off[v] + 7) >> 3, r = rg[v];
#pragma unroll
      for (int j = 0; j < kRanges; ++j) s[j] += r == j ? ng : 0;
    }
  }
#pragma unroll
  for (int j = 0; j < kRanges; ++j) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s[j] += __shfl_xor(s[j], o);
  }
  if (lane < kRanges) {
    int x = s[0];
#pragma unroll
    for (int j = 1; j < kRanges; ++j) x = lane == j ? s[j] : x;
    ntiles[(size_t)row * kRanges + lane] = (x + 3) >> 2;
  }
}

// Exclusive scan of n ints in three launches: per-block sums (kScanBlock values per
// workgroup), a scan of the block sums, then the in-block scans plus the block offsets.
constexpr int kScanBlock = 4096;

__device__ __forceinline__ int block_excl_scan(int x, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int ex = incl - x, tot = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
    ex += i < w ? wsum[i] : 0;
    tot += wsum[i];
  }
  *total = tot;
  return ex;
}

// Chunk tables of clustered query blocks (one workgroup per head, two blocks per thread):
// block u of n_u queries is split into ceil(n_u / 64) chunks of consecutive positions.
constexpr int kQcPer = 2;
__global__ __launch_bounds__(1024) void k_qchunks(const int32_t* __restrict__ qoffsets, int N, int NQ, int maxc,
                                                  int4* __restrict__ chunks, int32_t* __restrict__ cbase,
                                                  int32_t* __restrict__ ctotal) {
  __shared__ int wsum[16];
  const int bh = blockIdx.x, t = threadIdx.x;
  const int32_t* off = qoffsets + (size_t)bh * (NQ + 1);
  int st[kQcPer], n[kQcPer], s = 0;
#pragma unroll
  for (int j = 0; j < kQcPer; ++j) {
    const int u = kQcPer * t + j;
    st[j] = 0;
    n[j] = 0;
    if (u < NQ) {
      const int a = min(max(off[u], 0), N), b = min(max(off[u + 1], a), N);
      st[j] = a;
      n[j] = b - a;
    }
    s += (n[j] + 63) >> 6;
  }
  int tot;
  int c = block_excl_scan(s, wsum, &tot);
  int32_t* cb = cbase + (size_t)bh * (NQ + 1);
#pragma unroll
  for (int j = 0; j < kQcPer; ++j) {
    const int u = kQcPer * t + j;
    if (u < NQ) {
      cb[u] = min(c, maxc);
      for (int k = 0; k < n[j]; k += 64, ++c)
        if (c < maxc) chunks[(size_t)bh * maxc + c] = make_int4(u, st[j] + k, min(64, n[j] - k), 0);
    }
  }
  if (t == 0) {
    cb[NQ] = min(tot, maxc);
    ctotal[bh] = min(tot, maxc);
  }
}

hipError_t launch_qchunks(const int32_t* qoffsets, int BH, int N, int NQ, int maxc, int4* chunks,
                          int32_t* cbase, int32_t* ctotal, hipStream_t st) {
  if (NQ > kQcPer * 1024) return hipErrorInvalidValue;
  k_qchunks<<<BH, 1024, 0, st>>>(qoffsets, N, NQ, maxc, chunks, cbase, ctotal);
  return hipGetLastError();
}

__global__ __launch_bounds__(1024) void k_scan_blocks(const int32_t* __restrict__ x, int n, int32_t* __restrict__ bsum) {
  __shared__ int wsum[16];
  const int b0 = blockIdx.x * kScanBlock + threadIdx.x * 4;
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += b0 + i < n ? x[b0 + i] : 0;
  int tot;
  block_excl_scan(s, wsum, &tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

__global__ __launch_bounds__(1024) void k_scan_top(int32_t* __restrict__ bsum, int nb, int32_t* __restrict__ ictr) {
  __shared__ int wsum[16];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  if (threadIdx.x < kRanges) ictr[threadIdx.x] = 0;   // the attention kernel's item counters
  __syncthreads();
  for (int c = 0; c < nb; c += 1024) {
    const int i = c + threadIdx.x;
    const int x = i < nb ? bsum[i] : 0;
    int tot;
    const int ex = block_excl_scan(x, wsum, &tot);
    const int base = carry;
    if (i < nb) bsum[i] = base + ex;
    __syncthreads();
    if (threadIdx.x == 0) carry = base + tot;
    __syncthreads();
  }
}

__global__ __launch_bounds__(1024) void k_scan_final(const int32_t* __restrict__ x, int n,
                                                     const int32_t* __restrict__ boff, int32_t* __restrict__ out) {
  __shared__ int wsum[16];
  const int b0 = blockIdx.x * kScanBlock + threadIdx.x * 4;
  int v[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = b0 + i < n ? x[b0 + i] : 0; s += v[i]; }
  int tot;
  int ex = block_excl_scan(s, wsum, &tot) + boff[blockIdx.x];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (b0 + i < n) out[b0 + i] = ex;
    ex += v[i];
  }
  if (b0 <= n - 1 && n - 1 < b0 + 4) out[n] = ex;   // the thread holding the last value
}

__global__ __launch_bounds__(256) void k_plan_fill(const int32_t* __restrict__ list, const int32_t* __restrict__ count,
                                                   const int32_t* __restrict__ offsets, const int32_t* __restrict__ gstart,
                                                   const int32_t* __restrict__ rng, int nk, int NQ, int rows, int Gcap,
                                                   const int32_t* __restrict__ tbase, int32_t* __restrict__ plan) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int bh = row / NQ;
  const int cnt = min(max(count[row], 0), nk);
  const int32_t* lst = list + (size_t)row * nk;
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  const int32_t* gs = gstart + (size_t)bh * (nk + 1);
  const int32_t* rg = rng + (size_t)bh * nk;
  const int32_t* tb = tbase + (size_t)row * kRanges;
  int run[kRanges];   // groups placed so far in each range
#pragma unroll
  for (int j = 0; j < kRanges; ++j) run[j] = 0;
  // two chunks of 64 entries per pass, all of their loads in flight together (branch-free:
  // indices clamped, entries past the count or out of range count as empty)
  for (int i00 = 0; i00 < cnt; i00 += 128) {
    int vv[2], nn[2], gg[2], rr[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) vv[k] = lst[min(i00 + 64 * k + lane, nk - 1)];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bool ok = i00 + 64 * k + lane < cnt && vv[k] >= 0 && vv[k] < nk;
      const int v = ok ? vv[k] : 0;
      const int o0 = off[v], o1 = off[v + 1];
      gg[k] = gs[v];
      rr[k] = ok ? rg[v] : 0;
      nn[k] = ok ? o1 - o0 : 0;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i0 = i00 + 64 * k;
      if (i0 >= cnt) break;
      const int n = nn[k], g0 = gg[k], r = rr[k];
      const int ng = (n + 7) >> 3;
      int pos = 0;
#pragma unroll
      for (int j = 0; j < kRanges; ++j) {
        const int x = r == j ? ng : 0;
        int incl = x;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_up(incl, o);
          if (lane >= o) incl += t;
        }
        if (r == j) pos = run[j] + incl - x;
        run[j] += __shfl(incl, 63);
      }
      int32_t* pl = plan + (size_t)tb[r] * 4 + pos;
      for (int jj = 0; jj < ng; ++jj) pl[jj] = ((g0 + jj) << 4) | min(8, n - 8 * jj);
    }
  }
  // fill the tail of each range's last tile
  if (lane < kRanges) {
    int used = run[0];
#pragma unroll
    for (int j = 1; j < kRanges; ++j) used = lane == j ? run[j] : used;
    int32_t* pl = plan + (size_t)tb[lane] * 4;
    for (int j = used; j < 4 * (tb[lane + 1] - tb[lane]); ++j) pl[j] = Gcap << 4;
  }
}

// ---------------------------------------------------------------------------------------
// Step 4: attention over one item's tiles.  One wave per (head, query block, key range),
// holding all 64 queries of the block, so every K or V fragment it reads feeds two MFMAs:
//   S^T = K Q^T      (A: 32 keys x 16 columns in bf16; B: Q^T fragments of query halves 0 and
//                     1 in registers; the accumulators start at 0 / -inf, which masks padding)
//   O^T += V^T P^T   (A: V^T in bf16; B: P^T from the S^T accumulators, rounded to bf16)
// Keys and values are loaded from the packed groups straight into the MFMA operand registers
// (every lane loads exactly the 16 bytes it feeds to the matrix unit, one coalesced 1 KB piece
// per instruction), about one and a half tiles ahead of their use; no operand passes through
// LDS, which holds only a small table of score starts.
// Row swap inside each 16-row chunk of a tile (rows 4..7 <-> 8..11): with it, the 8 rows of
// S^T an MFMA lane holds for one 16-key chunk are 8 consecutive keys of one group, which is
// the P^T operand layout.
// Softmax: probabilities are taken against a per-query reference m, set to the row maximum
// of the first tile.  They are rounded to bf16 for the P V product; the sum of exactly those
// bf16 weights (v_dot2, accumulated in float) normalises O, and the float sum of the
// unrounded probabilities gives the log-sum-exp.  The reference only moves (with a rescale of
// the accumulators) when a lane's float sum for a tile leaves [0, 2^60]; the row maximum is
// then recovered from the probabilities themselves (m + log2 of the largest), and only if
// one overflowed float are the scores recomputed.  The partial state of the item is
// O_r = O^T / lb in fp16 (in units of the head's value unit, so |O_r| <= 1), and (m, l) with
// l the float sum.
__device__ __forceinline__ int sigma16(int x) { return (x & ~12) | ((x >> 1) & 4) | ((x << 1) & 8); }

// LDS of one wave: the score start table (row n: 0 for the first n slots of a group, -inf
// for its padding)
template <int D>
struct AttnLds {
  __attribute__((aligned(16))) float btab[9][8];
};

// One item: the partial softmax state of 64 queries over one key range's tiles.
template <int D, bool FUSED>
__device__ __forceinline__ void attn_item(const int item, AttnLds<D>& sm, const bf16* __restrict__ Q,
                                          const bf16* __restrict__ Kp, const bf16* __restrict__ Vp,
                                          const int32_t* __restrict__ plan, const int32_t* __restrict__ tbase,
                                          const float* __restrict__ vmax, int N, int NQ, int Gcap, float scale2,
                                          f16* __restrict__ Opart, float2* __restrict__ ML,
                                          const int4* __restrict__ chunks, const int32_t* __restrict__ ctotal,
                                          const int32_t* __restrict__ qperm, int maxc, bf16* __restrict__ Ofin,
                                          float* __restrict__ lse, int item0) {
  constexpr bool fused = FUSED;
  constexpr int KC = D / 16, DT = D / 32;
  constexpr uint32_t GB = 16 * D;   // bytes per packed group (K or V)
  static_assert(KC == 2 * DT, "K and V batches have the same size");
  auto& btab = sm.btab;
  // fused: the item is a whole row (all its ranges' tiles, which are contiguous in the plan),
  // so it writes the final output and log-sum-exp itself (no partial states, no merge)
  const int rr = fused ? 0 : item % kRanges;
  const int row = fused ? item : item / kRanges;
  const int lane = threadIdx.x, l32 = lane & 31, h = lane >> 5;
  // The item's queries: 64-token blocks (chunks == NULL): block u = item / kRanges of the
  // plan rows, tokens 64u + i.  Clustered query blocks: item / kRanges = (head, chunk slot);
  // chunk (u, p0, n) of block u holds positions p0 .. p0 + n - 1 of qperm, and the plan row
  // is block u's.
  int bh, prow, p0, nq;
  if (chunks) {
    const int cr = row;
    bh = cr / maxc;
    const int c = cr - bh * maxc;
    if (c >= ctotal[bh]) return;
    const int4 ch = chunks[(size_t)bh * maxc + c];
    prow = bh * NQ + ch.x;
    p0 = ch.y;
    nq = ch.z;
  } else {
    prow = row;
    bh = prow / NQ;
    p0 = 64 * (prow - bh * NQ);
    nq = min(64, N - p0);
  }
  const size_t hrow = (size_t)bh * N;
  // the head's largest |value| (the partial states' unit), loaded early: it is used at the end
  const float vmax_h = fused ? 0.0f : vmax[bh];
  // query index of position i < nq of the item
  auto query = [&](int i) __attribute__((always_inline)) {
    return qperm ? min(max(qperm[hrow + p0 + i], 0), N - 1) : p0 + i;
  };
  // Q^T fragments of query halves 0 and 1 in registers (qrow: this lane's query of each
  // half, -1 past the item's queries), issued before the item's tile range is read
  bf16x8 qf[2][KC];
  int qrow[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) qrow[h2] = 32 * h2 + l32 < nq ? query(32 * h2 + l32) : -1;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if (qrow[h2] >= 0) {
        qf[h2][kc] = load_bf16x8(Q + (hrow + qrow[h2]) * D + kc * 16 + 8 * h);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[h2][kc][i] = (bf16)0.0f;
      }
    }
  }

  PARK_ATTN_STAMP(clk_start);
  const int t0 = tbase[(size_t)prow * kRanges + rr];
  const int nt = tbase[(size_t)prow * kRanges + (fused ? kRanges : rr + 1)] - t0;
  if (nt <= 0) {
    if (lane < nq) {
      if constexpr (FUSED) {
        // no key selected: O = 0, lse = -inf
        bf16x8 z;
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
        bf16* orow = Ofin + (hrow + query(lane)) * D;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) *reinterpret_cast<bf16x8*>(orow + 8 * c) = z;
        if (lse) lse[hrow + query(lane)] = -INFINITY;
      } else {
        ML[(hrow + query(lane)) * kRanges + rr] = make_float2(-INFINITY, 0.0f);
      }
    }
    return;
  }
  const int32_t* pl = plan + (size_t)t0 * 4;
  const char* Kb = reinterpret_cast<const char*>(Kp + (size_t)bh * (Gcap + 1) * 8 * D);
  const char* Vb = reinterpret_cast<const char*>(Vp + (size_t)bh * (Gcap + 1) * 8 * D);
  // A row l32 of S^T is tile key kk: group kk / 8 of the tile, slot kk % 8
  const int kk = 16 * (l32 >> 4) + sigma16(l32 & 15);
  const int kj = kk >> 3;
  const uint32_t koff = (uint32_t)((kk & 7) * 32 + h * 16);
  const uint32_t voff = (uint32_t)(l32 * 16);

  // plan entries of tile t (clamped to the item, so loads past its last tile read that tile
  // again; they are never used): one 16-byte load with a uniform address, made uniform
  auto load_entries = [&](int t) __attribute__((always_inline)) {
    return *reinterpret_cast<const int4*>(pl + 4 * min(t, nt - 1));
  };
  auto uniform = [](const int4& e) __attribute__((always_inline)) {
    return make_int4(__builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y),
                     __builtin_amdgcn_readfirstlane(e.z), __builtin_amdgcn_readfirstlane(e.w));
  };
  auto entries = [&](int t) __attribute__((always_inline)) { return uniform(load_entries(t)); };
  // group ids are clamped to the head's packed groups: entries read from past an item's
  // plan (only ever used for unused loads) may hold anything
  auto key_offset = [&](const int4& e) __attribute__((always_inline)) {
    const int g01 = (kj & 1) ? e.y : e.x, g23 = (kj & 1) ? e.w : e.z;
    return (uint32_t)min((uint32_t)((kj & 2) ? g23 : g01) >> 4, (uint32_t)Gcap) * GB + koff;
  };
  // A operands of a tile straight from the packed groups into registers: the keys of S^T
  // (KC fragments) and the values of O^T (2 DT fragments).  Every lane loads exactly the 16
  // bytes of each fragment it feeds to the MFMA (one coalesced 1 KB piece per instruction),
  // so no operand passes through LDS.
  auto load_k = [&](const int4& e, bf16x8 (&kf)[KC]) __attribute__((always_inline)) {
    const char* src = Kb + key_offset(e);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) kf[kc] = *reinterpret_cast<const bf16x8*>(src + kc * 256);
  };
  auto load_v = [&](const int4& e, bf16x8 (&vf)[2 * DT]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int g = c ? (h ? e.w : e.z) : (h ? e.y : e.x);
      const char* src = Vb + min((uint32_t)g >> 4, (uint32_t)Gcap) * GB + voff;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vf[c * DT + dt] = *reinterpret_cast<const bf16x8*>(src + dt * 512);
    }
  };

  f32x16 oacc[2][DT];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[h2][dt][r] = 0.0f;
  // per lane and query half: reference m (log2 units), float sum of the probabilities (for
  // the log-sum-exp) and sum of the bf16 weights the P V product used (O normalisation)
  float m[2], lsum[2], lb[2];
  const float kBig = __builtin_amdgcn_ldexpf(1.0f, 60);
  const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};

  // Scores and probabilities share registers: sc holds S^T of a tile after its MFMAs and,
  // after the exponentials (taken in place), its probabilities.  The accumulators start at 0
  // for real keys and -inf for padding (lane element r < 8 is slot r of group h, element
  // 8 + r slot r of group 2 + h).
  f32x16 sc[2];
  auto init_scores = [&](const int4& e) __attribute__((always_inline)) {
    const int nva = (h ? e.y : e.x) & 15, nvb = (h ? e.w : e.z) & 15;
    const f32x4* b0 = reinterpret_cast<const f32x4*>(&btab[nva][0]);
    const f32x4* b1 = reinterpret_cast<const f32x4*>(&btab[nvb][0]);
    const f32x4 x0 = b0[0], x1 = b0[1], x2 = b1[0], x3 = b1[1];
    f32x16 init;
#pragma unroll
    for (int i = 0; i < 4; ++i) { init[i] = x0[i]; init[4 + i] = x1[i]; init[8 + i] = x2[i]; init[12 + i] = x3[i]; }
    return init;
  };
  // scores of tile t into out, from its key fragments kf
  auto scores_of = [&](const int4& e, const bf16x8 (&kf)[KC], f32x16 (&out)[2]) __attribute__((always_inline)) {
    out[0] = init_scores(e);
    out[1] = out[0];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      out[0] = mfma32(kf[kc], qf[0][kc], out[0]);
      out[1] = mfma32(kf[kc], qf[1][kc], out[1]);
    }
  };
  // scores of tile t read afresh from the packed groups (the rare rescale path)
  auto scores = [&](int t, f32x16 (&out)[2]) __attribute__((always_inline)) {
    const int4 e = entries(t);
    bf16x8 kf[KC];
    load_k(e, kf);
    scores_of(e, kf, out);
  };
  auto prob = [&](float x, int h2) __attribute__((always_inline)) { return fast_exp2(fmaf(x, scale2, -m[h2])); };
  // bf16 weights of the probabilities in sc
  auto to_bf16 = [&](bf16x8 (&pb)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[h2][c][i] = (bf16)sc[h2][8 * c + i];
  };
  auto weight_sums = [&](const bf16x8 (&pb)[2][2], float (&wb)[2], int h2) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x2 pair = {pb[h2][c][2 * i], pb[h2][c][2 * i + 1]};
        wb[h2] = __builtin_amdgcn_fdot2_f32_bf16(pair, one2, wb[h2], false);
      }
  };
  // Tile t's probabilities are in sc, their per-lane float sums in ps, their bf16 weights in pb
  // with sums wb.  Final unless a float sum left [0, 2^60]: then m moves to the row maximum
  // where that is larger (recovered from the probabilities, or from recomputed scores if one
  // overflowed), the accumulators are rescaled, and the tile's weights are rescaled with them.
  // Adds the tile to lsum and lb.
  auto settle = [&](int t, bf16x8 (&pb)[2][2], float (&ps)[2], float (&wb)[2]) __attribute__((always_inline)) {
    if (__builtin_expect(__any(!(ps[0] <= kBig) || !(ps[1] <= kBig)), 0)) {
      asm volatile("" ::: "memory");   // keep this rare path a branch (no if-conversion)
      float pmax[2];
      bool finite = true;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        float x = sc[h2][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) x = fmaxf(x, sc[h2][r]);
        pmax[h2] = fmaxf(x, __shfl_xor(x, 32));
        finite = finite && pmax[h2] <= 3.0e38f;
      }
      float mx[2];
      if (__all(finite)) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) mx[h2] = m[h2] + __log2f(pmax[h2]);
      } else {
        f32x16 st[2];
        scores(t, st);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          float x = st[h2][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) x = fmaxf(x, st[h2][r]);
          mx[h2] = fmaxf(x, __shfl_xor(x, 32)) * scale2;
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[h2][r] = fast_exp2(fmaf(st[h2][r], scale2, -mx[h2]));
        }
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const float mnew = fmaxf(m[h2], mx[h2]);
        const float alpha = fast_exp2(m[h2] - mnew);
        const float beta = __all(finite) ? alpha : fast_exp2(mx[h2] - mnew);
        lsum[h2] *= alpha;
        lb[h2] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[h2][dt][r] *= alpha;
        m[h2] = mnew;
        ps[h2] = 0.0f;
        wb[h2] = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[h2][r] *= beta;
          ps[h2] += sc[h2][r];
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int i = 0; i < 8; ++i) pb[h2][c][i] = (bf16)sc[h2][8 * c + i];
      }
      weight_sums(pb, wb, 0);
      weight_sums(pb, wb, 1);
    }
    lsum[0] += ps[0];
    lsum[1] += ps[1];
    lb[0] += wb[0];
    lb[1] += wb[1];
  };

  // Operand registers: the keys of tile t live in kbuf[t & 1], its values in vbuf[t & 1].
  // One pipeline step t (tile t + 1 exists) finds the keys of tiles t + 1 and t + 2 and the
  // values of tiles t and t + 1 loaded or in flight, tile t's bf16 weights settled in pb, and
  // in the order written (scheduling fences keep it; with one wave per SIMD the matrix and
  // vector units overlap only through this interleave):
  //   A1: S^T MFMAs of tile t + 1, query half 0;
  //   A2: S^T MFMAs of tile t + 1, query half 1, with the exponentials of half 0;
  //   then the loads of tile t + 3's keys into the buffer A just freed, and of the plan
  //   entries of tile t + 4;
  //   B:  P V MFMAs of tile t (O^T += V^T P^T) with the exponentials of half 1 and the bf16
  //       conversion and weight sums of half 0;
  //   then the loads of tile t + 2's values into the buffer B just freed, the conversion and
  //   sums of half 1 and the check of tile t + 1's weights (the rare rescale), leaving them
  //   settled in pb.
  // A key buffer is refilled about 1.4 steps before its use, a value buffer about 1.5 (the
  // compiler's memory counter waits cover exactly the loads each use needs).
  constexpr int kNPV = 4 * DT;             // P V MFMAs: 2 key chunks x DT x 2 query halves
  bf16x8 kbuf[2][KC], vbuf[2][2 * DT];
  bf16x8 pb[2][2];
  // uniform plan entries of tile t + 2 (values loaded in step t), the plan entries of tile
  // t + 3 in flight (made uniform in step t, for its keys) and the score start of tile t + 1
  int4 e2, pe3;
  f32x16 init;
  auto step = [&](auto par, int t) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;   // t & 1
    bf16x8 (&Kx)[KC] = kbuf[P ^ 1];           // tile t + 1
    bf16x8 (&Vx)[2 * DT] = vbuf[P];           // tile t
    __builtin_amdgcn_sched_barrier(0);
    // A1
    sc[0] = init;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      sc[0] = mfma32(Kx[kc], qf[0][kc], sc[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // A2: the 16 exponentials (and float sums) of half 0
    float acc[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
    sc[1] = init;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      sc[1] = mfma32(Kx[kc], qf[1][kc], sc[1]);
#pragma unroll
      for (int r = kc * 16 / KC; r < (kc + 1) * 16 / KC; ++r) {
        sc[0][r] = prob(sc[0][r], 0);
        acc[0][r & 1] += sc[0][r];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // keys of tile t + 3 into the buffer of tile t + 1, plan entries of tile t + 4
    const int4 e3 = uniform(pe3);
    load_k(e3, Kx);
    pe3 = load_entries(t + 4);
    __builtin_amdgcn_sched_barrier(0);
    // B: 16 exponentials (and sums) of half 1, then 8 conversions (pairs) and 8 weight sums of
    // half 0
    bf16x8 pn[2][2];
    float wn[2] = {0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < kNPV; ++j) {
      const int c = j / (2 * DT), dt = (j / 2) % DT, h2 = j & 1;
      oacc[h2][dt] = mfma32(Vx[c * DT + dt], pb[h2][c], oacc[h2][dt]);
#pragma unroll
      for (int w = j * 32 / kNPV; w < (j + 1) * 32 / kNPV; ++w) {
        if (w < 16) {
          sc[1][w] = prob(sc[1][w], 1);
          acc[1][w & 1] += sc[1][w];
        } else if (w < 24) {
          const int cc = (w - 16) >> 2, i = (w - 16) & 3;
          pn[0][cc][2 * i] = (bf16)sc[0][8 * cc + 2 * i];
          pn[0][cc][2 * i + 1] = (bf16)sc[0][8 * cc + 2 * i + 1];
        } else {
          const int cc = (w - 24) >> 2, i = (w - 24) & 3;
          const bf16x2 pair = {pn[0][cc][2 * i], pn[0][cc][2 * i + 1]};
          wn[0] = __builtin_amdgcn_fdot2_f32_bf16(pair, one2, wn[0], false);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // values of tile t + 2 into the buffer of tile t
    load_v(e2, Vx);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) pn[1][c][i] = (bf16)sc[1][8 * c + i];
    weight_sums(pn, wn, 1);
    float ps[2] = {acc[0][0] + acc[0][1], acc[1][0] + acc[1][1]};
    settle(t + 1, pn, ps, wn);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int c = 0; c < 2; ++c) pb[h2][c] = pn[h2][c];
    init = init_scores(e2);   // tile t + 2, the next step's score tile
    e2 = e3;
  };
  // the last tile t: P V
  auto last = [&](auto par, int t) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    const bf16x8 (&Vx)[2 * DT] = vbuf[P];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        oacc[0][dt] = mfma32(Vx[c * DT + dt], pb[0][c], oacc[0][dt]);
        oacc[1][dt] = mfma32(Vx[c * DT + dt], pb[1][c], oacc[1][dt]);
      }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  {
    const int4 e0 = entries(0), e1 = entries(1);
    e2 = entries(2);
    load_k(e0, kbuf[0]);
    load_v(e0, vbuf[0]);
    load_k(e1, kbuf[1]);
    load_v(e1, vbuf[1]);
    pe3 = load_entries(3);
    // tile 0: m starts at the row maximum of its scores (every tile holds a real key), so its
    // probabilities are at most 1 and need no check
    scores_of(e0, kbuf[0], sc);
    load_k(e2, kbuf[0]);
    init = init_scores(e1);
  }
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    float mx = sc[h2][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[h2][r]);
    m[h2] = fmaxf(mx, __shfl_xor(mx, 32)) * scale2;
    lsum[h2] = 0.0f;
    lb[h2] = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[h2][r] = prob(sc[h2][r], h2);
      lsum[h2] += sc[h2][r];
    }
  }
  to_bf16(pb);
  weight_sums(pb, lb, 0);
  weight_sums(pb, lb, 1);
  PARK_ATTN_STAMP(clk_loop);
  int t = 0;
  for (; t + 2 < nt; t += 2) {
    step(P0{}, t);
    step(P1{}, t + 1);
  }
  if (t + 1 < nt) {
    step(P0{}, t);
    last(P1{}, t + 1);
  } else {
    last(P0{}, t);
  }
  PARK_ATTN_STAMP(clk_tiles);

  if constexpr (FUSED) {
    // the whole row: O = O^T / lb in bf16, lse = ln 2 (m + log2 l) (what the merge gives for
    // a single live state)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const float l = lsum[h2] + __shfl_xor(lsum[h2], 32);
      const float lbs = lb[h2] + __shfl_xor(lb[h2], 32);
      if (qrow[h2] >= 0) {
        const float inv = lbs > 0.0f ? 1.0f / lbs : 0.0f;
        bf16* orow = Ofin + (hrow + qrow[h2]) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (bf16)(oacc[h2][dt][4 * g + i] * inv);
            *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * g + 4 * h) = o;
          }
        if (lse && h == 0) lse[hrow + qrow[h2]] = l > 0.0f ? (m[h2] + __log2f(l)) * kLn2 : -INFINITY;
      }
    }
    return;
  }
  // partial state: O_r = O^T / lb stored as fp16 in units of the head's value unit (so
  // |stored| <= 1), and (m, l) in float
  const float unit = value_unit(vmax_h);
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const float l = lsum[h2] + __shfl_xor(lsum[h2], 32);
    const float lbs = lb[h2] + __shfl_xor(lb[h2], 32);
    if (qrow[h2] >= 0) {
      const float inv = lbs > 0.0f ? 1.0f / (lbs * unit) : 0.0f;
      f16* orow = Opart + ((hrow + qrow[h2]) * kRanges + rr) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f16x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = (f16)(oacc[h2][dt][4 * g + i] * inv);
          *reinterpret_cast<f16x4*>(orow + 32 * dt + 8 * g + 4 * h) = o;
        }
      if (h == 0) ML[(hrow + qrow[h2]) * kRanges + rr] = make_float2(m[h2], l);
    }
  }
#ifdef PARK_ATTN_CLOCKS
  PARK_ATTN_STAMP(clk_end);
  if (lane == 0 && ((size_t)item0 + item) * 5 + 5 <= kAttnClockWords) {
    unsigned long long* o = attn_clock + ((size_t)item0 + item) * 5;
    o[0] = clk_start;
    o[1] = clk_loop;
    o[2] = clk_tiles;
    o[3] = clk_end;
    o[4] = ((unsigned long long)blockIdx.x << 32) | (unsigned)nt;
  }
#endif
}

// Persistent waves, one per workgroup: wave b starts with item b and then takes items of its
// key range r = b % kRanges (items of range r run on the XCDs x with x % kRanges == r:
// workgroups are dealt to the XCDs round robin and the grid size is a multiple of kRanges,
// and of 8 whenever there are enough items to fill the chip) from a per-range counter, in item
// order: items gridDim.x + r + kRanges k for k = 0, 1, ...  The next index is taken as an
// item starts and used when it ends.  A wave whose range is exhausted moves on to the next
// ranges' counters (the ranges' total work differs a little).  No wave waits for another, so
// every wave ends once it has found every counter past its last item, whatever the number of
// resident waves.  FUSED (clustered query blocks): the items are whole rows (all ranges),
// counter r hands out rows r per .. (r + 1) per - 1 (per = items / kRanges; indices past frows
// are skipped).
template <int D, bool FUSED>
__global__ __launch_bounds__(64) void k_attn_items(const bf16* __restrict__ Q, const bf16* __restrict__ Kp,
                                                   const bf16* __restrict__ Vp, const int32_t* __restrict__ plan,
                                                   const int32_t* __restrict__ tbase, const float* __restrict__ vmax,
                                                   int N, int NQ, int Gcap, float scale2, f16* __restrict__ Opart,
                                                   float2* __restrict__ ML, int items, int32_t* __restrict__ ictr,
                                                   const int4* __restrict__ chunks, const int32_t* __restrict__ ctotal,
                                                   const int32_t* __restrict__ qperm, int maxc, int frows,
                                                   bf16* __restrict__ Ofin, float* __restrict__ lse, int item0) {
  __shared__ AttnLds<D> sm;
  const int lane = threadIdx.x;
  for (int i = lane; i < 72; i += 64) sm.btab[i >> 3][i & 7] = (i & 7) < (i >> 3) ? 0.0f : -INFINITY;
  int xr = blockIdx.x % kRanges;
  int item = blockIdx.x;
  for (int moved = 0;;) {
    if (item >= items) {
      // this range is done: help the next ones (their keys are not in this XCD's L2, but only
      // the last items of the launch run this way)
      if (++moved >= kRanges) break;
      xr = (xr + 1) % kRanges;
      int k = 0;
      if (lane == 0) k = atomicAdd(&ictr[xr], 1);
      item = (int)gridDim.x + xr + kRanges * __builtin_amdgcn_readfirstlane(k);
      continue;
    }
    int nxt = 0;
    if (lane == 0) nxt = atomicAdd(&ictr[xr], 1);
    if constexpr (FUSED) {
      // fused rows: counter r walks rows [r per, (r + 1) per), so the rows of a head (and
      // the tiles they share) stay on one XCD
      const int per = items / kRanges;
      const int row = (item % kRanges) * per + item / kRanges;
      if (row < frows)
        attn_item<D, true>(row, sm, Q, Kp, Vp, plan, tbase, vmax, N, NQ, Gcap, scale2, Opart, ML, chunks, ctotal,
                           qperm, maxc, Ofin, lse, item0);
    } else {
      attn_item<D, false>(item, sm, Q, Kp, Vp, plan, tbase, vmax, N, NQ, Gcap, scale2, Opart, ML, chunks, ctotal,
                          qperm, maxc, Ofin, lse, item0);
    }
    item = (int)gridDim.x + xr + kRanges * __builtin_amdgcn_readfirstlane(nxt);
  }
}

// Step 5: merge the kRanges partial states of every query:
//   M = max_r m_r,  w_r = l_r 2^(m_r - M),  O = unit sum_r w_r O_r / sum_r w_r,
//   lse = ln 2 (M + log2 sum_r w_r).
// Ranges with l_r = 0 contribute nothing (their O_r is never read), and neither is O_r read
// when w_r < 2^-20 sum_r w_r: |O_r| <= 1, so skipping it moves O by at most 2^-20 unit, far
// below the bf16 output's resolution.  D / 8 threads per query, 8 columns each.
template <int D>
__global__ __launch_bounds__(256) void k_attn_merge(const f16* __restrict__ Opart, const float2* __restrict__ ML,
                                                    const float* __restrict__ vmax, int rows, int N,
                                                    bf16* __restrict__ O, float* __restrict__ lse) {
  constexpr int TPQ = D / 8;
  const int gt = blockIdx.x * 256 + threadIdx.x;
  const int q = gt / TPQ, part = gt % TPQ;
  if (q >= rows) return;
  const float vm = vmax[q / N];
  float2 st[kRanges];
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < kRanges; ++j) {
    st[j] = ML[(size_t)q * kRanges + j];
    if (st[j].y > 0.0f) M = fmaxf(M, st[j].x);
  }
  float w[kRanges], wsum = 0.0f;
#pragma unroll
  for (int j = 0; j < kRanges; ++j) {
    w[j] = st[j].y > 0.0f ? st[j].y * fast_exp2(st[j].x - M) : 0.0f;
    wsum += w[j];
  }
  const float cut = wsum * 0x1p-20f;
  // every range's piece loaded at once (branch-free): a skipped range reads the first piece of
  // the buffer instead (cached, so no memory traffic) and its value is discarded
  f16x8 o[kRanges];
#pragma unroll
  for (int j = 0; j < kRanges; ++j)
    o[j] = *reinterpret_cast<const f16x8*>(Opart + (w[j] > cut ? ((size_t)q * kRanges + j) * D + part * 8 : 0));
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < kRanges; ++j) {
    const bool use = w[j] > cut;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = use ? fmaf(w[j], (float)o[j][i], acc[i]) : acc[i];
  }
  const float scale = wsum > 0.0f ? value_unit(vm) / wsum : 0.0f;
  bf16x8 out;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = (bf16)(acc[i] * scale);
  *reinterpret_cast<bf16x8*>(O + (size_t)q * D + part * 8) = out;
  if (lse && part == 0) lse[q] = wsum > 0.0f ? (M + __log2f(wsum)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------------------
// float path: one workgroup of 128 threads per (query block, head); threads 0..63 each own
// one query; all threads stage 64-key tiles of K and V in LDS.  Float arithmetic throughout.
template <int D>
__global__ __launch_bounds__(128) void k_attn_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                  const float* __restrict__ V, const int32_t* __restrict__ perm,
                                                  const int32_t* __restrict__ offsets,
                                                  const int32_t* __restrict__ list,
                                                  const int32_t* __restrict__ count, int N, int nk, int NQ,
                                                  float scale2, float* __restrict__ O, float* __restrict__ lse,
                                                  const int4* __restrict__ chunks, const int32_t* __restrict__ ctotal,
                                                  const int32_t* __restrict__ qperm, int maxc) {
  __shared__ float Ks[64][D + 1];
  __shared__ float Vs[64][D + 1];
  __shared__ int pre[PARK_MAX_CLUSTERS + 1];
  __shared__ int kidx[64];
  __shared__ int wsum[2];
  const int bh = blockIdx.y, tid = threadIdx.x;
  // workgroup blockIdx.x: 64-token block u (chunks == NULL), or chunk (u, p0, n) of a
  // clustered query block (positions p0 .. p0 + n - 1 of qperm)
  int u, p0, nq;
  if (chunks) {
    if ((int)blockIdx.x >= ctotal[bh]) return;
    const int4 ch = chunks[(size_t)bh * maxc + blockIdx.x];
    u = ch.x;
    p0 = ch.y;
    nq = ch.z;
  } else {
    u = blockIdx.x;
    p0 = 64 * u;
    nq = min(64, N - p0);
  }
  const size_t row = (size_t)bh * NQ + u;
  const int cnt = min(max(count[row], 0), nk);
  const int32_t* lst = list + row * nk;
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  const int32_t* pm = perm + (size_t)bh * N;
  const int T = selected_prefix(lst, off, cnt, nk, pre, wsum);
  const bool active = tid < nq;
  const int qrow = !active ? 0 : qperm ? min(max(qperm[(size_t)bh * N + p0 + tid], 0), N - 1) : p0 + tid;
  float q[D], o[D];
#pragma unroll
  for (int a = 0; a < D; ++a) {
    q[a] = active ? Q[((size_t)bh * N + qrow) * D + a] : 0.0f;
    o[a] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  const int ntiles = (T + 63) / 64;
  for (int t = 0; t < ntiles; ++t) {
    if (tid < 64) {
      const int p = t * 64 + tid;
      kidx[tid] = p < T ? selected_key(p, pre, cnt, lst, off, pm) : -1;
    }
    __syncthreads();
    for (int e = tid; e < 64 * D; e += 128) {
      const int r = e / D, a = e % D;
      const int key = kidx[r];
      Ks[r][a] = key >= 0 ? K[((size_t)bh * N + key) * D + a] : 0.0f;
      Vs[r][a] = key >= 0 ? V[((size_t)bh * N + key) * D + a] : 0.0f;
    }
    __syncthreads();
    const int nv = min(64, T - t * 64);
    if (active) {
      for (int j = 0; j < nv; ++j) {
        float dot = 0.0f;
#pragma unroll
        for (int a = 0; a < D; ++a) dot = fmaf(q[a], Ks[j][a], dot);
        const float s = dot * scale2;
        const float mnew = fmaxf(m, s);
        const float alpha = exp2f(m - mnew);
        const float p = exp2f(s - mnew);
        l = l * alpha + p;
#pragma unroll
        for (int a = 0; a < D; ++a) o[a] = fmaf(o[a], alpha, p * Vs[j][a]);
        m = mnew;
      }
    }
    __syncthreads();
  }
  if (active) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int a = 0; a < D; ++a) O[((size_t)bh * N + qrow) * D + a] = o[a] * inv;
    if (lse) lse[(size_t)bh * N + qrow] = T > 0 ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

static inline int group_cap(const Shape& s) { return (s.N + 7) / 8 + s.nk; }

struct AttnWs {
  int32_t *gstart, *rng, *ntiles, *tbase, *bsum, *plan, *ictr;
  float* vmax;
  bf16 *Kp, *Vp;
  f16* Opart;
  float2* ML;
  int4* chunks;               // clustered query blocks only
  int32_t *cbase, *ctotal;
};

// Workspace layout; the float path needs only the chunk tables of clustered query blocks.
static AttnWs carve_attn(const Shape& s, const QueryBlocks* qb, void* base, size_t* total) {
  char* p = static_cast<char*>(base);
  auto take = [&](size_t bytes) { char* q = p; p += align256(bytes); return q; };
  AttnWs w{};
  if (qb) {
    const int maxc = chunk_slots(s.N, qb->NQ);
    w.chunks = reinterpret_cast<int4*>(take((size_t)s.BH * maxc * sizeof(int4)));
    w.cbase = reinterpret_cast<int32_t*>(take((size_t)s.BH * (qb->NQ + 1) * sizeof(int32_t)));
    w.ctotal = reinterpret_cast<int32_t*>(take((size_t)s.BH * sizeof(int32_t)));
  }
  if (s.dtype != 1) {
    if (total) *total = (size_t)(p - static_cast<char*>(base));
    return w;
  }
  // plan rows: one per query block
  const size_t rows = (size_t)s.BH * (qb ? qb->NQ : n_qblocks(s.N));
  const size_t items = rows * kRanges;
  const size_t kv = (size_t)s.BH * (group_cap(s) + 1) * 8 * s.d * sizeof(bf16);
  // plan entries of one query block: at most every group of its head, plus the filler of
  // one partial tile per range
  const size_t per_row = (size_t)group_cap(s) + 4 * kRanges;
  w.ntiles = reinterpret_cast<int32_t*>(take(items * sizeof(int32_t)));
  w.tbase = reinterpret_cast<int32_t*>(take((items + 1) * sizeof(int32_t)));
  w.bsum = reinterpret_cast<int32_t*>(take(((items + kScanBlock - 1) / kScanBlock) * sizeof(int32_t)));
  w.ictr = reinterpret_cast<int32_t*>(take(kRanges * sizeof(int32_t)));
  // (+ slack; the attention kernel reads plan entries clamped to each item's own tiles)
  w.plan = reinterpret_cast<int32_t*>(take((rows * per_row + 128) * sizeof(int32_t)));
  w.Kp = reinterpret_cast<bf16*>(take(kv));
  w.Vp = reinterpret_cast<bf16*>(take(kv));
  if (!qb) {   // clustered query blocks: whole-row items write O and lse themselves
    w.Opart = reinterpret_cast<f16*>(take((size_t)s.BH * s.N * kRanges * s.d * sizeof(f16)));
    w.ML = reinterpret_cast<float2*>(take((size_t)s.BH * s.N * kRanges * sizeof(float2)));
  }
  if (total) *total = (size_t)(p - static_cast<char*>(base));
  return w;
}

// compute units of the current device (read once per device)
static int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
  if (dev >= 0) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev >= 0) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Per-head tables computed once for all heads before the passes (bf16 only): each cluster's
// first packed group (gstart [BH][nk+1]), its key range (rng [BH][nk]) and the head's largest
// |value| (vmax [BH]).  They sit at the front of the workspace.
static size_t head_tabs_bytes(const Shape& s) {
  if (s.dtype != 1) return 0;
  return align256((size_t)s.BH * (s.nk + 1) * sizeof(int32_t)) + align256((size_t)s.BH * s.nk * sizeof(int32_t)) +
         align256((size_t)s.BH * sizeof(float));
}

// The call walks the heads in passes; the workspace holds one pass's packed keys and values,
// tile plan and partial states (every one of them per head), so a pass takes as many heads as
// fit in kAttnPassBytes (at least one), and the passes are balanced.  Each pass is the whole
// computation for its heads: heads are independent.
constexpr size_t kAttnPassBytes = size_t(5) << 29;   // 2.5 GiB

int attn_heads_per_pass(const Shape& s, const QueryBlocks* qb) {
  Shape one = s;
  one.BH = 1;
  size_t per = 0;
  carve_attn(one, qb, nullptr, &per);
  const long long fit = std::max<long long>(1, (long long)(kAttnPassBytes / std::max<size_t>(per, 1)));
  const long long passes = (s.BH + fit - 1) / fit;
  return (int)((s.BH + passes - 1) / passes);
}

int attn_passes(const Shape& s, const QueryBlocks* qb) {
  const int hpp = attn_heads_per_pass(s, qb);
  return (s.BH + hpp - 1) / hpp;
}

// (carve_attn of h heads is at most h times carve_attn of one head: each buffer is per head,
// rounded up to 256 bytes)
size_t attn_workspace(const Shape& s, const QueryBlocks* qb) {
  Shape sp = s;
  sp.BH = attn_heads_per_pass(s, qb);
  size_t total = 0;
  carve_attn(sp, qb, nullptr, &total);
  return head_tabs_bytes(s) + total;
}

// One pass: the heads of s (pointers already offset to the pass's first head); item0 = the
// first head's first item, for the clock-stamped build's record.
static hipError_t attn_pass(const Shape& s, const void* Q, const void* K, const void* V, const int32_t* perm,
                            const int32_t* offsets, const int32_t* list, const int32_t* count, float scale,
                            void* O, float* lse, void* ws, hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end,
                            const QueryBlocks* qb, int item0, int32_t* gstart, int32_t* rng, float* vmax) {
  // query blocks per head (plan rows) and chunk slots per head (clustered blocks)
  const int NQ = qb ? qb->NQ : n_qblocks(s.N);
  const int maxc = qb ? chunk_slots(s.N, qb->NQ) : 0;
  const float scale2 = scale * kLog2e;
  AttnWs w = carve_attn(s, qb, ws, nullptr);
  w.gstart = gstart;   // (the pass's heads of the per-head tables)
  w.rng = rng;
  w.vmax = vmax;
  const int32_t* qperm = qb ? qb->qperm : nullptr;
  if (qb) {
    hipError_t e = launch_qchunks(qb->qoffsets, s.BH, s.N, NQ, maxc, w.chunks, w.cbase, w.ctotal, st);
    if (e != hipSuccess) return e;
  }
  if (s.dtype == 1) {
    const int Gcap = group_cap(s);
    const int rows = s.BH * NQ;
    const int items = rows * kRanges;
    // attention items: (plan row, range); for clustered blocks whole (head, chunk slot) rows
    // over all ranges (their selections are small: split into ranges, items would hold a
    // few tiles each), kRanges ceil(rows / kRanges) of them
    const long long frows = qb ? (long long)s.BH * maxc : 0;
    const long long aitems = qb ? (frows + kRanges - 1) / kRanges * kRanges : (long long)items;
    if (aitems >= (1LL << 31)) return hipErrorInvalidValue;
    auto k = reinterpret_cast<const bf16*>(K);
    auto v = reinterpret_cast<const bf16*>(V);
    auto q = reinterpret_cast<const bf16*>(Q);
    auto o = reinterpret_cast<bf16*>(O);
    hipError_t e;
#define PARK_CHECK() do { e = hipGetLastError(); if (e != hipSuccess) return e; } while (0)
    dim3 pgrid(s.nk, s.BH);
    if (s.d == 128) k_pack_kv<128><<<pgrid, 128, 0, st>>>(k, v, perm, offsets, w.gstart, s.N, s.nk, Gcap, w.Kp, w.Vp, w.vmax);
    else k_pack_kv<64><<<pgrid, 128, 0, st>>>(k, v, perm, offsets, w.gstart, s.N, s.nk, Gcap, w.Kp, w.Vp, w.vmax);
    PARK_CHECK();
    k_plan_count<<<(rows + 3) / 4, 256, 0, st>>>(list, count, offsets, w.rng, s.nk, NQ, rows, w.ntiles);
    PARK_CHECK();
    const int nb = (items + kScanBlock - 1) / kScanBlock;
    k_scan_blocks<<<nb, 1024, 0, st>>>(w.ntiles, items, w.bsum);
    PARK_CHECK();
    k_scan_top<<<1, 1024, 0, st>>>(w.bsum, nb, w.ictr);
    PARK_CHECK();
    k_scan_final<<<nb, 1024, 0, st>>>(w.ntiles, items, w.bsum, w.tbase);
    PARK_CHECK();
    k_plan_fill<<<(rows + 3) / 4, 256, 0, st>>>(list, count, offsets, w.gstart, w.rng, s.nk, NQ, rows, Gcap,
                                                 w.tbase, w.plan);
    PARK_CHECK();
    if (ev_begin && (e = hipEventRecord(ev_begin, st)) != hipSuccess) return e;
    // persistent waves: as many as the chip holds (one per SIMD, bound by the registers), a
    // multiple of kRanges (items is one)
    const int waves = (int)std::min<long long>(aitems, 4 * compute_units() / kRanges * kRanges);
#define PARK_ITEMS(DD, FF)                                                                                  \
  k_attn_items<DD, FF><<<waves, 64, 0, st>>>(q, w.Kp, w.Vp, w.plan, w.tbase, w.vmax, s.N, NQ, Gcap, scale2, w.Opart, \
                                             w.ML, (int)aitems, w.ictr, w.chunks, w.ctotal, qperm, maxc, (int)frows, o, lse, \
                                             item0)
    if (s.d == 128) {
      if (qb) PARK_ITEMS(128, true); else PARK_ITEMS(128, false);
    } else {
      if (qb) PARK_ITEMS(64, true); else PARK_ITEMS(64, false);
    }
#undef PARK_ITEMS
    PARK_CHECK();
    if (ev_end && (e = hipEventRecord(ev_end, st)) != hipSuccess) return e;
    if (!qb) {   // clustered blocks: the fused rows wrote O and lse themselves
      const int total_rows = s.BH * s.N;
      const long long mthreads = (long long)total_rows * (s.d / 8);
      const unsigned mblocks = (unsigned)((mthreads + 255) / 256);
      if (s.d == 128) k_attn_merge<128><<<mblocks, 256, 0, st>>>(w.Opart, w.ML, w.vmax, total_rows, s.N, o, lse);
      else k_attn_merge<64><<<mblocks, 256, 0, st>>>(w.Opart, w.ML, w.vmax, total_rows, s.N, o, lse);
      PARK_CHECK();
    }
#undef PARK_CHECK
  } else {
    dim3 grid(qb ? maxc : NQ, s.BH);
    auto q = reinterpret_cast<const float*>(Q);
    auto k = reinterpret_cast<const float*>(K);
    auto v = reinterpret_cast<const float*>(V);
    auto o = reinterpret_cast<float*>(O);
    if (s.d == 128)
      k_attn_f32<128><<<grid, 128, 0, st>>>(q, k, v, perm, offsets, list, count, s.N, s.nk, NQ, scale2, o, lse,
                                            w.chunks, w.ctotal, qperm, maxc);
    else
      k_attn_f32<64><<<grid, 128, 0, st>>>(q, k, v, perm, offsets, list, count, s.N, s.nk, NQ, scale2, o, lse,
                                           w.chunks, w.ctotal, qperm, maxc);
  }
  return hipGetLastError();
}

hipError_t launch_attn(const Shape& s, const void* Q, const void* K, const void* V, const int32_t* perm,
                       const int32_t* offsets, const int32_t* list, const int32_t* count, float scale,
                       void* O, float* lse, void* ws, hipStream_t st, const hipEvent_t* ev_begin,
                       const hipEvent_t* ev_end, int n_events, const QueryBlocks* qb) {
  const int hpp = attn_heads_per_pass(s, qb);
  const int NQ = qb ? qb->NQ : n_qblocks(s.N);
  const size_t esz = s.dtype == 1 ? 2 : 4, N = s.N, d = s.d;
  // the per-head tables of every head, then the passes' workspace
  char* const tabs = static_cast<char*>(ws);
  int32_t* const gstart = reinterpret_cast<int32_t*>(tabs);
  int32_t* const rng = reinterpret_cast<int32_t*>(tabs + align256((size_t)s.BH * (s.nk + 1) * sizeof(int32_t)));
  float* const vmax = reinterpret_cast<float*>(tabs + align256((size_t)s.BH * (s.nk + 1) * sizeof(int32_t)) +
                                               align256((size_t)s.BH * s.nk * sizeof(int32_t)));
  void* const pws = tabs + head_tabs_bytes(s);
  if (s.dtype == 1) {
    // each cluster's first packed group and the head's |value| maximum (reset here, raised by
    // the packing), and the clusters' key ranges, for all heads at once
    k_group_scan<<<s.BH, 256, 0, st>>>(offsets, s.nk, gstart, vmax);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_range_assign<<<s.BH, 1024, 0, st>>>(list, count, offsets, s.nk, NQ, rng);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  for (int h0 = 0, p = 0; h0 < s.BH; h0 += hpp, ++p) {
    Shape sp = s;
    sp.BH = std::min(hpp, s.BH - h0);
    const size_t tok = (size_t)h0 * N;
    QueryBlocks qp{};
    if (qb) qp = QueryBlocks{qb->qperm + tok, qb->qoffsets + (size_t)h0 * (NQ + 1), NQ};
    const hipError_t e = attn_pass(
        sp, static_cast<const char*>(Q) + tok * d * esz, static_cast<const char*>(K) + tok * d * esz,
        static_cast<const char*>(V) + tok * d * esz, perm + tok, offsets + (size_t)h0 * (s.nk + 1),
        list + (size_t)h0 * NQ * s.nk, count + (size_t)h0 * NQ, scale, static_cast<char*>(O) + tok * d * esz,
        lse ? lse + tok : nullptr, pws, st, ev_begin && p < n_events ? ev_begin[p] : nullptr,
        ev_end && p < n_events ? ev_end[p] : nullptr, qb ? &qp : nullptr,
        (int)std::min<long long>((long long)h0 * NQ * kRanges, INT_MAX), gstart + (size_t)h0 * (s.nk + 1),
        rng + (size_t)h0 * s.nk, vmax + h0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------------------
// Exact block importance (section 3.2, Eq. (3)), a retrieval-accuracy diagnostic:
//   W_uv = (1/n_u) sum_{i in block u} sum_{j in cluster v} softmax_j(scale q_i . k_j),
// softmax over all N keys.  The attention kernel computes it: with values V_j = the one-hot
// vector of key j's cluster (restricted to a chunk of d clusters) and every key selected, O_i
// is query i's attention mass on each cluster of the chunk.  Dense attention is the selection
// of nk_dense runs of consecutive keys (identity permutation), so every key range has work.
constexpr int kDenseRuns = 64;

// lab[bh][perm[p]] = v for the positions p of cluster v
__global__ __launch_bounds__(256) void k_key_labels(const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
                                                    int N, int nk, int32_t* __restrict__ lab) {
  const int v = blockIdx.x, bh = blockIdx.y;
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  const int a = min(max(off[v], 0), N), b = min(max(off[v + 1], a), N);
  for (int p = a + (int)threadIdx.x; p < b; p += 256) {
    const int j = perm[(size_t)bh * N + p];
    if (j >= 0 && j < N) lab[(size_t)bh * N + j] = v;
  }
}

// identity permutation, kDenseRuns runs of consecutive keys, every run listed for every block
__global__ __launch_bounds__(256) void k_dense_lists(int N, int NQ, int runs, int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ list,
                                                     int32_t* __restrict__ count) {
  const int bh = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < N) perm[(size_t)bh * N + t] = t;
  if (t <= runs) offsets[(size_t)bh * (runs + 1) + t] = (int)(((long long)t * N) / runs);
  if (t < NQ * runs) list[(size_t)bh * NQ * runs + t] = t % runs;
  if (t < NQ) count[(size_t)bh * NQ + t] = runs;
}

// V[bh][j][a] = 1 if key j is in cluster c0 + a, else 0
template <typename T>
__global__ __launch_bounds__(256) void k_onehot(const int32_t* __restrict__ lab, int N, int d, int c0,
                                                T* __restrict__ V) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)N * d) return;
  const size_t bhj = (size_t)blockIdx.y * N + e / d;
  const int a = (int)(e % d);
  V[bhj * d + a] = (T)(lab[bhj] == c0 + a ? 1.0f : 0.0f);
}

__global__ __launch_bounds__(256) void k_fill_i32(int32_t* __restrict__ x, size_t n, int v) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n) x[e] = v;
}

// W[bh][u][c0 + a] = mean over block u's rows of O[bh][i][a], for a < min(d, nk - c0)
template <typename T>
__global__ __launch_bounds__(128) void k_block_mean(const T* __restrict__ O, int N, int d, int nk, int c0, int NQ,
                                                    float* __restrict__ W) {
  const int u = blockIdx.x, bh = blockIdx.y, a = threadIdx.x;
  if (a >= d || c0 + a >= nk) return;
  const int i0 = 64 * u, i1 = min(N, i0 + 64);
  float acc = 0.0f;
  for (int i = i0; i < i1; ++i) acc += to_f32(O[((size_t)bh * N + i) * d + a]);
  W[((size_t)bh * NQ + u) * nk + c0 + a] = acc / (float)(i1 - i0);
}

size_t importance_workspace(const Shape& s) {
  const size_t BH = s.BH, N = s.N, NQ = n_qblocks(s.N), esz = s.dtype == 1 ? 2 : 4;
  Shape sd = s;
  sd.nk = kDenseRuns < s.N ? kDenseRuns : s.N;
  size_t b = 0;
  b += align256(BH * N * 4) * 2;                            // labels, identity permutation
  b += align256(BH * (sd.nk + 1) * 4);                      // run offsets
  b += align256(BH * NQ * sd.nk * 4) + align256(BH * NQ * 4);  // lists, counts
  b += align256(BH * N * s.d * esz) * 2;                    // one-hot values, outputs
  b += attn_workspace(sd);
  return b;
}

hipError_t launch_importance(const Shape& s, const void* Q, const void* K, const int32_t* perm,
                             const int32_t* offsets, float scale, float* W, void* ws, hipStream_t st) {
  const int N = s.N, NQ = n_qblocks(N), d = s.d;
  const size_t BH = s.BH, esz = s.dtype == 1 ? 2 : 4;
  Shape sd = s;
  sd.nk = kDenseRuns < N ? kDenseRuns : N;
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t bytes) { char* q = p; p += align256(bytes); return q; };
  int32_t* lab = reinterpret_cast<int32_t*>(take(BH * N * 4));
  int32_t* pid = reinterpret_cast<int32_t*>(take(BH * N * 4));
  int32_t* offd = reinterpret_cast<int32_t*>(take(BH * (sd.nk + 1) * 4));
  int32_t* lst = reinterpret_cast<int32_t*>(take(BH * NQ * sd.nk * 4));
  int32_t* cnt = reinterpret_cast<int32_t*>(take(BH * NQ * 4));
  void* V = take(BH * N * d * esz);
  void* O = take(BH * N * d * esz);
  void* aws = p;
  hipError_t e;
  k_dense_lists<<<dim3((unsigned)((std::max<long long>((long long)N, (long long)NQ * sd.nk) + 256) / 256), s.BH),
                  256, 0, st>>>(N, NQ, sd.nk, pid, offd, lst, cnt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // keys of no cluster (inconsistent perm) keep label -1
  k_fill_i32<<<dim3((unsigned)((BH * N + 255) / 256)), 256, 0, st>>>(lab, BH * N, -1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_key_labels<<<dim3(s.nk, s.BH), 256, 0, st>>>(perm, offsets, N, s.nk, lab);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int c0 = 0; c0 < s.nk; c0 += d) {
    const dim3 og((unsigned)(((size_t)N * d + 255) / 256), s.BH);
    if (s.dtype == 1) k_onehot<bf16><<<og, 256, 0, st>>>(lab, N, d, c0, static_cast<bf16*>(V));
    else k_onehot<float><<<og, 256, 0, st>>>(lab, N, d, c0, static_cast<float*>(V));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_attn(sd, Q, K, V, pid, offd, lst, cnt, scale, O, nullptr, aws, st)) != hipSuccess) return e;
    if (s.dtype == 1) k_block_mean<bf16><<<dim3(NQ, s.BH), 128, 0, st>>>(static_cast<const bf16*>(O), N, d, s.nk, c0, NQ, W);
    else k_block_mean<float><<<dim3(NQ, s.BH), 128, 0, st>>>(static_cast<const float*>(O), N, d, s.nk, c0, NQ, W);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------------------
// Centred log-mass error (appendix B, M2; section 4.2), a retrieval-accuracy diagnostic:
//   S*_iv = log sum_{j in cluster v} exp(scale q_i . k_j),   S_iv = log n_v + scale q_i . c_v,
//   D_iv = S*_iv - S_iv over the non-empty clusters, centred per query (minus its mean over v);
//   RMSE over all (i, v) of the centred D.
// One wave per (64-query block, head) walks every cluster's keys through perm in 32-key tiles:
// S^T = K Q^T by MFMA (bf16 products exact, float sums), a lane holds 16 of a tile's keys for
// its query and the swap with lane l ^ 32 completes the tile's log-sum-exp, which is folded
// into the cluster's.  q . c_v in float (each lane half takes 64 of the d columns).  Per block:
// (sum over queries of the centred sum of squares, number of (i, v) pairs) in double.
template <int D>
__global__ __launch_bounds__(64) void k_logmass(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                                const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
                                                const float* __restrict__ cent, const int32_t* __restrict__ counts,
                                                int N, int nk, float scale, double2* __restrict__ stats) {
  constexpr int KC = D / 16;
  const int u = blockIdx.x, bh = blockIdx.y, NQ = gridDim.x;
  const int lane = threadIdx.x, l32 = lane & 31, h = lane >> 5;
  const size_t hrow = (size_t)bh * N;
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  const int32_t* pm = perm + hrow;
  bf16x8 qf[2][KC];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int qrow = 64 * u + 32 * h2 + l32;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if (qrow < N) {
        qf[h2][kc] = load_bf16x8(Q + (hrow + qrow) * D + kc * 16 + 8 * h);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[h2][kc][i] = (bf16)0.0f;
      }
    }
  }
  double sd[2] = {0.0, 0.0}, sd2[2] = {0.0, 0.0};
  int pairs = 0;
  for (int v = 0; v < nk; ++v) {
    const int a = min(max(off[v], 0), N), b = min(max(off[v + 1], a), N);
    const int n = counts[(size_t)bh * nk + v];
    if (b <= a || n <= 0) continue;
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.0f, 0.0f};   // running log-sum-exp of cluster v
    for (int p0 = a; p0 < b; p0 += 32) {
      const int p = p0 + l32;
      bf16x8 kf[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if (p < b) {
          kf[kc] = load_bf16x8(K + (hrow + min(max(pm[p], 0), N - 1)) * D + kc * 16 + 8 * h);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) kf[kc][i] = (bf16)0.0f;
        }
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) acc = mfma32(kf[kc], qf[h2][kc], acc);
        // this lane's keys of the tile: rows c_row(r, lane)
        float tm = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (p0 + c_row(r, lane) < b) tm = fmaxf(tm, acc[r] * scale);
        float ts = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (p0 + c_row(r, lane) < b) ts += __expf(acc[r] * scale - tm);
        // the other 16 keys sit in lane l ^ 32
        const float om = __shfl_xor(tm, 32), os = __shfl_xor(ts, 32);
        const float mm = fmaxf(fmaxf(tm, om), m[h2]);
        l[h2] = (m[h2] == -INFINITY ? 0.0f : l[h2] * __expf(m[h2] - mm)) +
                (tm == -INFINITY ? 0.0f : ts * __expf(tm - mm)) + (om == -INFINITY ? 0.0f : os * __expf(om - mm));
        m[h2] = mm;
      }
    }
    // S_iv = log n_v + scale q_i . c_v (this lane half's 64 columns, then the swap)
    const float* c = cent + ((size_t)bh * nk + v) * D;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      float dot = 0.0f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int i = 0; i < 8; ++i) dot = fmaf((float)qf[h2][kc][i], c[kc * 16 + 8 * h + i], dot);
      dot += __shfl_xor(dot, 32);
      const double dlt = ((double)m[h2] + log((double)l[h2])) - (log((double)n) + (double)scale * (double)dot);
      sd[h2] += dlt;
      sd2[h2] += dlt * dlt;
    }
    ++pairs;
  }
  // per query: sum over v of (D - mean D)^2 = sum D^2 - (sum D)^2 / pairs; lanes of half h = 0
  // hold each query once
  double ss = 0.0;
  int np = 0;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int qrow = 64 * u + 32 * h2 + l32;
    if (h == 0 && qrow < N && pairs > 0) {
      ss += fmax(sd2[h2] - sd[h2] * sd[h2] / pairs, 0.0);
      np += pairs;
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    ss += __shfl_xor(ss, o);
    np += __shfl_xor(np, o);
  }
  if (lane == 0) stats[(size_t)bh * NQ + u] = make_double2(ss, (double)np);
}

// rmse[bh] = sqrt(sum of the blocks' centred squares / their pairs)
__global__ void k_logmass_rmse(const double2* __restrict__ stats, int BH, int NQ, float* __restrict__ rmse) {
  const int bh = blockIdx.x * blockDim.x + threadIdx.x;
  if (bh >= BH) return;
  double s = 0.0, n = 0.0;
  for (int u = 0; u < NQ; ++u) {
    s += stats[(size_t)bh * NQ + u].x;
    n += stats[(size_t)bh * NQ + u].y;
  }
  rmse[bh] = n > 0.0 ? (float)sqrt(s / n) : 0.0f;
}

size_t logmass_workspace(const Shape& s) { return align256((size_t)s.BH * n_qblocks(s.N) * sizeof(double2)); }

hipError_t launch_logmass(const Shape& s, const void* Q, const void* K, const int32_t* perm, const int32_t* offsets,
                          const float* cent, const int32_t* counts, float scale, float* rmse, void* ws,
                          hipStream_t st) {
  if (s.dtype != 1) return hipErrorInvalidValue;
  const int NQ = n_qblocks(s.N);
  double2* stats = static_cast<double2*>(ws);
  auto q = static_cast<const bf16*>(Q);
  auto k = static_cast<const bf16*>(K);
  if (s.d == 128) k_logmass<128><<<dim3(NQ, s.BH), 64, 0, st>>>(q, k, perm, offsets, cent, counts, s.N, s.nk, scale, stats);
  else k_logmass<64><<<dim3(NQ, s.BH), 64, 0, st>>>(q, k, perm, offsets, cent, counts, s.N, s.nk, scale, stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_logmass_rmse<<<(s.BH + 63) / 64, 64, 0, st>>>(stats, s.BH, NQ, rmse);
  return hipGetLastError();
}

}  // namespace park

#ifdef PARK_ATTN_CLOCKS
extern "C" __attribute__((visibility("default"))) size_t park_attn_clock_words(void) {
  return park::kAttnClockWords;
}
extern "C" __attribute__((visibility("default"))) int park_attn_clock_read(void* host, size_t words) {
  if (!host || words > park::kAttnClockWords) return PARK_ERR_INVALID;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(park::attn_clock), words * sizeof(unsigned long long), 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? PARK_OK : PARK_ERR_HIP;
}
#endif
