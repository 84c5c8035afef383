// Block-sparse attention (PARK section 3.1, E1/E2 with the softmax renormalised over the
// selected keys): every query block walks the concatenation of its selected key clusters,
// cut into 64-key tiles (only the last tile of a block is partial), gathering keys and
// values through the cluster permutation.
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
// bf16 path, step 1: pack the keys and values of every cluster, in cluster order, into
// 8-key groups (a cluster of n keys takes ceil(n / 8) groups; the tail of its last group is
// zero padding).  Kp[g] is 8 key rows of D; Vp[g] is the same 8 values transposed, D rows
// of 8 keys, which is the operand layout of the P V product.  gstart[v] is the first group
// of cluster v (exclusive scan of ceil(n_v / 8)).
__global__ __launch_bounds__(256) void k_group_scan(const int32_t* __restrict__ offsets, int nk,
                                                    int32_t* __restrict__ gstart) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, bh = blockIdx.x;
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

template <int D>
__global__ __launch_bounds__(128) void k_pack_kv(const bf16* __restrict__ K, const bf16* __restrict__ V,
                                                 const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ gstart, int N, int nk, int Gcap,
                                                 bf16* __restrict__ Kp, bf16* __restrict__ Vp) {
  constexpr int NS = D / 8;
  const int v = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  const int a = off[v], n = off[v + 1] - a;
  const int ng = (n + 7) >> 3;
  const int g0 = gstart[(size_t)bh * (nk + 1) + v];
  const int32_t* pm = perm + (size_t)bh * N + a;
  const bf16* Kh = K + (size_t)bh * N * D;
  const bf16* Vh = V + (size_t)bh * N * D;
  bf16* Kph = Kp + ((size_t)bh * Gcap + g0) * 8 * D;
  bf16* Vph = Vp + ((size_t)bh * Gcap + g0) * 8 * D;
  for (int e = tid; e < ng * 8 * NS; e += 128) {
    const int slot = e / NS, sg = e % NS;
    bf16x8 val;
    if (slot < n) {
      val = load_bf16x8(Kh + (size_t)pm[slot] * D + sg * 8);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) val[i] = (bf16)0.0f;
    }
    *reinterpret_cast<bf16x8*>(Kph + (size_t)slot * D + sg * 8) = val;
  }
  for (int e = tid; e < ng * NS; e += 128) {
    const int j = e / NS, sg = e % NS;
    bf16x8 rows[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slot = 8 * j + i;
      if (slot < n) {
        rows[i] = load_bf16x8(Vh + (size_t)pm[slot] * D + sg * 8);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) rows[i][t] = (bf16)0.0f;
      }
    }
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      bf16x8 col;
#pragma unroll
      for (int i = 0; i < 8; ++i) col[i] = rows[i][dd];
      *reinterpret_cast<bf16x8*>(Vph + (size_t)j * 8 * D + (size_t)(sg * 8 + dd) * 8) = col;
    }
  }
}

// Row swap inside each 16-row chunk (rows 4..7 <-> 8..11): with it, the 8 rows of S^T that
// an MFMA lane holds for one 16-key chunk are 8 consecutive keys, so the matching V^T
// operand is one 16-byte read.
__device__ __forceinline__ int sigma16(int x) { return (x & ~12) | ((x >> 1) & 4) | ((x << 1) & 8); }

// bf16 path, step 2.  One workgroup (4 waves) per (query block, head).  Wave w = 2 kw + qw
// owns queries 32 qw .. 32 qw + 31 of the block and keys 32 kw .. 32 kw + 31 of every
// 64-key tile (8 groups); each wave keeps its own online-softmax state and the two key
// halves are merged at the end.  Tiles are double-buffered in LDS: the loads of tile t+1
// are issued before the MFMA work on tile t.
//   S^T = K Q^T  (A: K rows from LDS in sigma16 order, B: Q^T fragments in registers)
//   O^T += V^T P^T  (A: V^T rows from LDS, B: P^T straight from the S^T accumulators)
template <int D>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(const bf16* __restrict__ Q, const bf16* __restrict__ Kp,
                                                      const bf16* __restrict__ Vp, const int32_t* __restrict__ gstart,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ list,
                                                      const int32_t* __restrict__ count, int N, int nk, int NQ,
                                                      int Gcap, float scale2, bf16* __restrict__ O,
                                                      float* __restrict__ lse) {
  constexpr int KP = D + 8;
  constexpr int VP = 64 + 8;
  constexpr int NS = D / 8;
  constexpr int KCH = 64 * NS / 256;  // 16-byte K chunks per thread per tile
  constexpr int VCH = 8 * D / 256;    // 16-byte V chunks per thread per tile
  __shared__ bf16 Ks[2][64 * KP];
  __shared__ bf16 Vt[2][D * VP];
  __shared__ int pre[PARK_MAX_CLUSTERS + 1];
  __shared__ int tgrp[3][8];
  __shared__ int tval[3][8];
  __shared__ int wsum[4];

  const uint32_t lb = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lb / NQ, u = lb % NQ;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int qw = w & 1, kw = w >> 1;
  const size_t row = (size_t)bh * NQ + u;
  const int cnt = min(max(count[row], 0), nk);
  const int32_t* lst = list + row * nk;
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  const int32_t* gst = gstart + (size_t)bh * (nk + 1);
  const bf16* Kph = Kp + (size_t)bh * Gcap * 8 * D;
  const bf16* Vph = Vp + (size_t)bh * Gcap * 8 * D;

  // prefix of the group counts of the selected clusters (ids outside [0, nk) count as empty)
  auto csize = [&](int i) {
    const int v = lst[i];
    return (v >= 0 && v < nk) ? off[v + 1] - off[v] : 0;
  };
  int TG;
  {
    const int per = (cnt + 255) / 256;
    const int b0 = min(tid * per, cnt), b1 = min(b0 + per, cnt);
    int s = 0;
    for (int i = b0; i < b1; ++i) s += (csize(i) + 7) >> 3;
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
    for (int i = b0; i < b1; ++i) {
      pre[i] = ex;
      ex += (csize(i) + 7) >> 3;
    }
    TG = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (tid == 0) pre[cnt] = TG;
    __syncthreads();
  }
  const int ntiles = (TG + 7) >> 3;

  // group ids and valid-key counts of tile t into ring slot t % 3 (threads 0..7)
  auto tile_info = [&](int t) {
    if (tid < 8) {
      const int j = 8 * t + tid;
      int g = -1, nv = 0;
      if (j < TG) {
        int lo = 0, hi = cnt - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (pre[mid] <= j) lo = mid; else hi = mid - 1;
        }
        const int jj = j - pre[lo];
        const int v = lst[lo];          // non-empty, hence a valid id
        g = gst[v] + jj;
        nv = min(8, off[v + 1] - off[v] - 8 * jj);
      }
      tgrp[t % 3][tid] = g;
      tval[t % 3][tid] = nv;
    }
  };

  bf16x8 kreg[KCH], vreg[VCH];
  auto load_tile = [&](int t) {
    const int sl = t % 3;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int e = tid + 256 * c;          // 0 .. 64*NS-1
      const int gi = e / (8 * NS);          // group within the tile
      const int g = tgrp[sl][gi];
      if (g >= 0) {
        kreg[c] = load_bf16x8(Kph + (size_t)g * 8 * D + (e % (8 * NS)) * 8);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) kreg[c][i] = (bf16)0.0f;
      }
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int e = tid + 256 * c;          // 0 .. 8*D-1
      const int gi = e / D, d = e % D;
      const int g = tgrp[sl][gi];
      if (g >= 0) {
        vreg[c] = load_bf16x8(Vph + (size_t)g * 8 * D + (size_t)d * 8);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) vreg[c][i] = (bf16)0.0f;
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int e = tid + 256 * c;
      const int r = e / NS, sg = e % NS;    // key slot (group-major) and segment
      *reinterpret_cast<bf16x8*>(&Ks[buf][r * KP + sg * 8]) = kreg[c];
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int e = tid + 256 * c;
      const int gi = e / D, d = e % D;
      *reinterpret_cast<bf16x8*>(&Vt[buf][d * VP + 8 * gi]) = vreg[c];
    }
  };

  const int qrow = 64 * u + 32 * qw + l32;
  const bool qvalid = qrow < N;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    if (qvalid) {
      qf[kc] = load_bf16x8(Q + ((size_t)bh * N + qrow) * D + kc * 16 + 8 * h);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[kc][i] = (bf16)0.0f;
    }
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
  constexpr float kNoMax = -1e30f;
  float m = kNoMax, lsum = 0.0f;

  if (ntiles > 0) {
    tile_info(0);
    if (ntiles > 1) tile_info(1);
    __syncthreads();
    load_tile(0);
    store_tile(0);
    __syncthreads();
  }
  const int arow = 32 * kw + 16 * (l32 >> 4) + sigma16(l32 & 15);
  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    if (t + 2 < ntiles) tile_info(t + 2);

    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[cur][arow * KP + kc * 16 + 8 * h]);
      sacc = mfma32(a, qf[kc], sacc);
    }
    // lane element r = 8c + i is key 32 kw + 16 c + 8 h + i, i.e. slot i of group 4 kw + 2 c + h
    const int nv0 = tval[t % 3][4 * kw + h], nv1 = tval[t % 3][4 * kw + 2 + h];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int nv = r < 8 ? nv0 : nv1;
      const float x = (r & 7) < nv ? sacc[r] * scale2 : -INFINITY;
      sacc[r] = x;
      mx = fmaxf(mx, x);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // rescale only when the running maximum grows by more than 2^8
    const bool grow = mx > m + 8.0f;
    if (__any(grow)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = fast_exp2(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      m = mnew;
    }
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(sacc[r] - m);
      sacc[r] = p;
      ps += p;
    }
    lsum += ps;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = (bf16)sacc[8 * c + i];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Vt[cur][(32 * dt + l32) * VP + 32 * kw + 16 * c + 8 * h]);
        oacc[dt] = mfma32(a, pb, oacc[dt]);
      }
    }
    if (t + 1 < ntiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  // merge the two key halves: waves kw = 1 hand (m, l, O^T) to waves kw = 0 through LDS
  float* xch = reinterpret_cast<float*>(&Ks[0][0]);  // 2 waves x 64 lanes x (2 + D/2) floats
  constexpr int XS = 2 + D / 2;
  if (kw == 1) {
    float* x = xch + ((size_t)qw * 64 + lane) * XS;
    x[0] = m;
    x[1] = lsum;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[2 + 16 * dt + r] = oacc[dt][r];
  }
  __syncthreads();
  if (kw == 0) {
    const float* x = xch + ((size_t)qw * 64 + lane) * XS;
    const float m1 = x[0], l1 = x[1];
    const float mt = fmaxf(m, m1);
    const float a0 = fast_exp2(m - mt), a1 = fast_exp2(m1 - mt);
    float l = lsum * a0 + l1 * a1;
    l += __shfl_xor(l, 32);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (qvalid) {
      bf16* orow = O + ((size_t)bh * N + qrow) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            o[i] = (bf16)((oacc[dt][r] * a0 + x[2 + 16 * dt + r] * a1) * inv);
          }
          *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * g + 4 * h) = o;
        }
      if (lse && h == 0) lse[(size_t)bh * N + qrow] = l > 0.0f ? (mt + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
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
                                                  float scale2, float* __restrict__ O, float* __restrict__ lse) {
  __shared__ float Ks[64][D + 1];
  __shared__ float Vs[64][D + 1];
  __shared__ int pre[PARK_MAX_CLUSTERS + 1];
  __shared__ int kidx[64];
  __shared__ int wsum[2];
  const int bh = blockIdx.y, u = blockIdx.x, tid = threadIdx.x;
  const size_t row = (size_t)bh * NQ + u;
  const int cnt = min(max(count[row], 0), nk);
  const int32_t* lst = list + row * nk;
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  const int32_t* pm = perm + (size_t)bh * N;
  const int T = selected_prefix(lst, off, cnt, nk, pre, wsum);
  const int qrow = 64 * u + tid;
  const bool active = tid < 64 && qrow < N;
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

size_t attn_workspace(const Shape& s) {
  if (s.dtype != 1) return 0;
  const size_t kv = (size_t)s.BH * group_cap(s) * 8 * s.d * sizeof(bf16);
  return align256((size_t)s.BH * (s.nk + 1) * sizeof(int32_t)) + 2 * align256(kv);
}

hipError_t launch_attn(const Shape& s, const void* Q, const void* K, const void* V, const int32_t* perm,
                       const int32_t* offsets, const int32_t* list, const int32_t* count, float scale,
                       void* O, float* lse, void* ws, hipStream_t st) {
  const int NQ = n_qblocks(s.N);
  const float scale2 = scale * kLog2e;
  if (s.dtype == 1) {
    const int Gcap = group_cap(s);
    char* p = static_cast<char*>(ws);
    int32_t* gstart = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)s.BH * (s.nk + 1) * sizeof(int32_t));
    bf16* Kp = reinterpret_cast<bf16*>(p);
    p += align256((size_t)s.BH * Gcap * 8 * s.d * sizeof(bf16));
    bf16* Vp = reinterpret_cast<bf16*>(p);
    auto k = reinterpret_cast<const bf16*>(K);
    auto v = reinterpret_cast<const bf16*>(V);
    k_group_scan<<<s.BH, 256, 0, st>>>(offsets, s.nk, gstart);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 pgrid(s.nk, s.BH);
    if (s.d == 128) k_pack_kv<128><<<pgrid, 128, 0, st>>>(k, v, perm, offsets, gstart, s.N, s.nk, Gcap, Kp, Vp);
    else k_pack_kv<64><<<pgrid, 128, 0, st>>>(k, v, perm, offsets, gstart, s.N, s.nk, Gcap, Kp, Vp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)(NQ * s.BH));
    auto q = reinterpret_cast<const bf16*>(Q);
    auto o = reinterpret_cast<bf16*>(O);
    if (s.d == 128)
      k_attn_bf16<128><<<grid, 256, 0, st>>>(q, Kp, Vp, gstart, offsets, list, count, s.N, s.nk, NQ, Gcap, scale2, o, lse);
    else
      k_attn_bf16<64><<<grid, 256, 0, st>>>(q, Kp, Vp, gstart, offsets, list, count, s.N, s.nk, NQ, Gcap, scale2, o, lse);
  } else {
    dim3 grid(NQ, s.BH);
    auto q = reinterpret_cast<const float*>(Q);
    auto k = reinterpret_cast<const float*>(K);
    auto v = reinterpret_cast<const float*>(V);
    auto o = reinterpret_cast<float*>(O);
    if (s.d == 128)
      k_attn_f32<128><<<grid, 128, 0, st>>>(q, k, v, perm, offsets, list, count, s.N, s.nk, NQ, scale2, o, lse);
    else
      k_attn_f32<64><<<grid, 128, 0, st>>>(q, k, v, perm, offsets, list, count, s.N, s.nk, NQ, scale2, o, lse);
  }
  return hipGetLastError();
}

}  // namespace park
