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
  bf16* Kph = Kp + (size_t)bh * (Gcap + 1) * 8 * D;
  bf16* Vph = Vp + (size_t)bh * (Gcap + 1) * 8 * D;
  if (v == 0) {  // group Gcap of every head is all zeros: the filler of partial tiles
    for (int e = tid; e < D; e += 128) {
      bf16x8 z;
#pragma unroll
      for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
      *reinterpret_cast<bf16x8*>(Kph + (size_t)Gcap * 8 * D + e * 8) = z;
      *reinterpret_cast<bf16x8*>(Vph + (size_t)Gcap * 8 * D + e * 8) = z;
    }
  }
  Kph += (size_t)g0 * 8 * D;
  Vph += (size_t)g0 * 8 * D;
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

// ---------------------------------------------------------------------------------------
// bf16 path, step 2: the tile plan.  For every (head, query block) the concatenation of its
// selected clusters' groups is cut into 64-key tiles of 8 groups; plan entry (g << 4) | nv
// names a packed group g and its number of real keys nv (0..8).  The last tile of a block is
// filled with the all-zero group Gcap.  tbase is the exclusive scan of tiles per block.
__global__ __launch_bounds__(256) void k_plan_count(const int32_t* __restrict__ list, const int32_t* __restrict__ count,
                                                    const int32_t* __restrict__ offsets, int nk, int NQ, int rows,
                                                    int32_t* __restrict__ ntiles) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int bh = row / NQ;
  const int cnt = min(max(count[row], 0), nk);
  const int32_t* lst = list + (size_t)row * nk;
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  int s = 0;
  for (int i = lane; i < cnt; i += 64) {
    const int v = lst[i];
    if (v >= 0 && v < nk) s += (off[v + 1] - off[v] + 7) >> 3;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) ntiles[row] = (s + 7) >> 3;
}

__global__ __launch_bounds__(1024) void k_plan_scan(const int32_t* __restrict__ ntiles, int rows,
                                                    int32_t* __restrict__ tbase) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (rows + 1023) / 1024;
  const int b0 = min(tid * per, rows), b1 = min(b0 + per, rows);
  int s = 0;
  for (int i = b0; i < b1; ++i) s += ntiles[i];
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
    tbase[i] = ex;
    ex += ntiles[i];
  }
  if (tid == 1023) tbase[rows] = ex;
}

__global__ __launch_bounds__(256) void k_plan_fill(const int32_t* __restrict__ list, const int32_t* __restrict__ count,
                                                   const int32_t* __restrict__ offsets, const int32_t* __restrict__ gstart,
                                                   int nk, int NQ, int rows, int Gcap, const int32_t* __restrict__ tbase,
                                                   int32_t* __restrict__ plan) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int bh = row / NQ;
  const int cnt = min(max(count[row], 0), nk);
  const int32_t* lst = list + (size_t)row * nk;
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  const int32_t* gs = gstart + (size_t)bh * (nk + 1);
  int32_t* pl = plan + (size_t)tbase[row] * 8;
  int run = 0;
  for (int i0 = 0; i0 < cnt; i0 += 64) {
    const int i = i0 + lane;
    int n = 0, g0 = 0;
    if (i < cnt) {
      const int v = lst[i];
      if (v >= 0 && v < nk) { n = off[v + 1] - off[v]; g0 = gs[v]; }
    }
    const int ng = (n + 7) >> 3;
    int incl = ng;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const int ex = run + incl - ng;
    for (int jj = 0; jj < ng; ++jj) pl[ex + jj] = ((g0 + jj) << 4) | min(8, n - 8 * jj);
    run += __shfl(incl, 63);
  }
  const int end = (run + 7) & ~7;
  for (int j = run + lane; j < end; j += 64) pl[j] = Gcap << 4;
}

// ---------------------------------------------------------------------------------------
// bf16 path, step 3: attention over the planned tiles.  One workgroup (4 waves) per
// (query block, head); wave w = 2 kw + qw owns queries 32 qw .. 32 qw + 31 of the block and
// keys 32 kw .. 32 kw + 31 of every 64-key tile, with its own online-softmax state (the two
// key halves are merged at the end).  Tiles are copied global -> LDS by the LDS DMA path
// (global_load_lds_dwordx4), double-buffered: the copy of tile t+1 runs under the MFMA
// work of tile t.  LDS holds K group-major and row-major with an XOR swizzle of the
// 16-byte chunks (conflict-free A reads), and V^T group-major exactly as packed.
//   S^T = K Q^T  (A: K rows in sigma16 order, B: Q^T fragments in registers; the MFMA
//                 accumulator starts at 0 / -inf so padding keys are masked for free)
//   O^T += V^T P^T  (A: V^T from LDS, B: P^T straight from the S^T accumulators)
// Row swap inside each 16-row chunk (rows 4..7 <-> 8..11): with it, the 8 rows of S^T that
// an MFMA lane holds for one 16-key chunk are 8 consecutive keys, so the matching V^T
// operand is one 16-byte read.
__device__ __forceinline__ int sigma16(int x) { return (x & ~12) | ((x >> 1) & 4) | ((x << 1) & 8); }

typedef __attribute__((address_space(3))) void* lds_vptr;
typedef __attribute__((address_space(1))) void* gbl_vptr;

__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_vptr)src, (lds_vptr)lds_wave_base, 16, 0, 0);
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(const bf16* __restrict__ Q, const bf16* __restrict__ Kp,
                                                      const bf16* __restrict__ Vp, const int32_t* __restrict__ plan,
                                                      const int32_t* __restrict__ tbase, int N, int NQ, int Gcap,
                                                      float scale2, bf16* __restrict__ O, float* __restrict__ lse) {
  constexpr int NS = D / 8;        // 16-byte chunks per K row
  constexpr int GE = 8 * D;        // bf16 elements per group (K or V)
  constexpr int CPG = GE / 8 / 64; // DMA instructions (64 lanes x 16 B) per group
  // Four distinct LDS objects, so the compiler can tell the tile being computed from the one
  // the DMA is filling and does not wait for the copy before reading.
  __shared__ __attribute__((aligned(16))) bf16 K0[64 * D];   // rows, chunk c of row R at (c ^ (R % NS))
  __shared__ __attribute__((aligned(16))) bf16 K1[64 * D];
  __shared__ __attribute__((aligned(16))) bf16 V0[64 * D];   // [8 groups][D][8]
  __shared__ __attribute__((aligned(16))) bf16 V1[64 * D];
  __shared__ __attribute__((aligned(16))) float btab[9][8];

  int bh, u;
  if (!xcd_head_sync(blockIdx.x, NQ, &bh, &u)) return;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qw = w & 1, kw = w >> 1;
  const int row = bh * NQ + u;
  const int t0 = tbase[row];
  const int nt = tbase[row + 1] - t0;
  const int32_t* pl = plan + (size_t)t0 * 8;
  const bf16* Kph = Kp + (size_t)bh * (Gcap + 1) * GE;
  const bf16* Vph = Vp + (size_t)bh * (Gcap + 1) * GE;

  if (tid < 72) btab[tid >> 3][tid & 7] = (tid & 7) < (tid >> 3) ? 0.0f : -INFINITY;

  // copy tile t into (Kb, Vb): wave w moves groups 2w and 2w+1 (K and V)
  auto issue = [&](int t, bf16* Kb, bf16* Vb) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gi = 2 * w + j;
      const int g = pl[8 * t + gi] >> 4;
      const bf16* ksrc = Kph + (size_t)g * GE;
      const bf16* vsrc = Vph + (size_t)g * GE;
#pragma unroll
      for (int c = 0; c < CPG; ++c) {
        const int pc = 64 * c + lane;            // physical chunk within the group
        const int r = pc / NS, R = 8 * gi + r;   // row within group / tile
        const int seg = (pc % NS) ^ (R % NS);    // logical chunk stored there
        dma16(ksrc + r * D + seg * 8, Kb + (size_t)gi * GE + c * 512);
        dma16(vsrc + pc * 8, Vb + (size_t)gi * GE + c * 512);
      }
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
  const float kBig = __builtin_amdgcn_ldexpf(1.0f, 60);
  float m = kNoMax, lsum = 0.0f;
  // lacc: V^T P^T with V^T replaced by ones, i.e. the row sums of the bf16 weights that the
  // PV product used (every element of a lane holds its query's sum); O is normalised by it,
  // the log-sum-exp by the float sum lsum
  f32x16 lacc;
#pragma unroll
  for (int r = 0; r < 16; ++r) lacc[r] = 0.0f;
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (bf16)1.0f;
  const int arow = 32 * kw + 16 * (l32 >> 4) + sigma16(l32 & 15);
  const int aswz = arow % NS;

  auto compute = [&](int t, const bf16* Kb, const bf16* Vb) {
    // plan entries through the scalar path (wave-uniform addresses)
    const int* pt = pl + __builtin_amdgcn_readfirstlane(8 * t + 4 * kw);
    const int e0 = pt[0], e1 = pt[1], e2 = pt[2], e3 = pt[3];
    // lane element r = 8c + i is key 32 kw + 16 c + 8 h + i: slot i of group 4 kw + 2 c + h
    const int nv0 = (h ? e1 : e0) & 15, nv1 = (h ? e3 : e2) & 15;
    f32x16 sacc;
    {
      const f32x4* b0 = reinterpret_cast<const f32x4*>(&btab[nv0][0]);
      const f32x4* b1 = reinterpret_cast<const f32x4*>(&btab[nv1][0]);
      const f32x4 x0 = b0[0], x1 = b0[1], x2 = b1[0], x3 = b1[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) { sacc[i] = x0[i]; sacc[4 + i] = x1[i]; sacc[8 + i] = x2[i]; sacc[12 + i] = x3[i]; }
    }
    const bf16* kb = Kb + arow * D;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + (((2 * kc + h) ^ aswz) * 8));
      sacc = mfma32(a, qf[kc], sacc);
    }
    // probabilities against the running reference m; the reference only moves (with a
    // rescale of the accumulators) when a row sum leaves [0, 2^60], which happens on the
    // first tile (m starts at -1e30) and when a score exceeds m by about 60 (log2 units)
    f32x16 pr;
    float ps;
    auto probs = [&]() {
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = fast_exp2(fmaf(sacc[r], scale2, -m));
      const float s0 = (pr[0] + pr[1]) + (pr[2] + pr[3]), s1 = (pr[4] + pr[5]) + (pr[6] + pr[7]);
      const float s2 = (pr[8] + pr[9]) + (pr[10] + pr[11]), s3 = (pr[12] + pr[13]) + (pr[14] + pr[15]);
      ps = (s0 + s1) + (s2 + s3);
    };
    probs();
    if (__builtin_expect(__any(!(ps <= kBig)), 0)) {
      asm volatile("" ::: "memory");   // keep this rare path a branch (no if-conversion)
      float mx = sacc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale2;
      const float mnew = fmaxf(m, mx);
      const float alpha = fast_exp2(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      m = mnew;
      probs();
    }
    lsum += ps;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = (bf16)pr[8 * c + i];
      const bf16* vg = Vb + (size_t)(4 * kw + 2 * c + h) * GE;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vg + (32 * dt + l32) * 8);
        oacc[dt] = mfma32(a, pb, oacc[dt]);
      }
      lacc = mfma32(ones, pb, lacc);
    }
  };

  if (nt > 0) issue(0, K0, V0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < nt; t += 2) {
    if (t + 1 < nt) issue(t + 1, K1, V1);
    compute(t, K0, V0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 >= nt) break;
    if (t + 2 < nt) issue(t + 2, K0, V0);
    compute(t + 1, K1, V1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // merge the two key halves: waves kw = 1 hand (m, l, O^T) to waves kw = 0 through LDS
  float* xo = reinterpret_cast<float*>(K0);  // K0 and K1 hold 2 waves x 64 lanes x D/2 floats
  float* xm = reinterpret_cast<float*>(V0);  // 2 waves x 64 lanes x (m, l, l of the bf16 weights)
  auto xo_at = [&](int qq, int ln, int k) -> float* {  // lane-contiguous: no bank conflicts
    const int idx = k * 128 + qq * 64 + ln;
    return idx < 32 * D ? xo + idx : reinterpret_cast<float*>(K1) + (idx - 32 * D);
  };
  if (kw == 1) {
    xm[(qw * 64 + lane) * 3] = m;
    xm[(qw * 64 + lane) * 3 + 1] = lsum;
    xm[(qw * 64 + lane) * 3 + 2] = lacc[0];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) *xo_at(qw, lane, 16 * dt + r) = oacc[dt][r];
  }
  __syncthreads();
  if (kw == 0) {
    const float m1 = xm[(qw * 64 + lane) * 3], l1 = xm[(qw * 64 + lane) * 3 + 1];
    const float lb1 = xm[(qw * 64 + lane) * 3 + 2];
    const float mt = fmaxf(m, m1);
    const float a0 = fast_exp2(m - mt), a1 = fast_exp2(m1 - mt);
    float l = lsum * a0 + l1 * a1;
    l += __shfl_xor(l, 32);
    const float lb = lacc[0] * a0 + lb1 * a1;   // already summed over both lane halves
    const float inv = lb > 0.0f ? 1.0f / lb : 0.0f;
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
            o[i] = (bf16)((oacc[dt][r] * a0 + *xo_at(qw, lane, 16 * dt + r) * a1) * inv);
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
// most 64-key tiles one query block can need (every cluster selected)
static inline int max_tiles_per_block(const Shape& s) { return (group_cap(s) + 7) / 8; }

struct AttnWs {
  int32_t *gstart, *ntiles, *tbase, *plan;
  bf16 *Kp, *Vp;
};

static AttnWs carve_attn(const Shape& s, void* base, size_t* total) {
  const int rows = s.BH * n_qblocks(s.N);
  const size_t kv = (size_t)s.BH * (group_cap(s) + 1) * 8 * s.d * sizeof(bf16);
  char* p = static_cast<char*>(base);
  auto take = [&](size_t bytes) { char* q = p; p += align256(bytes); return q; };
  AttnWs w;
  w.gstart = reinterpret_cast<int32_t*>(take((size_t)s.BH * (s.nk + 1) * sizeof(int32_t)));
  w.ntiles = reinterpret_cast<int32_t*>(take((size_t)rows * sizeof(int32_t)));
  w.tbase = reinterpret_cast<int32_t*>(take((size_t)(rows + 1) * sizeof(int32_t)));
  w.plan = reinterpret_cast<int32_t*>(take((size_t)rows * max_tiles_per_block(s) * 8 * sizeof(int32_t)));
  w.Kp = reinterpret_cast<bf16*>(take(kv));
  w.Vp = reinterpret_cast<bf16*>(take(kv));
  if (total) *total = (size_t)(p - static_cast<char*>(base));
  return w;
}

size_t attn_workspace(const Shape& s) {
  if (s.dtype != 1) return 0;
  size_t total = 0;
  carve_attn(s, nullptr, &total);
  return total;
}

hipError_t launch_attn(const Shape& s, const void* Q, const void* K, const void* V, const int32_t* perm,
                       const int32_t* offsets, const int32_t* list, const int32_t* count, float scale,
                       void* O, float* lse, void* ws, hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
  const int NQ = n_qblocks(s.N);
  const float scale2 = scale * kLog2e;
  if (s.dtype == 1) {
    const int Gcap = group_cap(s);
    const int rows = s.BH * NQ;
    AttnWs w = carve_attn(s, ws, nullptr);
    auto k = reinterpret_cast<const bf16*>(K);
    auto v = reinterpret_cast<const bf16*>(V);
    hipError_t e;
#define PARK_CHECK() do { e = hipGetLastError(); if (e != hipSuccess) return e; } while (0)
    k_group_scan<<<s.BH, 256, 0, st>>>(offsets, s.nk, w.gstart);
    PARK_CHECK();
    dim3 pgrid(s.nk, s.BH);
    if (s.d == 128) k_pack_kv<128><<<pgrid, 128, 0, st>>>(k, v, perm, offsets, w.gstart, s.N, s.nk, Gcap, w.Kp, w.Vp);
    else k_pack_kv<64><<<pgrid, 128, 0, st>>>(k, v, perm, offsets, w.gstart, s.N, s.nk, Gcap, w.Kp, w.Vp);
    PARK_CHECK();
    k_plan_count<<<(rows + 3) / 4, 256, 0, st>>>(list, count, offsets, s.nk, NQ, rows, w.ntiles);
    PARK_CHECK();
    k_plan_scan<<<1, 1024, 0, st>>>(w.ntiles, rows, w.tbase);
    PARK_CHECK();
    k_plan_fill<<<(rows + 3) / 4, 256, 0, st>>>(list, count, offsets, w.gstart, s.nk, NQ, rows, Gcap, w.tbase, w.plan);
    PARK_CHECK();
    dim3 grid((unsigned)(s.BH * 8 * ((NQ + 7) / 8)));
    auto q = reinterpret_cast<const bf16*>(Q);
    auto o = reinterpret_cast<bf16*>(O);
    if (ev_begin && (e = hipEventRecord(ev_begin, st)) != hipSuccess) return e;
    if (s.d == 128)
      k_attn_bf16<128><<<grid, 256, 0, st>>>(q, w.Kp, w.Vp, w.plan, w.tbase, s.N, NQ, Gcap, scale2, o, lse);
    else
      k_attn_bf16<64><<<grid, 256, 0, st>>>(q, w.Kp, w.Vp, w.plan, w.tbase, s.N, NQ, Gcap, scale2, o, lse);
    PARK_CHECK();
#undef PARK_CHECK
    if (ev_end && (e = hipEventRecord(ev_end, st)) != hipSuccess) return e;
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
