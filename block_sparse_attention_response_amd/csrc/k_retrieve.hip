// Block retrieval kernels: PAMA scores (PARK section 5.1, E7/E8), the pooled-query
// baseline (section 4.1), and top-p selection with a top-k floor (section 6.1; floor rule
// from the SCOPE appendix "Online Per-Head Top-k Selection").
#include "park_device.h"
#include "park_internal.h"

namespace park {

// ---------------------------------------------------------------------------------------
// Centroids for the PAMA product, pre-multiplied by scale2 = scale log2(e), so that the matrix
// product with the queries gives scale log2(e) q_i . c_v; the fused kernel starts each cluster's
// accumulators at log2 n_v (lg, -inf for an empty cluster), so the logits come out as
//   S_iv (log2 units) = scale log2(e) q_i . c_v + log2 n_v.
// Each value is stored as an unevaluated sum of two bf16 numbers (hi + lo), so a bf16 product
// with the exact-bf16 queries carries about 16 mantissa bits of it.  Layout: fragment-major
// over the d columns; rows nk..nkp-1 are empty clusters.
__global__ void k_centroid_split(const float* __restrict__ C, const int32_t* __restrict__ counts,
                                 int nk, int nkp, int d, float scale2, bf16* __restrict__ Chi,
                                 bf16* __restrict__ Clo, float* __restrict__ lg) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < nkp * d) {
    const int v = e / d, c = e % d;
    const float x = v < nk ? C[((size_t)bh * nk + v) * d + c] * scale2 : 0.0f;
    const bf16 hi = (bf16)x;
    const bf16 lo = (bf16)(x - (float)hi);
    const size_t o = (size_t)bh * nkp * d + frag_offset(v, c, d);
    Chi[o] = hi;
    Clo[o] = lo;
  }
  if (e < nkp) {
    const int n = e < nk ? counts[(size_t)bh * nk + e] : 0;
    lg[(size_t)bh * nkp + e] = n > 0 ? __log2f((float)n) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------
// Fused PAMA: one workgroup per (query block, head), 64 queries, nw waves; wave w owns
// clusters [32 VT w, 32 VT (w+1)).  The 64 x (32 VT) logit slab of a wave stays in
// registers (MFMA accumulators) through the softmax and the block mean; only W goes out.
//   P_iv = 2^(S_iv - max_r S_ir) / sum_r 2^(S_ir - max_r S_ir)
//   W_uv = (1/n_u) sum_i P_iv
// Row maxima and sums: in-lane over the wave's tiles, over the wave's 32 columns by a
// transpose through LDS (one query row per lane), then across the waves through LDS.
// PROBS (the unfused ablation, 64-token blocks only): instead of the block's column sums, every
// query row's normalised probabilities P_i. go to W, laid out [BH][N][nk]; k_rows_mean then
// forms the block means from them in a second pass over HBM.
template <int D, int VT, bool QF32, bool PROBS = false>
__global__ __launch_bounds__(512) void k_pama(const void* __restrict__ Qv, const bf16* __restrict__ Chi,
                                              const bf16* __restrict__ Clo, const float* __restrict__ lg,
                                              int N, int nk, int nkp, int NQ,
                                              float* __restrict__ W, const int4* __restrict__ chunks,
                                              const int32_t* __restrict__ ctotal,
                                              const int32_t* __restrict__ qperm, int maxc) {
  constexpr int DK = D;            // columns of the product
  constexpr int KC = DK / 16;
  constexpr int QP = DK + 8;       // padded LDS row
  __shared__ bf16 qs[64 * QP];
  __shared__ bf16 qlo[QF32 ? 64 * QP : 8];
  __shared__ float red[8][64];
  __shared__ float rowm[64];
  __shared__ float rowinv[64];
  // per wave: a 64-row transpose buffer for the row reductions over the wave's 32 columns
  constexpr int TP = 36;   // row pitch in floats (16-byte aligned rows)
  __shared__ __attribute__((aligned(16))) float tbuf[8][64 * TP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int u = blockIdx.x, bh = blockIdx.y;
  // 64-token blocks: block u is tokens [64u, 64u + 64) and W row u gets the mean.  Clustered
  // query blocks (chunks != NULL): workgroup u is chunk u of the head, positions
  // [q0, q0 + nu) of qperm, and its W row gets the chunk's column sums (k_pama_reduce then
  // adds the chunks of each block and divides by n_u).
  int q0, nu;
  if (chunks) {
    if (u >= ctotal[bh]) return;
    const int4 ch = chunks[(size_t)bh * maxc + u];
    q0 = ch.y;
    nu = ch.z;
  } else {
    q0 = u * 64;
    nu = min(64, N - q0);
  }

  for (int e = tid; e < 64 * (DK / 8); e += blockDim.x) {
    const int row = e / (DK / 8), seg = e % (DK / 8);
    bf16x8 hi, lo;
#pragma unroll
    for (int i = 0; i < 8; ++i) { hi[i] = (bf16)0.0f; lo[i] = (bf16)0.0f; }
    {
      if (row < nu) {
        const int qi = qperm ? min(max(qperm[(size_t)bh * N + q0 + row], 0), N - 1) : q0 + row;
        const size_t off = ((size_t)bh * N + qi) * D + seg * 8;
        if constexpr (QF32) {
          const float* q = reinterpret_cast<const float*>(Qv) + off;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            hi[i] = (bf16)q[i];
            lo[i] = (bf16)(q[i] - (float)hi[i]);
          }
        } else {
          hi = load_bf16x8(reinterpret_cast<const bf16*>(Qv) + off);
        }
      }
    }
    *reinterpret_cast<bf16x8*>(&qs[row * QP + seg * 8]) = hi;
    if constexpr (QF32) *reinterpret_cast<bf16x8*>(&qlo[row * QP + seg * 8]) = lo;
  }
  __syncthreads();

  const int v0 = w * VT * 32;
  // every accumulator of a lane belongs to one cluster column: it starts at log2 n_v
  f32x16 acc[2][VT];
#pragma unroll
  for (int vt = 0; vt < VT; ++vt) {
    const int v = v0 + 32 * vt + l32;
    const float l2n = v < nkp ? lg[(size_t)bh * nkp + v] : -INFINITY;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qt][vt][r] = l2n;
  }
  // B operand fragments (fragment-major Chi / Clo); spare tiles past nkp re-read tile 0: their
  // accumulators start at -inf, as an empty cluster's do, and the finite products leave them
  // there
  size_t crow[VT];
#pragma unroll
  for (int vt = 0; vt < VT; ++vt) {
    const int t = v0 + 32 * vt < nkp ? (v0 >> 5) + vt : 0;
    crow[vt] = (size_t)bh * nkp * DK + frag_lane(t, 0, lane, DK);
  }

  // B fragments stream from L2 PF 16-column steps ahead of their products, through PF + 1
  // named register buffers (the step loop is unrolled, so every buffer index is a constant);
  // the scheduling fences keep the compiler from sinking the loads to their first use
  // (with more than four tiles the registers are short: the loads go just before their use)
  constexpr int PF = VT <= 4 ? 1 : 0;
  bf16x8 bhi[PF + 1][VT], blo[PF + 1][VT];   // (used when PF > 0)
  const auto load_step = [&](int kc, bf16x8 (&hi)[VT], bf16x8 (&lo)[VT]) __attribute__((always_inline)) {
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      hi[vt] = load_bf16x8(Chi + crow[vt] + kc * 512);
      lo[vt] = load_bf16x8(Clo + crow[vt] + kc * 512);
    }
  };
  const auto products = [&](int kc, const bf16x8 (&hi)[VT], const bf16x8 (&lo)[VT]) __attribute__((always_inline)) {
    const int col = kc * 16 + 8 * h;
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&qs[l32 * QP + col]);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&qs[(32 + l32) * QP + col]);
    bf16x8 a0l, a1l;
    if constexpr (QF32) {
      a0l = *reinterpret_cast<const bf16x8*>(&qlo[l32 * QP + col]);
      a1l = *reinterpret_cast<const bf16x8*>(&qlo[(32 + l32) * QP + col]);
    }
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      acc[0][vt] = mfma32(a0, hi[vt], acc[0][vt]);
      acc[1][vt] = mfma32(a1, hi[vt], acc[1][vt]);
      acc[0][vt] = mfma32(a0, lo[vt], acc[0][vt]);
      acc[1][vt] = mfma32(a1, lo[vt], acc[1][vt]);
      if constexpr (QF32) {
        acc[0][vt] = mfma32(a0l, hi[vt], acc[0][vt]);
        acc[1][vt] = mfma32(a1l, hi[vt], acc[1][vt]);
      }
    }
  };
  if constexpr (PF > 0) {
#pragma unroll
    for (int kc = 0; kc < PF; ++kc) load_step(kc, bhi[kc], blo[kc]);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if (kc + PF < KC) load_step(kc + PF, bhi[(kc + PF) % (PF + 1)], blo[(kc + PF) % (PF + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      products(kc, bhi[kc % (PF + 1)], blo[kc % (PF + 1)]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int col = kc * 16 + 8 * h;
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&qs[l32 * QP + col]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&qs[(32 + l32) * QP + col]);
      bf16x8 a0l, a1l;
      if constexpr (QF32) {
        a0l = *reinterpret_cast<const bf16x8*>(&qlo[l32 * QP + col]);
        a1l = *reinterpret_cast<const bf16x8*>(&qlo[(32 + l32) * QP + col]);
      }
      bf16x8 hi[VT], lo[VT];
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        hi[vt] = load_bf16x8(Chi + crow[vt] + kc * 512);
        lo[vt] = load_bf16x8(Clo + crow[vt] + kc * 512);
      }
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        acc[0][vt] = mfma32(a0, hi[vt], acc[0][vt]);
        acc[1][vt] = mfma32(a1, hi[vt], acc[1][vt]);
        acc[0][vt] = mfma32(a0, lo[vt], acc[0][vt]);
        acc[1][vt] = mfma32(a1, lo[vt], acc[1][vt]);
        if constexpr (QF32) {
          acc[0][vt] = mfma32(a0l, hi[vt], acc[0][vt]);
          acc[1][vt] = mfma32(a1l, hi[vt], acc[1][vt]);
        }
      }
    }
  }

  // Row reductions over the wave's 32 cluster columns through LDS: lane (h, l32) holds
  // t[16 qt + r] for query row 32 qt + c_row(r, lane) and column l32; the values are written
  // transposed (row-major, one row per query), and lane L then combines row L's 32 values in
  // column order.  Two LDS rounds instead of five dependent shuffle rounds and their selects.
  float* tb = tbuf[w];
  const auto row_reduce = [&](const float (&t)[32], bool is_max) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 32; ++i) tb[(32 * (i >> 4) + c_row(i & 15, lane)) * TP + l32] = t[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float x = is_max ? -INFINITY : 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(&tb[lane * TP + 4 * k]);
#pragma unroll
      for (int z = 0; z < 4; ++z) x = is_max ? fmaxf(x, v[z]) : x + v[z];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return x;
  };
  float t[32];

  // row maxima
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float mx = acc[qt][0][r];
#pragma unroll
      for (int vt = 1; vt < VT; ++vt) mx = fmaxf(mx, acc[qt][vt][r]);
      t[16 * qt + r] = mx;
    }
  red[w][lane] = row_reduce(t, true);
  __syncthreads();
  if (tid < 64) {
    float m = -INFINITY;
    for (int i = 0; i < nw; ++i) m = fmaxf(m, red[i][tid]);
    rowm[tid] = (m == -INFINITY) ? 0.0f : m;
  }
  __syncthreads();

  // probabilities (unnormalised) and row sums
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 m4 = *reinterpret_cast<const f32x4*>(&rowm[32 * qt + 8 * g + 4 * h]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        float ps = 0.0f;
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
          const float p = fast_exp2(acc[qt][vt][r] - m4[i]);
          acc[qt][vt][r] = p;
          ps += p;
        }
        t[16 * qt + r] = ps;
      }
    }
  red[w][lane] = row_reduce(t, false);
  __syncthreads();
  if (tid < 64) {
    float l = 0.0f;
    for (int i = 0; i < nw; ++i) l += red[i][tid];
    rowinv[tid] = (tid < nu && l > 0.0f) ? 1.0f / l : 0.0f;
  }
  __syncthreads();

  // block mean over the queries: each lane owns one cluster column per tile
  float ri[2][16];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(&rowinv[32 * qt + 8 * g + 4 * h]);
#pragma unroll
      for (int i = 0; i < 4; ++i) ri[qt][4 * g + i] = x[i];
    }
  if constexpr (PROBS) {
    // element r of tile (qt, vt) is query row 32 qt + 8 (r / 4) + 4 h + r % 4, cluster column
    // v0 + 32 vt + l32: each store instruction writes two 128-byte row segments
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      const int v = v0 + 32 * vt + l32;
      if (v >= nk) continue;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * qt + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row < nu) W[((size_t)bh * N + q0 + row) * nk + v] = acc[qt][vt][r] * ri[qt][r];
        }
    }
    return;
  }
  const float inv_nu = chunks ? 1.0f : 1.0f / (float)nu;
  const size_t wrow = (size_t)bh * (chunks ? maxc : NQ) + u;
#pragma unroll
  for (int vt = 0; vt < VT; ++vt) {
    float cs = 0.0f;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) cs = fmaf(acc[qt][vt][r], ri[qt][r], cs);
    cs += __shfl_xor(cs, 32);
    const int v = v0 + 32 * vt + l32;
    if (h == 0 && v < nk) W[wrow * nk + v] = cs * inv_nu;
  }
}

// Unfused ablation, second pass: W_uv = (1/n_u) sum_{i in block u} P_iv over the materialised
// probabilities P [BH][N][nk] (rows in order, float).  grid (ceil(nk / 256), NQ, BH).
__global__ __launch_bounds__(256) void k_rows_mean(const float* __restrict__ P, int N, int nk, int NQ,
                                                   float* __restrict__ W) {
  const int v = blockIdx.x * 256 + threadIdx.x, u = blockIdx.y, bh = blockIdx.z;
  if (v >= nk) return;
  const int i0 = 64 * u, nu = min(64, N - i0);
  const float* p = P + ((size_t)bh * N + i0) * nk + v;
  float acc = 0.0f;
  for (int i = 0; i < nu; ++i) acc += p[(size_t)i * nk];
  W[((size_t)bh * NQ + u) * nk + v] = acc / (float)nu;
}

// Clustered query blocks: W_uv = (1/n_u) sum over the chunks of block u of their column sums
// (chunks in order, float).  grid (ceil(nk / 256), NQ, BH).
__global__ __launch_bounds__(256) void k_pama_reduce(const float* __restrict__ Wp, const int4* __restrict__ chunks,
                                                     const int32_t* __restrict__ cbase, int nk, int NQ, int maxc,
                                                     float* __restrict__ W) {
  const int v = blockIdx.x * 256 + threadIdx.x, u = blockIdx.y, bh = blockIdx.z;
  if (v >= nk) return;
  const int32_t* cb = cbase + (size_t)bh * (NQ + 1);
  const int c0 = cb[u], c1 = cb[u + 1];
  float acc = 0.0f;
  int n = 0;
  for (int c = c0; c < c1; ++c) {
    acc += Wp[((size_t)bh * maxc + c) * nk + v];
    n += chunks[(size_t)bh * maxc + c].z;
  }
  W[((size_t)bh * NQ + u) * nk + v] = n > 0 ? acc / (float)n : 0.0f;
}

// ---------------------------------------------------------------------------------------
// Pooled-query baseline: qbar_u = mean of the block's queries; W_uv = softmax_v(scale
// qbar_u . c_v + log n_v).  One workgroup per (query block, head).
template <typename T>
__global__ __launch_bounds__(256) void k_pooled(const T* __restrict__ Q, const float* __restrict__ C,
                                                const float* __restrict__ lg, int N, int d, int nk,
                                                int nkp, int NQ, float scale2, float* __restrict__ W) {
  extern __shared__ float sm[];
  float* qbar = sm;          // d
  float* s = sm + 128;       // nk
  __shared__ float redv[4];
  const int tid = threadIdx.x, u = blockIdx.x, bh = blockIdx.y;
  const int q0 = u * 64, nu = min(64, N - q0);
  for (int a = tid; a < d; a += blockDim.x) {
    double acc = 0.0;
    for (int i = 0; i < nu; ++i) acc += (double)to_f32(Q[((size_t)bh * N + q0 + i) * d + a]);
    qbar[a] = (float)(acc / nu);
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int v = tid; v < nk; v += blockDim.x) {
    const float* c = C + ((size_t)bh * nk + v) * d;
    float dot = 0.0f;
    for (int a = 0; a < d; ++a) dot = fmaf(qbar[a], c[a], dot);
    const float x = fmaf(dot, scale2, lg[(size_t)bh * nkp + v]);
    s[v] = x;
    mx = fmaxf(mx, x);
  }
  mx = max64(mx);
  if ((tid & 63) == 0) redv[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(redv[0], redv[1]), fmaxf(redv[2], redv[3]));
  __syncthreads();
  float ps = 0.0f;
  for (int v = tid; v < nk; v += blockDim.x) {
    const float p = fast_exp2(s[v] - mx);
    s[v] = p;
    ps += p;
  }
  ps = sum64(ps);
  if ((tid & 63) == 0) redv[tid >> 6] = ps;
  __syncthreads();
  const float inv = 1.0f / (redv[0] + redv[1] + redv[2] + redv[3]);
  for (int v = tid; v < nk; v += blockDim.x) W[((size_t)bh * NQ + u) * nk + v] = s[v] * inv;
}

// ---------------------------------------------------------------------------------------
// Selection per (query block, head), one wave per row.  Clusters are ranked by the key
//   K = (hi << 11) | id,  hi = 0x7F800000 - bits(max(W, 0)) for a non-empty cluster, all ones
// for an empty one, so ascending K is (W descending, id ascending, empty last).  Masses are
// integers in units of 2^-56, so every prefix sum is exact and independent of the order of
// the additions.  t_p is the smallest t whose ranking prefix reaches top_p * total; the
// count is min(max(t_p, top_k), non-empty); the selected set is the `count` smallest keys.
// Both cuts are found by a radix descent over K with 6-bit digits: a 64-bin LDS histogram of
// the candidates' next digit (count and mass), a wave scan over the bins, and the first bin
// that reaches the target; the descent stops as soon as one candidate is left.
constexpr int kKeyBits = 43;   // 32 bits of hi + 11 bits of id (nk <= 2048)

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t t = __shfl_up(x, o);
    if (lane >= o) x += t;
  }
  return x;
}

template <int EPL>
__global__ __launch_bounds__(256) void k_select(const float* __restrict__ W, const int32_t* __restrict__ counts,
                                                int nk, int NQ, int rows, float top_p, int top_k,
                                                uint8_t* __restrict__ mask, int32_t* __restrict__ list,
                                                int32_t* __restrict__ count, const int32_t* __restrict__ floors) {
  __shared__ uint32_t hcnt[4][64];
  __shared__ uint64_t hmass[4][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + w;
  if (row >= rows) return;
  const int bh = row / NQ;
  const float* Wr = W + (size_t)row * nk;
  uint32_t* hc = hcnt[w];
  uint64_t* hm = hmass[w];

  uint64_t key[EPL], ms[EPL];
  int ne = 0;
  uint64_t msum = 0;
  // every count and weight of the row loaded at once (branch-free: indices clamped to the
  // row, entries past it or of empty clusters masked afterwards)
  int cn[EPL];
  float wr[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int i = min(lane + 64 * j, nk - 1);
    cn[j] = counts[(size_t)bh * nk + i];
    wr[j] = Wr[i];
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int i = lane + 64 * j;
    uint32_t hi = 0xFFFFFFFFu;
    uint64_t m = 0;
    if (i < nk && cn[j] > 0) {
      const float wv = (wr[j] > 0.0f) ? wr[j] : 0.0f;   // also maps NaN to 0
      hi = 0x7F800000u - __float_as_uint(wv);
      m = (uint64_t)((double)fminf(wv, 64.0f) * 72057594037927936.0);   // 2^56
      ++ne;
    }
    key[j] = ((uint64_t)hi << 11) | (uint32_t)i;   // i < 2048
    ms[j] = m;
    msum += m;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ne += __shfl_xor(ne, o);
    msum += __shfl_xor(msum, o);
  }
  const double total = (double)msum;

  // smallest key kappa with (sum over keys <= kappa of the weight) >= target, where the
  // weight is the mass (by_mass) or 1; returns kappa and the number of keys <= kappa
  auto descend = [&](bool by_mass, double target, uint64_t* kappa, int* rank) {
    uint64_t prefix = 0;          // key bits above `shift` fixed so far
    uint64_t below = 0;           // weight of the keys below the candidate range
    int nbelow = 0;               // number of keys below the candidate range
    for (int shift = kKeyBits - 6; ; shift -= 6) {
      const int sh = shift > 0 ? shift : 0;
      const int width = shift + 6 - sh;              // digit bits at this level
      const uint64_t hmask = (1ull << width) - 1;
      hc[lane] = 0;
      hm[lane] = 0;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        if ((key[j] >> (sh + width)) == prefix) {
          const int d = (int)((key[j] >> sh) & hmask);
          atomicAdd(&hc[d], 1u);
          if (by_mass) atomicAdd((unsigned long long*)&hm[d], (unsigned long long)ms[j]);
        }
      }
      __builtin_amdgcn_wave_barrier();
      const uint32_t c = hc[lane];
      const uint64_t wt = by_mass ? hm[lane] : (uint64_t)c;
      const uint64_t cw = wave_incl_scan_u64(wt, lane);
      int cc = (int)c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(cc, o);
        if (lane >= o) cc += t;
      }
      const bool reach = (double)(below + cw) >= target;
      const uint64_t bal = __ballot(reach);
      const int d = bal ? __ffsll((unsigned long long)bal) - 1 : 63;
      const uint64_t cw_before = d > 0 ? __shfl(cw, d - 1) : 0;
      const int cc_before = d > 0 ? __shfl(cc, d - 1) : 0;
      const uint32_t cd = __shfl(c, d);
      below += cw_before;
      nbelow += cc_before;
      prefix = (prefix << width) | (uint64_t)d;
      if (sh == 0 || cd == 1) {
        if (sh > 0) {
          // one candidate left: its key completes the prefix
          uint64_t k = 0;
#pragma unroll
          for (int j = 0; j < EPL; ++j)
            if ((key[j] >> sh) == prefix) k = key[j];
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) k |= __shfl_xor(k, o);
          prefix = k;
        }
        *kappa = prefix;
        *rank = nbelow + 1;
        return;
      }
      __builtin_amdgcn_wave_barrier();
    }
  };

  int tp = 0;
  uint64_t kp = 0;
  int cnt;
  if (floors) {
    // second pass of the online per-head top-k: `count` holds this row's first selection
    // b = min(max(t_p, top_k), ne).  A row at or above the head's floor keeps it; a row below
    // is extended to the floor, which exceeds t_p, so only the count descent is needed.
    const int b = count[row], kf = max(top_k, floors[bh]);
    if (b >= kf) return;
    cnt = min(kf, ne);
    if (cnt == b) return;
  } else {
    if (top_p > 0.0f && ne > 0) descend(true, (double)top_p * total, &kp, &tp);
    cnt = min(tp > top_k ? tp : top_k, ne);
  }
  uint64_t kc = kp;
  if (cnt > 0 && cnt != tp) {
    int rk;
    descend(false, (double)cnt, &kc, &rk);
  }

  // mask and ascending id list
  int base = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int i = lane + 64 * j;
    const bool sel = cnt > 0 && key[j] <= kc;
    if (i < nk) mask[(size_t)row * nk + i] = (uint8_t)sel;
    const uint64_t b = __ballot(sel && i < nk);
    const int pos = base + __popcll(b & ((1ull << lane) - 1));
    if (sel && i < nk) list[(size_t)row * nk + pos] = i;
    base += __popcll(b);
  }
  for (int i = cnt + lane; i < nk; i += 64) list[(size_t)row * nk + i] = -1;
  if (lane == 0) count[row] = cnt;
}

// ---------------------------------------------------------------------------------------
size_t retrieve_workspace(const Shape& s, bool need_scores) {
  const int nkp = nk_pad32(s.nk);
  size_t b = 0;
  b += align256((size_t)s.BH * nkp * s.d * sizeof(bf16)) * 2;  // Chi, Clo
  b += align256((size_t)s.BH * nkp * sizeof(float));           // lg
  if (need_scores) b += align256((size_t)s.BH * n_qblocks(s.N) * s.nk * sizeof(float));
  b += align256((size_t)s.BH * sizeof(int32_t));                // online per-head floors
  return b;
}

// chunks == nullptr: 64-token blocks, W [BH][NQ][nk] means; otherwise one workgroup per chunk
// slot, W [BH][maxc][nk] column sums
template <int D, bool QF32, bool PROBS = false>
static hipError_t launch_pama_d(const Shape& s, const void* Q, const bf16* Chi, const bf16* Clo, const float* lg,
                                float* W, hipStream_t st, const int4* chunks = nullptr,
                                const int32_t* ctotal = nullptr, const int32_t* qperm = nullptr, int maxc = 0) {
  const int nkp = nk_pad32(s.nk), NQ = n_qblocks(s.N);
  const int vt = (nkp + 255) / 256;
  const int nw = (nkp + 32 * vt - 1) / (32 * vt);
  dim3 grid(chunks ? maxc : NQ, s.BH), block(64 * nw);
  switch (vt) {
#define PARK_PAMA_CASE(V) \
  case V: k_pama<D, V, QF32, PROBS><<<grid, block, 0, st>>>(Q, Chi, Clo, lg, s.N, s.nk, nkp, NQ, W, chunks, ctotal, qperm, maxc); \
    break;
    PARK_PAMA_CASE(1) PARK_PAMA_CASE(2) PARK_PAMA_CASE(3) PARK_PAMA_CASE(4) PARK_PAMA_CASE(5) PARK_PAMA_CASE(6)
#undef PARK_PAMA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// workspace of the clustered-block retrieval: Chi, Clo, lg, W (when not returned), per-chunk
// column sums and the chunk tables
size_t retrieve_clustered_workspace(const Shape& s, int NQ, bool need_scores) {
  const int nkp = nk_pad32(s.nk), maxc = chunk_slots(s.N, NQ);
  size_t b = 0;
  b += align256((size_t)s.BH * nkp * s.d * sizeof(bf16)) * 2;  // Chi, Clo
  b += align256((size_t)s.BH * nkp * sizeof(float));           // lg
  if (need_scores) b += align256((size_t)s.BH * NQ * s.nk * sizeof(float));
  b += align256((size_t)s.BH * maxc * s.nk * sizeof(float));   // chunk column sums
  b += align256((size_t)s.BH * sizeof(int32_t));                // online per-head floors
  b += align256((size_t)s.BH * maxc * sizeof(int4));           // chunks
  b += align256((size_t)s.BH * (NQ + 1) * sizeof(int32_t));     // cbase
  b += align256((size_t)s.BH * sizeof(int32_t));                // ctotal
  return b;
}

// Online per-head top-k (SCOPE, appendix "Online Per-Head Top-k Selection"): from the base
// counts b_u of a first selection, floor[bh] = ceil(sum_u n_u b_u / sum_u n_u), the
// query-size-weighted mean; n_u = 64-token block sizes, or the clustered blocks' sizes.
__global__ __launch_bounds__(256) void k_online_floor(const int32_t* __restrict__ count, int NQ, int N,
                                                      const int32_t* __restrict__ qoffsets,
                                                      int32_t* __restrict__ floors) {
  __shared__ long long sw[4], sn[4];
  const int bh = blockIdx.x, tid = threadIdx.x;
  long long w = 0, n = 0;
  for (int u = tid; u < NQ; u += 256) {
    long long nu;
    if (qoffsets) {
      const int32_t* off = qoffsets + (size_t)bh * (NQ + 1);
      const int a = min(max(off[u], 0), N), b = min(max(off[u + 1], a), N);
      nu = b - a;
    } else {
      nu = min(64, N - 64 * u);
    }
    w += nu * (long long)count[(size_t)bh * NQ + u];
    n += nu;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    w += __shfl_xor(w, o);
    n += __shfl_xor(n, o);
  }
  if ((tid & 63) == 0) { sw[tid >> 6] = w; sn[tid >> 6] = n; }
  __syncthreads();
  if (tid == 0) {
    const long long W = sw[0] + sw[1] + sw[2] + sw[3], Nn = sn[0] + sn[1] + sn[2] + sn[3];
    floors[bh] = Nn > 0 ? (int)((W + Nn - 1) / Nn) : 0;
  }
}

// top-p / top-k selection of `rows` score rows (NQ per head); floors (per head) or NULL
static hipError_t select_rows(const float* W, const int32_t* counts, int nk, int NQ, int rows, float top_p,
                              int top_k, uint8_t* mask, int32_t* list, int32_t* count, hipStream_t st,
                              const int32_t* floors = nullptr);

// the selection, then (online) the per-head floors from its counts and the selection again
static hipError_t select_all(const Shape& s, const float* W, const int32_t* counts, int NQ, float top_p, int top_k,
                             uint8_t* mask, int32_t* list, int32_t* count, bool online, const int32_t* qoffsets,
                             int32_t* floors, hipStream_t st) {
  hipError_t e = select_rows(W, counts, s.nk, NQ, s.BH * NQ, top_p, top_k, mask, list, count, st);
  if (e != hipSuccess || !online) return e;
  k_online_floor<<<s.BH, 256, 0, st>>>(count, NQ, s.N, qoffsets, floors);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return select_rows(W, counts, s.nk, NQ, s.BH * NQ, top_p, top_k, mask, list, count, st, floors);
}

static hipError_t select_rows(const float* W, const int32_t* counts, int nk, int NQ, int rows, float top_p,
                              int top_k, uint8_t* mask, int32_t* list, int32_t* count, hipStream_t st,
                              const int32_t* floors) {
  const int sgrid = (rows + 3) / 4;
  const int epl = (nk + 63) / 64;
  switch (epl <= 1 ? 1 : epl <= 2 ? 2 : epl <= 4 ? 4 : epl <= 8 ? 8 : epl <= 16 ? 16 : 32) {
#define PARK_SEL_CASE(E) \
  case E: k_select<E><<<sgrid, 256, 0, st>>>(W, counts, nk, NQ, rows, top_p, top_k, mask, list, count, floors); break;
    PARK_SEL_CASE(1) PARK_SEL_CASE(2) PARK_SEL_CASE(4) PARK_SEL_CASE(8) PARK_SEL_CASE(16) PARK_SEL_CASE(32)
#undef PARK_SEL_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_retrieve(const Shape& s, const void* Q, const float* cent, const int32_t* counts,
                           float scale, float top_p, int top_k, bool pooled, float* scores,
                           uint8_t* mask, int32_t* list, int32_t* count, void* ws, hipStream_t st, bool online,
                           float* probs, hipEvent_t ev_begin, hipEvent_t ev_end) {
  const int nkp = nk_pad32(s.nk), NQ = n_qblocks(s.N);
  char* p = static_cast<char*>(ws);
  bf16* Chi = reinterpret_cast<bf16*>(p); p += align256((size_t)s.BH * nkp * s.d * sizeof(bf16));
  bf16* Clo = reinterpret_cast<bf16*>(p); p += align256((size_t)s.BH * nkp * s.d * sizeof(bf16));
  float* lg = reinterpret_cast<float*>(p); p += align256((size_t)s.BH * nkp * sizeof(float));
  float* W = scores;
  if (!W) { W = reinterpret_cast<float*>(p); p += align256((size_t)s.BH * NQ * s.nk * sizeof(float)); }
  int32_t* floors = reinterpret_cast<int32_t*>(p);
  const float scale2 = scale * kLog2e;
  {
    dim3 grid((nkp * s.d + 255) / 256, s.BH);
    k_centroid_split<<<grid, 256, 0, st>>>(cent, counts, s.nk, nkp, s.d, scale2, Chi, Clo, lg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e;
  if (pooled) {
    dim3 grid(NQ, s.BH);
    const size_t shm = (128 + (size_t)s.nk) * sizeof(float);
    if (s.dtype == 1)
      k_pooled<bf16><<<grid, 256, shm, st>>>(reinterpret_cast<const bf16*>(Q), cent, lg, s.N, s.d, s.nk, nkp, NQ, scale2, W);
    else
      k_pooled<float><<<grid, 256, shm, st>>>(reinterpret_cast<const float*>(Q), cent, lg, s.N, s.d, s.nk, nkp, NQ, scale2, W);
    e = hipGetLastError();
  } else if (probs) {
    // unfused ablation: probabilities to HBM, then the block means in a second kernel
    if (s.d == 128)
      e = s.dtype == 1 ? launch_pama_d<128, false, true>(s, Q, Chi, Clo, lg, probs, st)
                       : launch_pama_d<128, true, true>(s, Q, Chi, Clo, lg, probs, st);
    else
      e = s.dtype == 1 ? launch_pama_d<64, false, true>(s, Q, Chi, Clo, lg, probs, st)
                       : launch_pama_d<64, true, true>(s, Q, Chi, Clo, lg, probs, st);
    if (e == hipSuccess) {
      k_rows_mean<<<dim3((s.nk + 255) / 256, NQ, s.BH), 256, 0, st>>>(probs, s.N, s.nk, NQ, W);
      e = hipGetLastError();
    }
  } else {
    if (ev_begin && (e = hipEventRecord(ev_begin, st)) != hipSuccess) return e;
    if (s.d == 128)
      e = s.dtype == 1 ? launch_pama_d<128, false>(s, Q, Chi, Clo, lg, W, st)
                       : launch_pama_d<128, true>(s, Q, Chi, Clo, lg, W, st);
    else
      e = s.dtype == 1 ? launch_pama_d<64, false>(s, Q, Chi, Clo, lg, W, st)
                       : launch_pama_d<64, true>(s, Q, Chi, Clo, lg, W, st);
    if (e == hipSuccess && ev_end) e = hipEventRecord(ev_end, st);
  }
  if (e != hipSuccess) return e;
  return select_all(s, W, counts, NQ, top_p, top_k, mask, list, count, online, nullptr, floors, st);
}

hipError_t launch_retrieve_clustered(const Shape& s, const void* Q, const float* cent, const int32_t* counts,
                                     const QueryBlocks& qb, float scale, float top_p, int top_k, float* scores,
                                     uint8_t* mask, int32_t* list, int32_t* count, void* ws, hipStream_t st,
                                     bool online) {
  const int nkp = nk_pad32(s.nk), NQ = qb.NQ, maxc = chunk_slots(s.N, NQ);
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t bytes) { char* q = p; p += align256(bytes); return q; };
  bf16* Chi = reinterpret_cast<bf16*>(take((size_t)s.BH * nkp * s.d * sizeof(bf16)));
  bf16* Clo = reinterpret_cast<bf16*>(take((size_t)s.BH * nkp * s.d * sizeof(bf16)));
  float* lg = reinterpret_cast<float*>(take((size_t)s.BH * nkp * sizeof(float)));
  float* W = scores ? scores : reinterpret_cast<float*>(take((size_t)s.BH * NQ * s.nk * sizeof(float)));
  float* Wp = reinterpret_cast<float*>(take((size_t)s.BH * maxc * s.nk * sizeof(float)));
  int4* chunks = reinterpret_cast<int4*>(take((size_t)s.BH * maxc * sizeof(int4)));
  int32_t* cbase = reinterpret_cast<int32_t*>(take((size_t)s.BH * (NQ + 1) * sizeof(int32_t)));
  int32_t* ctotal = reinterpret_cast<int32_t*>(take((size_t)s.BH * sizeof(int32_t)));
  int32_t* floors = reinterpret_cast<int32_t*>(take((size_t)s.BH * sizeof(int32_t)));
  const float scale2 = scale * kLog2e;
  {
    dim3 grid((nkp * s.d + 255) / 256, s.BH);
    k_centroid_split<<<grid, 256, 0, st>>>(cent, counts, s.nk, nkp, s.d, scale2, Chi, Clo, lg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_qchunks(qb.qoffsets, s.BH, s.N, NQ, maxc, chunks, cbase, ctotal, st);
  if (e != hipSuccess) return e;
  if (s.d == 128)
    e = s.dtype == 1 ? launch_pama_d<128, false>(s, Q, Chi, Clo, lg, Wp, st, chunks, ctotal, qb.qperm, maxc)
                     : launch_pama_d<128, true>(s, Q, Chi, Clo, lg, Wp, st, chunks, ctotal, qb.qperm, maxc);
  else
    e = s.dtype == 1 ? launch_pama_d<64, false>(s, Q, Chi, Clo, lg, Wp, st, chunks, ctotal, qb.qperm, maxc)
                     : launch_pama_d<64, true>(s, Q, Chi, Clo, lg, Wp, st, chunks, ctotal, qb.qperm, maxc);
  if (e != hipSuccess) return e;
  k_pama_reduce<<<dim3((s.nk + 255) / 256, NQ, s.BH), 256, 0, st>>>(Wp, chunks, cbase, s.nk, NQ, maxc, W);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return select_all(s, W, counts, NQ, top_p, top_k, mask, list, count, online, qb.qoffsets, floors, st);
}

}  // namespace park
