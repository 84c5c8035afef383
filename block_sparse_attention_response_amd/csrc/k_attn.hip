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
// bf16 path.  One workgroup (2 waves) per (query block, head); wave w owns queries
// 32w .. 32w+31 of the block.  Per 64-key tile:  S^T = K Q^T  (A = K rows from LDS,
// B = Q^T fragments kept in registers), online softmax per query column, then
// O^T += V^T P^T with P^T taken straight from the S^T accumulators (the MFMA k index is
// permuted consistently on both operands) and V^T staged transposed in LDS.
template <int D>
__global__ __launch_bounds__(128) void k_attn_bf16(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                                   const bf16* __restrict__ V, const int32_t* __restrict__ perm,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ list,
                                                   const int32_t* __restrict__ count, int N, int nk, int NQ,
                                                   float scale2, bf16* __restrict__ O, float* __restrict__ lse) {
  constexpr int KP = D + 8;
  constexpr int VP = 64 + 8;
  constexpr int NS = D / 8;  // 16-byte segments per row
  __shared__ bf16 Ks[64 * KP];
  __shared__ bf16 Vt[D * VP];
  __shared__ int pre[PARK_MAX_CLUSTERS + 1];
  __shared__ int kidx[64];
  __shared__ int wsum[2];

  const uint32_t lb = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lb / NQ, u = lb % NQ;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const size_t row = (size_t)bh * NQ + u;
  const int cnt = min(max(count[row], 0), nk);
  const int32_t* lst = list + row * nk;
  const int32_t* off = offsets + (size_t)bh * (nk + 1);
  const int32_t* pm = perm + (size_t)bh * N;
  const bf16* Kh = K + (size_t)bh * N * D;
  const bf16* Vh = V + (size_t)bh * N * D;

  const int T = selected_prefix(lst, off, cnt, nk, pre, wsum);

  const int qrow = 64 * u + 32 * w + l32;
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
  float m = -INFINITY, lsum = 0.0f;

  const int ntiles = (T + 63) / 64;
  for (int t = 0; t < ntiles; ++t) {
    if (tid < 64) {
      const int p = t * 64 + tid;
      kidx[tid] = p < T ? selected_key(p, pre, cnt, lst, off, pm) : -1;
    }
    __syncthreads();
    for (int e = tid; e < 64 * NS; e += 128) {
      const int r = e / NS, sg = e % NS;
      const int key = kidx[r];
      bf16x8 val;
      if (key >= 0) {
        val = load_bf16x8(Kh + (size_t)key * D + sg * 8);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) val[i] = (bf16)0.0f;
      }
      *reinterpret_cast<bf16x8*>(&Ks[r * KP + sg * 8]) = val;
    }
    for (int e = tid; e < 16 * NS; e += 128) {
      const int kq = e & 15, sg = e >> 4;
      bf16x8 rv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kidx[4 * kq + i];
        if (key >= 0) {
          rv[i] = load_bf16x8(Vh + (size_t)key * D + sg * 8);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) rv[i][j] = (bf16)0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16x4 col;
        col[0] = rv[0][j]; col[1] = rv[1][j]; col[2] = rv[2][j]; col[3] = rv[3][j];
        *reinterpret_cast<bf16x4*>(&Vt[(sg * 8 + j) * VP + 4 * kq]) = col;
      }
    }
    __syncthreads();

    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.0f;
#pragma unroll
      for (int kc = 0; kc < D / 16; ++kc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[(32 * kt + l32) * KP + kc * 16 + 8 * h]);
        sacc[kt] = mfma32(a, qf[kc], sacc[kt]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = t * 64 + 32 * kt + c_row(r, lane);
        const float x = p < T ? sacc[kt][r] * scale2 : -INFINITY;
        sacc[kt][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mnew);
    float ps = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(sacc[kt][r] - mnew);
        sacc[kt][r] = p;
        ps += p;
      }
    lsum = lsum * alpha + ps;
    m = mnew;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;

#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = (bf16)sacc[kt][8 * c + i];
        const int base = 32 * kt + 16 * c;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int dr = 32 * dt + l32;
          const bf16x4 x0 = *reinterpret_cast<const bf16x4*>(&Vt[dr * VP + base + 4 * h]);
          const bf16x4 x1 = *reinterpret_cast<const bf16x4*>(&Vt[dr * VP + base + 8 + 4 * h]);
          bf16x8 a;
          a[0] = x0[0]; a[1] = x0[1]; a[2] = x0[2]; a[3] = x0[3];
          a[4] = x1[0]; a[5] = x1[1]; a[6] = x1[2]; a[7] = x1[3];
          oacc[dt] = mfma32(a, pb, oacc[dt]);
        }
      }
    __syncthreads();
  }

  lsum += __shfl_xor(lsum, 32);
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  if (qvalid) {
    bf16* orow = O + ((size_t)bh * N + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (bf16)(oacc[dt][4 * g + i] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * g + 4 * h) = o;
      }
    if (lse && h == 0) lse[(size_t)bh * N + qrow] = T > 0 ? (m + __log2f(lsum)) * kLn2 : -INFINITY;
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

size_t attn_workspace(const Shape&) { return 0; }

hipError_t launch_attn(const Shape& s, const void* Q, const void* K, const void* V, const int32_t* perm,
                       const int32_t* offsets, const int32_t* list, const int32_t* count, float scale,
                       void* O, float* lse, void*, hipStream_t st) {
  const int NQ = n_qblocks(s.N);
  const float scale2 = scale * kLog2e;
  if (s.dtype == 1) {
    dim3 grid((unsigned)(NQ * s.BH));
    auto q = reinterpret_cast<const bf16*>(Q);
    auto k = reinterpret_cast<const bf16*>(K);
    auto v = reinterpret_cast<const bf16*>(V);
    auto o = reinterpret_cast<bf16*>(O);
    if (s.d == 128)
      k_attn_bf16<128><<<grid, 128, 0, st>>>(q, k, v, perm, offsets, list, count, s.N, s.nk, NQ, scale2, o, lse);
    else
      k_attn_bf16<64><<<grid, 128, 0, st>>>(q, k, v, perm, offsets, list, count, s.N, s.nk, NQ, scale2, o, lse);
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
