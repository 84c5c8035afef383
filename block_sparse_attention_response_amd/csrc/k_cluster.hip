// Query-response key clustering (PARK section 5.2 and App. D.2):
//   G_Q = Q^T Q / N,  Gs = (1 - alpha) G_Q + (alpha + eps) s_Q I = R R^T,  k~ = R^T k,
//   Lloyd k-means on k~ (assign: MFMA distance screen + exact float refine; update:
//   stable counting sort by label + per-cluster sums), then the key permutation, offsets,
//   counts and original-space centroids.
#include "park_device.h"
#include "park_internal.h"

namespace park {

constexpr int kGramChunk = 4096;   // tokens per Gram partial
constexpr int kSortChunk = 256;    // keys per counting-sort chunk
constexpr int kCandPerKey = 16;    // screened candidates kept per key before the slow path
constexpr double kEps = 1e-6;      // Cholesky stability term (times s_Q)
constexpr double kSMin = 1e-6;     // floor of s_Q

struct ClusterWs {
  double* gpart;  // [BH][nch_g][D][D]
  double* R64;    // [BH][D][D] lower-triangular factor
  double* Rt64;   // [BH][D][D] its transpose
  bf16* Rsp;      // [BH][3][D][D] Rt as a sum of three bf16 matrices
  float* Kt;      // [BH][N][D] transformed keys
  float4* knorm;  // [BH][N] (|k|, |k - bf16(k)|, |k~|, 0)
  float* ctil;    // [BH][nkp][D] centroids in the transformed space
  bf16* gneg2;    // [BH][nkp][D] bf16(-2 R c~)
  float4* cinfo;  // [BH][nkp] (|c~|^2, |R c~|, |R c~ - bf16(R c~)|, 0)
  int32_t* hist;  // [BH][nch_s][nk] counting-sort histograms, then bases
  int nch_g, nch_s, nkp;
};

static ClusterWs carve(const Shape& s, void* base) {
  ClusterWs w{};
  w.nch_g = (s.N + kGramChunk - 1) / kGramChunk;
  w.nch_s = (s.N + kSortChunk - 1) / kSortChunk;
  w.nkp = nk_pad32(s.nk);
  const size_t D = s.d, BH = s.BH;
  char* p = static_cast<char*>(base);
  auto take = [&](size_t bytes) { char* q = p; p += align256(bytes); return q; };
  w.gpart = reinterpret_cast<double*>(take(BH * w.nch_g * D * D * sizeof(double)));
  w.R64 = reinterpret_cast<double*>(take(BH * D * D * sizeof(double)));
  w.Rt64 = reinterpret_cast<double*>(take(BH * D * D * sizeof(double)));
  w.Rsp = reinterpret_cast<bf16*>(take(BH * 3 * D * D * sizeof(bf16)));
  w.Kt = reinterpret_cast<float*>(take(BH * (size_t)s.N * D * sizeof(float)));
  w.knorm = reinterpret_cast<float4*>(take(BH * (size_t)s.N * sizeof(float4)));
  w.ctil = reinterpret_cast<float*>(take(BH * w.nkp * D * sizeof(float)));
  w.gneg2 = reinterpret_cast<bf16*>(take(BH * w.nkp * D * sizeof(bf16)));
  w.cinfo = reinterpret_cast<float4*>(take(BH * w.nkp * sizeof(float4)));
  w.hist = reinterpret_cast<int32_t*>(take(BH * (size_t)w.nch_s * s.nk * sizeof(int32_t)));
  if (base == nullptr) w.gpart = reinterpret_cast<double*>(p);  // total size in the pointer
  return w;
}

size_t cluster_workspace(const Shape& s) {
  ClusterWs w = carve(s, nullptr);
  return reinterpret_cast<size_t>(w.gpart);
}

// ---------------------------------------------------------------------------------------
// a1: Gram partials of bf16 queries.  One workgroup per (4096-token chunk, head); 64-token
// sub-chunks are staged transposed in LDS; products are exact in float, each sub-chunk is
// summed in float by the MFMA and then added into double accumulators.
template <int D>
__global__ __launch_bounds__(256) void k_gram_bf16(const bf16* __restrict__ Q, int N, int nch, double* __restrict__ gpart) {
  constexpr int TP = 64 + 8;
  constexpr int NT = D / 32;
  constexpr int TPW = NT * NT / 4;  // output tiles per wave
  __shared__ bf16 Qt[D * TP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int bh = blockIdx.y, ch = blockIdx.x;
  const int c0 = ch * kGramChunk, c1 = min(c0 + kGramChunk, N);
  double acc64[TPW][16];
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc64[j][r] = 0.0;
  for (int sub = c0; sub < c1; sub += 64) {
    for (int e = tid; e < 64 * (D / 8); e += 256) {
      const int tok = e & 63, sg = e >> 6;
      bf16x8 val;
      if (sub + tok < c1) {
        val = load_bf16x8(Q + ((size_t)bh * N + sub + tok) * D + sg * 8);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) val[i] = (bf16)0.0f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) Qt[(sg * 8 + i) * TP + tok] = val[i];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int id = w * TPW + j, mt = id / NT, nt = id % NT;
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Qt[(32 * mt + l32) * TP + 16 * kc + 8 * h]);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(&Qt[(32 * nt + l32) * TP + 16 * kc + 8 * h]);
        acc = mfma32(a, b, acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc64[j][r] += (double)acc[r];
    }
    __syncthreads();
  }
  double* out = gpart + ((size_t)bh * nch + ch) * D * D;
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int id = w * TPW + j, mt = id / NT, nt = id % NT;
#pragma unroll
    for (int r = 0; r < 16; ++r) out[(32 * mt + c_row(r, lane)) * D + 32 * nt + l32] = acc64[j][r];
  }
}

// a1 for float queries: plain double sums (small workloads only).
template <int D>
__global__ __launch_bounds__(256) void k_gram_f32(const float* __restrict__ Q, int N, int nch, double* __restrict__ gpart) {
  __shared__ float Qs[64][D];
  constexpr int PER = D * D / 256;
  const int tid = threadIdx.x, bh = blockIdx.y, ch = blockIdx.x;
  const int c0 = ch * kGramChunk, c1 = min(c0 + kGramChunk, N);
  double acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0;
  for (int sub = c0; sub < c1; sub += 64) {
    for (int e = tid; e < 64 * D; e += 256) {
      const int tok = e / D, a = e % D;
      Qs[tok][a] = sub + tok < c1 ? Q[((size_t)bh * N + sub + tok) * D + a] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = tid + 256 * i, a = p / D, b = p % D;
      double s = 0.0;
      for (int t = 0; t < 64; ++t) s += (double)Qs[t][a] * (double)Qs[t][b];
      acc[i] += s;
    }
    __syncthreads();
  }
  double* out = gpart + ((size_t)bh * nch + ch) * D * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) out[tid + 256 * i] = acc[i];
}

// ---------------------------------------------------------------------------------------
// a2: shrinkage and Cholesky factor, one workgroup per head, double precision in LDS.
//   G = sum of partials / N;  s = max(tr G / D, s_min);  Gs = (1-alpha) G + (alpha+eps) s I;
//   Gs = R R^T (left-looking, in place, row pitch D+1).  On failure (non-positive or
//   non-finite pivot) the head gets R = I and status 1.  metric 1 (Euclidean) writes R = I.
template <int D>
__global__ __launch_bounds__(256) void k_chol(const double* __restrict__ gpart, int nch, int N, int metric,
                                              double alpha, double* __restrict__ R64, double* __restrict__ Rt64,
                                              bf16* __restrict__ Rsp, int32_t* __restrict__ status) {
  constexpr int P = D + 1;
  __shared__ double A[D * P];
  __shared__ double red[4];
  __shared__ int fail;
  const int tid = threadIdx.x, bh = blockIdx.x;
  if (tid == 0) fail = 0;
  if (metric == 0) {
    for (int e = tid; e < D * D; e += 256) {
      double s = 0.0;
      for (int c = 0; c < nch; ++c) s += gpart[((size_t)bh * nch + c) * D * D + e];
      A[(e / D) * P + e % D] = s / (double)N;
    }
    __syncthreads();
    double tr = 0.0;
    for (int i = tid; i < D; i += 256) tr += A[i * P + i];
    tr = sum64d(tr);
    if ((tid & 63) == 0) red[tid >> 6] = tr;
    __syncthreads();
    double sq = (red[0] + red[1] + red[2] + red[3]) / D;
    if (!(sq > kSMin)) sq = kSMin;
    for (int e = tid; e < D * D; e += 256) {
      const int i = e / D, j = e % D;
      A[i * P + j] = (1.0 - alpha) * A[i * P + j] + (i == j ? (alpha + kEps) * sq : 0.0);
    }
    __syncthreads();
    for (int j = 0; j < D; ++j) {
      if (tid == 0) {
        double s = A[j * P + j];
        for (int k = 0; k < j; ++k) s -= A[j * P + k] * A[j * P + k];
        if (!(s > 0.0) || !isfinite(s)) { fail = 1; s = 1.0; }
        A[j * P + j] = sqrt(s);
      }
      __syncthreads();
      const double piv = A[j * P + j];
      for (int i = j + 1 + tid; i < D; i += 256) {
        double s = A[i * P + j];
        for (int k = 0; k < j; ++k) s -= A[i * P + k] * A[j * P + k];
        A[i * P + j] = s / piv;
      }
      __syncthreads();
    }
  }
  const bool ident = metric != 0 || fail;
  for (int e = tid; e < D * D; e += 256) {
    const int i = e / D, j = e % D;
    const double r = ident ? (i == j ? 1.0 : 0.0) : (j <= i ? A[i * P + j] : 0.0);
    R64[(size_t)bh * D * D + e] = r;                       // R[i][j]
    Rt64[(size_t)bh * D * D + (size_t)j * D + i] = r;      // Rt[j][i] = R[i][j]
    // Rsp[s][out a][in c] = split of Rt[a][c] = R[c][a]: here a = j, c = i
    const bf16 s0 = (bf16)(float)r;
    const double r1 = r - (double)(float)s0;
    const bf16 s1 = (bf16)(float)r1;
    const double r2 = r1 - (double)(float)s1;
    const bf16 s2 = (bf16)(float)r2;
    bf16* rs = Rsp + (size_t)bh * 3 * D * D + (size_t)j * D + i;
    rs[0] = s0;
    rs[(size_t)D * D] = s1;
    rs[(size_t)2 * D * D] = s2;
  }
  if (status && tid == 0) status[bh] = (metric == 0 && fail) ? 1 : 0;
}

// ---------------------------------------------------------------------------------------
// a3: k~ = R^T k for bf16 keys, as K . Rt^T with Rt split into three bf16 matrices (so the
// float accumulation sees R to ~24 bits).  64 keys per workgroup, 4 waves.
template <int D>
__global__ __launch_bounds__(256) void k_transform_bf16(const bf16* __restrict__ K, const bf16* __restrict__ Rsp,
                                                        int N, float* __restrict__ Kt) {
  constexpr int NT = D / 32;
  constexpr int TPW = 2 * NT / 4;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int bh = blockIdx.y, k0 = blockIdx.x * 64;
  const bf16* rs = Rsp + (size_t)bh * 3 * D * D;
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int id = w * TPW + j, kt = id / NT, ct = id % NT;
    const int key = k0 + 32 * kt + l32;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      bf16x8 a;
      if (key < N) {
        a = load_bf16x8(K + ((size_t)bh * N + key) * D + 16 * kc + 8 * h);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = (bf16)0.0f;
      }
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        const bf16x8 b = load_bf16x8(rs + (size_t)s * D * D + (size_t)(32 * ct + l32) * D + 16 * kc + 8 * h);
        acc = mfma32(a, b, acc);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = k0 + 32 * kt + c_row(r, lane);
      if (kr < N) Kt[((size_t)bh * N + kr) * D + 32 * ct + l32] = acc[r];
    }
  }
}

// a3 for float keys: one thread per output, double sums.
template <int D>
__global__ __launch_bounds__(256) void k_transform_f32(const float* __restrict__ K, const double* __restrict__ R64,
                                                       int N, float* __restrict__ Kt) {
  const int bh = blockIdx.y;
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)N * D) return;
  const int j = e / D, a = e % D;
  const double* R = R64 + (size_t)bh * D * D;
  const float* k = K + ((size_t)bh * N + j) * D;
  double s = 0.0;
  for (int c = 0; c < D; ++c) s += R[(size_t)c * D + a] * (double)k[c];
  Kt[((size_t)bh * N + j) * D + a] = (float)s;
}

// Per-key norms for the screening bound: |k|, |k - bf16(k)| (0 for bf16 keys), |k~|.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_key_norms(const T* __restrict__ K, const float* __restrict__ Kt, int N,
                                                   float4* __restrict__ knorm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, bh = blockIdx.y;
  for (int r = w; r < 64; r += 4) {
    const int j = blockIdx.x * 64 + r;
    if (j >= N) break;
    double a2 = 0.0, e2 = 0.0, t2 = 0.0;
    for (int c = lane; c < D; c += 64) {
      const float x = to_f32(K[((size_t)bh * N + j) * D + c]);
      const float xb = (float)(bf16)x;
      const float y = Kt[((size_t)bh * N + j) * D + c];
      a2 += (double)x * x;
      e2 += (double)(x - xb) * (x - xb);
      t2 += (double)y * y;
    }
    a2 = sum64d(a2); e2 = sum64d(e2); t2 = sum64d(t2);
    if (lane == 0) knorm[(size_t)bh * N + j] = make_float4((float)sqrt(a2), (float)sqrt(e2), (float)sqrt(t2), 0.0f);
  }
}

// ---------------------------------------------------------------------------------------
// Centroid preparation (D threads): from c~_v (float, in LDS) compute g = R c~ in double,
// gneg2 = bf16(-2 g), |c~|^2, |g| and |g - bf16(g)|.  Pad rows (v >= nk) get cc = +inf.
template <int D>
__device__ void centroid_prep(int bh, int v, int nk, int nkp, const float* cs, const double* __restrict__ Rt64,
                              bf16* __restrict__ gneg2, float4* __restrict__ cinfo, double* red) {
  const int i = threadIdx.x;
  const double* Rt = Rt64 + (size_t)bh * D * D;
  double g = 0.0;
  for (int k = 0; k < D; ++k) g += Rt[(size_t)k * D + i] * (double)cs[k];
  const bf16 gb = (bf16)(float)g;
  gneg2[((size_t)bh * nkp + v) * D + i] = (bf16)(-2.0f * (float)gb);
  const double df = g - (double)(float)gb;
  double cc = (double)cs[i] * cs[i], gn = g * g, f = df * df;
  cc = sum64d(cc); gn = sum64d(gn); f = sum64d(f);
  const int w = i >> 6;
  if ((i & 63) == 0) { red[3 * w] = cc; red[3 * w + 1] = gn; red[3 * w + 2] = f; }
  __syncthreads();
  if (i == 0) {
    for (int k = 1; k < D / 64; ++k) { cc += red[3 * k]; gn += red[3 * k + 1]; f += red[3 * k + 2]; }
    const float up = 1.0f + 1.0f / 1048576.0f;
    cinfo[(size_t)bh * nkp + v] = make_float4((float)cc, (float)sqrt(gn) * up, (float)sqrt(f) * up, 0.0f);
  }
  __syncthreads();
}

// a4: initial centroids c~_v = k~ at floor(v N / nk) (or init_idx[v], clamped to [0, N)).
template <int D>
__global__ __launch_bounds__(D) void k_km_init(const float* __restrict__ Kt, const int32_t* __restrict__ init_idx,
                                               int N, int nk, int nkp, const double* __restrict__ Rt64,
                                               float* __restrict__ ctil, bf16* __restrict__ gneg2,
                                               float4* __restrict__ cinfo) {
  __shared__ float cs[D];
  __shared__ double red[6];
  const int v = blockIdx.x, bh = blockIdx.y, i = threadIdx.x;
  if (v >= nk) {  // padding rows
    ctil[((size_t)bh * nkp + v) * D + i] = 0.0f;
    gneg2[((size_t)bh * nkp + v) * D + i] = (bf16)0.0f;
    if (i == 0) cinfo[(size_t)bh * nkp + v] = make_float4(INFINITY, 0.0f, 0.0f, 0.0f);
    return;
  }
  long j = init_idx ? (long)init_idx[v] : (long)(((long long)v * N) / nk);
  j = j < 0 ? 0 : (j >= N ? N - 1 : j);
  const float x = Kt[((size_t)bh * N + j) * D + i];
  cs[i] = x;
  ctil[((size_t)bh * nkp + v) * D + i] = x;
  __syncthreads();
  centroid_prep<D>(bh, v, nk, nkp, cs, Rt64, gneg2, cinfo, red);
}

// ---------------------------------------------------------------------------------------
// a5: assignment a_j = argmin_v |k~_j - c~_v|^2, ties to the lowest v.
// Screen: score_jv = |c~_v|^2 - 2 k_j . bf16(R c~_v) on bf16 MFMA (S^T layout: rows are
// clusters, columns keys), which equals |k~_j - c~_v|^2 - |k~_j|^2 up to a per-key bound
//   E_j = 2 (e_j G + a_j F + e_j F) + 2^-12 (2 a_j G + CC + t_j^2)
// (a_j = |k_j|, e_j = |k_j - bf16(k_j)|, t_j = |k~_j|, G = max |R c~|, F = max bf16 error of
// R c~, CC = max |c~|^2).  Every cluster whose score is within 2 E_j of the key's minimum is
// a candidate; the true argmin always is one.  A single candidate is the answer; otherwise
// the candidates are compared with exact float distances (k~ and c~ as stored), then by id.
template <int D, int VT, bool KF32>
__global__ __launch_bounds__(512) void k_km_assign(const void* __restrict__ Kv, const float* __restrict__ Kt,
                                                   const float4* __restrict__ knorm, const float* __restrict__ ctil,
                                                   const bf16* __restrict__ gneg2, const float4* __restrict__ cinfo,
                                                   int N, int nk, int nkp, int32_t* __restrict__ labels) {
  constexpr int KP = D + 8;
  __shared__ bf16 Ks[64 * KP];
  __shared__ float red[8][64];
  __shared__ float thr[64];
  __shared__ unsigned int bmax[3];
  __shared__ int ccount[64];
  __shared__ int cand[64][kCandPerKey];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int bh = blockIdx.y, k0 = blockIdx.x * 64;
  const float4* ci = cinfo + (size_t)bh * nkp;

  if (tid < 3) bmax[tid] = 0u;
  if (tid < 64) ccount[tid] = 0;
  __syncthreads();
  {
    float g = 0.0f, f = 0.0f, cc = 0.0f;
    for (int v = tid; v < nk; v += blockDim.x) {
      const float4 c = ci[v];
      cc = fmaxf(cc, c.x); g = fmaxf(g, c.y); f = fmaxf(f, c.z);
    }
    g = max64(g); f = max64(f); cc = max64(cc);
    if (lane == 0) {
      atomicMax(&bmax[0], __float_as_uint(g));
      atomicMax(&bmax[1], __float_as_uint(f));
      atomicMax(&bmax[2], __float_as_uint(cc));
    }
  }
  for (int e = tid; e < 64 * (D / 8); e += blockDim.x) {
    const int r = e / (D / 8), sg = e % (D / 8);
    bf16x8 val;
    if (k0 + r < N) {
      const size_t off = ((size_t)bh * N + k0 + r) * D + sg * 8;
      if constexpr (KF32) val = load_f32x8_as_bf16(reinterpret_cast<const float*>(Kv) + off);
      else val = load_bf16x8(reinterpret_cast<const bf16*>(Kv) + off);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) val[i] = (bf16)0.0f;
    }
    *reinterpret_cast<bf16x8*>(&Ks[r * KP + sg * 8]) = val;
  }
  __syncthreads();

  const int v0 = w * VT * 32;
  f32x16 acc[2][VT];
#pragma unroll
  for (int vt = 0; vt < VT; ++vt) {
    float init[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = v0 + 32 * vt + c_row(r, lane);
      init[r] = v < nkp ? ci[v].x : INFINITY;
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qt][vt][r] = init[r];
  }
#pragma unroll 2
  for (int kc = 0; kc < D / 16; ++kc) {
    const int col = 16 * kc + 8 * h;
    const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(&Ks[l32 * KP + col]);
    const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(&Ks[(32 + l32) * KP + col]);
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      if (v0 + 32 * vt < nkp) {
        const bf16x8 a = load_bf16x8(gneg2 + ((size_t)bh * nkp + v0 + 32 * vt + l32) * D + col);
        acc[0][vt] = mfma32(a, b0, acc[0][vt]);
        acc[1][vt] = mfma32(a, b1, acc[1][vt]);
      }
    }
  }
  // per-key minimum over this wave's clusters, then over the waves
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float mn = INFINITY;
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mn = fminf(mn, acc[qt][vt][r]);
    mn = fminf(mn, __shfl_xor(mn, 32));
    if (h == 0) red[w][32 * qt + l32] = mn;
  }
  __syncthreads();
  if (tid < 64) {
    float mn = INFINITY;
    for (int i = 0; i < nw; ++i) mn = fminf(mn, red[i][tid]);
    const float G = __uint_as_float(bmax[0]), F = __uint_as_float(bmax[1]), CC = __uint_as_float(bmax[2]);
    float E = 0.0f;
    if (k0 + tid < N) {
      const float4 kn = knorm[(size_t)bh * N + k0 + tid];
      E = 2.0f * (kn.y * G + kn.x * F + kn.y * F) +
          (1.0f / 4096.0f) * (2.0f * kn.x * G + CC + kn.z * kn.z);
    }
    thr[tid] = mn + 2.0f * E * (1.0f + 1.0f / 65536.0f);
  }
  __syncthreads();
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int kl = 32 * qt + l32;
    const float t = thr[kl];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = v0 + 32 * vt + c_row(r, lane);
        if (acc[qt][vt][r] <= t && v < nk) {
          const int c = atomicAdd(&ccount[kl], 1);
          if (c < kCandPerKey) cand[kl][c] = v;
        }
      }
  }
  __syncthreads();
  // refine: one wave per key, exact float distance, (distance, id) minimum
  for (int kl = w; kl < 64; kl += nw) {
    const int j = k0 + kl;
    if (j >= N) break;
    const int n = ccount[kl];
    int best;
    if (n == 1) {
      best = cand[kl][0];
    } else {
      const float* x = Kt + ((size_t)bh * N + j) * D;
      float xv[D / 64];
#pragma unroll
      for (int i = 0; i < D / 64; ++i) xv[i] = x[lane + 64 * i];
      // no candidate (only with non-finite data) or too many: compare every cluster
      const bool listed = n >= 1 && n <= kCandPerKey;
      const int nc = listed ? n : nk;
      uint64_t bk = ~0ull;
      for (int c = 0; c < nc; ++c) {
        const int v = listed ? cand[kl][c] : c;
        const float* y = ctil + ((size_t)bh * nkp + v) * D;
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
          const float dd = xv[i] - y[lane + 64 * i];
          s = fmaf(dd, dd, s);
        }
        s = sum64(s);
        const uint64_t k = ((uint64_t)__float_as_uint(s) << 32) | (uint32_t)v;
        bk = k < bk ? k : bk;
      }
      best = (int)(uint32_t)bk;
    }
    if (lane == 0) labels[(size_t)bh * N + j] = best;
  }
}

// ---------------------------------------------------------------------------------------
// Stable counting sort of the keys by label: per-chunk histograms, a per-head scan, and a
// scatter that keeps the key order inside each label.  Gives counts, offsets and perm.
__global__ __launch_bounds__(256) void k_sort_hist(const int32_t* __restrict__ labels, int N, int nk, int nch,
                                                   int32_t* __restrict__ hist) {
  extern __shared__ int hs[];
  const int tid = threadIdx.x, bh = blockIdx.y, ch = blockIdx.x;
  for (int v = tid; v < nk; v += 256) hs[v] = 0;
  __syncthreads();
  const int j = ch * kSortChunk + tid;
  if (j < N) atomicAdd(&hs[labels[(size_t)bh * N + j]], 1);
  __syncthreads();
  for (int v = tid; v < nk; v += 256) hist[((size_t)bh * nch + ch) * nk + v] = hs[v];
}

__global__ __launch_bounds__(1024) void k_sort_scan(int32_t* __restrict__ hist, int N, int nk, int nch,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  extern __shared__ int tot[];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, bh = blockIdx.x;
  int32_t* hb = hist + (size_t)bh * nch * nk;
  for (int v = tid; v < nk; v += 1024) {
    int s = 0;
    for (int c = 0; c < nch; ++c) s += hb[(size_t)c * nk + v];
    tot[v] = s;
    counts[(size_t)bh * nk + v] = s;
  }
  __syncthreads();
  // exclusive scan of tot over v (each thread a contiguous range)
  const int per = (nk + 1023) / 1024;
  const int b0 = min(tid * per, nk), b1 = min(b0 + per, nk);
  int s = 0;
  for (int v = b0; v < b1; ++v) s += tot[v];
  int incl = s;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += wsum[i];
  int ex = base + incl - s;
  for (int v = b0; v < b1; ++v) {
    const int t = tot[v];
    tot[v] = ex;
    offsets[(size_t)bh * (nk + 1) + v] = ex;
    ex += t;
  }
  if (tid == 0) offsets[(size_t)bh * (nk + 1) + nk] = N;
  __syncthreads();
  for (int v = tid; v < nk; v += 1024) {
    int b = tot[v];
    for (int c = 0; c < nch; ++c) {
      const int t = hb[(size_t)c * nk + v];
      hb[(size_t)c * nk + v] = b;
      b += t;
    }
  }
}

__global__ __launch_bounds__(64) void k_sort_scatter(const int32_t* __restrict__ labels, const int32_t* __restrict__ hist,
                                                     int N, int nk, int nch, int32_t* __restrict__ perm) {
  extern __shared__ int cur[];
  const int lane = threadIdx.x, bh = blockIdx.y, ch = blockIdx.x;
  for (int v = lane; v < nk; v += 64) cur[v] = hist[((size_t)bh * nch + ch) * nk + v];
  __syncthreads();
  for (int st = 0; st < kSortChunk / 64; ++st) {
    const int j = ch * kSortChunk + 64 * st + lane;
    const int lab = j < N ? labels[(size_t)bh * N + j] : -1;
    int rank = 0;
    bool last = true;
    for (int i = 0; i < 64; ++i) {
      const int li = __shfl(lab, i);
      if (li == lab) {
        if (i < lane) ++rank;
        if (i > lane) last = false;
      }
    }
    if (lab >= 0) {
      const int pos = cur[lab] + rank;
      perm[(size_t)bh * N + pos] = j;
      if (last) cur[lab] = pos + 1;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// a6/a7: per-cluster update.  The members (a contiguous run of perm) are summed in double in
// key order; the original-space mean is the cluster centroid output, and c~_v = R^T mean
// (the same value as the mean of R^T k_j).  Empty clusters keep c~ and output 0.
template <int D, typename T>
__global__ __launch_bounds__(D) void k_km_update(const T* __restrict__ K, const int32_t* __restrict__ perm,
                                                 const int32_t* __restrict__ offsets, int N, int nk, int nkp,
                                                 const double* __restrict__ R64, const double* __restrict__ Rt64,
                                                 float* __restrict__ ctil, bf16* __restrict__ gneg2,
                                                 float4* __restrict__ cinfo, float* __restrict__ cent) {
  __shared__ double mean[D];
  __shared__ float cs[D];
  __shared__ double red[6];
  const int v = blockIdx.x, bh = blockIdx.y, i = threadIdx.x;
  const int a = offsets[(size_t)bh * (nk + 1) + v], b = offsets[(size_t)bh * (nk + 1) + v + 1];
  const int32_t* pm = perm + (size_t)bh * N;
  const T* Kh = K + (size_t)bh * N * D;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int p = a;
  for (; p + 3 < b; p += 4) {
    s0 += (double)to_f32(Kh[(size_t)pm[p] * D + i]);
    s1 += (double)to_f32(Kh[(size_t)pm[p + 1] * D + i]);
    s2 += (double)to_f32(Kh[(size_t)pm[p + 2] * D + i]);
    s3 += (double)to_f32(Kh[(size_t)pm[p + 3] * D + i]);
  }
  for (; p < b; ++p) s0 += (double)to_f32(Kh[(size_t)pm[p] * D + i]);
  const int n = b - a;
  const double m = n > 0 ? ((s0 + s1) + (s2 + s3)) / (double)n : 0.0;
  if (cent) cent[((size_t)bh * nk + v) * D + i] = (float)m;
  if (n == 0) return;  // block-uniform
  mean[i] = m;
  __syncthreads();
  const double* R = R64 + (size_t)bh * D * D;
  double t = 0.0;
  for (int k = 0; k < D; ++k) t += R[(size_t)k * D + i] * mean[k];  // (R^T m)_i
  const float tf = (float)t;
  cs[i] = tf;
  ctil[((size_t)bh * nkp + v) * D + i] = tf;
  __syncthreads();
  centroid_prep<D>(bh, v, nk, nkp, cs, Rt64, gneg2, cinfo, red);
}

// ---------------------------------------------------------------------------------------
template <int D>
static hipError_t launch_assign(const Shape& s, const ClusterWs& w, const void* K, int32_t* labels, hipStream_t st) {
  const int vt = (w.nkp + 255) / 256;
  const int nw = (w.nkp + 32 * vt - 1) / (32 * vt);
  dim3 grid((s.N + 63) / 64, s.BH), block(64 * nw);
  const bool f32 = s.dtype == 0;
  switch (vt) {
#define PARK_ASSIGN_CASE(V)                                                                                   \
  case V:                                                                                                     \
    if (f32) k_km_assign<D, V, true><<<grid, block, 0, st>>>(K, w.Kt, w.knorm, w.ctil, w.gneg2, w.cinfo, s.N, s.nk, w.nkp, labels); \
    else k_km_assign<D, V, false><<<grid, block, 0, st>>>(K, w.Kt, w.knorm, w.ctil, w.gneg2, w.cinfo, s.N, s.nk, w.nkp, labels); \
    break;
    PARK_ASSIGN_CASE(1) PARK_ASSIGN_CASE(2) PARK_ASSIGN_CASE(3) PARK_ASSIGN_CASE(4) PARK_ASSIGN_CASE(5) PARK_ASSIGN_CASE(6)
#undef PARK_ASSIGN_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_cluster_d(const Shape& s, const void* Q, const void* K, int iters, int metric, float alpha,
                                   const int32_t* init_idx, float* cent, int32_t* counts, int32_t* labels,
                                   int32_t* perm, int32_t* offsets, int32_t* status, const ClusterWs& w,
                                   hipStream_t st) {
  const bool f32 = s.dtype == 0;
  hipError_t e;
#define PARK_CHECK() do { e = hipGetLastError(); if (e != hipSuccess) return e; } while (0)
  if (metric == 0) {
    dim3 grid(w.nch_g, s.BH);
    if (f32) k_gram_f32<D><<<grid, 256, 0, st>>>(reinterpret_cast<const float*>(Q), s.N, w.nch_g, w.gpart);
    else k_gram_bf16<D><<<grid, 256, 0, st>>>(reinterpret_cast<const bf16*>(Q), s.N, w.nch_g, w.gpart);
    PARK_CHECK();
  }
  k_chol<D><<<s.BH, 256, 0, st>>>(w.gpart, w.nch_g, s.N, metric, (double)alpha, w.R64, w.Rt64, w.Rsp, status);
  PARK_CHECK();
  if (f32) {
    dim3 grid((unsigned)(((size_t)s.N * D + 255) / 256), s.BH);
    k_transform_f32<D><<<grid, 256, 0, st>>>(reinterpret_cast<const float*>(K), w.R64, s.N, w.Kt);
  } else {
    dim3 grid((s.N + 63) / 64, s.BH);
    k_transform_bf16<D><<<grid, 256, 0, st>>>(reinterpret_cast<const bf16*>(K), w.Rsp, s.N, w.Kt);
  }
  PARK_CHECK();
  {
    dim3 grid((s.N + 63) / 64, s.BH);
    if (f32) k_key_norms<float, D><<<grid, 256, 0, st>>>(reinterpret_cast<const float*>(K), w.Kt, s.N, w.knorm);
    else k_key_norms<bf16, D><<<grid, 256, 0, st>>>(reinterpret_cast<const bf16*>(K), w.Kt, s.N, w.knorm);
    PARK_CHECK();
  }
  k_km_init<D><<<dim3(w.nkp, s.BH), D, 0, st>>>(w.Kt, init_idx, s.N, s.nk, w.nkp, w.Rt64, w.ctil, w.gneg2, w.cinfo);
  PARK_CHECK();
  const size_t shm_nk = (size_t)s.nk * sizeof(int);
  for (int it = 0; it < iters; ++it) {
    e = launch_assign<D>(s, w, K, labels, st);
    if (e != hipSuccess) return e;
    k_sort_hist<<<dim3(w.nch_s, s.BH), 256, shm_nk, st>>>(labels, s.N, s.nk, w.nch_s, w.hist);
    PARK_CHECK();
    k_sort_scan<<<s.BH, 1024, shm_nk, st>>>(w.hist, s.N, s.nk, w.nch_s, counts, offsets);
    PARK_CHECK();
    k_sort_scatter<<<dim3(w.nch_s, s.BH), 64, shm_nk, st>>>(labels, w.hist, s.N, s.nk, w.nch_s, perm);
    PARK_CHECK();
    float* co = (it == iters - 1) ? cent : nullptr;
    if (f32)
      k_km_update<D, float><<<dim3(s.nk, s.BH), D, 0, st>>>(reinterpret_cast<const float*>(K), perm, offsets, s.N, s.nk, w.nkp, w.R64, w.Rt64, w.ctil, w.gneg2, w.cinfo, co);
    else
      k_km_update<D, bf16><<<dim3(s.nk, s.BH), D, 0, st>>>(reinterpret_cast<const bf16*>(K), perm, offsets, s.N, s.nk, w.nkp, w.R64, w.Rt64, w.ctil, w.gneg2, w.cinfo, co);
    PARK_CHECK();
  }
#undef PARK_CHECK
  return hipSuccess;
}

hipError_t launch_cluster(const Shape& s, const void* Q, const void* K, int iters, int metric, float alpha,
                          const int32_t* init_idx, float* cent, int32_t* counts, int32_t* labels, int32_t* perm,
                          int32_t* offsets, int32_t* status, void* ws, hipStream_t st) {
  const ClusterWs w = carve(s, ws);
  if (s.d == 128)
    return launch_cluster_d<128>(s, Q, K, iters, metric, alpha, init_idx, cent, counts, labels, perm, offsets, status, w, st);
  return launch_cluster_d<64>(s, Q, K, iters, metric, alpha, init_idx, cent, counts, labels, perm, offsets, status, w, st);
}

}  // namespace park
