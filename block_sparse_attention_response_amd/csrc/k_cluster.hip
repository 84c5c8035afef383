// Query-response key clustering (PARK section 5.2 and App. D.2):
//   G_Q = Q^T Q / N,  Gs = (1 - alpha) G_Q + (alpha + eps) s_Q I = R R^T,  k~ = R^T k,
//   Lloyd k-means on k~ (assign: MFMA distance screen + exact float refine; update:
//   stable counting sort by label + per-cluster sums), then the key permutation, offsets,
//   counts and original-space centroids.
#include "park_device.h"
#include "park_internal.h"
#include "../../include/park.h"

namespace park {

typedef __attribute__((address_space(3))) void* lds_vptr_c;
typedef __attribute__((address_space(1))) void* gbl_vptr_c;

constexpr int kGramChunk = 4096;   // tokens per Gram partial
constexpr int kSortChunk = 1024;   // keys per counting-sort chunk
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
  float* ccv;     // [BH][nkp] |c~|^2 (+inf for padding rows)
  double* cmean;  // [BH][nkp][D] original-space member means
  uint32_t* hmax; // [BH][4] float bits of max |R c~|, max bf16 error of R c~, max |c~|^2
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
  w.ccv = reinterpret_cast<float*>(take(BH * w.nkp * sizeof(float)));
  w.cmean = reinterpret_cast<double*>(take(BH * w.nkp * D * sizeof(double)));
  w.hmax = reinterpret_cast<uint32_t*>(take(BH * 4 * sizeof(uint32_t)));
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
constexpr int kTfKeys = 256;   // keys per workgroup of the bf16 key transform

// Sum over the 32 lanes of a wave half of v[i] (i < 16): lanes l and l ^ 1 end up holding
// the sum for i = (l % 32) / 2 (a reduce-scatter: 16 shuffles instead of 16 x 5).
__device__ __forceinline__ float reduce_scatter16(float (&v)[16], int l32) {
#pragma unroll
  for (int step = 0; step < 4; ++step) {
    const int mask = 16 >> step, half = 8 >> step;
    // lanes with the mask bit keep the upper half; bitwise selects on values (a ternary on
    // array elements would become dynamic register indexing)
    const uint32_t sel = (l32 & mask) ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const uint32_t lo = __float_as_uint(v[i]), hi = __float_as_uint(v[i + half]);
      const float send = __uint_as_float((lo & sel) | (hi & ~sel));
      const float keep = __uint_as_float((hi & sel) | (lo & ~sel));
      v[i] = keep + __shfl_xor(send, mask);
    }
  }
  return v[0] + __shfl_xor(v[0], 1);
}

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
// a1 (end): G = (sum of the chunk partials, in chunk order) / N, one thread per entry.
template <int D>
__global__ __launch_bounds__(256) void k_gram_reduce(const double* __restrict__ gpart, int nch, int N,
                                                     double* __restrict__ G) {
  const int bh = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  double s = 0.0;
  for (int c = 0; c < nch; ++c) s += gpart[((size_t)bh * nch + c) * D * D + e];
  G[(size_t)bh * D * D + e] = s / (double)N;
}

// a2: shrinkage and Cholesky factor, one workgroup per head, double precision in LDS.
//   s = max(tr G / D, s_min);  Gs = (1-alpha) G + (alpha+eps) s I;  Gs = R R^T computed
//   right-looking in place (row pitch D+1): for each column the pivot is square-rooted, the
//   column below it scaled, and the trailing lower triangle updated by all threads at once.
//   On failure (non-positive or non-finite pivot) the head gets R = I and status 1.
//   metric 1 (Euclidean) writes R = I.  G may alias Rt64 (it is read before Rt64 is written).
template <int D>
__global__ __launch_bounds__(256) void k_chol(const double* G, int metric, double alpha, double* __restrict__ R64,
                                              double* Rt64, bf16* __restrict__ Rsp, int32_t* __restrict__ status) {
  constexpr int P = D + 1;
  __shared__ double A[D * P];
  __shared__ double red[4];
  __shared__ int fail;
  const int tid = threadIdx.x, bh = blockIdx.x;
  if (tid == 0) fail = 0;
  if (metric == 0) {
    for (int e = tid; e < D * D; e += 256) A[(e / D) * P + e % D] = G[(size_t)bh * D * D + e];
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
      double piv = A[j * P + j];
      if (!(piv > 0.0) || !isfinite(piv)) {
        if (tid == 0) fail = 1;
        piv = 1.0;
      }
      const double dj = sqrt(piv);
      __syncthreads();
      if (tid == 0) A[j * P + j] = dj;
      for (int i = j + 1 + tid; i < D; i += 256) A[i * P + j] /= dj;
      __syncthreads();
      // trailing lower triangle, 16 x 16 thread grid
      const int ty = tid >> 4, tx = tid & 15;
      for (int i = j + 1 + ty; i < D; i += 16) {
        const double lij = A[i * P + j];
        for (int k = j + 1 + tx; k <= i; k += 16) A[i * P + k] -= lij * A[k * P + j];
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
// float accumulation sees R to ~24 bits).  kTfKeys keys per workgroup of 4 waves.
template <int D>
__global__ __launch_bounds__(256) void k_transform_bf16(const bf16* __restrict__ K, const bf16* __restrict__ Rsp,
                                                        int N, float* __restrict__ Kt, float4* __restrict__ knorm) {
  // k~ = R^T k for kTfKeys keys per workgroup, and the key norms (|k|, 0, |k~|) on the way.
  // The workgroup's keys are copied to LDS once (rows padded by 16 bytes: the 16 rows one
  // 16-lane pass of a fragment read touches start in distinct banks); wave w computes output
  // columns [32 ct, 32 ct + 32) (ct = w % NT) of the key tiles with parity w / NT, with its B
  // fragments (three bf16 splits of R^T for those columns) in registers.
  constexpr int NT = D / 32;            // 32-column output tiles
  constexpr int KC = D / 16;
  constexpr int PAR = 4 / NT;           // waves per output tile
  constexpr int KTILES = kTfKeys / 32;
  constexpr int KP = D + 8;             // padded LDS row (bf16)
  __shared__ bf16 ks[kTfKeys * KP];
  __shared__ float tpart[NT][kTfKeys];  // |k~|^2 partial sums per output tile
  __shared__ float ksq[kTfKeys];        // |k|^2
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int ct = w % NT, par = w / NT;
  const int bh = blockIdx.y, k0 = blockIdx.x * kTfKeys;
  // the keys: 16-byte pieces, consecutive threads on consecutive pieces of a row
  for (int e = tid; e < kTfKeys * (D / 8); e += 256) {
    const int r = e / (D / 8), c = e % (D / 8);
    bf16x8 x;
    if (k0 + r < N) {
      x = load_bf16x8(K + ((size_t)bh * N + k0 + r) * D + 8 * c);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (bf16)0.0f;
    }
    *reinterpret_cast<bf16x8*>(&ks[r * KP + 8 * c]) = x;
  }
  const bf16* rs = Rsp + (size_t)bh * 3 * D * D + (size_t)(32 * ct + l32) * D + 8 * h;
  bf16x8 bfr[3][KC];
#pragma unroll
  for (int sp = 0; sp < 3; ++sp)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) bfr[sp][kc] = load_bf16x8(rs + (size_t)sp * D * D + 16 * kc);
  __syncthreads();
  const int my_row = c_row(l32 >> 1, lane);   // tile row of this lane after the reduce-scatter
  for (int kt = par; kt < KTILES; kt += PAR) {
    bf16x8 a[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) a[kc] = *reinterpret_cast<const bf16x8*>(&ks[(32 * kt + l32) * KP + 16 * kc + 8 * h]);
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int sp = 0; sp < 3; ++sp) acc = mfma32(a[kc], bfr[sp][kc], acc);
    float sq[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = k0 + 32 * kt + c_row(r, lane);
      if (kr < N) Kt[((size_t)bh * N + kr) * D + 32 * ct + l32] = acc[r];
      sq[r] = acc[r] * acc[r];
    }
    // row sums of squares over this wave's 32 columns: lanes l and l ^ 1 get row my_row
    const float t = reduce_scatter16(sq, l32);
    if ((l32 & 1) == 0) tpart[ct][32 * kt + my_row] = t;
    if (ct == 0) {   // |k|^2 from the A fragments: this lane's half of key l32's row
      float s2 = 0.0f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int i = 0; i < 8; ++i) { const float x = (float)a[kc][i]; s2 = fmaf(x, x, s2); }
      s2 += __shfl_xor(s2, 32);
      if (h == 0) ksq[32 * kt + l32] = s2;
    }
  }
  __syncthreads();
  for (int i = tid; i < kTfKeys; i += 256) {
    const int key = k0 + i;
    if (key < N) {
      float t2 = 0.0f;
#pragma unroll
      for (int c = 0; c < NT; ++c) t2 += tpart[c][i];
      knorm[(size_t)bh * N + key] = make_float4(sqrtf(ksq[i]), 0.0f, sqrtf(t2), 0.0f);
    }
  }
}

// a3 for the Euclidean metric with bf16 keys: R = I, so k~ = k exactly (a widening copy) and
// |k~| = |k|.  D / 8 threads per key, 64 keys per workgroup.
template <int D>
__global__ __launch_bounds__(256) void k_copy_keys_bf16(const bf16* __restrict__ K, int N, float* __restrict__ Kt,
                                                        float4* __restrict__ knorm) {
  constexpr int TPK = D / 8;             // threads per key
  constexpr int KPS = 256 / TPK;         // keys per pass
  const int tid = threadIdx.x, bh = blockIdx.y;
  const int sub = tid / TPK, c = tid % TPK;
  for (int r = sub; r < 64; r += KPS) {
    const int j = blockIdx.x * 64 + r;
    float s2 = 0.0f;
    if (j < N) {
      const size_t off = ((size_t)bh * N + j) * D + 8 * c;
      const bf16x8 x = load_bf16x8(K + off);
      f32x4 lo, hi;
#pragma unroll
      for (int i = 0; i < 4; ++i) { lo[i] = (float)x[i]; hi[i] = (float)x[4 + i]; }
#pragma unroll
      for (int i = 0; i < 8; ++i) s2 = fmaf((float)x[i], (float)x[i], s2);
      *reinterpret_cast<f32x4*>(Kt + off) = lo;
      *reinterpret_cast<f32x4*>(Kt + off + 4) = hi;
    }
#pragma unroll
    for (int o = 1; o < TPK; o <<= 1) s2 += __shfl_xor(s2, o);
    if (j < N && c == 0) {
      const float n = sqrtf(s2);
      knorm[(size_t)bh * N + j] = make_float4(n, 0.0f, n, 0.0f);
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

// a4: initial centroids c~_v = k~ at floor(v N / nk) (or init_idx[v], clamped to [0, N));
// padding rows (v >= nk) are zero.  The screen operands follow from k_km_ctx.
template <int D>
__global__ __launch_bounds__(D) void k_km_init(const float* __restrict__ Kt, const int32_t* __restrict__ init_idx,
                                               int N, int nk, int nkp, float* __restrict__ ctil) {
  const int v = blockIdx.x, bh = blockIdx.y, i = threadIdx.x;
  float x = 0.0f;
  if (v < nk) {
    long j = init_idx ? (long)init_idx[v] : (long)(((long long)v * N) / nk);
    j = j < 0 ? 0 : (j >= N ? N - 1 : j);
    x = Kt[((size_t)bh * N + j) * D + i];
  }
  ctil[((size_t)bh * nkp + v) * D + i] = x;
}

// Per-head maxima of |R c~|, its bf16 error and |c~|^2 over all clusters (empty ones
// included: they keep their centroid and stay candidates), read by the next assignment.
__global__ __launch_bounds__(256) void k_bound_max(const float4* __restrict__ cinfo, int nk, int nkp,
                                                   uint32_t* __restrict__ hmax) {
  __shared__ float red[3][4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, bh = blockIdx.x;
  float g = 0.0f, f = 0.0f, cc = 0.0f;
  for (int v = tid; v < nk; v += 256) {
    const float4 c = cinfo[(size_t)bh * nkp + v];
    cc = fmaxf(cc, c.x); g = fmaxf(g, c.y); f = fmaxf(f, c.z);
  }
  g = max64(g); f = max64(f); cc = max64(cc);
  if (lane == 0) { red[0][w] = g; red[1][w] = f; red[2][w] = cc; }
  __syncthreads();
  if (tid < 3) {
    const float m = fmaxf(fmaxf(red[tid][0], red[tid][1]), fmaxf(red[tid][2], red[tid][3]));
    hmax[4 * bh + tid] = __float_as_uint(tid == 2 ? m * (1.0f + 1.0f / 1048576.0f) : m);
  }
}

// ---------------------------------------------------------------------------------------
// a5: assignment a_j = argmin_v |k~_j - c~_v|^2, ties to the lowest v.
// Screen: score_jv = |c~_v|^2 - 2 k_j . bf16(R c~_v) on bf16 MFMA (S^T layout: rows are
// clusters, columns keys), which equals |k~_j - c~_v|^2 - |k~_j|^2 up to a per-key bound
//   E_j = 2 (e_j G + a_j F + e_j F) + 2^-14 (2 a_j G + CC + t_j^2)
// (a_j = |k_j|, e_j = |k_j - bf16(k_j)|, t_j = |k~_j|, G = max |R c~|, F = max bf16 error of
// R c~, CC = max |c~|^2).  Every cluster whose score is within 2 E_j of the key's minimum is
// a candidate; the true argmin always is one.
// One workgroup: 4 waves x 64 keys.  The cluster operand streams through LDS in 32-cluster
// tiles (LDS DMA, double-buffered, shared by the 4 waves); each wave keeps its keys' B
// fragments in registers and a running minimum per key, and records every score within 2 E_j
// of the running minimum in a small per-key list (a value that ends within 2 E_j of the final
// minimum was within 2 E_j of the running minimum when it was seen).  A single surviving
// candidate is the answer; otherwise the candidates are compared with exact float distances
// (k~ and c~ as stored, summed in dimension order), then by id; a key whose list overflowed
// compares every cluster.
constexpr int kAsgWaves = 4;
constexpr int kAsgKeys = 64 * kAsgWaves;   // keys per workgroup
constexpr int kAsgCap = 12;                // list entries per key and lane half (compacted when half full)

template <int D, bool KF32>
__global__ __launch_bounds__(256, 2) void k_km_assign(const void* __restrict__ Kv, const float* __restrict__ Kt,
                                                      const float4* __restrict__ knorm, const float* __restrict__ ctil,
                                                      const bf16* __restrict__ gneg2, const float* __restrict__ ccv,
                                                      const uint32_t* __restrict__ hmax, int N, int nk, int nkp,
                                                      int have_prev, const int32_t* __restrict__ order,
                                                      int32_t* __restrict__ labels) {
  constexpr int NF = D / 16;  // 16-column fragments per 32-cluster tile
  __shared__ int lcnt[kAsgKeys][2];
  __shared__ int lovf[kAsgKeys];
  __shared__ int2 lst[kAsgKeys][2][kAsgCap];   // one list per key and lane half (one writer each)
  __shared__ float ths[kAsgKeys];
  __shared__ unsigned long long best[kAsgKeys];
  __shared__ int2 pairs[kAsgKeys * 4];
  __shared__ int npairs;
  __shared__ __attribute__((aligned(16))) float ccs[PARK_MAX_CLUSTERS];
  __shared__ int kidx[kAsgKeys];   // key index of each slot (-1 past N)
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.y, k0 = blockIdx.x * kAsgKeys;
  const int nT = nkp >> 5;
  const bf16* gA = gneg2 + (size_t)bh * nkp * D + (size_t)lane * 8;  // this lane's piece of fragment 0
  // The loads that need no key index go first (the slot's key and |c~|^2); the LDS copies are
  // written once the key-dependent loads are in flight.
  // Slots walk the keys in `order` (the previous step's label order, so that the keys of a
  // tile share their nearest clusters and few tiles produce candidates) or in index order.
  const int kslot = k0 + tid < N ? (order ? order[(size_t)bh * N + k0 + tid] : k0 + tid) : -1;
  constexpr int MV = PARK_MAX_CLUSTERS / kAsgKeys;
  static_assert(MV * kAsgKeys == PARK_MAX_CLUSTERS, "cluster cap");
  float cvv[MV];
#pragma unroll
  for (int i = 0; i < MV; ++i) {
    const int v = tid + i * kAsgKeys;
    cvv[i] = v < nkp ? ccv[(size_t)bh * nkp + v] : 0.0f;
  }
  if (tid == 0) npairs = 0;

  // B fragments of this wave's 64 keys (two 32-key tiles)
  bf16x8 bfr[2][NF];
  float E[2];
  const float G = __uint_as_float(hmax[4 * bh]), F = __uint_as_float(hmax[4 * bh + 1]);
  const float CC = __uint_as_float(hmax[4 * bh + 2]);
  // the keys of slots 64 w + l32 and 64 w + 32 + l32 (-1 past N)
  const int keyi[2] = {__shfl(kslot, l32), __shfl(kslot, 32 + l32)};
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int pos = k0 + 64 * w + 32 * kt + l32;
    const int key = pos < N ? keyi[kt] : 0;
#pragma unroll
    for (int kc = 0; kc < NF; ++kc) {
      if (pos < N) {
        const size_t off = ((size_t)bh * N + key) * D + 16 * kc + 8 * h;
        if constexpr (KF32) bfr[kt][kc] = load_f32x8_as_bf16(reinterpret_cast<const float*>(Kv) + off);
        else bfr[kt][kc] = load_bf16x8(reinterpret_cast<const bf16*>(Kv) + off);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) bfr[kt][kc][i] = (bf16)0.0f;
      }
    }
    E[kt] = 0.0f;
    if (pos < N) {
      const float4 kn = knorm[(size_t)bh * N + key];
      // the second term covers the float accumulation of 129 terms (< 2^-16.9 of their
      // magnitudes), the rounding of |c~|^2 and of the stored k~, with a factor-7 margin
      E[kt] = 2.0f * (kn.y * G + kn.x * F + kn.y * F) + (1.0f / 16384.0f) * (2.0f * kn.x * G + CC + kn.z * kn.z);
      E[kt] *= 2.0f * (1.0f + 1.0f / 65536.0f);  // the window is twice the bound
    }
  }
  // Running minimum.  From the second step on it starts at the screen score of the key's
  // previous cluster (plus half the window, which covers the different summation order), an
  // upper bound of the final minimum: far fewer scores then fall inside the window.
  float mr[2] = {INFINITY, INFINITY};
  int cnt[2] = {0, 0};          // entries in this lane's list of each key (kept in registers)
  bool ovf[2] = {false, false};
  if (have_prev) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int pos = k0 + 64 * w + 32 * kt + l32;
      if (pos < N) {
        const int vp = labels[(size_t)bh * N + keyi[kt]];
        float dot = 0.0f;
#pragma unroll
        for (int kc = 0; kc < NF; ++kc) {
          const bf16x8 g = load_bf16x8(gneg2 + (size_t)bh * nkp * D + frag_offset(vp, 16 * kc + 8 * h, D));
#pragma unroll
          for (int i = 0; i < 8; ++i) dot = fmaf((float)bfr[kt][kc][i], (float)g[i], dot);
        }
        dot += __shfl_xor(dot, 32);
        mr[kt] = ccv[(size_t)bh * nkp + vp] + dot + 0.5f * E[kt];
      } else {
        mr[kt] = INFINITY;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < MV; ++i)
    if (tid + i * kAsgKeys < nkp) ccs[tid + i * kAsgKeys] = cvv[i];
  kidx[tid] = kslot;
  lovf[tid] = 0;
  best[tid] = ~0ull;
  __syncthreads();

  // stream the 32-cluster tiles straight from memory (fragment-major: 1 KB per fragment);
  // three named fragment buffers rotate (the loop is unrolled by 3), so tile t + 3 is loaded
  // into the buffer of tile t as soon as its products are issued, with no register copies
  auto load_tile = [&](int t, bf16x8 (&buf)[NF]) {
    const int tt = min(t, nT - 1);
#pragma unroll
    for (int kc = 0; kc < NF; ++kc) buf[kc] = load_bf16x8(gA + ((size_t)tt * NF + kc) * 512);
  };
  auto tile = [&](int t, bf16x8 (&a)[NF]) {
    f32x16 init;
#pragma unroll
    for (int g = 0; g < 4; ++g) {  // rows 8g + 4h + 0..3 of the tile
      const f32x4 c = *reinterpret_cast<const f32x4*>(&ccs[32 * t + 8 * g + 4 * h]);
#pragma unroll
      for (int i = 0; i < 4; ++i) init[4 * g + i] = c[i];
    }
    f32x16 acc[2];
    acc[0] = mfma32(a[0], bfr[0][0], init);
    acc[1] = mfma32(a[0], bfr[1][0], init);
#pragma unroll
    for (int kc = 1; kc < NF; ++kc) {
      acc[0] = mfma32(a[kc], bfr[0][kc], acc[0]);
      acc[1] = mfma32(a[kc], bfr[1][kc], acc[1]);
    }
    load_tile(t + 3, a);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float tm = fminf(fminf(acc[kt][0], acc[kt][1]), acc[kt][2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) tm = fminf(fminf(tm, acc[kt][r]), acc[kt][r + 1]);
      tm = fminf(tm, acc[kt][15]);
      tm = xor32_min(tm);
      mr[kt] = fminf(mr[kt], tm);
      const float th = mr[kt] + E[kt];
      if (__any(tm <= th)) {
        const int slot = 64 * w + 32 * kt + l32;
        int c = cnt[kt];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int v = 32 * t + c_row(r, lane);
          if (acc[kt][r] <= th && v < nk) {
            if (c < kAsgCap) lst[slot][h][c] = make_int2(v, __float_as_int(acc[kt][r]));
            else ovf[kt] = true;
            ++c;
          }
        }
        // the window only shrinks: drop entries that left it once a list is half full
        if (c > kAsgCap / 2 && !ovf[kt]) {
          int m = 0;
          for (int e = 0; e < c; ++e) {
            const int2 x = lst[slot][h][e];
            if (__int_as_float(x.y) <= th) lst[slot][h][m++] = x;
          }
          c = m;
        }
        cnt[kt] = c;
      }
    }
  };
  bf16x8 fa[NF], fb[NF], fc[NF];
  load_tile(0, fa);
  load_tile(1, fb);
  load_tile(2, fc);
  int t = 0;
  for (; t + 2 < nT; t += 3) {
    tile(t, fa);
    tile(t + 1, fb);
    tile(t + 2, fc);
  }
  if (t < nT) tile(t, fa);
  if (t + 1 < nT) tile(t + 1, fb);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int slot = 64 * w + 32 * kt + l32;
    lcnt[slot][h] = min(cnt[kt], kAsgCap);
    if (ovf[kt]) lovf[slot] = 1;
  }
  if (h == 0) {
    ths[64 * w + l32] = mr[0] + E[0];
    ths[64 * w + 32 + l32] = mr[1] + E[1];
  }
  __syncthreads();
  // survivors per key: list entries within the window of the final minimum; keys with two
  // or more add their (key, cluster) pairs to the refine list
  int n_surv = 0, only = 0;
  const int j = k0 + tid;
  {
    const float th = ths[tid];
    for (int hh = 0; hh < 2; ++hh) {
      const int n = lcnt[tid][hh];
      for (int c = 0; c < n; ++c) {
        const int2 e = lst[tid][hh][c];
        if (__int_as_float(e.y) <= th) { ++n_surv; only = e.x; }
      }
    }
    if (j < N && !lovf[tid] && n_surv >= 2) {
      const int base = atomicAdd(&npairs, n_surv);
      int m = 0;
      for (int hh = 0; hh < 2; ++hh) {
        const int n = lcnt[tid][hh];
        for (int c = 0; c < n; ++c) {
          const int2 e = lst[tid][hh][c];
          if (__int_as_float(e.y) <= th) {
            if (base + m < kAsgKeys * 4) pairs[base + m] = make_int2(tid, e.x);
            ++m;
          }
        }
      }
    }
  }
  // exact comparison of every cluster where the list overflowed, the pair list is full or no
  // entry survived (only possible with non-finite data)
  bool slow = lovf[tid] != 0 || n_surv == 0;
  __syncthreads();
  const int np = npairs;
  if (np > kAsgKeys * 4 && n_surv >= 2) slow = true;
  lovf[tid] = slow ? 1 : 0;
  __syncthreads();
  // refine: 4 lanes per (key, cluster) pair, exact float distance; each lane sums D/4
  // consecutive dimensions in order and the 4 partial sums are added in a fixed tree
  const int npl = min(np, kAsgKeys * 4);
  for (int p0 = 0; p0 < npl; p0 += kAsgKeys / 4) {
    const int p = p0 + tid / 4, q = tid & 3;
    float s = 0.0f;
    int2 pr = make_int2(0, 0);
    if (p < npl) {
      pr = pairs[p];
      const f32x4* x = reinterpret_cast<const f32x4*>(Kt + ((size_t)bh * N + kidx[pr.x]) * D + q * (D / 4));
      const f32x4* y = reinterpret_cast<const f32x4*>(ctil + ((size_t)bh * nkp + pr.y) * D + q * (D / 4));
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        const f32x4 a = x[i], b = y[i];
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          const float dd = a[z] - b[z];
          s = fmaf(dd, dd, s);
        }
      }
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (p < npl && q == 0 && !lovf[pr.x])
      atomicMin(&best[pr.x], ((unsigned long long)__float_as_uint(s) << 32) | (uint32_t)pr.y);
  }
  // slots w + 4 i of this wave that take the exhaustive path (lane i looks at slot w + 4 i)
  static_assert(kAsgKeys == 64 * kAsgWaves, "one slot per lane and wave");
  uint64_t todo = __ballot(k0 + w + kAsgWaves * lane < N && lovf[w + kAsgWaves * lane]);
  for (; todo; todo &= todo - 1) {
    const int kl = w + kAsgWaves * __builtin_ctzll(todo);
    const f32x4* x = reinterpret_cast<const f32x4*>(Kt + ((size_t)bh * N + kidx[kl]) * D);
    unsigned long long bk = ~0ull;
    for (int v = lane; v < nk; v += 64) {
      const f32x4* y = reinterpret_cast<const f32x4*>(ctil + ((size_t)bh * nkp + v) * D);
      float s = 0.0f;
      for (int i = 0; i < D / 4; ++i) {
        const f32x4 a = x[i], b = y[i];
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          const float dd = a[z] - b[z];
          s = fmaf(dd, dd, s);
        }
      }
      const unsigned long long k = ((unsigned long long)__float_as_uint(s) << 32) | (uint32_t)v;
      bk = k < bk ? k : bk;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long t = __shfl_xor(bk, o);
      bk = t < bk ? t : bk;
    }
    if (lane == 0) best[kl] = bk;
  }
  __syncthreads();
  if (j < N) labels[(size_t)bh * N + kidx[tid]] = (!slow && n_surv == 1) ? only : (int)(uint32_t)best[tid];
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
  for (int j = ch * kSortChunk + tid; j < min(N, (ch + 1) * kSortChunk); j += 256)
    atomicAdd(&hs[labels[(size_t)bh * N + j]], 1);
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
#pragma unroll 8
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
#pragma unroll 8
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
  const int nbits = nk > 1 ? 32 - __builtin_clz((unsigned)(nk - 1)) : 0;   // bits of a label
  // every label of the chunk is loaded before the first is ranked
  constexpr int kSteps = kSortChunk / 64;
  int labs[kSteps];
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int j = ch * kSortChunk + 64 * st + lane;
    labs[st] = j < N ? labels[(size_t)bh * N + j] : -1;
  }
  for (int v = lane; v < nk; v += 64) cur[v] = hist[((size_t)bh * nch + ch) * nk + v];
  __syncthreads();
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int j = ch * kSortChunk + 64 * st + lane;
    const int lab = labs[st];
    // lanes holding the same label: one ballot per label bit (and one for validity)
    uint64_t same = __ballot(lab >= 0);
    if (lab < 0) same = ~same;
    for (int b = 0; b < nbits; ++b) {
      const uint64_t bl = __ballot((lab >> b) & 1);
      same &= ((lab >> b) & 1) ? bl : ~bl;
    }
    const uint64_t below = (1ull << lane) - 1;
    const int rank = __builtin_popcountll(same & below);
    const bool last = (same & ~below & ~(1ull << lane)) == 0;
    if (lab >= 0) {
      const int pos = cur[lab] + rank;
      perm[(size_t)bh * N + pos] = j;
      if (last) cur[lab] = pos + 1;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// a6/a7: per-cluster update, step 1: member sums.  One 256-thread workgroup per cluster;
// the members (a run of perm) are read 16 bytes per thread, RPI rows at a time; each thread
// sums its dimensions in double over its rows, and the RPI partial sums are added in a
// fixed order, so the result does not depend on scheduling.  Writes the original-space mean
// (double) for step 2 and, on the last iteration, the float centroid output (0 if empty).
template <int D, typename T>
__global__ __launch_bounds__(256) void k_km_sums(const T* __restrict__ K, const int32_t* __restrict__ perm,
                                                 const int32_t* __restrict__ offsets, int N, int nk, int nkp,
                                                 double* __restrict__ cmean, float* __restrict__ cent) {
  constexpr int TPR = D / 8;         // threads per row (8 dimensions each)
  constexpr int RPI = 256 / TPR;     // rows in flight per step
  __shared__ double part[RPI][D];
  const int v = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int a = offsets[(size_t)bh * (nk + 1) + v], b = offsets[(size_t)bh * (nk + 1) + v + 1];
  const int n = b - a;
  if (n == 0) {
    if (cent && tid < D) cent[((size_t)bh * nk + v) * D + tid] = 0.0f;
    return;
  }
  const int32_t* pm = perm + (size_t)bh * N + a;
  const T* Kh = K + (size_t)bh * N * D;
  const int rg = tid / TPR, c8 = (tid % TPR) * 8;
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
#pragma unroll 4
  for (int r = rg; r < n; r += RPI) {
    const T* src = Kh + (size_t)pm[r] * D + c8;
    float x[8];
    if constexpr (sizeof(T) == 2) {
      const bf16x8 q = load_bf16x8(reinterpret_cast<const bf16*>(src));
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (float)q[i];
    } else {
      const f32x4 q0 = *reinterpret_cast<const f32x4*>(src);
      const f32x4 q1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) { x[i] = q0[i]; x[4 + i] = q1[i]; }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += (double)x[i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[rg][c8 + i] = acc[i];
  __syncthreads();
  if (tid < D) {
    double sum = 0.0;
    for (int g = 0; g < RPI; ++g) sum += part[g][tid];
    const double m = sum / (double)n;
    cmean[((size_t)bh * nkp + v) * D + tid] = m;
    if (cent) cent[((size_t)bh * nk + v) * D + tid] = (float)m;
  }
}

// Step 2, per (32-cluster tile, head): c~_v = R^T mean_v rounded to float (or, for the
// initial centroids, c~_v as stored), then the screen operand g_v = R c~_v in double,
// gneg2 = bf16(-2 g) (fragment-major), |c~|^2, |g|, |g - bf16(g)|.  Clusters without keys
// keep everything from the previous step; padding rows (v >= nk) get |c~|^2 = +inf.
// Thread (i, vh) owns dimension i of the clusters NVH j + vh of the tile, so each R element
// read from memory serves several clusters.
template <int D>
__global__ __launch_bounds__(256) void k_km_ctx(const double* __restrict__ cmean, const int32_t* __restrict__ counts,
                                                 int nk, int nkp, int init_mode, const double* __restrict__ R64,
                                                 const double* __restrict__ Rt64, float* __restrict__ ctil,
                                                 bf16* __restrict__ gneg2, float4* __restrict__ cinfo,
                                                 float* __restrict__ ccv) {
  // thread (cg, dg): clusters 4 cg .. 4 cg + 3 of the 32-cluster tile, columns DPT dg .. + DPT - 1
  constexpr int DPT = D / 32;
  __shared__ double ms[32][D + 1];     // means, then g
  __shared__ float cs[32][D + 1];
  __shared__ int live_s[32];
  const int tid = threadIdx.x, bh = blockIdx.y, v0 = blockIdx.x * 32;
  const int cg = tid >> 5, dg = tid & 31, c0 = 4 * cg, i0 = DPT * dg;
  if (tid < 32) {
    const int v = v0 + tid;
    live_s[tid] = v < nk && (init_mode || counts[(size_t)bh * nk + v] > 0);
  }
  // acc[c][d] = sum_k M[k][i0 + d] rhs(c0 + c, k), 8 rows of M loaded ahead of their use
  auto matvec = [&](const double* M, auto&& rhs, double (&acc)[4][DPT]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int d = 0; d < DPT; ++d) acc[c][d] = 0.0;
    for (int k0 = 0; k0 < D; k0 += 8) {
      double r[8][DPT];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int d = 0; d < DPT; ++d) r[u][d] = M[(size_t)(k0 + u) * D + i0 + d];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        double x[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = rhs(c0 + c, k0 + u);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int d = 0; d < DPT; ++d) acc[c][d] = fma(r[u][d], x[c], acc[c][d]);
      }
    }
  };
  if (init_mode) {
    for (int e = tid; e < 32 * D; e += 256) {
      const int vv = e / D, k = e % D;
      cs[vv][k] = ctil[((size_t)bh * nkp + v0 + vv) * D + k];
    }
    __syncthreads();
  } else {
    for (int e = tid; e < 32 * D; e += 256) {
      const int vv = e / D, k = e % D;
      const int v = v0 + vv;
      ms[vv][k] = v < nk ? cmean[((size_t)bh * nkp + v) * D + k] : 0.0;
    }
    __syncthreads();
    double t[4][DPT];   // (R^T m)_i = sum_k R[k][i] m_k
    matvec(R64 + (size_t)bh * D * D, [&](int vv, int k) { return ms[vv][k]; }, t);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int d = 0; d < DPT; ++d) cs[c0 + c][i0 + d] = (float)t[c][d];
    __syncthreads();
  }
  {
    double g[4][DPT];   // Rt[k][i] = R[i][k]: (R c~)_i
    matvec(Rt64 + (size_t)bh * D * D, [&](int vv, int k) { return (double)cs[vv][k]; }, g);
    __syncthreads();  // ms is reused for g
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int vv = c0 + c, v = v0 + vv;
#pragma unroll
      for (int d = 0; d < DPT; ++d) {
        const int i = i0 + d;
        ms[vv][i] = g[c][d];
        if (live_s[vv]) {
          ctil[((size_t)bh * nkp + v) * D + i] = cs[vv][i];
          gneg2[(size_t)bh * nkp * D + frag_offset(v, i, D)] = (bf16)(-2.0f * (float)(bf16)(float)g[c][d]);
        } else if (v >= nk) {
          gneg2[(size_t)bh * nkp * D + frag_offset(v, i, D)] = (bf16)0.0f;
        }
      }
    }
  }
  __syncthreads();
  // per cluster |c~|^2, |g| and the bf16 rounding residual of g: 8 threads per cluster, each
  // summing D/8 consecutive columns in order, then a fixed butterfly
  {
    const int vv = tid >> 3, part = tid & 7;
    double cc = 0.0, gn = 0.0, f = 0.0;
    for (int k = part * (D / 8); k < (part + 1) * (D / 8); ++k) {
      const double c = cs[vv][k], g = ms[vv][k];
      const double df = g - (double)(float)(bf16)(float)g;
      cc += c * c; gn += g * g; f += df * df;
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      cc += __shfl_xor(cc, o);
      gn += __shfl_xor(gn, o);
      f += __shfl_xor(f, o);
    }
    const int v = v0 + vv;
    if (part == 0) {
      if (v >= nk) {
        cinfo[(size_t)bh * nkp + v] = make_float4(INFINITY, 0.0f, 0.0f, 0.0f);
        ccv[(size_t)bh * nkp + v] = INFINITY;
      } else if (live_s[vv]) {
        const float up = 1.0f + 1.0f / 1048576.0f;
        const float4 ci = make_float4((float)cc, (float)sqrt(gn) * up, (float)sqrt(f) * up, 0.0f);
        cinfo[(size_t)bh * nkp + v] = ci;
        ccv[(size_t)bh * nkp + v] = ci.x;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
template <int D>
static hipError_t launch_assign(const Shape& s, const ClusterWs& w, const void* K, int have_prev,
                                const int32_t* order, int32_t* labels, hipStream_t st) {
  dim3 grid((s.N + kAsgKeys - 1) / kAsgKeys, s.BH);
  if (s.dtype == 0)
    k_km_assign<D, true><<<grid, 64 * kAsgWaves, 0, st>>>(K, w.Kt, w.knorm, w.ctil, w.gneg2, w.ccv, w.hmax, s.N, s.nk,
                                                         w.nkp, have_prev, order, labels);
  else
    k_km_assign<D, false><<<grid, 64 * kAsgWaves, 0, st>>>(K, w.Kt, w.knorm, w.ctil, w.gneg2, w.ccv, w.hmax, s.N,
                                                          s.nk, w.nkp, have_prev, order, labels);
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
  if (metric == 0) {
    k_gram_reduce<D><<<dim3((D * D + 255) / 256, s.BH), 256, 0, st>>>(w.gpart, w.nch_g, s.N, w.Rt64);
    PARK_CHECK();
  }
  k_chol<D><<<s.BH, 256, 0, st>>>(w.Rt64, metric, (double)alpha, w.R64, w.Rt64, w.Rsp, status);
  PARK_CHECK();
  if (f32) {
    dim3 grid((unsigned)(((size_t)s.N * D + 255) / 256), s.BH);
    k_transform_f32<D><<<grid, 256, 0, st>>>(reinterpret_cast<const float*>(K), w.R64, s.N, w.Kt);
    PARK_CHECK();
    dim3 ngrid((s.N + 63) / 64, s.BH);
    k_key_norms<float, D><<<ngrid, 256, 0, st>>>(reinterpret_cast<const float*>(K), w.Kt, s.N, w.knorm);
  } else if (metric != 0) {
    k_copy_keys_bf16<D><<<dim3((s.N + 63) / 64, s.BH), 256, 0, st>>>(reinterpret_cast<const bf16*>(K), s.N, w.Kt,
                                                                     w.knorm);
  } else {
    dim3 grid((s.N + kTfKeys - 1) / kTfKeys, s.BH);
    k_transform_bf16<D><<<grid, 256, 0, st>>>(reinterpret_cast<const bf16*>(K), w.Rsp, s.N, w.Kt, w.knorm);
  }
  PARK_CHECK();
  k_km_init<D><<<dim3(w.nkp, s.BH), D, 0, st>>>(w.Kt, init_idx, s.N, s.nk, w.nkp, w.ctil);
  PARK_CHECK();
  k_km_ctx<D><<<dim3(w.nkp / 32, s.BH), 256, 0, st>>>(w.cmean, counts, s.nk, w.nkp, 1, w.R64, w.Rt64, w.ctil,
                                                      w.gneg2, w.cinfo, w.ccv);
  PARK_CHECK();
  k_bound_max<<<s.BH, 256, 0, st>>>(w.cinfo, s.nk, w.nkp, w.hmax);
  PARK_CHECK();
  const size_t shm_nk = (size_t)s.nk * sizeof(int);
  for (int it = 0; it < iters; ++it) {
    // from the second step on, the keys are visited in the previous step's label order (perm)
    e = launch_assign<D>(s, w, K, it > 0 ? 1 : 0, it > 0 ? perm : nullptr, labels, st);
    if (e != hipSuccess) return e;
    k_sort_hist<<<dim3(w.nch_s, s.BH), 256, shm_nk, st>>>(labels, s.N, s.nk, w.nch_s, w.hist);
    PARK_CHECK();
    k_sort_scan<<<s.BH, 1024, shm_nk, st>>>(w.hist, s.N, s.nk, w.nch_s, counts, offsets);
    PARK_CHECK();
    k_sort_scatter<<<dim3(w.nch_s, s.BH), 64, shm_nk, st>>>(labels, w.hist, s.N, s.nk, w.nch_s, perm);
    PARK_CHECK();
    float* co = (it == iters - 1) ? cent : nullptr;
    if (f32)
      k_km_sums<D, float><<<dim3(s.nk, s.BH), 256, 0, st>>>(reinterpret_cast<const float*>(K), perm, offsets, s.N, s.nk, w.nkp, w.cmean, co);
    else
      k_km_sums<D, bf16><<<dim3(s.nk, s.BH), 256, 0, st>>>(reinterpret_cast<const bf16*>(K), perm, offsets, s.N, s.nk, w.nkp, w.cmean, co);
    PARK_CHECK();
    if (it + 1 < iters) {  // the transformed centroids only feed the next assignment
      k_km_ctx<D><<<dim3(w.nkp / 32, s.BH), 256, 0, st>>>(w.cmean, counts, s.nk, w.nkp, 0, w.R64, w.Rt64, w.ctil, w.gneg2, w.cinfo, w.ccv);
      PARK_CHECK();
    }
    if (it + 1 < iters) {
      k_bound_max<<<s.BH, 256, 0, st>>>(w.cinfo, s.nk, w.nkp, w.hmax);
      PARK_CHECK();
    }
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
