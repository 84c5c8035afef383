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
  float4* knorm;  // [BH][N] (|k|, |k - fp16(k)|, |k~|, 0)
  float* ctil;    // [BH][nkp][D] centroids in the transformed space
  f16* gneg2;     // [BH][nkp][D] fp16(-2 R c~)
  float4* cinfo;  // [BH][nkp] (|c~|^2, |R c~|, |R c~ - fp16(R c~)|, 0)
  float* ccv;     // [BH][nkp] |c~|^2 (+inf for padding rows)
  double* cmean;  // [BH][nkp][D] original-space member means
  double* csum;   // [BH][nkp][D] original-space member sums (carried from step to step)
  int32_t *lalt, *palt, *oalt, *calt;   // the other step's labels, perm, offsets, counts
  uint32_t* hmax; // [BH][4] float bits of max |R c~|, max fp16 error of R c~, max |c~|^2
  int32_t* hist;  // [BH][nch_s][nk] counting-sort histograms, then bases
  int32_t* wlab;  // [BH][ceil(N / kAsgKeys)] label at the first position of each assignment workgroup
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
  w.gneg2 = reinterpret_cast<f16*>(take(BH * w.nkp * D * sizeof(f16)));
  w.cinfo = reinterpret_cast<float4*>(take(BH * w.nkp * sizeof(float4)));
  w.ccv = reinterpret_cast<float*>(take(BH * w.nkp * sizeof(float)));
  w.cmean = reinterpret_cast<double*>(take(BH * w.nkp * D * sizeof(double)));
  w.csum = reinterpret_cast<double*>(take(BH * w.nkp * D * sizeof(double)));
  w.lalt = reinterpret_cast<int32_t*>(take(BH * (size_t)s.N * sizeof(int32_t)));
  w.palt = reinterpret_cast<int32_t*>(take(BH * (size_t)s.N * sizeof(int32_t)));
  w.oalt = reinterpret_cast<int32_t*>(take(BH * (size_t)(s.nk + 1) * sizeof(int32_t)));
  w.calt = reinterpret_cast<int32_t*>(take(BH * (size_t)s.nk * sizeof(int32_t)));
  w.hmax = reinterpret_cast<uint32_t*>(take(BH * 4 * sizeof(uint32_t)));
  w.hist = reinterpret_cast<int32_t*>(take(BH * (size_t)w.nch_s * s.nk * sizeof(int32_t)));
  w.wlab = reinterpret_cast<int32_t*>(take(BH * (size_t)((s.N + 255) / 256) * sizeof(int32_t)));
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

// One wave per 32x32 output tile ((D/32)^2 waves per workgroup), so a lane holds the double
// sums of one tile only and the workgroup has many waves to hide the loads; every thread
// loads its share of each 64-token sub-chunk kGramAhead sub-chunks ahead into registers.
// The sums are taken in the same order as ever: per sub-chunk the MFMA's float sum over the
// 64 tokens, then the sub-chunks in order in double.
constexpr int kGramAhead = 4;
template <int D>
__global__ __launch_bounds__(64 * (D / 32) * (D / 32)) void k_gram_bf16(const bf16* __restrict__ Q, int N, int nch,
                                                                        double* __restrict__ gpart) {
  constexpr int TP = 64 + 8;
  constexpr int NT = D / 32;
  constexpr int NTH = 64 * NT * NT;            // threads
  constexpr int LPT = (64 * (D / 8)) / NTH;    // 16-byte loads per thread and sub-chunk
  static_assert(LPT * NTH == 64 * (D / 8) && LPT >= 1, "sub-chunk split");
  __shared__ bf16 Qt[D * TP];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), mt = w / NT, nt = w % NT;
  const int bh = blockIdx.y, ch = blockIdx.x;
  const int c0 = ch * kGramChunk, c1 = min(c0 + kGramChunk, N);
  const int nsub = (c1 - c0 + 63) / 64;
  // this thread's loads of a sub-chunk: element e = tid + NTH l, token e % 64, 8 columns at 8 (e / 64)
  auto load_sub = [&](int sidx, bf16x8 (&v)[LPT]) {
#pragma unroll
    for (int l = 0; l < LPT; ++l) {
      const int e = tid + NTH * l, tok = e & 63, sg = e >> 6;
      const int t = c0 + 64 * sidx + tok;
      if (sidx < nsub && t < c1) {
        v[l] = load_bf16x8(Q + ((size_t)bh * N + t) * D + sg * 8);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[l][i] = (bf16)0.0f;
      }
    }
  };
  bf16x8 ring[kGramAhead][LPT];
#pragma unroll
  for (int a = 0; a < kGramAhead; ++a) load_sub(a, ring[a]);
  double acc64[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc64[r] = 0.0;
  for (int s0 = 0; s0 < nsub; s0 += kGramAhead) {
#pragma unroll
    for (int a = 0; a < kGramAhead; ++a) {
      const int sidx = s0 + a;
      if (sidx < nsub) {   // uniform over the workgroup
#pragma unroll
        for (int l = 0; l < LPT; ++l) {
          const int e = tid + NTH * l, tok = e & 63, sg = e >> 6;
#pragma unroll
          for (int i = 0; i < 8; ++i) Qt[(sg * 8 + i) * TP + tok] = ring[a][l][i];
        }
        __syncthreads();
        load_sub(sidx + kGramAhead, ring[a]);   // the slot is free: kGramAhead sub-chunks ahead
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(&Qt[(32 * mt + l32) * TP + 16 * kc + 8 * h]);
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&Qt[(32 * nt + l32) * TP + 16 * kc + 8 * h]);
          acc = mfma32(av, bv, acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) acc64[r] += (double)acc[r];
        __syncthreads();
      }
    }
  }
  double* out = gpart + ((size_t)bh * nch + ch) * D * D;
#pragma unroll
  for (int r = 0; r < 16; ++r) out[(32 * mt + c_row(r, lane)) * D + 32 * nt + l32] = acc64[r];
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

// a2: shrinkage and Cholesky factor, one workgroup per head, double precision in registers.
//   s = max(tr G / D, s_min);  Gs = (1-alpha) G + (alpha+eps) s I;  Gs = R R^T computed
//   right-looking: thread (ty, tx) of a 16 x 16 grid holds the entries (ty + 16a, tx + 16b) of
//   the matrix.  For each column j the threads holding it publish it in LDS, every thread takes
//   the square root of the pivot and one thread per row divides its entry by it, and then every
//   thread updates its entries to the right of column j with the new column (each entry gets its
//   updates one FMA at a time in column order).  Entries above the diagonal are updated too and
//   ignored.  On failure (non-positive or non-finite pivot) the head gets R = I and status 1.
//   metric 1 (Euclidean) writes R = I.  G may alias Rt64 (every read of G precedes the first
//   barrier, every write of Rt64 follows the last).
template <int D>
__global__ __launch_bounds__(256) void k_chol(const double* G, int metric, double alpha, double* __restrict__ R64,
                                              double* Rt64, bf16* __restrict__ Rsp, int32_t* __restrict__ status) {
  constexpr int NB = D / 16;  // rows (and columns) per thread
  __shared__ double col[D], lcol[D];
  __shared__ double red[4];
  const int tid = threadIdx.x, bh = blockIdx.x, ty = tid >> 4, tx = tid & 15;
  double acc[NB][NB];
  bool fail = false;
  if (metric == 0) {
    const double* g = G + (size_t)bh * D * D;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[a][b] = g[(ty + 16 * a) * D + tx + 16 * b];
    double tr = tid < D ? g[tid * D + tid] : 0.0;
    tr = sum64d(tr);
    if ((tid & 63) == 0) red[tid >> 6] = tr;
    __syncthreads();
    double sq = (red[0] + red[1] + red[2] + red[3]) / D;
    if (!(sq > kSMin)) sq = kSMin;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int i = ty + 16 * a, j = tx + 16 * b;
        acc[a][b] = (1.0 - alpha) * acc[a][b] + (i == j ? (alpha + kEps) * sq : 0.0);
      }
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
#pragma unroll 1
      for (int jj = 0; jj < 16; ++jj) {
        const int j = 16 * jb + jj;
        if (tx == jj) {
#pragma unroll
          for (int a = 0; a < NB; ++a) col[ty + 16 * a] = acc[a][jb];
        }
        __syncthreads();
        double piv = col[j];
        if (!(piv > 0.0) || !isfinite(piv)) {
          fail = true;
          piv = 1.0;
        }
        const double dj = sqrt(piv);
        if (tid < D) lcol[tid] = tid > j ? col[tid] / dj : (tid == j ? dj : 0.0);
        __syncthreads();
        double li[NB];
#pragma unroll
        for (int a = 0; a < NB; ++a) li[a] = lcol[ty + 16 * a];
        if (tx == jj) {
#pragma unroll
          for (int a = 0; a < NB; ++a)
            if (ty + 16 * a >= j) acc[a][jb] = li[a];
        }
        // columns k = tx + 16 b > j: b > jb always, b == jb when tx > jj
#pragma unroll
        for (int b = jb; b < NB; ++b) {
          if (b == jb && tx <= jj) continue;
          const double lk = lcol[tx + 16 * b];
#pragma unroll
          for (int a = 0; a < NB; ++a) acc[a][b] -= li[a] * lk;
        }
      }
    }
  }
  const bool ident = metric != 0 || fail;
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = ty + 16 * a, j = tx + 16 * b;
      const double r = ident ? (i == j ? 1.0 : 0.0) : (j <= i ? acc[a][b] : 0.0);
      R64[(size_t)bh * D * D + (size_t)i * D + j] = r;       // R[i][j]
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
  // k~ = R^T k for kTfKeys keys per workgroup, and the key norms (|k|, |k - fp16(k)|, |k~|) on
  // the way.
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
  __shared__ float kerr[kTfKeys];       // |k - fp16(k)|^2
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int ct = w % NT, par = w / NT;
  const int bh = blockIdx.y, k0 = blockIdx.x * kTfKeys;
  // the keys: 16-byte pieces, consecutive threads on consecutive pieces of a row; every load
  // of a thread is issued before the first is written to LDS
  constexpr int PPT = kTfKeys * (D / 8) / 256;   // pieces per thread
  static_assert(PPT * 256 == kTfKeys * (D / 8), "key pieces");
  {
    bf16x8 x[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int e = tid + 256 * j, r = e / (D / 8), c = e % (D / 8);
      if (k0 + r < N) {
        x[j] = load_bf16x8(K + ((size_t)bh * N + k0 + r) * D + 8 * c);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[j][i] = (bf16)0.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int e = tid + 256 * j, r = e / (D / 8), c = e % (D / 8);
      *reinterpret_cast<bf16x8*>(&ks[r * KP + 8 * c]) = x[j];
    }
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
    if (ct == 0) {   // |k|^2 and |k - fp16(k)|^2 from the A fragments: this lane's half of key l32's row
      float s2 = 0.0f, e2 = 0.0f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = (float)a[kc][i], dx = x - (float)(f16)x;
          s2 = fmaf(x, x, s2);
          e2 = fmaf(dx, dx, e2);
        }
      s2 += __shfl_xor(s2, 32);
      e2 += __shfl_xor(e2, 32);
      if (h == 0) { ksq[32 * kt + l32] = s2; kerr[32 * kt + l32] = e2; }
    }
  }
  __syncthreads();
  for (int i = tid; i < kTfKeys; i += 256) {
    const int key = k0 + i;
    if (key < N) {
      float t2 = 0.0f;
#pragma unroll
      for (int c = 0; c < NT; ++c) t2 += tpart[c][i];
      knorm[(size_t)bh * N + key] = make_float4(sqrtf(ksq[i]), sqrtf(kerr[i]), sqrtf(t2), 0.0f);
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
    float s2 = 0.0f, e2 = 0.0f;
    if (j < N) {
      const size_t off = ((size_t)bh * N + j) * D + 8 * c;
      const bf16x8 x = load_bf16x8(K + off);
      f32x4 lo, hi;
#pragma unroll
      for (int i = 0; i < 4; ++i) { lo[i] = (float)x[i]; hi[i] = (float)x[4 + i]; }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xf = (float)x[i], dx = xf - (float)(f16)xf;
        s2 = fmaf(xf, xf, s2);
        e2 = fmaf(dx, dx, e2);
      }
      *reinterpret_cast<f32x4*>(Kt + off) = lo;
      *reinterpret_cast<f32x4*>(Kt + off + 4) = hi;
    }
#pragma unroll
    for (int o = 1; o < TPK; o <<= 1) {
      s2 += __shfl_xor(s2, o);
      e2 += __shfl_xor(e2, o);
    }
    if (j < N && c == 0) {
      const float n = sqrtf(s2);
      knorm[(size_t)bh * N + j] = make_float4(n, sqrtf(e2), n, 0.0f);
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

// Per-key norms for the screening bound: |k|, |k - fp16(k)|, |k~|.
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
      const float xb = (float)(f16)x;
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

// Per-head maxima of |R c~|, its fp16 error and |c~|^2 over all clusters (empty ones
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
// Screen: score_jv = |c~_v|^2 + fp16(k_j) . fp16(-2 R c~_v) on fp16 MFMA (S^T layout: rows are
// clusters, columns keys), which equals |k~_j - c~_v|^2 - |k~_j|^2 up to a per-key bound
//   E_j = 2 (e_j G + a_j F + e_j F) + 2^-14 (2 a_j G + CC + t_j^2)
// (a_j = |k_j|, e_j = |k_j - fp16(k_j)|, t_j = |k~_j|, G = max |R c~|, F = max fp16 error of
// R c~, CC = max |c~|^2).  fp16 operands rather than bf16 (the same MFMA rate) make the first
// term, the larger one, about 8 times smaller, and with it the keys left with several
// candidates.  A key whose bound is not finite (values beyond the fp16 range), or any key of
// a head with G >= 2^14 (where -2 R c~ could leave it), compares every cluster exactly.  Every cluster whose score is within 2 E_j of the key's minimum is
// a candidate; the true argmin always is one.
// One workgroup: 4 waves x 64 keys.  The cluster operand streams through a three-slot LDS ring
// in 32-cluster tiles (LDS DMA, each wave copying a quarter of every tile, one barrier per
// tile), shared by the 4 waves; each wave keeps its keys' B fragments in registers and a
// running minimum per key, and records every score within 2 E_j of the running minimum in a
// small per-key list (a value that ends within 2 E_j of the final minimum was within 2 E_j of
// the running minimum when it was seen).  From the second step on, keys are visited in the
// previous step's label order and the screen starts at the tile of the workgroup's first
// previous cluster, so the running minimum is tight from the first tile on.  A single
// surviving candidate is the answer; otherwise the candidates are compared with exact float
// distances (k~ and c~ as stored, summed in dimension order), then by id; a key whose list
// overflowed compares every cluster.
constexpr int kAsgWaves = 4;
constexpr int kAsgKeys = 64 * kAsgWaves;   // keys per workgroup
static_assert(kAsgKeys == 256, "the workspace sizes the per-workgroup start labels for 256 keys per workgroup");
constexpr int kAsgCap = 10;                // list entries per key and lane half (compacted when half full)

// global -> LDS copy of 16 bytes per lane: lane i reads base + off_i and writes lds + 16 i
// (the LDS address goes in m0, bound as an operand so that the compiler sets it).  Inline
// assembly, so that the compiler does not guard later LDS reads with a wait for all
// outstanding copies; the kernel waits for exactly the copies it needs (copies complete in
// issue order).  The instruction has no register results.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_copies() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// every LDS read this wave has issued has returned
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

template <int D, bool KF32>
__global__ __launch_bounds__(256, 2) void k_km_assign(const void* __restrict__ Kv, const float* __restrict__ Kt,
                                                      const float4* __restrict__ knorm, const float* __restrict__ ctil,
                                                      const f16* __restrict__ gneg2, const float* __restrict__ ccv,
                                                      const uint32_t* __restrict__ hmax, int N, int nk, int nkp,
                                                      const int32_t* __restrict__ order,
                                                      const int32_t* __restrict__ wlab, int32_t* __restrict__ labels) {
  constexpr int NF = D / 16;  // 16-column fragments per 32-cluster tile
  __shared__ int lcnt[kAsgKeys][2];
  __shared__ int lovf[kAsgKeys];
  __shared__ int2 lst[kAsgKeys][2][kAsgCap];   // one list per key and lane half (one writer each)
  __shared__ float ths[kAsgKeys];
  __shared__ unsigned long long best[kAsgKeys];
  // the three-slot ring of screen tiles; after the screen it holds the refine pairs
  constexpr int kRingBytes = 3 * NF * 1024;
  static_assert(kRingBytes >= kAsgKeys * 4 * (int)sizeof(int2), "pairs fit the ring");
  __shared__ __attribute__((aligned(16))) char ring[kRingBytes];
  int2* const pairs = reinterpret_cast<int2*>(ring);
  __shared__ int npairs;
  __shared__ __attribute__((aligned(16))) float ccs[PARK_MAX_CLUSTERS];
  __shared__ int kidx[kAsgKeys];   // key index of each slot (-1 past N)
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.y, k0 = blockIdx.x * kAsgKeys;
  const int nT = nkp >> 5;
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
  int t0 = 0;
  if (wlab) t0 = __builtin_amdgcn_readfirstlane(min(max(wlab[(size_t)bh * gridDim.x + blockIdx.x], 0), nkp - 1) >> 5);

  // The 32-cluster tiles of the screen operand (fragment-major: 1 KB per fragment) pass through
  // a three-slot LDS ring shared by the workgroup's waves: the tile of turn i sits in slot
  // i % 3, each wave copies NF / 4 of its fragments two turns ahead, and one barrier per turn
  // both publishes a tile and frees the slot the next copy refills.  Every fragment crosses
  // the memory path once per workgroup instead of once per wave.  The first three turns are
  // copied before the keys are loaded, so that the two overlap.
  // tile of turn i (rotated start)
  auto tile_of = [&](int i) { const int j = t0 + i; return j >= nT ? j - nT : j; };
  constexpr int FPW = NF / kAsgWaves;   // fragments each wave copies per turn
  static_assert(FPW * kAsgWaves == NF, "fragments per wave");
  const char* gtiles = reinterpret_cast<const char*>(gneg2 + (size_t)bh * nkp * D);
  const uint32_t ring0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring;
  auto copy_turn = [&](int i) {
    const char* src = gtiles + (size_t)tile_of(i) * NF * 1024;
    const uint32_t dst = ring0 + (uint32_t)((i % 3) * NF * 1024);
#pragma unroll
    for (int f = 0; f < FPW; ++f) {
      const int kc = w * FPW + f;
      dma16(src + kc * 1024, (uint32_t)lane * 16u, dst + (uint32_t)kc * 1024u);
    }
  };
  copy_turn(0);
  if (nT > 1) copy_turn(1);
  if (nT > 2) copy_turn(2);

  // B fragments of this wave's 64 keys (two 32-key tiles) and their bounds: every load in
  // flight at once (branch-free: slots past N load key 0 and take zeros)
  f16x8 bfr[2][NF];
  float E[2];
  bool exact_all[2];
  const float G = __uint_as_float(hmax[4 * bh]), F = __uint_as_float(hmax[4 * bh + 1]);
  const float CC = __uint_as_float(hmax[4 * bh + 2]);
  // the keys of slots 64 w + l32 and 64 w + 32 + l32 (-1 past N)
  const int keyi[2] = {__shfl(kslot, l32), __shfl(kslot, 32 + l32)};
  float4 kn[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int pos = k0 + 64 * w + 32 * kt + l32;
    const int key = pos < N ? keyi[kt] : 0;
    kn[kt] = knorm[(size_t)bh * N + key];
#pragma unroll
    for (int kc = 0; kc < NF; ++kc) {
      const size_t off = ((size_t)bh * N + key) * D + 16 * kc + 8 * h;
      if constexpr (KF32) bfr[kt][kc] = load_f32x8_as_f16(reinterpret_cast<const float*>(Kv) + off);
      else bfr[kt][kc] = load_bf16x8_as_f16(reinterpret_cast<const bf16*>(Kv) + off);
    }
  }
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const bool real = k0 + 64 * w + 32 * kt + l32 < N;
    // (only a key tile that runs past N has slots to clear: a wave-uniform test, so the other
    // tiles skip the 64 selects)
    if (k0 + 64 * w + 32 * kt + 32 > N) {
#pragma unroll
      for (int kc = 0; kc < NF; ++kc)
#pragma unroll
        for (int i = 0; i < 8; ++i) bfr[kt][kc][i] = real ? bfr[kt][kc][i] : (f16)0.0f;
    }
    // the second term covers the float accumulation of 129 terms (< 2^-16.9 of their
    // magnitudes), the rounding of |c~|^2 and of the stored k~, with a factor-7 margin
    const float4 k4 = kn[kt];
    float e = 2.0f * (k4.y * G + k4.x * F + k4.y * F) + (1.0f / 16384.0f) * (2.0f * k4.x * G + CC + k4.z * k4.z);
    e *= 2.0f * (1.0f + 1.0f / 65536.0f);  // the window is twice the bound
    // no finite bound: no candidates, the exact comparison of every cluster instead
    exact_all[kt] = real && !(e <= 3.0e38f && G < 16384.0f);
    E[kt] = !real ? 0.0f : (exact_all[kt] ? -INFINITY : e);
  }
  // Running minimum and candidate lists.  From the second step on the keys are visited in the
  // previous step's label order, so the workgroup's keys share a few consecutive previous
  // clusters; the screen starts at the 32-cluster tile holding the previous cluster of the
  // workgroup's first key (wlab), which makes the running minimum tight from the first tile
  // on.  The candidate set does not depend on the tile order: every score within the final
  // window is recorded whatever its turn (the window only shrinks).
  float mr[2] = {INFINITY, INFINITY};
  int cnt[2] = {0, 0};          // entries in this lane's list of each key (kept in registers)
  bool ovf[2] = {exact_all[0], exact_all[1]};
#pragma unroll
  for (int i = 0; i < MV; ++i)
    if (tid + i * kAsgKeys < nkp) ccs[tid + i * kAsgKeys] = cvv[i];
  kidx[tid] = kslot;
  lovf[tid] = 0;
  best[tid] = ~0ull;
  __syncthreads();

  // the screen products of turn i's tile into acc
  auto products = [&](int i, const f16x8 (&a)[NF], f32x16 (&acc)[2]) {
    const int t = tile_of(i);
    f32x16 init;
#pragma unroll
    for (int g = 0; g < 4; ++g) {  // rows 8g + 4h + 0..3 of the tile
      const f32x4 c = *reinterpret_cast<const f32x4*>(&ccs[32 * t + 8 * g + 4 * h]);
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) init[4 * g + i2] = c[i2];
    }
    acc[0] = mfma32(a[0], bfr[0][0], init);
    acc[1] = mfma32(a[0], bfr[1][0], init);
#pragma unroll
    for (int kc = 1; kc < NF; ++kc) {
      acc[0] = mfma32(a[kc], bfr[0][kc], acc[0]);
      acc[1] = mfma32(a[kc], bfr[1][kc], acc[1]);
    }
  };
  // minima of turn i's products per key (lane halves combined), into tm
  auto minima = [&](const f32x16 (&acc)[2], float (&tm)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float x = fminf(fminf(acc[kt][0], acc[kt][1]), acc[kt][2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) x = fminf(fminf(x, acc[kt][r]), acc[kt][r + 1]);
      tm[kt] = xor32_min(fminf(x, acc[kt][15]));
    }
  };
  // running minimum and candidate lists from turn i's products and minima
  auto candidates = [&](int i, const f32x16 (&acc)[2], const float (&tm)[2]) {
    const int t = tile_of(i);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      mr[kt] = fminf(mr[kt], tm[kt]);
      const float th = mr[kt] + E[kt];
      if (__any(tm[kt] <= th)) {
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
  // fragments of turn i from its slot
  auto read_turn = [&](int i, f16x8 (&a)[NF]) {
    const f16x8* tl = reinterpret_cast<const f16x8*>(ring + (i % 3) * NF * 1024);
#pragma unroll
    for (int kc = 0; kc < NF; ++kc) a[kc] = tl[kc * 64 + lane];
  };
  // Software pipeline over the turns (two named sets of fragment and product registers, the
  // loop unrolled by two).  Iteration i: a barrier (before it every wave has its LDS reads
  // returned and its copies of turn i + 2 landed; after it turn i + 2 is whole and the slot of
  // turn i + 1, read an iteration earlier, is free for the copy of turn i + 4); then, as one
  // block whose instructions are interleaved (scheduling group barriers), the products of turn
  // i + 1, the LDS reads of turn i + 2 and the minima of turn i's products, so the matrix
  // unit works on the next tile while the vector unit reduces this one; last the candidate
  // lists of turn i (a branch taken only when a score falls inside a key's window).
  f16x8 fa[NF], fb[NF];
  f32x16 pa[2], pb[2];
  auto iteration = [&](int i, f16x8 (&fi)[NF], f16x8 (&fn)[NF], f32x16 (&pi)[2], f32x16 (&pn)[2]) {
    float tm[2];
    if (i + 2 < nT) {
      wait_lds();
      if (i + 3 < nT) wait_copies<FPW>(); else wait_copies<0>();
      __syncthreads();
      if (i + 4 < nT) copy_turn(i + 4);
      products(i + 1, fn, pn);
      read_turn(i + 2, fi);
      minima(pi, tm);
#pragma unroll
      for (int k = 0; k < 2 * NF; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // two VALU
        if (k < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
      }
    } else {
      if (i + 1 < nT) products(i + 1, fn, pn);
      minima(pi, tm);
    }
    candidates(i, pi, tm);
  };
  if (nT > 2) wait_copies<FPW>(); else wait_copies<0>();
  __syncthreads();
  read_turn(0, fa);
  if (nT > 1) read_turn(1, fb);
  products(0, fa, pa);
  if (nT > 3) {   // turn 3 goes to the slot of turn 0, once every wave has read it
    wait_lds();
    __syncthreads();
    copy_turn(3);
  }
  int i = 0;
  for (; i + 1 < nT; i += 2) {
    iteration(i, fa, fb, pa, pb);
    iteration(i + 1, fb, fa, pb, pa);
  }
  if (i < nT) iteration(i, fa, fb, pa, pb);
  wait_copies<0>();
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
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ wlab) {
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
  const int nwg = (N + kAsgKeys - 1) / kAsgKeys;
  for (int v = b0; v < b1; ++v) {
    const int t = tot[v];
    tot[v] = ex;
    offsets[(size_t)bh * (nk + 1) + v] = ex;
    // the next step's assignment workgroups whose first position lies in cluster v
    for (int g = (ex + kAsgKeys - 1) / kAsgKeys; g < nwg && g * kAsgKeys < ex + t; ++g) wlab[(size_t)bh * nwg + g] = v;
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

// Stable scatter of one chunk by four waves: wave w takes the chunk's keys [256 w, 256 w + 256)
// and counts them per label in LDS; the counts are turned into each wave's starting position
// per label (the chunk's base, then the waves in order), and each wave ranks its keys among
// equal labels with one ballot per label bit, 64 keys at a time, in key order.
constexpr int kScatWaves = 4;
__global__ __launch_bounds__(64 * kScatWaves) void k_sort_scatter(const int32_t* __restrict__ labels,
                                                                  const int32_t* __restrict__ hist, int N, int nk,
                                                                  int nch, int32_t* __restrict__ perm) {
  extern __shared__ int wpos[];   // [kScatWaves][nk]: keys per label, then starting positions
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, bh = blockIdx.y, ch = blockIdx.x;
  const int nbits = nk > 1 ? 32 - __builtin_clz((unsigned)(nk - 1)) : 0;   // bits of a label
  constexpr int kSteps = kSortChunk / (64 * kScatWaves);
  static_assert(kSteps * 64 * kScatWaves == kSortChunk, "chunk split");
  const int j0 = ch * kSortChunk + w * (kSortChunk / kScatWaves);
  int labs[kSteps];
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int j = j0 + 64 * st + lane;
    labs[st] = j < N ? labels[(size_t)bh * N + j] : -1;
  }
  for (int v = tid; v < kScatWaves * nk; v += 64 * kScatWaves) wpos[v] = 0;
  __syncthreads();
#pragma unroll
  for (int st = 0; st < kSteps; ++st)
    if (labs[st] >= 0) atomicAdd(&wpos[w * nk + labs[st]], 1);
  __syncthreads();
  for (int v = tid; v < nk; v += 64 * kScatWaves) {
    int b = hist[((size_t)bh * nch + ch) * nk + v];
#pragma unroll
    for (int ww = 0; ww < kScatWaves; ++ww) {
      const int t = wpos[ww * nk + v];
      wpos[ww * nk + v] = b;
      b += t;
    }
  }
  __syncthreads();
  int* cur = wpos + w * nk;   // this wave's next position per label
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int j = j0 + 64 * st + lane;
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
    // (a wave's LDS accesses complete in order: every lane reads its label's position before
    // the last lane of the label moves it, and the next step reads the moved value)
    if (lab >= 0) {
      const int pos = cur[lab] + rank;
      perm[(size_t)bh * N + pos] = j;
      if (last) cur[lab] = pos + 1;
    }
  }
}

// ---------------------------------------------------------------------------------------
// a6/a7: per-cluster update, step 1: member sums.  One 256-thread workgroup per cluster;
// the members (a run of perm) are read 16 bytes per thread, RPI rows at a time; each thread
// sums its dimensions in double over its rows, and the RPI partial sums are added in a
// fixed order, so the result does not depend on scheduling.  Writes the original-space mean
// (double) for step 2, the sum (csum, when given) for the next k-means step's update and,
// on the last iteration, the float centroid output (0 if empty).
template <int D, typename T>
__global__ __launch_bounds__(256) void k_km_sums(const T* __restrict__ K, const int32_t* __restrict__ perm,
                                                 const int32_t* __restrict__ offsets, int N, int nk, int nkp,
                                                 double* __restrict__ cmean, double* __restrict__ csum,
                                                 float* __restrict__ cent) {
  constexpr int TPR = D / 8;         // threads per row (8 dimensions each)
  constexpr int RPI = 256 / TPR;     // rows in flight per step
  __shared__ double part[RPI][D];
  const int v = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int a = offsets[(size_t)bh * (nk + 1) + v], b = offsets[(size_t)bh * (nk + 1) + v + 1];
  const int n = b - a;
  if (n == 0) {
    if (cent && tid < D) cent[((size_t)bh * nk + v) * D + tid] = 0.0f;
    if (csum && tid < D) csum[((size_t)bh * nkp + v) * D + tid] = 0.0;
    return;
  }
  const int32_t* pm = perm + (size_t)bh * N + a;
  const T* Kh = K + (size_t)bh * N * D;
  const int rg = tid / TPR, c8 = (tid % TPR) * 8;
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  // rows rg, rg + RPI, ... in order, U at a time: their member indices, then their values,
  // all in flight together (branch-free: indices clamped to the cluster, rows past it add 0)
  constexpr int U = 8;
  for (int r0 = rg; r0 < n; r0 += U * RPI) {
    int src[U];
#pragma unroll
    for (int u = 0; u < U; ++u) src[u] = pm[min(r0 + u * RPI, n - 1)];
    float x[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const T* row = Kh + (size_t)src[u] * D + c8;
      if constexpr (sizeof(T) == 2) {
        const bf16x8 q = load_bf16x8(reinterpret_cast<const bf16*>(row));
#pragma unroll
        for (int i = 0; i < 8; ++i) x[u][i] = (float)q[i];
      } else {
        const f32x4 q0 = *reinterpret_cast<const f32x4*>(row);
        const f32x4 q1 = *reinterpret_cast<const f32x4*>(row + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[u][i] = q0[i]; x[u][4 + i] = q1[i]; }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = r0 + u * RPI < n;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += in ? (double)x[u][i] : 0.0;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[rg][c8 + i] = acc[i];
  __syncthreads();
  if (tid < D) {
    double sum = 0.0;
    for (int g = 0; g < RPI; ++g) sum += part[g][tid];
    const double m = sum / (double)n;
    cmean[((size_t)bh * nkp + v) * D + tid] = m;
    if (csum) csum[((size_t)bh * nkp + v) * D + tid] = sum;
    if (cent) cent[((size_t)bh * nk + v) * D + tid] = (float)m;
  }
}

// a6 from the second k-means step on, for bf16 keys: a cluster's member sum changes only by
// the keys that joined it (members now, of another cluster before) and the keys that left it
// (members before, of another cluster now), so csum_v += sum(joined) - sum(left), and the
// mean is csum_v / n_v as before.  A sum of bf16 values in double is exact while the partial
// sums stay within 53 bits of the smallest term's last place (for these key magnitudes, terms
// of magnitude 2^-24 and up), so the carried sum equals the sum over the current members; in
// late steps only a few percent of the keys change cluster, and only their rows are read.
// One wave per cluster (four per workgroup), every step's loads issued together: the two
// member runs (now, then before) are walked as one list, the member indices and labels of 256
// positions at a time; the changed keys of each 64-position window are compacted in list
// order into LDS, and their rows read 16 bytes per lane, four rows per instruction, up to 8
// rows in flight; lane l adds the rows of the window's list positions = l / 16 (mod 4), in
// order, for dimensions 8 (l % 16) .. + 7, and the four row groups are added by a fixed
// butterfly at the end.  Writes csum and, for a
// non-empty cluster, the mean; on the last iteration the float centroid output (0 if empty).
template <int D>
__global__ __launch_bounds__(256) void k_km_sums_delta(const bf16* __restrict__ K, const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ labels,
                                                       const int32_t* __restrict__ perm_prev,
                                                       const int32_t* __restrict__ offsets_prev,
                                                       const int32_t* __restrict__ labels_prev, int N, int nk,
                                                       int nkp, double* __restrict__ cmean,
                                                       double* __restrict__ csum, float* __restrict__ cent) {
  static_assert(D == 64 || D == 128, "head dimension");
  constexpr int LPR = D / 8;        // lanes per row (16 bytes each)
  constexpr int RPW = 64 / LPR;     // rows per wave instruction
  constexpr int U = 2;              // row instructions in flight
  __shared__ int clist[4][64];      // per wave: changed keys of the window, sign in bit 31
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, bh = blockIdx.y;
  const int v = blockIdx.x * 4 + w;
  if (v >= nk) return;              // (whole waves; no workgroup barrier below)
  const int32_t* on = offsets + (size_t)bh * (nk + 1);
  const int32_t* op = offsets_prev + (size_t)bh * (nk + 1);
  const int an = on[v], bn = on[v + 1], ap = op[v], bp = op[v + 1];
  const int nn = bn - an, ntot = nn + (bp - ap);
  const int rl = lane / LPR, c8 = (lane % LPR) * 8;
  const size_t crow = ((size_t)bh * nkp + v) * D + c8;
  const bf16* Kh = K + (size_t)bh * N * D;
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  constexpr int XW = 4;             // list windows of 64 positions whose loads go out together
  for (int x0 = 0; x0 < ntot; x0 += 64 * XW) {
    int jj[XW], oth[XW];
#pragma unroll
    for (int q = 0; q < XW; ++q) {   // the run now (joined keys), then the run before (left keys)
      const int x = min(x0 + 64 * q + lane, ntot - 1);
      const bool joined = x < nn;
      const int pos = joined ? an + x : ap + (x - nn);
      jj[q] = min(max((joined ? perm : perm_prev)[(size_t)bh * N + pos], 0), N - 1);
    }
#pragma unroll
    for (int q = 0; q < XW; ++q) {
      const bool joined = min(x0 + 64 * q + lane, ntot - 1) < nn;
      oth[q] = (joined ? labels_prev : labels)[(size_t)bh * N + jj[q]];
    }
#pragma unroll
    for (int q = 0; q < XW; ++q) {
    const int x = x0 + 64 * q + lane;
    if (x0 + 64 * q >= ntot) break;   // (uniform)
    int key = -1, neg = 0;
    if (x < ntot && oth[q] != v) { key = jj[q]; neg = x < nn ? 0 : 1; }
    const uint64_t m = __ballot(key >= 0);
    const int nch = __builtin_popcountll(m);
    if (key >= 0) clist[w][__builtin_popcountll(m & ((1ull << lane) - 1))] = key | (neg << 31);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int r0 = 0; r0 < nch; r0 += U * RPW) {
      float xv[U][8];
      int sg[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * RPW + rl;
        const int e = clist[w][min(r, nch - 1)];
        sg[u] = r < nch ? ((e < 0) ? -1 : 1) : 0;
        const bf16x8 q = load_bf16x8(Kh + (size_t)(e & 0x7FFFFFFF) * D + c8);
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[u][i] = (float)q[i];
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += sg[u] > 0 ? (double)xv[u][i] : (sg[u] < 0 ? -(double)xv[u][i] : 0.0);
    }
    __builtin_amdgcn_wave_barrier();   // the list is rewritten by the next window
    }
  }
  // the row groups' partial sums, by a fixed butterfly over the lanes of equal c8
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], o);
  if (rl == 0) {
    const bool live = nn > 0;
    double sm[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sm[i] = csum[crow + i] + acc[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) csum[crow + i] = sm[i];
    if (live)
#pragma unroll
      for (int i = 0; i < 8; ++i) cmean[crow + i] = sm[i] / (double)nn;
    if (cent)
#pragma unroll
      for (int i = 0; i < 8; ++i) cent[((size_t)bh * nk + v) * D + c8 + i] = live ? (float)(sm[i] / (double)nn) : 0.0f;
  }
}

// Step 2, per (32-cluster tile, head): c~_v = R^T mean_v rounded to float (or, for the
// initial centroids, c~_v as stored), then the screen operand g_v = R c~_v in double,
// gneg2 = fp16(-2 g) (fragment-major), |c~|^2, |g|, |g - fp16(g)|.  Clusters without keys
// keep everything from the previous step; padding rows (v >= nk) get |c~|^2 = +inf.
// Both products are double GEMMs on the matrix cores (16 x 16 x 4 double MFMAs): wave w takes
// the 16 clusters v0 + 16 (w & 1) .. + 15 and the D / 2 columns of half w >> 1, as D / 32
// output blocks of 16 columns.  Lane l holds the A element (cluster l % 16, k) and the B
// element (k, column l % 16) for k in [(l / 16) KS, (l / 16 + 1) KS), KS = D / 4, one k of
// that range per MFMA step, so each lane reads contiguous rows: the means (or c~), and rows
// of R^T (first product) or R (second).  The MFMA output element (cluster 4 r + l / 16,
// column l % 16) sits in lane l, register r.
template <int D>
__global__ __launch_bounds__(256, 2) void k_km_ctx(const double* __restrict__ cmean, const int32_t* __restrict__ counts,
                                                    int nk, int nkp, int init_mode, const double* __restrict__ R64,
                                                    const double* __restrict__ Rt64, float* __restrict__ ctil,
                                                    f16* __restrict__ gneg2, float4* __restrict__ cinfo,
                                                    float* __restrict__ ccv) {
  constexpr int NBW = D / 32;  // 16-column output blocks per wave
  constexpr int KS = D / 4;    // MFMA steps
  constexpr int SP = 2;        // steps per B load (16 bytes per lane and block)
  __shared__ __attribute__((aligned(16))) float cs[32][D + 4];   // c~ of the tile's clusters
  __shared__ __attribute__((aligned(16))) f16 gs[32][D + 8];     // fp16(-2 g) of the tile's clusters
  __shared__ double red[2][32][2];     // per column half: |g|^2 and residual sums of each cluster
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, lg = lane >> 4;
  const int cg = w & 1, ch = w >> 1;
  const int bh = blockIdx.y, t0 = blockIdx.x * 32, v0 = t0 + 16 * cg;
  const int k0 = lg * KS;
  // live32 bit c: cluster t0 + c has keys (or is an initial centroid); write32 bit c: its
  // outputs are written (live, or a padding row)
  const int vl = t0 + (lane & 31);
  const bool lv = vl < nk && (init_mode || counts[(size_t)bh * nk + vl] > 0);
  const uint32_t live32 = (uint32_t)__ballot(lv && lane < 32);
  const uint32_t write32 = (uint32_t)__ballot((lv || vl >= nk) && lane < 32);
  // out[b] = A (a[s], step s) x B (row 16 (NBW ch + b) + l % 16 of M, columns k0 + s)
  auto gemm = [&](const double (&a)[KS], const double* __restrict__ M, f64x4 (&out)[NBW]) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < NBW; ++b) out[b] = f64x4{0.0, 0.0, 0.0, 0.0};
    const double* mrow = M + (size_t)bh * D * D + (size_t)(16 * NBW * ch + li) * D + k0;
    // B in chunks of SP steps (16 bytes per lane and block), kAhead chunks in flight; scheduling
    // fences keep each chunk's loads together and ahead of the MFMAs
    constexpr int kAhead = 3, NC = KS / SP;
    f64x2 bq[kAhead + 1][NBW];
#pragma unroll
    for (int c = 0; c < kAhead; ++c)
#pragma unroll
      for (int b = 0; b < NBW; ++b) bq[c][b] = *reinterpret_cast<const f64x2*>(mrow + (size_t)16 * b * D + SP * c);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      __builtin_amdgcn_sched_barrier(0);
      if (c + kAhead < NC) {
#pragma unroll
        for (int b = 0; b < NBW; ++b)
          bq[(c + kAhead) % (kAhead + 1)][b] = *reinterpret_cast<const f64x2*>(mrow + (size_t)16 * b * D + SP * (c + kAhead));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ss = 0; ss < SP; ++ss)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
          out[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[SP * c + ss], bq[c % (kAhead + 1)][b][ss], out[b], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  double a[KS];
  if (init_mode) {
    const float* src = ctil + ((size_t)bh * nkp + v0 + li) * D + k0;
#pragma unroll
    for (int s = 0; s < KS; s += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + s);
#pragma unroll
      for (int u = 0; u < 4; ++u) a[s + u] = (double)x[u];
    }
  } else {
    // first product: c~ = R^T m, i.e. c~[v][i] = sum_k m[v][k] Rt[i][k]
    const bool real = v0 + li < nk;
    const double* src = cmean + ((size_t)bh * nkp + v0 + li) * D + k0;
#pragma unroll
    for (int s = 0; s < KS; s += 2) {
      const f64x2 x = real ? *reinterpret_cast<const f64x2*>(src + s) : f64x2{0.0, 0.0};
      a[s] = x[0];
      a[s + 1] = x[1];
    }
    f64x4 t[NBW];
    gemm(a, Rt64, t);
#pragma unroll
    for (int b = 0; b < NBW; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) cs[16 * cg + 4 * r + lg][16 * (NBW * ch + b) + li] = (float)t[b][r];
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KS; s += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(&cs[16 * cg + li][k0 + s]);
#pragma unroll
      for (int u = 0; u < 4; ++u) a[s + u] = (double)x[u];
    }
    // c~ of the live clusters to ctil, 16 bytes per store (piece p: row p / (D / 4), columns
    // 4 (p % (D / 4)) .. + 3)
#pragma unroll
    for (int q = 0; q < (32 * D / 4) / 256; ++q) {
      const int p = tid + 256 * q, row = p / (D / 4), c4 = 4 * (p % (D / 4));
      if ((live32 >> row) & 1)
        *reinterpret_cast<f32x4*>(ctil + ((size_t)bh * nkp + t0 + row) * D + c4) =
            *reinterpret_cast<const f32x4*>(&cs[row][c4]);
    }
  }
  // |c~|^2 of cluster v0 + li: this lane's KS columns in order, then the four column ranges
  double cc = 0.0;
#pragma unroll
  for (int s = 0; s < KS; ++s) cc += a[s] * a[s];
  cc += __shfl_xor(cc, 16);
  cc += __shfl_xor(cc, 32);
  // second product: g = R c~, i.e. g[v][i] = sum_k c~[v][k] R[i][k]
  f64x4 g[NBW];
  gemm(a, R64, g);
  // fp16(-2 g) into LDS; the per-cluster |g|^2 and residual sums of this column half: columns
  // in block order per lane, then the 16 lanes of the cluster's group by a fixed butterfly
  double gn[4] = {0.0, 0.0, 0.0, 0.0}, fr[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int b = 0; b < NBW; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = 16 * cg + 4 * r + lg, i = 16 * (NBW * ch + b) + li;
      const double gv = g[b][r];
      const f16 gb = (f16)(float)gv;
      const double df = gv - (double)(float)gb;
      gn[r] += gv * gv;
      fr[r] += df * df;
      gs[c][i] = t0 + c < nk ? (f16)(-2.0f * (float)gb) : (f16)0.0f;
    }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      gn[r] += __shfl_xor(gn[r], o);
      fr[r] += __shfl_xor(fr[r], o);
    }
  if (li < 4) {   // lane (li = r, lg) holds cluster 4 r + lg's sums
    double gsel = gn[0], fsel = fr[0];
#pragma unroll
    for (int r = 1; r < 4; ++r) {
      gsel = li == r ? gn[r] : gsel;
      fsel = li == r ? fr[r] : fsel;
    }
    red[ch][16 * cg + 4 * li + lg][0] = gsel;
    red[ch][16 * cg + 4 * li + lg][1] = fsel;
  }
  __syncthreads();
  // gneg2 of the written rows: the tile's D / 16 fragments (1 KB each, contiguous), 16 bytes
  // per store: lane l of fragment kc holds row l % 32, columns 16 kc + 8 (l / 32) .. + 7
#pragma unroll
  for (int q = 0; q < (32 * D / 8) / 256; ++q) {
    const int p = tid + 256 * q, kc = p >> 6, l = p & 63, row = l & 31, col = 16 * kc + 8 * (l >> 5);
    if ((write32 >> row) & 1)
      *reinterpret_cast<f16x8*>(gneg2 + (size_t)bh * nkp * D + frag_lane(blockIdx.x, kc, l, D)) =
          *reinterpret_cast<const f16x8*>(&gs[row][col]);
  }
  // lane c < 16 of the first column half writes cluster v0 + c (column halves added in order)
  if (ch == 0 && lg == 0) {
    const int v = v0 + li, c = 16 * cg + li;
    const double gnc = red[0][c][0] + red[1][c][0];
    const double frc = red[0][c][1] + red[1][c][1];
    if (v >= nk) {
      cinfo[(size_t)bh * nkp + v] = make_float4(INFINITY, 0.0f, 0.0f, 0.0f);
      ccv[(size_t)bh * nkp + v] = INFINITY;
    } else if ((live32 >> c) & 1) {
      const float up = 1.0f + 1.0f / 1048576.0f;
      const float4 ci = make_float4((float)cc, (float)sqrt(gnc) * up, (float)sqrt(frc) * up, 0.0f);
      cinfo[(size_t)bh * nkp + v] = ci;
      ccv[(size_t)bh * nkp + v] = ci.x;
    }
  }
}

// ---------------------------------------------------------------------------------------
template <int D>
static hipError_t launch_assign(const Shape& s, const ClusterWs& w, const void* K, const int32_t* order,
                                const int32_t* wlab, int32_t* labels, hipStream_t st) {
  dim3 grid((s.N + kAsgKeys - 1) / kAsgKeys, s.BH);
  if (s.dtype == 0)
    k_km_assign<D, true><<<grid, 64 * kAsgWaves, 0, st>>>(K, w.Kt, w.knorm, w.ctil, w.gneg2, w.ccv, w.hmax, s.N, s.nk,
                                                         w.nkp, order, wlab, labels);
  else
    k_km_assign<D, false><<<grid, 64 * kAsgWaves, 0, st>>>(K, w.Kt, w.knorm, w.ctil, w.gneg2, w.ccv, w.hmax, s.N,
                                                          s.nk, w.nkp, order, wlab, labels);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_cluster_d(const Shape& s, const void* Q, const void* K, int iters, int metric, float alpha,
                                   const int32_t* init_idx, float* cent, int32_t* counts, int32_t* labels,
                                   int32_t* perm, int32_t* offsets, int32_t* status, const ClusterWs& w,
                                   hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
  const bool f32 = s.dtype == 0;
  hipError_t e;
#define PARK_CHECK() do { e = hipGetLastError(); if (e != hipSuccess) return e; } while (0)
  if (metric == 0) {
    dim3 grid(w.nch_g, s.BH);
    if (f32) k_gram_f32<D><<<grid, 256, 0, st>>>(reinterpret_cast<const float*>(Q), s.N, w.nch_g, w.gpart);
    else k_gram_bf16<D><<<grid, 64 * (D / 32) * (D / 32), 0, st>>>(reinterpret_cast<const bf16*>(Q), s.N, w.nch_g, w.gpart);
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
  // Labels, perm, offsets and counts alternate between the caller's arrays and the workspace
  // from step to step (the last step writes the caller's), so that each step's update sees
  // the previous step's clustering beside its own.
  int32_t* const lab2[2] = {labels, w.lalt};
  int32_t* const perm2[2] = {perm, w.palt};
  int32_t* const off2[2] = {offsets, w.oalt};
  int32_t* const cnt2[2] = {counts, w.calt};
  for (int it = 0; it < iters; ++it) {
    const int cur = (iters - 1 - it) & 1, prv = cur ^ 1;
    // from the second step on, the keys are visited in the previous step's label order (perm)
    const bool timed = it == iters - 1;
    if (timed && ev_begin && (e = hipEventRecord(ev_begin, st)) != hipSuccess) return e;
    e = launch_assign<D>(s, w, K, it > 0 ? perm2[prv] : nullptr, it > 0 ? w.wlab : nullptr, lab2[cur], st);
    if (e != hipSuccess) return e;
    if (timed && ev_end && (e = hipEventRecord(ev_end, st)) != hipSuccess) return e;
    k_sort_hist<<<dim3(w.nch_s, s.BH), 256, shm_nk, st>>>(lab2[cur], s.N, s.nk, w.nch_s, w.hist);
    PARK_CHECK();
    k_sort_scan<<<s.BH, 1024, shm_nk, st>>>(w.hist, s.N, s.nk, w.nch_s, cnt2[cur], off2[cur], w.wlab);
    PARK_CHECK();
    k_sort_scatter<<<dim3(w.nch_s, s.BH), 64 * kScatWaves, kScatWaves * shm_nk, st>>>(lab2[cur], w.hist, s.N, s.nk,
                                                                                   w.nch_s, perm2[cur]);
    PARK_CHECK();
    float* co = (it == iters - 1) ? cent : nullptr;
    // carried sums (one wave per cluster walks both member runs) pay off for small clusters;
    // clusters of more than 128 keys on average (the query blocks' k-means, say) are summed
    // afresh by a workgroup each
    const bool carry = (long long)s.N <= 128LL * s.nk;
    if (f32)
      k_km_sums<D, float><<<dim3(s.nk, s.BH), 256, 0, st>>>(reinterpret_cast<const float*>(K), perm2[cur], off2[cur],
                                                            s.N, s.nk, w.nkp, w.cmean, nullptr, co);
    else if (it == 0 || !carry)
      k_km_sums<D, bf16><<<dim3(s.nk, s.BH), 256, 0, st>>>(reinterpret_cast<const bf16*>(K), perm2[cur], off2[cur],
                                                           s.N, s.nk, w.nkp, w.cmean, w.csum, co);
    else
      k_km_sums_delta<D><<<dim3((s.nk + 3) / 4, s.BH), 256, 0, st>>>(reinterpret_cast<const bf16*>(K), perm2[cur],
                                                                     off2[cur], lab2[cur], perm2[prv], off2[prv],
                                                                     lab2[prv], s.N, s.nk, w.nkp, w.cmean, w.csum, co);
    PARK_CHECK();
    if (it + 1 < iters) {  // the transformed centroids only feed the next assignment
      k_km_ctx<D><<<dim3(w.nkp / 32, s.BH), 256, 0, st>>>(w.cmean, cnt2[cur], s.nk, w.nkp, 0, w.R64, w.Rt64, w.ctil,
                                                          w.gneg2, w.cinfo, w.ccv);
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
                          int32_t* offsets, int32_t* status, void* ws, hipStream_t st, hipEvent_t ev_begin,
                          hipEvent_t ev_end) {
  const ClusterWs w = carve(s, ws);
  if (s.d == 128)
    return launch_cluster_d<128>(s, Q, K, iters, metric, alpha, init_idx, cent, counts, labels, perm, offsets, status, w,
                                 st, ev_begin, ev_end);
  return launch_cluster_d<64>(s, Q, K, iters, metric, alpha, init_idx, cent, counts, labels, perm, offsets, status, w,
                              st, ev_begin, ev_end);
}

}  // namespace park
