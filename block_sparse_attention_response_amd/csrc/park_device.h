// Device-side helpers shared by the libpark kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace park {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// 32x32x16 bf16 matrix FMA (gfx950).  Operand layout per lane l (h = l / 32):
//   A (32 x 16, row-major M x K): row l % 32, k = 8h .. 8h+7
//   B (16 x 32, K x N):           col l % 32, k = 8h .. 8h+7
//   C (32 x 32): element r of the lane is row 8 (r / 4) + 4 h + (r % 4), col l % 32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// the same shape with fp16 operands
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int c_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Fragment-major layout of a [rows][D] bf16 operand that is read as 32x16 MFMA fragments:
// the 64 lanes' 16-byte pieces of one (32-row tile, 16-column chunk) sit in 1 KB of
// contiguous memory, so every fragment load is fully coalesced.  Lane l of the fragment
// holds row 32 t + (l % 32), columns 16 kc + 8 (l / 32) .. + 7.
__device__ __forceinline__ size_t frag_offset(int row, int col, int D) {
  const int t = row >> 5, r = row & 31, kc = col >> 4, hh = (col >> 3) & 1, i = col & 7;
  return ((size_t)(t * (D / 16) + kc) * 64 + r + 32 * hh) * 8 + i;
}
// Start of the fragment (tile t, chunk kc) for lane `lane`.
__device__ __forceinline__ size_t frag_lane(int t, int kc, int lane, int D) {
  return ((size_t)(t * (D / 16) + kc) * 64 + lane) * 8;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// min of x over lanes l and l ^ 32 in one VALU exchange (v_permlane32_swap) instead of
// a round trip through the LDS crossbar: the swap of x with itself leaves lanes l and l ^ 32
// of the two results holding x_l and x_(l^32) in some order.
__device__ __forceinline__ float xor32_min(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// 8 float or bf16 values as fp16 (round to nearest even; beyond the fp16 range they become inf)
__device__ __forceinline__ f16x8 load_f32x8_as_f16(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f16x8 r;
  r[0] = (f16)a[0]; r[1] = (f16)a[1]; r[2] = (f16)a[2]; r[3] = (f16)a[3];
  r[4] = (f16)b[0]; r[5] = (f16)b[1]; r[6] = (f16)b[2]; r[7] = (f16)b[3];
  return r;
}
__device__ __forceinline__ f16x8 load_bf16x8_as_f16(const bf16* p) {
  const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (f16)(float)x[i];
  return r;
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 x) { return (float)x; }

// Butterfly reductions over the 32 lanes that share lane / 32 (masks 1..16), or over the
// whole wave (masks 1..32).
__device__ __forceinline__ float max32(float v) {
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float sum32(float v) {
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float sum64(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ double sum64d(double v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float max64(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// XCD-aware block order for grids of per-head work items (NQ items per head).  The
// dispatcher hands consecutive workgroups to the 8 XCDs in turn, so workgroup b runs on XCD
// b % 8.  This mapping gives XCD x the items [x S, (x+1) S) of each head (S = ceil(NQ / 8))
// and walks all XCDs through the heads together: the blocks in flight at any moment belong
// to one or two heads (whose packed keys and values then stay in the shared cache), and the
// neighbouring query blocks of one XCD share its L2.  The grid must have 8 S workgroups per
// head; returns false for the padding slots.
__device__ __forceinline__ bool xcd_head_sync(uint32_t bid, int NQ, int* head, int* item) {
  const int S = (NQ + 7) / 8;
  const int x = bid % 8u, slot = bid / 8u;
  *head = slot / S;
  *item = x * S + slot % S;
  return *item < NQ;
}

}  // namespace park
