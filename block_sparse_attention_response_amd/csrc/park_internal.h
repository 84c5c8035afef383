// Internal launch interface between the libpark host code and its kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace park {

// Shape of one call: B*H independent heads of N tokens of dimension d.
struct Shape {
  int BH, N, d, nk;  // nk = number of key clusters
  int dtype;         // 0 float, 1 bfloat16
};

inline int nk_pad32(int nk) { return (nk + 31) / 32 * 32; }
inline int n_qblocks(int N) { return (N + 63) / 64; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ----- retrieval (PAMA, pooled baseline, selection)
size_t retrieve_workspace(const Shape& s, bool need_scores);
hipError_t launch_retrieve(const Shape& s, const void* Q, const float* cent, const int32_t* counts,
                           float scale, float top_p, int top_k, bool pooled, float* scores,
                           uint8_t* mask, int32_t* list, int32_t* count, void* ws, hipStream_t st);

// ----- block-sparse attention
size_t attn_workspace(const Shape& s);
hipError_t launch_attn(const Shape& s, const void* Q, const void* K, const void* V, const int32_t* perm,
                       const int32_t* offsets, const int32_t* list, const int32_t* count, float scale,
                       void* O, float* lse, void* ws, hipStream_t st, hipEvent_t ev_begin = nullptr,
                       hipEvent_t ev_end = nullptr);

// ----- key clustering
size_t cluster_workspace(const Shape& s);
hipError_t launch_cluster(const Shape& s, const void* Q, const void* K, int iters, int metric,
                          float alpha, const int32_t* init_idx, float* cent, int32_t* counts,
                          int32_t* labels, int32_t* perm, int32_t* offsets, int32_t* status,
                          void* ws, hipStream_t st);

}  // namespace park
