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

// Clustered query blocks: block u of head bh holds the queries
// qperm[bh][qoffsets[bh][u] .. qoffsets[bh][u+1]) (n_u of them).  Kernels walk a block as
// chunks of at most 64 consecutive positions; a head has at most chunk_slots() chunks.
struct QueryBlocks {
  const int32_t* qperm;     // [BH][N]
  const int32_t* qoffsets;  // [BH][NQ+1]
  int NQ;                   // query blocks per head
};
inline int chunk_slots(int N, int NQ) { return n_qblocks(N) + NQ; }

// Chunk tables of clustered query blocks, per head: chunks[c] = (block u, first position,
// count, 0) for c < ctotal, blocks in order; cbase[u] = first chunk of block u
// (cbase[NQ] = ctotal).  Offsets are clamped to [0, N], so inconsistent ones cannot lead to
// an access out of range.
hipError_t launch_qchunks(const int32_t* qoffsets, int BH, int N, int NQ, int maxc, int4* chunks,
                          int32_t* cbase, int32_t* ctotal, hipStream_t st);

// ----- retrieval (PAMA, pooled baseline, selection)
size_t retrieve_workspace(const Shape& s, bool need_scores);
// online: SCOPE's online per-head top-k floor on top of the fixed one; probs [BH][N][nk] (or
// NULL): the unfused ablation, which materialises the probabilities there and averages them in
// a second kernel
// ev_begin / ev_end (optional): recorded on st right before and after the fused PAMA kernel
hipError_t launch_retrieve(const Shape& s, const void* Q, const float* cent, const int32_t* counts,
                           float scale, float top_p, int top_k, bool pooled, float* scores,
                           uint8_t* mask, int32_t* list, int32_t* count, void* ws, hipStream_t st,
                           bool online = false, float* probs = nullptr, hipEvent_t ev_begin = nullptr,
                           hipEvent_t ev_end = nullptr);
// PAMA and the same selection over clustered query blocks
size_t retrieve_clustered_workspace(const Shape& s, int NQ, bool need_scores);
hipError_t launch_retrieve_clustered(const Shape& s, const void* Q, const float* cent, const int32_t* counts,
                                     const QueryBlocks& qb, float scale, float top_p, int top_k, float* scores,
                                     uint8_t* mask, int32_t* list, int32_t* count, void* ws, hipStream_t st,
                                     bool online = false);

// ----- block-sparse attention
// qb == nullptr: 64-token query blocks; otherwise clustered query blocks.  The heads are
// computed in attn_passes() passes of at most attn_heads_per_pass() heads; the workspace holds
// one pass.  ev_begin[p] / ev_end[p] (optional, p < n_events): recorded on st right before and
// after pass p's attention kernel.
int attn_heads_per_pass(const Shape& s, const QueryBlocks* qb = nullptr);
int attn_passes(const Shape& s, const QueryBlocks* qb = nullptr);
size_t attn_workspace(const Shape& s, const QueryBlocks* qb = nullptr);
hipError_t launch_attn(const Shape& s, const void* Q, const void* K, const void* V, const int32_t* perm,
                       const int32_t* offsets, const int32_t* list, const int32_t* count, float scale,
                       void* O, float* lse, void* ws, hipStream_t st, const hipEvent_t* ev_begin = nullptr,
                       const hipEvent_t* ev_end = nullptr, int n_events = 0, const QueryBlocks* qb = nullptr);

// ----- exact block importance (section 3.2, Eq. (3)) for 64-token blocks, a diagnostic
size_t importance_workspace(const Shape& s);
hipError_t launch_importance(const Shape& s, const void* Q, const void* K, const int32_t* perm,
                             const int32_t* offsets, float scale, float* W, void* ws, hipStream_t st);

// ----- centred log-mass RMSE (appendix B, M2) per head, a diagnostic (bf16 inputs)
size_t logmass_workspace(const Shape& s);
hipError_t launch_logmass(const Shape& s, const void* Q, const void* K, const int32_t* perm, const int32_t* offsets,
                          const float* cent, const int32_t* counts, float scale, float* rmse, void* ws,
                          hipStream_t st);

// ----- key clustering
size_t cluster_workspace(const Shape& s);
// ev_begin / ev_end (optional): recorded on st right before and after the last step's
// assignment kernel
hipError_t launch_cluster(const Shape& s, const void* Q, const void* K, int iters, int metric,
                          float alpha, const int32_t* init_idx, float* cent, int32_t* counts,
                          int32_t* labels, int32_t* perm, int32_t* offsets, int32_t* status,
                          void* ws, hipStream_t st, hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr);

}  // namespace park
