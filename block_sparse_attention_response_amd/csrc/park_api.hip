// libpark C ABI: argument validation, workspace sizing and kernel launches.
#include <math.h>
#include "../../include/park.h"
#include "park_internal.h"

using park::Shape;

namespace {

bool finite_f(float x) { return isfinite(x) != 0; }

int check_common(int dtype, int B, int H, int N, int d, int n_clusters, bool* unsupported) {
  *unsupported = false;
  if (dtype != PARK_F32 && dtype != PARK_BF16) return PARK_ERR_INVALID;
  if (B < 1 || H < 1 || N < 1 || d < 1 || n_clusters < 1 || n_clusters > N) return PARK_ERR_INVALID;
  // B H N d < 2^31, multiplied one factor at a time: every partial product stays below
  // 2^31 before the next factor (< 2^31), so none overflows
  long long elems = B;
  for (const int f : {H, N, d}) {
    elems *= f;
    if (elems >= (1LL << 31)) { *unsupported = true; return PARK_ERR_UNSUPPORTED; }
  }
  if (d != 64 && d != 128) { *unsupported = true; return PARK_ERR_UNSUPPORTED; }
  if (n_clusters > PARK_MAX_CLUSTERS) { *unsupported = true; return PARK_ERR_UNSUPPORTED; }
  return PARK_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return PARK_OK;
  if (ws == nullptr || have < need) return PARK_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return PARK_ERR_WORKSPACE;
  return PARK_OK;
}

Shape make_shape(int dtype, int B, int H, int N, int d, int nk) {
  Shape s;
  s.BH = B * H; s.N = N; s.d = d; s.nk = nk; s.dtype = dtype;
  return s;
}

int retrieve_impl(bool pooled, const void* Q, int dtype, int B, int H, int N, int d, const float* centroids,
                  const int32_t* counts, int n_clusters, int q_block, float top_p, int top_k, float scale,
                  float* scores, uint8_t* mask, int32_t* block_list, int32_t* block_count, void* workspace,
                  size_t workspace_bytes, void* stream, float* probs = nullptr, void* ev_begin = nullptr,
                  void* ev_end = nullptr) {
  bool uns;
  int st = check_common(dtype, B, H, N, d, n_clusters, &uns);
  if (st != PARK_OK) return st;
  if (!Q || !centroids || !counts || !mask || !block_list || !block_count) return PARK_ERR_INVALID;
  if (!finite_f(top_p) || top_p < 0.0f || top_p > 1.0f || top_k < 0 || !finite_f(scale)) return PARK_ERR_INVALID;
  if (q_block != PARK_QUERY_BLOCK) return PARK_ERR_UNSUPPORTED;
  const Shape s = make_shape(dtype, B, H, N, d, n_clusters);
  st = check_ws(workspace, workspace_bytes, park::retrieve_workspace(s, scores == nullptr));
  if (st != PARK_OK) return st;
  if (scale <= 0.0f) scale = 1.0f / sqrtf((float)d);
  hipError_t e = park::launch_retrieve(s, Q, centroids, counts, scale, top_p, top_k, pooled, scores, mask,
                                       block_list, block_count, workspace, static_cast<hipStream_t>(stream), false,
                                       probs, static_cast<hipEvent_t>(ev_begin), static_cast<hipEvent_t>(ev_end));
  return e == hipSuccess ? PARK_OK : PARK_ERR_HIP;
}

// clustered query blocks: n_qblocks in [1, min(N, PARK_MAX_QUERY_BLOCKS)], both tables given
int check_qblocks(int N, const int32_t* q_perm, const int32_t* q_offsets, int n_qblocks) {
  if (!q_perm || !q_offsets || n_qblocks < 1 || n_qblocks > N) return PARK_ERR_INVALID;
  if (n_qblocks > PARK_MAX_QUERY_BLOCKS) return PARK_ERR_UNSUPPORTED;
  return PARK_OK;
}

}  // namespace

extern "C" {

int park_abi_version(void) { return PARK_ABI_VERSION; }

const char* park_status_string(int status) {
  switch (status) {
    case PARK_OK: return "PARK_OK";
    case PARK_ERR_INVALID: return "PARK_ERR_INVALID";
    case PARK_ERR_UNSUPPORTED: return "PARK_ERR_UNSUPPORTED";
    case PARK_ERR_WORKSPACE: return "PARK_ERR_WORKSPACE";
    case PARK_ERR_HIP: return "PARK_ERR_HIP";
    case PARK_ERR_NUMERIC: return "PARK_ERR_NUMERIC";
    default: return "PARK_ERR_UNKNOWN";
  }
}

size_t park_workspace_bytes(int op, int B, int H, int N, int d, int n_clusters) {
  bool uns;
  if (check_common(PARK_BF16, B, H, N, d, n_clusters, &uns) != PARK_OK) return 0;
  const Shape s = make_shape(PARK_BF16, B, H, N, d, n_clusters);
  switch (op) {
    case PARK_OP_CLUSTER_KEYS: return park::cluster_workspace(s);
    case PARK_OP_RETRIEVE_BLOCKS: return park::retrieve_workspace(s, true);
    case PARK_OP_BLOCK_SPARSE_ATTN: return park::attn_workspace(s);
    case PARK_OP_BLOCK_IMPORTANCE: return park::importance_workspace(s);
    default: return 0;
  }
}

int park_block_importance_exact(const void* Q, const void* K, int dtype, int B, int H, int N, int d,
                                const int32_t* perm, const int32_t* offsets, int n_clusters, float scale,
                                float* W, void* workspace, size_t workspace_bytes, void* stream) {
  bool uns;
  int st = check_common(dtype, B, H, N, d, n_clusters, &uns);
  if (st != PARK_OK) return st;
  if (!Q || !K || !perm || !offsets || !W || !finite_f(scale)) return PARK_ERR_INVALID;
  const Shape s = make_shape(dtype, B, H, N, d, n_clusters);
  st = check_ws(workspace, workspace_bytes, park::importance_workspace(s));
  if (st != PARK_OK) return st;
  if (scale <= 0.0f) scale = 1.0f / sqrtf((float)d);
  hipError_t e = park::launch_importance(s, Q, K, perm, offsets, scale, W, workspace,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PARK_OK : PARK_ERR_HIP;
}

size_t park_logmass_workspace_bytes(int B, int H, int N, int d, int n_clusters) {
  bool uns;
  if (check_common(PARK_BF16, B, H, N, d, n_clusters, &uns) != PARK_OK) return 0;
  return park::logmass_workspace(make_shape(PARK_BF16, B, H, N, d, n_clusters));
}

int park_logmass_rmse(const void* Q, const void* K, int dtype, int B, int H, int N, int d, const int32_t* perm,
                      const int32_t* offsets, int n_clusters, const float* centroids, const int32_t* counts,
                      float scale, float* rmse, void* workspace, size_t workspace_bytes, void* stream) {
  bool uns;
  int st = check_common(dtype, B, H, N, d, n_clusters, &uns);
  if (st != PARK_OK) return st;
  if (!Q || !K || !perm || !offsets || !centroids || !counts || !rmse || !finite_f(scale)) return PARK_ERR_INVALID;
  if (dtype != PARK_BF16) return PARK_ERR_UNSUPPORTED;
  const Shape s = make_shape(dtype, B, H, N, d, n_clusters);
  st = check_ws(workspace, workspace_bytes, park::logmass_workspace(s));
  if (st != PARK_OK) return st;
  if (scale <= 0.0f) scale = 1.0f / sqrtf((float)d);
  hipError_t e = park::launch_logmass(s, Q, K, perm, offsets, centroids, counts, scale, rmse, workspace,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PARK_OK : PARK_ERR_HIP;
}

size_t park_workspace_bytes_clustered(int op, int B, int H, int N, int d, int n_clusters, int n_qblocks) {
  bool uns;
  if (check_common(PARK_BF16, B, H, N, d, n_clusters, &uns) != PARK_OK) return 0;
  if (n_qblocks < 1 || n_qblocks > N || n_qblocks > PARK_MAX_QUERY_BLOCKS) return 0;
  const Shape s = make_shape(PARK_BF16, B, H, N, d, n_clusters);
  const park::QueryBlocks qb{nullptr, nullptr, n_qblocks};
  switch (op) {
    case PARK_OP_CLUSTER_KEYS: return park::cluster_workspace(s);
    case PARK_OP_RETRIEVE_BLOCKS: return park::retrieve_clustered_workspace(s, n_qblocks, true);
    case PARK_OP_BLOCK_SPARSE_ATTN: return park::attn_workspace(s, &qb);
    default: return 0;
  }
}

int park_cluster_queries(const void* Q, int dtype, int B, int H, int N, int d, int n_qblocks, int iters,
                         const int32_t* init_idx, float* centroids, int32_t* counts, int32_t* labels, int32_t* perm,
                         int32_t* offsets, void* workspace, size_t workspace_bytes, void* stream) {
  bool uns;
  int st = check_common(dtype, B, H, N, d, n_qblocks, &uns);
  if (st != PARK_OK) return st;
  if (!Q || !centroids || !counts || !labels || !perm || !offsets || iters < 1) return PARK_ERR_INVALID;
  const Shape s = make_shape(dtype, B, H, N, d, n_qblocks);
  st = check_ws(workspace, workspace_bytes, park::cluster_workspace(s));
  if (st != PARK_OK) return st;
  hipError_t e = park::launch_cluster(s, Q, Q, iters, PARK_METRIC_EUCLIDEAN, 0.0f, init_idx, centroids, counts, labels,
                                      perm, offsets, nullptr, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PARK_OK : PARK_ERR_HIP;
}

int park_cluster_keys_timed(const void* Q, const void* K, int dtype, int B, int H, int N, int d, int n_clusters,
                            int iters, int metric, float alpha, const int32_t* init_idx, float* centroids,
                            int32_t* counts, int32_t* labels, int32_t* perm, int32_t* offsets, int32_t* status,
                            void* workspace, size_t workspace_bytes, void* stream, void* ev_begin, void* ev_end) {
  bool uns;
  int st = check_common(dtype, B, H, N, d, n_clusters, &uns);
  if (st != PARK_OK) return st;
  if (!Q || !K || !centroids || !counts || !labels || !perm || !offsets) return PARK_ERR_INVALID;
  if (iters < 1 || (metric != PARK_METRIC_QRKC && metric != PARK_METRIC_EUCLIDEAN)) return PARK_ERR_INVALID;
  if (!finite_f(alpha) || alpha < 0.0f || alpha > 1.0f) return PARK_ERR_INVALID;
  const Shape s = make_shape(dtype, B, H, N, d, n_clusters);
  st = check_ws(workspace, workspace_bytes, park::cluster_workspace(s));
  if (st != PARK_OK) return st;
  hipError_t e = park::launch_cluster(s, Q, K, iters, metric, alpha, init_idx, centroids, counts, labels, perm,
                                      offsets, status, workspace, static_cast<hipStream_t>(stream),
                                      static_cast<hipEvent_t>(ev_begin), static_cast<hipEvent_t>(ev_end));
  return e == hipSuccess ? PARK_OK : PARK_ERR_HIP;
}

int park_cluster_keys(const void* Q, const void* K, int dtype, int B, int H, int N, int d, int n_clusters,
                      int iters, int metric, float alpha, const int32_t* init_idx, float* centroids,
                      int32_t* counts, int32_t* labels, int32_t* perm, int32_t* offsets, int32_t* status,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return park_cluster_keys_timed(Q, K, dtype, B, H, N, d, n_clusters, iters, metric, alpha, init_idx, centroids,
                                 counts, labels, perm, offsets, status, workspace, workspace_bytes, stream, nullptr,
                                 nullptr);
}

int park_retrieve_blocks(const void* Q, int dtype, int B, int H, int N, int d, const float* centroids,
                         const int32_t* counts, int n_clusters, int q_block, float top_p, int top_k, float scale,
                         float* scores, uint8_t* mask, int32_t* block_list, int32_t* block_count, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return retrieve_impl(false, Q, dtype, B, H, N, d, centroids, counts, n_clusters, q_block, top_p, top_k, scale,
                       scores, mask, block_list, block_count, workspace, workspace_bytes, stream);
}

int park_retrieve_blocks_timed(const void* Q, int dtype, int B, int H, int N, int d, const float* centroids,
                               const int32_t* counts, int n_clusters, int q_block, float top_p, int top_k,
                               float scale, float* scores, uint8_t* mask, int32_t* block_list, int32_t* block_count,
                               void* workspace, size_t workspace_bytes, void* stream, void* ev_begin, void* ev_end) {
  return retrieve_impl(false, Q, dtype, B, H, N, d, centroids, counts, n_clusters, q_block, top_p, top_k, scale,
                       scores, mask, block_list, block_count, workspace, workspace_bytes, stream, nullptr, ev_begin,
                       ev_end);
}

int park_retrieve_blocks_pooled(const void* Q, int dtype, int B, int H, int N, int d, const float* centroids,
                                const int32_t* counts, int n_clusters, int q_block, float top_p, int top_k,
                                float scale, float* scores, uint8_t* mask, int32_t* block_list,
                                int32_t* block_count, void* workspace, size_t workspace_bytes, void* stream) {
  return retrieve_impl(true, Q, dtype, B, H, N, d, centroids, counts, n_clusters, q_block, top_p, top_k, scale,
                       scores, mask, block_list, block_count, workspace, workspace_bytes, stream);
}

int park_retrieve_blocks_unfused(const void* Q, int dtype, int B, int H, int N, int d, const float* centroids,
                                 const int32_t* counts, int n_clusters, int q_block, float top_p, int top_k,
                                 float scale, float* probs, float* scores, uint8_t* mask, int32_t* block_list,
                                 int32_t* block_count, void* workspace, size_t workspace_bytes, void* stream) {
  if (!probs) return PARK_ERR_INVALID;
  return retrieve_impl(false, Q, dtype, B, H, N, d, centroids, counts, n_clusters, q_block, top_p, top_k, scale,
                       scores, mask, block_list, block_count, workspace, workspace_bytes, stream, probs);
}

int park_retrieve_blocks_clustered(const void* Q, int dtype, int B, int H, int N, int d, const float* centroids,
                                   const int32_t* counts, int n_clusters, const int32_t* q_perm,
                                   const int32_t* q_offsets, int n_qblocks, float top_p, int top_k, float scale,
                                   float* scores, uint8_t* mask, int32_t* block_list, int32_t* block_count,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  bool uns;
  int st = check_common(dtype, B, H, N, d, n_clusters, &uns);
  if (st != PARK_OK) return st;
  if (!Q || !centroids || !counts || !mask || !block_list || !block_count) return PARK_ERR_INVALID;
  if (!finite_f(top_p) || top_p < 0.0f || top_p > 1.0f || top_k < 0 || !finite_f(scale)) return PARK_ERR_INVALID;
  if ((st = check_qblocks(N, q_perm, q_offsets, n_qblocks)) != PARK_OK) return st;
  const Shape s = make_shape(dtype, B, H, N, d, n_clusters);
  st = check_ws(workspace, workspace_bytes, park::retrieve_clustered_workspace(s, n_qblocks, scores == nullptr));
  if (st != PARK_OK) return st;
  if (scale <= 0.0f) scale = 1.0f / sqrtf((float)d);
  const park::QueryBlocks qb{q_perm, q_offsets, n_qblocks};
  hipError_t e = park::launch_retrieve_clustered(s, Q, centroids, counts, qb, scale, top_p, top_k, scores, mask,
                                                 block_list, block_count, workspace,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PARK_OK : PARK_ERR_HIP;
}

int park_retrieve_blocks_online(const void* Q, int dtype, int B, int H, int N, int d, const float* centroids,
                                const int32_t* counts, int n_clusters, const int32_t* q_perm,
                                const int32_t* q_offsets, int n_qblocks, float top_p, int top_k, float scale,
                                float* scores, uint8_t* mask, int32_t* block_list, int32_t* block_count,
                                void* workspace, size_t workspace_bytes, void* stream) {
  bool uns;
  int st = check_common(dtype, B, H, N, d, n_clusters, &uns);
  if (st != PARK_OK) return st;
  if (!Q || !centroids || !counts || !mask || !block_list || !block_count) return PARK_ERR_INVALID;
  if (!finite_f(top_p) || top_p < 0.0f || top_p > 1.0f || top_k < 0 || !finite_f(scale)) return PARK_ERR_INVALID;
  const bool clustered = q_perm || q_offsets;
  if (clustered) {
    if ((st = check_qblocks(N, q_perm, q_offsets, n_qblocks)) != PARK_OK) return st;
  } else if (n_qblocks != 0 && n_qblocks != (N + PARK_QUERY_BLOCK - 1) / PARK_QUERY_BLOCK) {
    return PARK_ERR_INVALID;
  }
  const Shape s = make_shape(dtype, B, H, N, d, n_clusters);
  const size_t need = clustered ? park::retrieve_clustered_workspace(s, n_qblocks, scores == nullptr)
                                : park::retrieve_workspace(s, scores == nullptr);
  if ((st = check_ws(workspace, workspace_bytes, need)) != PARK_OK) return st;
  if (scale <= 0.0f) scale = 1.0f / sqrtf((float)d);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (clustered) {
    const park::QueryBlocks qb{q_perm, q_offsets, n_qblocks};
    e = park::launch_retrieve_clustered(s, Q, centroids, counts, qb, scale, top_p, top_k, scores, mask, block_list,
                                        block_count, workspace, hs, true);
  } else {
    e = park::launch_retrieve(s, Q, centroids, counts, scale, top_p, top_k, false, scores, mask, block_list,
                              block_count, workspace, hs, true);
  }
  return e == hipSuccess ? PARK_OK : PARK_ERR_HIP;
}

int park_block_sparse_attn_clustered(const void* Q, const void* K, const void* V, int dtype, int B, int H, int N,
                                     int d, const int32_t* perm, const int32_t* offsets, int n_clusters,
                                     const int32_t* q_perm, const int32_t* q_offsets, int n_qblocks,
                                     const int32_t* block_list, const int32_t* block_count, float scale, void* O,
                                     float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  bool uns;
  int st = check_common(dtype, B, H, N, d, n_clusters, &uns);
  if (st != PARK_OK) return st;
  if (!Q || !K || !V || !perm || !offsets || !block_list || !block_count || !O) return PARK_ERR_INVALID;
  if (!finite_f(scale)) return PARK_ERR_INVALID;
  if ((st = check_qblocks(N, q_perm, q_offsets, n_qblocks)) != PARK_OK) return st;
  const Shape s = make_shape(dtype, B, H, N, d, n_clusters);
  const park::QueryBlocks qb{q_perm, q_offsets, n_qblocks};
  st = check_ws(workspace, workspace_bytes, park::attn_workspace(s, &qb));
  if (st != PARK_OK) return st;
  if (scale <= 0.0f) scale = 1.0f / sqrtf((float)d);
  hipError_t e = park::launch_attn(s, Q, K, V, perm, offsets, block_list, block_count, scale, O, lse, workspace,
                                   static_cast<hipStream_t>(stream), nullptr, nullptr, 0, &qb);
  return e == hipSuccess ? PARK_OK : PARK_ERR_HIP;
}

static int attn_impl(const void* Q, const void* K, const void* V, int dtype, int B, int H, int N, int d,
                     const int32_t* perm, const int32_t* offsets, int n_clusters, const int32_t* block_list,
                     const int32_t* block_count, int q_block, float scale, void* O, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream, void* const* ev_begin, void* const* ev_end,
                     int n_events) {
  bool uns;
  int st = check_common(dtype, B, H, N, d, n_clusters, &uns);
  if (st != PARK_OK) return st;
  if (!Q || !K || !V || !perm || !offsets || !block_list || !block_count || !O) return PARK_ERR_INVALID;
  if (!finite_f(scale)) return PARK_ERR_INVALID;
  if (q_block != PARK_QUERY_BLOCK) return PARK_ERR_UNSUPPORTED;
  const Shape s = make_shape(dtype, B, H, N, d, n_clusters);
  st = check_ws(workspace, workspace_bytes, park::attn_workspace(s));
  if (st != PARK_OK) return st;
  if (scale <= 0.0f) scale = 1.0f / sqrtf((float)d);
  hipError_t e = park::launch_attn(s, Q, K, V, perm, offsets, block_list, block_count, scale, O, lse, workspace,
                                   static_cast<hipStream_t>(stream), reinterpret_cast<const hipEvent_t*>(ev_begin),
                                   reinterpret_cast<const hipEvent_t*>(ev_end), n_events);
  return e == hipSuccess ? PARK_OK : PARK_ERR_HIP;
}

int park_block_sparse_attn(const void* Q, const void* K, const void* V, int dtype, int B, int H, int N, int d,
                           const int32_t* perm, const int32_t* offsets, int n_clusters, const int32_t* block_list,
                           const int32_t* block_count, int q_block, float scale, void* O, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return attn_impl(Q, K, V, dtype, B, H, N, d, perm, offsets, n_clusters, block_list, block_count, q_block, scale, O,
                   lse, workspace, workspace_bytes, stream, nullptr, nullptr, 0);
}

int park_block_sparse_attn_timed(const void* Q, const void* K, const void* V, int dtype, int B, int H, int N,
                                 int d, const int32_t* perm, const int32_t* offsets, int n_clusters,
                                 const int32_t* block_list, const int32_t* block_count, int q_block, float scale,
                                 void* O, float* lse, void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* ev_begin, void* const* ev_end, int n_events) {
  if (n_events < 0 || (n_events > 0 && (!ev_begin || !ev_end))) return PARK_ERR_INVALID;
  return attn_impl(Q, K, V, dtype, B, H, N, d, perm, offsets, n_clusters, block_list, block_count, q_block, scale, O,
                   lse, workspace, workspace_bytes, stream, ev_begin, ev_end, n_events);
}

int park_attn_passes(int dtype, int B, int H, int N, int d, int n_clusters) {
  bool uns;
  if (check_common(dtype, B, H, N, d, n_clusters, &uns) != PARK_OK) return 0;
  return park::attn_passes(make_shape(dtype, B, H, N, d, n_clusters));
}

}  // extern "C"
