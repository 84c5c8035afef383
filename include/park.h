/*
 * park.h - C ABI of libpark: query-response key clustering, per-query attention-mass
 * block retrieval and block-sparse attention for one attention layer, on one MI355X
 * (gfx950) GPU.
 *
 * The method is PARK, "Accurate Block Retrieval for Sparse Attention in Video Diffusion
 * Transformers" (paperpeel.com/paper/2609.38978).  Section and equation names below refer
 * to that page.
 *
 * Conventions for every entry point
 *   - Tensors are caller-owned DEVICE memory, contiguous, in [B, H, N, d] (or the stated
 *     shape) row-major order; nothing is copied to or from the host.
 *   - libpark allocates no device memory.  Scratch space comes from the caller's
 *     `workspace` (device memory, 256-byte aligned, at least park_workspace_bytes()).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL means the default stream) and the
 *     call returns without synchronising.  Device-side faults surface at the caller's next
 *     synchronisation.  Calls hold no global state and may run concurrently on different
 *     streams with different workspaces.
 *   - Arguments are validated on the host before anything is launched; a failing check
 *     returns its status and launches nothing.  No C++ exception crosses the ABI.
 *   - dtype: PARK_F32 (inputs are float) or PARK_BF16 (inputs are bfloat16).
 *   - Head dimension d must be 64 or 128; the number of key clusters is at most
 *     PARK_MAX_CLUSTERS.  Query blocks are either 64 consecutive tokens (the entry points
 *     without a suffix) or clustered (the *_clustered entry points, PARK's own setting:
 *     Euclidean k-means of the queries, Figure 2 and section 6 "Implementations").
 */
#ifndef PARK_H
#define PARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define PARK_API __attribute__((visibility("default")))
#else
#define PARK_API
#endif

#define PARK_ABI_VERSION 2
#define PARK_MAX_CLUSTERS 1536
#define PARK_QUERY_BLOCK 64
#define PARK_MAX_QUERY_BLOCKS 1536   /* clustered query blocks per head */

typedef enum park_status {
  PARK_OK = 0,
  PARK_ERR_INVALID = 1,      /* a required pointer is NULL or a size/parameter is out of range */
  PARK_ERR_UNSUPPORTED = 2,  /* valid, but not built: d not in {64,128}, q_block != 64, ... */
  PARK_ERR_WORKSPACE = 3,    /* workspace NULL, misaligned or smaller than required */
  PARK_ERR_HIP = 4,          /* a kernel launch failed (hipGetLastError after the launch) */
  PARK_ERR_NUMERIC = 5       /* a per-head status flag is set (see park_cluster_keys); the
                                entry points themselves never return it, because the flag is
                                written on the device after they return */
} park_status;

typedef enum park_dtype { PARK_F32 = 0, PARK_BF16 = 1 } park_dtype;

typedef enum park_metric {
  PARK_METRIC_QRKC = 0,      /* query-response key clustering (section 5.2) */
  PARK_METRIC_EUCLIDEAN = 1  /* plain Euclidean k-means on the raw keys ("w/o QRKC", section 6.3) */
} park_metric;

typedef enum park_op {
  PARK_OP_CLUSTER_KEYS = 0,
  PARK_OP_RETRIEVE_BLOCKS = 1,
  PARK_OP_BLOCK_SPARSE_ATTN = 2,
  PARK_OP_BLOCK_IMPORTANCE = 3
} park_op;

/* PARK_ABI_VERSION of the loaded library. */
PARK_API int park_abi_version(void);

/* Static, NUL-terminated name of a park_status value ("PARK_OK", ...). */
PARK_API const char* park_status_string(int status);

/* Bytes of workspace the given entry point needs for these sizes (0 if none); returns 0
 * also for invalid sizes, which the entry point itself then rejects. */
PARK_API size_t park_workspace_bytes(int op, int B, int H, int N, int d, int n_clusters);

/*
 * park_cluster_keys - query-response key clustering (section 5.2, App. D.2), per (b, h):
 *   G_Q = (1/N) Q^T Q;  s_Q = max(tr(G_Q)/d, 1e-6);
 *   Gs  = (1 - alpha) G_Q + (alpha + 1e-6) s_Q I = R R^T  (Cholesky, R lower triangular);
 *   k~_j = R^T k_j;  Lloyd k-means with `iters` steps of (assign, update) on k~ from the
 *   anchors k~_{floor(v N / n_clusters)} (or k~_{init_idx[v]});  argmin ties go to the
 *   lowest cluster; an empty cluster keeps its centroid.  metric EUCLIDEAN uses R = I.
 * Outputs (all per (b, h)):
 *   centroids [B,H,n_clusters,d] float: c_v = mean of the ORIGINAL keys of cluster v
 *             (section 5.1, E7), 0 for an empty cluster;
 *   counts    [B,H,n_clusters]   int32: n_v;
 *   labels    [B,H,N]            int32: cluster of each key after the last step;
 *   perm      [B,H,N]            int32: key indices in (label, index) order, so cluster v
 *             is perm[offsets[v] .. offsets[v+1]);
 *   offsets   [B,H,n_clusters+1] int32: exclusive prefix sum of counts, offsets[n] = N;
 *   status    [B,H] int32 or NULL: 0, or 1 when the Cholesky factorisation failed (App. D.2
 *             "Numerically stable Cholesky factorization"); the head is then clustered with
 *             R = I, i.e. with the Euclidean metric.  For finite queries the (alpha + 1e-6) s_Q I
 *             term keeps Gs positive definite, so only non-finite input (or overflow) sets
 *             it.  It is written on `stream` after the call has returned PARK_OK: a caller
 *             that needs the outcome synchronises and reports PARK_ERR_NUMERIC for a non-zero
 *             flag (the Python binding's numeric_status does so).
 * init_idx: NULL or device int32 [n_clusters] of key indices in [0, N), shared by all heads.
 * With bf16 keys and clusters of at most 128 keys on average, each cluster's member sum is
 * carried from step to step (plus the keys that joined, minus those that left), which is exact
 * in double and gives the plain Lloyd step's means.
 * Errors: INVALID for NULL required pointers, B,H < 1, N < 1, n_clusters outside [1, N],
 * iters < 1, alpha outside [0, 1] or not finite, unknown dtype/metric; UNSUPPORTED for d
 * not in {64,128} or n_clusters > PARK_MAX_CLUSTERS; WORKSPACE; HIP.
 */
PARK_API int park_cluster_keys(const void* Q, const void* K, int dtype, int B, int H, int N, int d,
                      int n_clusters, int iters, int metric, float alpha, const int32_t* init_idx,
                      float* centroids, int32_t* counts, int32_t* labels, int32_t* perm,
                      int32_t* offsets, int32_t* status, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * park_cluster_keys_timed - park_cluster_keys for measurement: records the HIP events ev_begin
 * and ev_end (hipEvent_t, created by the caller; either may be NULL) on `stream` immediately
 * before and after the assignment kernel of the last k-means step, so that
 * hipEventElapsedTime gives one assignment launch's duration.  Otherwise identical to
 * park_cluster_keys (arguments, results, errors); a failed hipEventRecord is reported as HIP.
 */
PARK_API int park_cluster_keys_timed(const void* Q, const void* K, int dtype, int B, int H, int N, int d,
                                     int n_clusters, int iters, int metric, float alpha, const int32_t* init_idx,
                                     float* centroids, int32_t* counts, int32_t* labels, int32_t* perm,
                                     int32_t* offsets, int32_t* status, void* workspace, size_t workspace_bytes,
                                     void* stream, void* ev_begin, void* ev_end);

/*
 * park_retrieve_blocks - per-query attention-mass aggregation (PAMA, section 5.1, E7/E8)
 * followed by top-p selection with a top-k floor (section 6.1; the floor as in SCOPE,
 * paperpeel.com/paper/2608.12780, appendix "Online Per-Head Top-k Selection"), per (b, h):
 *   S_iv = scale q_i . c_v + log n_v  (-inf for n_v = 0);  P_iv = softmax_v S_iv;
 *   W_uv = (1/n_u) sum_{i in query block u} P_iv, query block u = tokens [64u, 64u+64) of N
 *   (the last block may be shorter);
 *   ranking of blocks v by (W_uv descending, v ascending), empty clusters last;
 *   t_p = shortest prefix with mass >= top_p * sum_v W_uv (0 if top_p = 0);
 *   count_u = min(max(t_p, top_k), number of non-empty clusters).
 * Inputs: Q [B,H,N,d]; centroids [B,H,n_clusters,d] float and counts [B,H,n_clusters] as
 * written by park_cluster_keys.  scale <= 0 selects 1/sqrt(d).
 * Outputs (NQ = ceil(N/64)):
 *   scores      [B,H,NQ,n_clusters] float or NULL: W^PAMA;
 *   mask        [B,H,NQ,n_clusters] uint8: 1 for selected (query block, cluster) pairs;
 *   block_list  [B,H,NQ,n_clusters] int32: selected cluster ids ascending, then -1;
 *   block_count [B,H,NQ] int32: count_u.
 * Errors: INVALID (NULL required pointers, sizes, top_p outside [0,1], top_k < 0, scale not
 * finite), UNSUPPORTED (d, q_block != 64, n_clusters > PARK_MAX_CLUSTERS), WORKSPACE, HIP.
 */
PARK_API int park_retrieve_blocks(const void* Q, int dtype, int B, int H, int N, int d,
                         const float* centroids, const int32_t* counts, int n_clusters,
                         int q_block, float top_p, int top_k, float scale, float* scores,
                         uint8_t* mask, int32_t* block_list, int32_t* block_count,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * park_retrieve_blocks_timed - park_retrieve_blocks for measurement: records the HIP events
 * ev_begin and ev_end (hipEvent_t, created by the caller; either may be NULL) on `stream`
 * immediately before and after the fused PAMA kernel (after the centroid preparation, before
 * the selection).  Otherwise identical to park_retrieve_blocks; a failed hipEventRecord is
 * reported as HIP.
 */
PARK_API int park_retrieve_blocks_timed(const void* Q, int dtype, int B, int H, int N, int d,
                                        const float* centroids, const int32_t* counts, int n_clusters,
                                        int q_block, float top_p, int top_k, float scale, float* scores,
                                        uint8_t* mask, int32_t* block_list, int32_t* block_count,
                                        void* workspace, size_t workspace_bytes, void* stream, void* ev_begin,
                                        void* ev_end);

/*
 * park_retrieve_blocks_pooled - the query-centroid estimate that PAMA replaces (section 4.1
 * and the "w/o PAMA" ablation of section 6.3), kept as a measurement baseline:
 *   qbar_u = mean of block u's queries;  W_uv = softmax_v(scale qbar_u . c_v + log n_v);
 * then the same selection as park_retrieve_blocks.  Same arguments, layouts and errors.
 */
PARK_API int park_retrieve_blocks_pooled(const void* Q, int dtype, int B, int H, int N, int d,
                                const float* centroids, const int32_t* counts, int n_clusters,
                                int q_block, float top_p, int top_k, float scale, float* scores,
                                uint8_t* mask, int32_t* block_list, int32_t* block_count,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * park_block_sparse_attn - attention restricted to the selected blocks (section 3.1, E1/E2
 * with the softmax renormalised over the selected keys), per (b, h) and query i in block u:
 *   J_u = union over r < block_count[u] of cluster block_list[u][r], i.e. the keys
 *         perm[offsets[v] .. offsets[v+1]);
 *   O_i = sum_{j in J_u} exp(s_ij - m_i) v_j / sum_{j in J_u} exp(s_ij - m_i),
 *   s_ij = scale q_i . k_j,  lse_i = m_i + log sum_{j in J_u} exp(s_ij - m_i);
 * an empty J_u gives O_i = 0 and lse_i = -inf.  O is in the original query order.
 * For bf16 inputs the call first copies every cluster's keys and values, in cluster order, into
 * the workspace as 8-key groups in matrix-operand order (the last group of a cluster
 * zero-padded), deals each head's clusters to 4 key ranges of about equal work (range r is
 * computed on XCDs r and r + 4, so each XCD's L2 holds a quarter of a head's keys), lists the
 * 32-key tiles of every (query block, range) pair, computes a partial softmax state per pair
 * and merges the 4 partial states of every query; float inputs are read in place through perm.
 * Inputs: Q, K, V [B,H,N,d] of `dtype`; perm/offsets from park_cluster_keys; block_list /
 * block_count from park_retrieve_blocks (ids must lie in [0, n_clusters); listing every
 * cluster gives dense attention).  scale <= 0 selects 1/sqrt(d).
 * Outputs: O [B,H,N,d] of `dtype`; lse [B,H,N] float or NULL (natural-log log-sum-exp).
 * Numerics: bf16 inputs use bf16 matrix products with float accumulation and a float
 * online softmax (probabilities rounded to bf16 before the PV product, O normalised by the
 * sum of those rounded weights, lse from the float sum); here (64-token blocks) the partial
 * outputs of the key ranges are kept in fp16, scaled by the head's largest |value|, and
 * merged in range order; float inputs are computed in float throughout.
 * The heads are computed in park_attn_passes() passes (each the whole computation for its
 * heads, heads being independent); the workspace holds one pass's packed keys and values, tile
 * plan and partial states, and a pass takes as many heads as fit in 2.5 GiB (at least one).
 * Workspace: park_workspace_bytes(PARK_OP_BLOCK_SPARSE_ATTN, ...) bytes (sized for any selection,
 * up to every cluster for every query block).
 * Errors: INVALID, UNSUPPORTED (d, q_block != 64, n_clusters > PARK_MAX_CLUSTERS),
 * WORKSPACE, HIP.
 */
PARK_API int park_block_sparse_attn(const void* Q, const void* K, const void* V, int dtype, int B, int H,
                           int N, int d, const int32_t* perm, const int32_t* offsets,
                           int n_clusters, const int32_t* block_list, const int32_t* block_count,
                           int q_block, float scale, void* O, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Number of passes over the heads that park_block_sparse_attn makes for these sizes (>= 1;
 * 0 for sizes the call rejects). */
PARK_API int park_attn_passes(int dtype, int B, int H, int N, int d, int n_clusters);

/*
 * park_block_sparse_attn_timed - park_block_sparse_attn for measurement: for each pass p <
 * n_events, records the HIP events ev_begin[p] and ev_end[p] (hipEvent_t, created by the
 * caller; host arrays of n_events handles, either handle may be NULL) on `stream` immediately
 * before and after that pass's attention kernel itself, i.e. after its packing and
 * tile-planning launches, so that the sum of hipEventElapsedTime over the passes gives the
 * kernel's duration.  Otherwise identical to park_block_sparse_attn (arguments, results,
 * errors); INVALID also for n_events < 0 or a NULL array with n_events > 0; a failed
 * hipEventRecord is reported as HIP.
 */
PARK_API int park_block_sparse_attn_timed(const void* Q, const void* K, const void* V, int dtype, int B, int H,
                                 int N, int d, const int32_t* perm, const int32_t* offsets,
                                 int n_clusters, const int32_t* block_list, const int32_t* block_count,
                                 int q_block, float scale, void* O, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream, void* const* ev_begin,
                                 void* const* ev_end, int n_events);

/*
 * park_block_importance_exact - a retrieval-accuracy diagnostic: the exact block importance
 * of section 3.2, Eq. (3), for 64-token query blocks,
 *   W_uv = (1/n_u) sum_{i in block u} sum_{j in cluster v} softmax_j(scale q_i . k_j)
 * (softmax over all N keys), the reference against which PARK's appendix A measures the
 * total-variation error of an estimated map (M1).  Computed with the block-sparse attention
 * kernel: every key selected (dense attention) and values equal to the one-hot vector of each
 * key's cluster, d clusters per pass (ceil(n_clusters / d) passes), then the mean over each
 * block's queries.  Numerics: as park_block_sparse_attn (for bf16 inputs the probabilities are
 * rounded to bf16 and the per-query masses are bf16 outputs, so |W error| stays near 1e-3).
 * Inputs: Q, K [B,H,N,d]; perm / offsets from park_cluster_keys.  scale <= 0 selects 1/sqrt(d).
 * Output: W [B,H,NQ,n_clusters] float.  Workspace: park_workspace_bytes(PARK_OP_BLOCK_IMPORTANCE,
 * ...).  Errors: INVALID, UNSUPPORTED (d, n_clusters > PARK_MAX_CLUSTERS), WORKSPACE, HIP.
 */
PARK_API int park_block_importance_exact(const void* Q, const void* K, int dtype, int B, int H, int N, int d,
                                         const int32_t* perm, const int32_t* offsets, int n_clusters, float scale,
                                         float* W, void* workspace, size_t workspace_bytes, void* stream);

/*
 * park_logmass_rmse - a retrieval-accuracy diagnostic: the centred log-mass error of the key
 * centroids (PARK appendix B, M2, with the quantities of section 4.2), per head:
 *   S*_iv = log sum_{j in cluster v} exp(scale q_i . k_j),  S_iv = log n_v + scale q_i . c_v,
 *   D_iv = S*_iv - S_iv for every query i and non-empty cluster v, centred per query (the
 *   mean over v subtracted: a softmax over clusters does not see a per-query constant);
 *   rmse = sqrt(mean over all (i, v) of the centred D^2).
 * One wave per 64-query block computes every (query, cluster) log-sum-exp from the keys
 * (bf16 products, float sums) - L^2 d work per head, a diagnostic rather than a step.
 * Inputs: Q, K [B,H,N,d] bf16; perm / offsets / centroids / counts from park_cluster_keys.
 * Output: rmse [B,H] float.  Workspace: park_logmass_workspace_bytes(...).
 * Errors: INVALID, UNSUPPORTED (float inputs, d, n_clusters > PARK_MAX_CLUSTERS), WORKSPACE, HIP.
 */
PARK_API size_t park_logmass_workspace_bytes(int B, int H, int N, int d, int n_clusters);
PARK_API int park_logmass_rmse(const void* Q, const void* K, int dtype, int B, int H, int N, int d,
                               const int32_t* perm, const int32_t* offsets, int n_clusters, const float* centroids,
                               const int32_t* counts, float scale, float* rmse, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * park_retrieve_blocks_unfused - park_retrieve_blocks without the fusion of PARK section 5.1
 * ("Efficient Kernel Implementation"): the per-query probabilities P_iv of E7 are written to
 * HBM (probs, [B,H,N,n_clusters] float, caller-allocated device memory, 4 N n_clusters bytes
 * per head) and a second kernel averages each 64-token block's rows into W.  Scores and
 * selection equal park_retrieve_blocks up to the order of the block sums; the call exists to
 * measure what the fusion saves.  Inputs, outputs, workspace and errors as
 * park_retrieve_blocks; INVALID also for a NULL probs.
 */
PARK_API int park_retrieve_blocks_unfused(const void* Q, int dtype, int B, int H, int N, int d,
                                          const float* centroids, const int32_t* counts, int n_clusters,
                                          int q_block, float top_p, int top_k, float scale, float* probs,
                                          float* scores, uint8_t* mask, int32_t* block_list, int32_t* block_count,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Clustered query blocks.  PARK groups the queries by plain Euclidean k-means (Figure 2;
 * N_Q = 128 in section 6, "Implementations") instead of taking runs of 64 tokens.  Query
 * block u of head (b, h) is then the set of queries
 *   q_perm[b,h][q_offsets[b,h][u] .. q_offsets[b,h][u+1])        (n_u of them),
 * which is what park_cluster_queries (or park_cluster_keys with metric EUCLIDEAN and K = Q)
 * writes as perm / offsets.  q_perm must hold each query index once and q_offsets must rise
 * from 0 to N; other contents give undefined results but never an access out of range
 * (offsets are clamped to [0, N] and indices to [0, N - 1]).  Internally every block is
 * walked as chunks of at most 64 consecutive positions of q_perm.
 * --------------------------------------------------------------------------------- */

/* Bytes of workspace the *_clustered entry points (op PARK_OP_RETRIEVE_BLOCKS or
 * PARK_OP_BLOCK_SPARSE_ATTN) or park_cluster_queries (op PARK_OP_CLUSTER_KEYS with
 * n_clusters = n_qblocks) need; 0 for invalid sizes. */
PARK_API size_t park_workspace_bytes_clustered(int op, int B, int H, int N, int d, int n_clusters, int n_qblocks);

/*
 * park_cluster_queries - the query blocks of PARK (Figure 2: the queries are clustered by
 * standard Euclidean k-means): park_cluster_keys with K = Q and metric EUCLIDEAN, i.e. Lloyd
 * k-means of the raw queries from the anchors q_{floor(u N / n_qblocks)} (or init_idx), ties
 * to the lowest block, empty blocks keeping their centroid.  Outputs as park_cluster_keys
 * with n_clusters = n_qblocks: centroids [B,H,n_qblocks,d] float (block means), counts
 * [B,H,n_qblocks] (n_u), labels [B,H,N], perm [B,H,N] (queries in (block, index) order) and
 * offsets [B,H,n_qblocks+1] - perm and offsets are the q_perm / q_offsets below.
 * Workspace: park_workspace_bytes(PARK_OP_CLUSTER_KEYS, B, H, N, d, n_qblocks).
 * Errors: INVALID (NULL required pointers, sizes, n_qblocks outside [1, N], iters < 1),
 * UNSUPPORTED (d, n_qblocks > PARK_MAX_CLUSTERS), WORKSPACE, HIP.
 */
PARK_API int park_cluster_queries(const void* Q, int dtype, int B, int H, int N, int d, int n_qblocks, int iters,
                                  const int32_t* init_idx, float* centroids, int32_t* counts, int32_t* labels,
                                  int32_t* perm, int32_t* offsets, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * park_retrieve_blocks_clustered - PAMA (section 5.1, E7/E8) and the top-p / top-k selection
 * of park_retrieve_blocks over clustered query blocks:
 *   W_uv = (1/n_u) sum_{i in block u} P_iv  (a zero row for an empty block).
 * The fused kernel computes, per chunk of a block, the column sums of the chunk's 64 x
 * n_clusters softmax in registers; a second kernel adds the chunks of each block in order
 * and divides by n_u.
 * Inputs: Q, centroids, counts as for park_retrieve_blocks; q_perm [B,H,N], q_offsets
 * [B,H,n_qblocks+1] int32 (device).
 * Outputs: scores [B,H,n_qblocks,n_clusters] float or NULL, mask [B,H,n_qblocks,n_clusters]
 * uint8, block_list [B,H,n_qblocks,n_clusters] int32, block_count [B,H,n_qblocks] int32, with
 * the meanings of park_retrieve_blocks.
 * Workspace: park_workspace_bytes_clustered(PARK_OP_RETRIEVE_BLOCKS, ...).
 * Errors: as park_retrieve_blocks; INVALID also for NULL q_perm / q_offsets or n_qblocks
 * outside [1, N]; UNSUPPORTED for n_qblocks > PARK_MAX_QUERY_BLOCKS.
 */
PARK_API int park_retrieve_blocks_clustered(const void* Q, int dtype, int B, int H, int N, int d,
                                            const float* centroids, const int32_t* counts, int n_clusters,
                                            const int32_t* q_perm, const int32_t* q_offsets, int n_qblocks,
                                            float top_p, int top_k, float scale, float* scores, uint8_t* mask,
                                            int32_t* block_list, int32_t* block_count, void* workspace,
                                            size_t workspace_bytes, void* stream);

/*
 * park_retrieve_blocks_online - the PAMA scores of park_retrieve_blocks (q_perm and q_offsets
 * NULL: 64-token query blocks, n_qblocks 0 or ceil(N/64)) or of park_retrieve_blocks_clustered
 * (both given), selected with SCOPE's online per-head top-k (SCOPE, section 3 "Online Per-Head
 * Top-k Estimation" and the appendix "Online Per-Head Top-k Selection"):
 *   1. b_u = the count of the top-p / fixed top-k selection of park_retrieve_blocks;
 *   2. per head, k_on = ceil(sum_u n_u b_u / sum_u n_u), n_u the size of query block u
 *      (64, the last block N - 64 (NQ - 1); or q_offsets[u+1] - q_offsets[u]);
 *   3. block u keeps max(b_u, min(k_on, non-empty clusters)) clusters: blocks below k_on are
 *      extended along the same ranking, the others keep their selection.
 * The counted unit is a key cluster (the unit PARK selects), where SCOPE counts keys.
 * Inputs, outputs, workspace (park_workspace_bytes or park_workspace_bytes_clustered with op
 * PARK_OP_RETRIEVE_BLOCKS) and errors as the two entry points above; INVALID also for a
 * non-zero n_qblocks other than ceil(N/64) without q_perm / q_offsets, and for only one of
 * q_perm / q_offsets given.
 */
PARK_API int park_retrieve_blocks_online(const void* Q, int dtype, int B, int H, int N, int d,
                                         const float* centroids, const int32_t* counts, int n_clusters,
                                         const int32_t* q_perm, const int32_t* q_offsets, int n_qblocks,
                                         float top_p, int top_k, float scale, float* scores, uint8_t* mask,
                                         int32_t* block_list, int32_t* block_count, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * park_block_sparse_attn_clustered - park_block_sparse_attn with clustered query blocks:
 * query i of block u attends to J_u, the keys of the clusters block_list[u][0 ..
 * block_count[u]), with the same formulas, numerics and output layout (O [B,H,N,d] and lse
 * [B,H,N] in the original query order).  block_list / block_count [B,H,n_qblocks,...] come
 * from park_retrieve_blocks_clustered.  The bf16 path packs keys and values and plans the
 * tiles of every block as park_block_sparse_attn does (the tile plan of a block serves all its
 * chunks); one wave computes a whole chunk over all its selected tiles in one pass and writes
 * the final O (bf16) and lse itself, so there are no partial states and no merge.  Queries are
 * read and results written through q_perm.  Heads are computed in passes as in
 * park_block_sparse_attn.
 * Workspace: park_workspace_bytes_clustered(PARK_OP_BLOCK_SPARSE_ATTN, ...).
 * Errors: as park_block_sparse_attn; INVALID also for NULL q_perm / q_offsets or n_qblocks
 * outside [1, N]; UNSUPPORTED for n_qblocks > PARK_MAX_QUERY_BLOCKS.
 */
PARK_API int park_block_sparse_attn_clustered(const void* Q, const void* K, const void* V, int dtype, int B,
                                              int H, int N, int d, const int32_t* perm, const int32_t* offsets,
                                              int n_clusters, const int32_t* q_perm, const int32_t* q_offsets,
                                              int n_qblocks, const int32_t* block_list,
                                              const int32_t* block_count, float scale, void* O, float* lse,
                                              void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).
 * --------------------------------------------------------------------------------- */

/* Size of the library's fixed per-GPU scratch array used by park_retrieve_blocks_noalloc:
 * 32 MiB, held on every GPU the library runs on until the process ends (enough for the
 * 75,600-token / 40-head / 1024-cluster and the 119,056-token / 24-head / 1536-cluster
 * shapes at d = 128). */
#define PARK_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* Bytes of that scratch park_retrieve_blocks_noalloc needs for these sizes (0 for invalid
 * sizes); the call works when this is at most PARK_NOALLOC_SCRATCH_BYTES. */
PARK_API size_t park_noalloc_scratch_bytes(int B, int H, int N, int d, int n_clusters);

/*
 * park_retrieve_blocks_noalloc - park_retrieve_blocks (same computation, same kernels,
 * same outputs) that allocates nothing and takes no workspace: its scratch (the centroid
 * operands of the fused PAMA kernel) is the library's static per-GPU array of
 * PARK_NOALLOC_SCRATCH_BYTES.  `scores` is required here (W is an output in caller memory,
 * not scratch).  The device address of the array is looked up once per device, on the first
 * call with that device current; `stream` (NULL: the current device's null stream) must
 * belong to the current device, whose copy of the array the call uses.  Every call on one
 * GPU uses the same array and overwrites
 * all of it that it reads, so calls that overlap on one GPU (several host threads, or
 * several streams running at once) race and must be serialised by the caller.
 * Errors: as park_retrieve_blocks; INVALID also for a NULL scores and for a stream of another
 * device; WORKSPACE when the sizes need more than PARK_NOALLOC_SCRATCH_BYTES
 * (park_noalloc_scratch_bytes); HIP also when the current device, the stream's device or the
 * scratch address cannot be obtained.
 */
PARK_API int park_retrieve_blocks_noalloc(const void* Q, int dtype, int B, int H, int N, int d,
                                          const float* centroids, const int32_t* counts, int n_clusters,
                                          int q_block, float top_p, int top_k, float scale, float* scores,
                                          uint8_t* mask, int32_t* block_list, int32_t* block_count,
                                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PARK_H */
