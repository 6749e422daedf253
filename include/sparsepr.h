/*
 * sparsepr.h -- C ABI of the MI355X (gfx950) SparsePR attention-call library.
 *
 * One SparsePR attention call ("Partition the Support, Reconstruct the
 * Residual: Training-Free Sparse Attention for Video Generation and World
 * Models", the SparsePR paper) runs five library calls in this order:
 *
 *   sparsepr_partition_layout  group-major permutation + gather + centroids
 *   sparsepr_route_cells       centroid-logit routing under a pair budget
 *   sparsepr_sparse_attn       renormalised hard-drop attention on the cells
 *   sparsepr_probe_fit         Algorithm A.1 probes, exact probe rows, ridge
 *                              fit and residual-subspace projection
 *   sparsepr_correct           corrected output in original token order
 *
 * probe_fit does not read the sparse-attention output, so it may run on a
 * second stream concurrently with sparse_attn (both only read what
 * partition_layout and route_cells wrote).
 *
 * The comments of this library number the steps of a call:
 *   S1 stable counting sort of the labels (permutation, group offsets)
 *   S2 gather of Q, K, V into group-major order (V as scaled fp16)
 *   S3 fp64 group centroids                       -- partition_layout
 *   S4 cell routing                               -- route_cells
 *   S5 sparse attention                           -- sparse_attn
 *   S6 probe selection (Algorithm A.1)
 *   S7 exact probe rows (retained / omitted sums)
 *   S8 weighted ridge fit and residual subspace   -- probe_fit
 *   S9 correction and restore to token order      -- correct
 *
 * Further entry points: sparsepr_rcp_partition builds the query and K/V
 * groups from the call's own activations (before S1), and
 * sparsepr_rcp_partition_ex does so across the calls of a layer;
 * sparsepr_route_cells_ex, sparsepr_probe_fit_ex and sparsepr_correct_ex
 * add the per-group routing rule, probe features and the restricted
 * residual estimators; sparsepr_probe_select with sparsepr_probe_fit_selected
 * split probe_fit in two, so that the probe selection (which reads only the
 * layout) can run while the cells are routed.
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer unless marked (host).
 *     Every buffer is allocated, owned and freed by the caller; the library
 *     keeps no pointer after a call returns and holds no mutable global
 *     state (except the device array of sparsepr_sparse_attn_noalloc).
 *     Calls are thread-safe.
 *   - Calls are asynchronous on `stream` and never synchronise the device;
 *     inputs must stay valid until the stream reaches the call.
 *   - Scratch memory is the caller's `ws` of `ws_bytes` bytes, at least
 *     sparsepr_workspace_bytes(call, dims, m, rank) (256-byte aligned).
 *     A workspace may be reused by the next call on the same stream.
 *   - Tensors listed as [H][N][d] are dense, row-major, head-major.
 *   - Data errors are the caller's contract: NaN/Inf inputs propagate into
 *     the outputs, and a label outside [0, C) is sorted as the nearest valid
 *     group (so every kernel stays inside its buffers, but the results are
 *     meaningless).  sparsepr_debug_check validates a call's integer data
 *     on the device and reports such errors in an error word.
 *   - Return value: SPARSEPR_OK, or an error code; on error nothing was
 *     launched.
 */
#ifndef SPARSEPR_H
#define SPARSEPR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SPARSEPR_OK = 0,
  SPARSEPR_ERR_INVALID = 1,      /* null pointer, bad size, m < 1, rank < 0, ... */
  SPARSEPR_ERR_UNSUPPORTED = 2,  /* head_dim not 64/128, dtype, C_q or C_k > 1024,
                                    N_k*d*(element bytes) or N_q*d*4 at or above 2^32 */
  SPARSEPR_ERR_WORKSPACE = 3,    /* ws_bytes smaller than required */
  SPARSEPR_ERR_HIP = 4           /* a kernel launch failed */
};

enum { SPARSEPR_BF16 = 0, SPARSEPR_F32 = 1 };

enum {
  SPARSEPR_CALL_PARTITION_LAYOUT = 0,
  SPARSEPR_CALL_ROUTE_CELLS = 1,
  SPARSEPR_CALL_SPARSE_ATTN = 2,
  SPARSEPR_CALL_PROBE_FIT = 3,
  SPARSEPR_CALL_CORRECT = 4,
  SPARSEPR_CALL_RCP_PARTITION = 5,
  SPARSEPR_CALL_PROBE_FIT_EX = 6,
  SPARSEPR_CALL_ROUTE_CELLS_EX = 7,
  SPARSEPR_CALL_SPARSE_ATTN_CORRECT = 8
};

/* Routing rules of sparsepr_route_cells_ex. */
enum {
  SPARSEPR_ROUTE_GLOBAL = 0,     /* sparsepr_route_cells: one pair budget per head */
  SPARSEPR_ROUTE_PER_GROUP = 1   /* a common key-token budget per query */
};

/* Residual estimators of sparsepr_probe_fit_ex (SparsePR paper §5 Table 4,
 * App. D.4): the full weighted ridge with output-subspace projection (the
 * default of sparsepr_probe_fit), the weighted mean residual, and the affine
 * variants with B = a I (scalar) and B = diag(b) (diagonal). */
enum {
  SPARSEPR_EST_FULL = 0,
  SPARSEPR_EST_MEAN = 1,
  SPARSEPR_EST_SCALAR = 2,
  SPARSEPR_EST_DIAGONAL = 3
};

/* Error bits of sparsepr_debug_check. */
enum {
  SPARSEPR_DBG_LABELS = 1,    /* a label outside [0, C_q) or [0, C_k) */
  SPARSEPR_DBG_OFFSETS = 2,   /* offsets not 0 .. N non-decreasing */
  SPARSEPR_DBG_PERM = 4,      /* perm not the stable counting sort of the labels */
  SPARSEPR_DBG_ROWPTR = 8,    /* cell_rowptr not 0 .. <= C_q*C_k non-decreasing */
  SPARSEPR_DBG_CELLS = 16,    /* a column outside [0, C_k), not ascending, an empty K/V
                                 group selected, or a query group with cells iff empty */
  SPARSEPR_DBG_ROUTE = 32,    /* routed_pairs[h] < 0: routing met non-finite scores */
  SPARSEPR_DBG_PROBES = 64    /* probe rows out of range, repeated, not -1 past
                                 min(m, N_q), or a token not perm_q of its row */
};

#define SPARSEPR_MAX_GROUPS 1024
#define SPARSEPR_MAX_PROBES 64
#define SPARSEPR_MAX_RANK 64

/*
 * Shape of one attention call (self-attention with N_q queries and N_k
 * paired key/value tokens per head, head dimension d; SparsePR paper §3
 * problem setup).  Strides describe the caller's q/k/v inputs in ELEMENTS,
 * so both [H][N][d] (stride_head = N*d, stride_tok = d) and [N][H][d]
 * (stride_head = d, stride_tok = H*d) model layouts are accepted; the last
 * dimension must be contiguous.  k and v share kv strides.
 */
typedef struct sparsepr_dims {
  int32_t heads;       /* H >= 1 */
  int32_t n_q;         /* N_q >= 1 */
  int32_t n_k;         /* N_k >= 1 */
  int32_t head_dim;    /* d: 64 or 128 */
  int32_t dtype;       /* SPARSEPR_BF16 or SPARSEPR_F32 (q, k, v and gathered copies) */
  int32_t c_q;         /* query groups, 1..1024 */
  int32_t c_k;         /* key/value groups, 1..1024 */
  int32_t reserved;    /* must be 0 */
  /* element strides of q (and of k, v); each a multiple of 16 bytes, with
   * stride_tok >= head_dim.  The q, k, v base pointers passed to the calls
   * must be 16-byte aligned (rows are read in 16-byte chunks); otherwise the
   * call returns SPARSEPR_ERR_INVALID. */
  int64_t q_stride_head, q_stride_tok;
  int64_t kv_stride_head, kv_stride_tok;
} sparsepr_dims;

/* Workspace bytes needed by one call (0 if it needs none).  m and rank are
 * only used by SPARSEPR_CALL_PROBE_FIT and SPARSEPR_CALL_PROBE_FIT_EX.
 * Returns 0 for invalid dims too; the call itself reports the error. */
size_t sparsepr_workspace_bytes(int32_t which_call, const sparsepr_dims* dims /* host */,
                                int32_t m, int32_t rank);

/* Human-readable text of a status code (static storage). */
const char* sparsepr_status_string(int32_t status);

/* ABI version: major*10000 + minor*100 + patch. */
int32_t sparsepr_version(void);

/*
 * S1-S3. Group-major layout.  (SparsePR paper §3: queries and keys are
 * partitioned into groups, each value follows its key; the review's step
 * (3): Q, K, V are permuted into group-major order before the varlen
 * block-sparse kernel.)
 *   labels_q [H][N_q], labels_kv [H][N_k]: int32 group ids in [0, C).
 *   q [.. per q strides], k, v [.. per kv strides]: dims.dtype.
 * Outputs
 *   perm_q [H][N_q], perm_kv [H][N_k]: int32 token index of each group-major
 *     row.  Groups in ascending id, tokens ascending inside a group (stable).
 *   offsets_q [H][C_q+1], offsets_kv [H][C_k+1]: int32 first row of each
 *     group; an empty group has offsets[a] == offsets[a+1].
 *   q_g [H][N_q][d], k_g [H][N_k][d]: dims.dtype, bit-exact copies.
 *   v_g [H][N_k][d] and v_shift [H] (int32): for SPARSEPR_F32, an fp32 copy
 *     and shift 0; for SPARSEPR_BF16, the fp16 operand of the PV product,
 *     v_g = fp16(v * 2^-v_shift[h]) with v_shift[h] chosen so the head's
 *     largest |v| lands in [2^14, 2^15): every bf16 value down to 2^-28 of
 *     that maximum converts exactly (smaller ones round to fp16 subnormals).
 *   centroid_q [H][C_q][d], centroid_k [H][C_k][d]: fp64 group means of q
 *     and k (exact fp64 sums of the inputs, divided by the group size);
 *     rows of empty groups are 0.
 */
int32_t sparsepr_partition_layout(const sparsepr_dims* dims /* host */,
                                  const int32_t* labels_q, const int32_t* labels_kv,
                                  const void* q, const void* k, const void* v,
                                  int32_t* perm_q, int32_t* offsets_q,
                                  int32_t* perm_kv, int32_t* offsets_kv,
                                  void* q_g, void* k_g, void* v_g, int32_t* v_shift,
                                  double* centroid_q, double* centroid_k,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * S4. Cell routing under a routed pair budget.  (SparsePR paper §4.3: each
 * cell G_a x G_b costs |G_a||G_b| interactions; the router keeps the
 * shortest prefix that reaches the budget; probe cost M/N_q is reserved, so
 * the caller passes budget = ceil((rho*N_q - M) * N_k).)
 * Score s_ab = centroid_q[a] . centroid_k[b] / sqrt(d) in fp64.  Every
 * non-empty query group first keeps its best non-empty cell (ties -> smaller
 * b); then the other non-empty cells are taken in (s desc, a asc, b asc)
 * order while the running pair count is below `routed_pair_budget`.  Empty
 * groups are never selected.
 * Outputs
 *   cell_rowptr [H][C_q+1]: int32, per-head CSR row pointers (start at 0).
 *   cell_col [H][C_q*C_k]: int32, selected b of query group a in
 *     cell_col[h][rowptr[a] .. rowptr[a+1]), ascending; slots past
 *     rowptr[C_q] are left untouched.
 *   routed_pairs [H]: int64, sum of |G_a||G_b| over selected cells; -1 if
 *     the head's scores were not finite (NaN/Inf inputs), in which case the
 *     head keeps only its forced cells.
 */
int32_t sparsepr_route_cells(const sparsepr_dims* dims /* host */,
                             const int32_t* offsets_q, const int32_t* offsets_kv,
                             const double* centroid_q, const double* centroid_k,
                             int64_t routed_pair_budget,
                             int32_t* cell_rowptr, int32_t* cell_col, int64_t* routed_pairs,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * S4 with a choice of rule.  SPARSEPR_ROUTE_GLOBAL is sparsepr_route_cells
 * (`budget` = routed pairs).  SPARSEPR_ROUTE_PER_GROUP is the rule of the
 * SparsePR paper §4.3: every non-empty query group ranks the non-empty K/V
 * groups by decreasing score s_ab (fp64 centroid logit; ties -> smaller b)
 * and keeps the shortest prefix whose key tokens sum(|G_b|) reach `budget`
 * (key tokens per query: the caller passes ceil((rho*N_q - M) * N_k / N_q));
 * a group keeps at least its top cell.  Outputs as sparsepr_route_cells.
 * Workspace: sparsepr_workspace_bytes(SPARSEPR_CALL_ROUTE_CELLS_EX, ...).
 */
int32_t sparsepr_route_cells_ex(const sparsepr_dims* dims /* host */, int32_t rule,
                                const int32_t* offsets_q, const int32_t* offsets_kv,
                                const double* centroid_q, const double* centroid_k,
                                int64_t budget,
                                int32_t* cell_rowptr, int32_t* cell_col, int64_t* routed_pairs,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * S5. Renormalised hard-drop attention.  (SparsePR paper §3: a query of
 * group a attends only to keys of the groups selected for a, with the
 * softmax normalised over those keys.)
 *   q_g, k_g, v_g, v_shift: group-major outputs of partition_layout.
 *   softmax_scale: logits are (q . k) * softmax_scale (1/sqrt(d) normally).
 * Outputs (group-major row order)
 *   o_sp [H][N_q][d]: fp32 sparse output.
 *   lse [H][N_q]: fp32 natural-log sum of exp of the scaled logits (may be NULL).
 * Every non-empty query group has at least one selected cell after
 * route_cells, so every row is written.
 */
int32_t sparsepr_sparse_attn(const sparsepr_dims* dims /* host */,
                             const int32_t* offsets_q, const int32_t* offsets_kv,
                             const int32_t* cell_rowptr, const int32_t* cell_col,
                             const void* q_g, const void* k_g, const void* v_g,
                             const int32_t* v_shift,
                             float softmax_scale, float* o_sp, float* lse,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * S5 for callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): as
 * sparsepr_sparse_attn, without a workspace.  The call allocates nothing;
 * its work-item table lives in a fixed device array of the library
 * (65537 int32 = 256 KiB, held on each GPU the library runs on until the
 * process ends), so H * C_q + 1 must not exceed 65537 (otherwise
 * SPARSEPR_ERR_UNSUPPORTED).  The table is rewritten in full by every call.
 * Every call on one GPU shares that array: calls that overlap on one GPU
 * (different streams, or threads) race and must be serialised by the
 * caller.  The first call on a device looks the array up with that device
 * current (SPARSEPR_ERR_HIP if the lookup fails).
 */
int32_t sparsepr_sparse_attn_noalloc(const sparsepr_dims* dims /* host */,
                                     const int32_t* offsets_q, const int32_t* offsets_kv,
                                     const int32_t* cell_rowptr, const int32_t* cell_col,
                                     const void* q_g, const void* k_g, const void* v_g,
                                     const int32_t* v_shift,
                                     float softmax_scale, float* o_sp, float* lse,
                                     hipStream_t stream);

/*
 * S6-S8. Probes and correction fit.  (SparsePR paper App. A.2, Algorithm
 * A.1: probe rows are taken per query group by increasing distance to the
 * group centroid, groups by decreasing size, round-robin, until
 * min(m, N_q) probes; exact rows against all keys give O_dense and the
 * residual R_p = O_dense - O_sp at the probes; coverage weights |G_a|/m_a;
 * weighted standardisation with sqrt(var + 1e-6); ridge with `lambda`;
 * projection on the top `rank` right singular vectors of the weighted
 * centred residuals (singular values <= 1e-10 * largest dropped).)
 * The distance uses the raw queries (features of the given partition) and
 * the fp64 centroids of partition_layout.  O_sp at a probe row is formed
 * here from the same pass that forms the dense row (retained and omitted
 * partial sums, SparsePR paper App. A.1), so this call does not read the
 * output of sparse_attn.
 *   m: 1..64 probes per head; rank: 0..64 (capped at min(m, d) columns).
 * Outputs
 *   probe_rows [H][m], probe_tokens [H][m]: int32 group-major row and token
 *     index of each probe in selection order; entries past min(m, N_q) = -1.
 *   o_probe_dense [H][m][d]: fp32 dense output of each probe row.
 *   o_probe_sparse [H][m][d]: fp32 hard-drop output at each probe (may be NULL).
 *   corr_a [H][d][rank], corr_psi_t [H][rank][d], corr_c [H][d]: fp32 folded
 *     correction  out = o + (o . A) Psi^T + c  with A = diag(1/s) B Psi and
 *     c = mu_R - (mu_x . A) Psi^T; dropped directions are zero columns.
 */
int32_t sparsepr_probe_fit(const sparsepr_dims* dims /* host */, int32_t m, int32_t rank,
                           double lambda,
                           const int32_t* offsets_q, const int32_t* offsets_kv,
                           const int32_t* perm_q,
                           const int32_t* cell_rowptr, const int32_t* cell_col,
                           const double* centroid_q,
                           const void* q_g, const void* k_g, const void* v_g,
                           const int32_t* v_shift, float softmax_scale,
                           int32_t* probe_rows, int32_t* probe_tokens,
                           float* o_probe_dense, float* o_probe_sparse,
                           float* corr_a, float* corr_psi_t, float* corr_c,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * S9. Correction and restore.  (Review step (5): unprobed rows get their
 * sparse output plus the predicted residual, probe rows their dense
 * output; the result returns to the original token order.)
 *   o_sp [H][N_q][d] fp32 group-major (sparse_attn output).
 *   out: [H][N_q][d]-shaped in ORIGINAL token order with element strides
 *     out_stride_head, out_stride_tok; out_dtype SPARSEPR_BF16 (nearest-even
 *     rounding) or SPARSEPR_F32.
 */
int32_t sparsepr_correct(const sparsepr_dims* dims /* host */, int32_t m, int32_t rank,
                         const int32_t* perm_q, const float* o_sp,
                         const int32_t* probe_tokens, const float* o_probe_dense,
                         const float* corr_a, const float* corr_psi_t, const float* corr_c,
                         void* out, int32_t out_dtype,
                         int64_t out_stride_head, int64_t out_stride_tok,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * S5 + S9 in one call: the probe-first order of a call.  (SparsePR paper
 * App. A.1: the exact probe rows come with their hard-drop rows from the
 * retained / omitted partial sums, so probe_fit does not need the output of
 * sparse_attn and can run before it; the review's step (5): unprobed rows get
 * their sparse output plus the predicted residual, probe rows their dense
 * output, in the original token order.)  Run sparsepr_probe_fit (or _ex)
 * first; this call then computes the hard-drop attention of every row and
 * writes
 *   out[h][perm_q[h][r]] = o + (o A) Psi^T + g * o + c   (unprobed rows)
 *   out[h][probe token]  = o_probe_dense                  (probe rows)
 * so no O_sp is stored.  Arguments as sparsepr_sparse_attn and
 * sparsepr_correct_ex (corr_g may be NULL: g = 0); lse may be NULL.
 * For bf16 inputs with rank <= 16 the correction runs in the attention
 * epilogue (exact fp32 products); otherwise the call keeps O_sp in its
 * workspace and runs the correction kernel after the attention.
 * Workspace: sparsepr_workspace_bytes(SPARSEPR_CALL_SPARSE_ATTN_CORRECT,
 * dims, m, rank).
 */
int32_t sparsepr_sparse_attn_correct(const sparsepr_dims* dims /* host */, int32_t m,
                                     int32_t rank, const int32_t* offsets_q,
                                     const int32_t* offsets_kv, const int32_t* cell_rowptr,
                                     const int32_t* cell_col, const void* q_g, const void* k_g,
                                     const void* v_g, const int32_t* v_shift,
                                     float softmax_scale, const int32_t* perm_q,
                                     const int32_t* probe_tokens, const float* o_probe_dense,
                                     const float* corr_a, const float* corr_psi_t,
                                     const float* corr_c, const float* corr_g, void* out,
                                     int32_t out_dtype, int64_t out_stride_head,
                                     int64_t out_stride_tok, float* lse, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/*
 * Partition step before S1: response-coupled partitioning.  (SparsePR paper
 * §4.1; App. B.1 key response metric; App. B.2 query response metric and
 * RMS normalisation; App. C.1 clustering on the GPU with initial centres
 * sampled from the feature rows.)  Per head:
 *   M_K = Q_s^T Q_s / M_s over the query rows floor(i N_q / m_s), i < m_s
 *     (every row when N_q <= m_s);
 *   F_K = the leading r_k eigenvectors of M_K, each scaled by
 *     sqrt(max(lambda, 0) / mean of the r_k retained eigenvalues);
 *   K/V labels = Lloyd's k-means (`iters` iterations, C_k = dims.c_k
 *     centres starting at rows init_k) on phi_K = k F_K;
 *   M_Q = K~^T K~ / C_nonempty, K~ = non-empty K/V group centroids in key
 *     space minus their mean; F_Q likewise with r_q;
 *   query labels = k-means (C_q = dims.c_q centres from init_q) on
 *     phi_Q = u / max(RMS(u), 1e-6), u = q F_Q.
 * One Lloyd iteration assigns every row to the centre with the smallest
 * |c|^2 - 2 x.c (x.c from the bf16 pair of each operand, three products,
 * fp32 accumulation; ties to the smaller index) and moves each centre to
 * the mean of its rows (an empty cluster keeps its centre); the labels are
 * those of the last assignment.  Metrics, factors and centroids are fp32.
 *   m_s >= 1; r_k, r_q in 1..min(64, d); iters >= 1.
 *   q, k: as for partition_layout (dims strides and dtype); v is not used.
 *   init_q [H][C_q], init_k [H][C_k]: int32 row indices (clamped to [0, N)).
 * Outputs
 *   labels_q [H][N_q], labels_kv [H][N_k]: int32 group ids (inputs of
 *     partition_layout); empty groups may occur.
 *   phi_q [H][N_q][r_q]: fp32 query coordinates in token order (may be NULL;
 *     the probe distances of a response-coupled partition use them, see
 *     sparsepr_probe_fit_ex).
 *   phi_k [H][N_k][r_k]: fp32 key coordinates in token order (may be NULL).
 */
int32_t sparsepr_rcp_partition(const sparsepr_dims* dims /* host */, int32_t m_s, int32_t r_k,
                               int32_t r_q, int32_t iters, const void* q, const void* k,
                               const int32_t* init_q, const int32_t* init_k,
                               int32_t* labels_q, int32_t* labels_kv, float* phi_q, float* phi_k,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Response-coupled partitioning across calls: a first call and later calls
 * of the same layer.  (SparsePR paper App. C.1: later calls start k-means
 * from the previous centroids in the original space projected into the
 * current response coordinates, and update the metric factors with two
 * subspace iterations started from the previous factors, using a Cholesky
 * factorisation.)  As sparsepr_rcp_partition, plus a state the call reads
 * (warm = 1) and always writes back:
 *   basis_k [H][d][r_k], basis_q [H][d][r_q] fp32: orthonormal bases of the
 *     response coordinates.  A first call (warm = 0) stores the leading
 *     eigenvectors; a later call runs two steps X <- Y L^-T, Y = M X,
 *     Y^T Y = L L^T (fp64; a Cholesky pivot at or below 1e-10 of the largest
 *     diagonal entry of Y^T Y drops its direction, which stays 0), and
 *     weights direction j by sqrt(max(x_j^T M x_j, 0) / mean over the r).
 *   cent_k [H][C_k][d], cent_q [H][C_q][d] fp32: each group's mean in the
 *     original key or query space.  A later call starts k-means at
 *     cent_k F_K and at phi_Q(cent_q) (RMS-normalised); a group left empty
 *     keeps its previous centroid, and on a first call its initial row.
 *   warm: 0 = first call (init_q, init_k required), 1 = later call (the
 *     state must hold a previous call's output for the same dims, r_k and
 *     r_q; init_q, init_k are not read and may be NULL).
 * The state buffers are read and overwritten in place; calls that share a
 * state must not overlap.  Every pointer but init_q, init_k, phi_q, phi_k is
 * required.  Workspace: sparsepr_workspace_bytes(SPARSEPR_CALL_RCP_PARTITION,
 * dims, 0, 0).
 */
int32_t sparsepr_rcp_partition_ex(const sparsepr_dims* dims /* host */, int32_t m_s, int32_t r_k,
                                  int32_t r_q, int32_t iters, int32_t warm, const void* q,
                                  const void* k, const int32_t* init_q, const int32_t* init_k,
                                  float* basis_q, float* basis_k, float* cent_q, float* cent_k,
                                  int32_t* labels_q, int32_t* labels_kv, float* phi_q,
                                  float* phi_k, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * S6-S8 with options.  As sparsepr_probe_fit, plus:
 *   probe_feat [H][N_q][feat_dim] fp32 token order (feat_dim 1..64), or
 *     NULL: when given, the distance of a row to its group's centroid is
 *     taken in that feature space (the coordinates that formed the partition;
 *     SparsePR paper App. B.2: the query-response coordinates stratify the
 *     probes), with fp64 feature means and distances; centroid_q is then not
 *     read (may be NULL).
 *   estimator: SPARSEPR_EST_*.  The restricted estimators use the weights,
 *     means and feature scale of the full fit and minimise the same weighted
 *     squared error with penalty lambda * |B|_F^2 (so lambda * d * a^2 for
 *     B = a I); the mean is not penalised and the output is not truncated
 *     (`rank` is ignored; corr_a and corr_psi_t are zeroed).
 *   corr_g [H][d] fp32: diagonal gain g = diag(B) / s of the folded
 *     correction out = o + (o A) Psi^T + g * o + c; zero for
 *     SPARSEPR_EST_FULL (may then be NULL), required otherwise.
 * Workspace: sparsepr_workspace_bytes(SPARSEPR_CALL_PROBE_FIT_EX, dims, m, rank).
 */
int32_t sparsepr_probe_fit_ex(const sparsepr_dims* dims /* host */, int32_t m, int32_t rank,
                              double lambda, int32_t estimator,
                              const int32_t* offsets_q, const int32_t* offsets_kv,
                              const int32_t* perm_q,
                              const int32_t* cell_rowptr, const int32_t* cell_col,
                              const double* centroid_q,
                              const float* probe_feat, int32_t feat_dim,
                              const void* q_g, const void* k_g, const void* v_g,
                              const int32_t* v_shift, float softmax_scale,
                              int32_t* probe_rows, int32_t* probe_tokens,
                              float* o_probe_dense, float* o_probe_sparse,
                              float* corr_a, float* corr_psi_t, float* corr_c, float* corr_g,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * S6-S8 in two calls.  (SparsePR paper App. A.2, Algorithm A.1: the probe
 * rows are chosen from the query partition alone, so the selection can run
 * before the routing is known; the exact probe rows and the fit of App. A.1,
 * A.2 and D.3 need the routed cells.)  sparsepr_probe_select followed by
 * sparsepr_probe_fit_selected on the same stream order, with the same dims,
 * m and ws, computes exactly what one sparsepr_probe_fit_ex call computes.
 *
 * sparsepr_probe_select: the probe plan and probe rows.  Arguments as in
 *   sparsepr_probe_fit_ex (probe_feat / feat_dim or centroid_q and q_g);
 *   writes probe_rows, probe_tokens and, in ws, the per-group probe counts
 *   and each probe's group.
 * sparsepr_probe_fit_selected: exact probe rows, merge and fit for the
 *   probes in probe_rows (read) and in ws, which must hold what the select
 *   call wrote (the caller orders the two calls and keeps ws untouched in
 *   between).  Other arguments as in sparsepr_probe_fit_ex.
 * Workspace: one buffer of sparsepr_workspace_bytes(SPARSEPR_CALL_PROBE_FIT_EX,
 * dims, m, rank) bytes for both calls (the fit call needs only the
 * SPARSEPR_CALL_PROBE_FIT size).
 */
int32_t sparsepr_probe_select(const sparsepr_dims* dims /* host */, int32_t m,
                              const int32_t* offsets_q, const int32_t* perm_q,
                              const double* centroid_q, const float* probe_feat,
                              int32_t feat_dim, const void* q_g, int32_t* probe_rows,
                              int32_t* probe_tokens, void* ws, size_t ws_bytes,
                              hipStream_t stream);

int32_t sparsepr_probe_fit_selected(const sparsepr_dims* dims /* host */, int32_t m,
                                    int32_t rank, double lambda, int32_t estimator,
                                    const int32_t* offsets_q, const int32_t* offsets_kv,
                                    const int32_t* cell_rowptr, const int32_t* cell_col,
                                    const void* q_g, const void* k_g, const void* v_g,
                                    const int32_t* v_shift, float softmax_scale,
                                    const int32_t* probe_rows, float* o_probe_dense,
                                    float* o_probe_sparse, float* corr_a, float* corr_psi_t,
                                    float* corr_c, float* corr_g, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/*
 * S9 with a diagonal gain: as sparsepr_correct with
 *   out = o + (o A) Psi^T + g * o + c
 * for unprobed rows (corr_g [H][d] from sparsepr_probe_fit_ex; NULL means
 * g = 0, which is sparsepr_correct).
 */
int32_t sparsepr_correct_ex(const sparsepr_dims* dims /* host */, int32_t m, int32_t rank,
                            const int32_t* perm_q, const float* o_sp,
                            const int32_t* probe_tokens, const float* o_probe_dense,
                            const float* corr_a, const float* corr_psi_t, const float* corr_c,
                            const float* corr_g,
                            void* out, int32_t out_dtype,
                            int64_t out_stride_head, int64_t out_stride_tok,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Debug validation of a call's integer data (read-only; for tests and
 * debugging, not needed by a correct caller).  The quantities are those of
 * the SparsePR paper's problem setup (§3: query and key index sets
 * partitioned into groups; cells G_a x G_b selected or not) and of its probe
 * step (App. A.2, Algorithm A.1: min(M, N_q) distinct probe rows).
 * Every array argument but error_word may be NULL, and is then not checked:
 *   labels_q [H][N_q], labels_kv [H][N_k]: in [0, C_q), [0, C_k).
 *   offsets_q [H][C_q+1], offsets_kv [H][C_k+1]: start at 0, non-decreasing,
 *     end at N.
 *   perm_q, perm_kv [H][N]: inside each group, tokens in [0, N), strictly
 *     ascending, each labelled with its group (needs offsets; labels if
 *     given).  With valid offsets this makes perm the stable counting sort.
 *   cell_rowptr [H][C_q+1], cell_col [H][C_q*C_k] (both or neither): CSR
 *     rows starting at 0 and within C_q*C_k, columns in [0, C_k) strictly
 *     ascending; with offsets also: no empty K/V group selected, and a query
 *     group has cells if and only if it is non-empty.
 *   routed_pairs [H]: not negative.
 *   probe_rows, probe_tokens [H][m] (m in 1..64): as sparsepr_probe_fit
 *     writes them; tokens are compared with perm_q when both are given.
 * error_word: one device uint32, overwritten with the OR of the
 *   SPARSEPR_DBG_* bits found (0 when everything checked is valid); read it
 *   after the stream reaches the call.  A value that fails a check is never
 *   used as an index; values are used as indices only after they have been
 *   checked against the extent of the array they index.
 */
int32_t sparsepr_debug_check(const sparsepr_dims* dims /* host */, int32_t m,
                             const int32_t* labels_q, const int32_t* labels_kv,
                             const int32_t* offsets_q, const int32_t* offsets_kv,
                             const int32_t* perm_q, const int32_t* perm_kv,
                             const int32_t* cell_rowptr, const int32_t* cell_col,
                             const int64_t* routed_pairs, const int32_t* probe_rows,
                             const int32_t* probe_tokens, uint32_t* error_word,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSEPR_H */
