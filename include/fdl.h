/*
 * fdl.h - C ABI of the Focus-dLLM sparse attention step on AMD Instinct MI355X (gfx950).
 *
 * One non-block-entry denoising step of a long-context diffusion LLM, as the
 * structured summary of "Focus-dLLM: Accelerating Long-Context Diffusion LLM
 * Inference via Confidence-Guided Context Focusing" (paper.rainbus.top/paper/
 * 2602.02159) describes it in its sections "Core method" and "Method steps"
 * (1)-(5):
 *   fdl_pcgi_select       (1) top-k masked positions by previous confidence, (2) windows
 *   fdl_dense_attention   (3) dense layers 1..l_dense, and the block-entry full refresh
 *   fdl_sink_identify     (3) attention sinks from layer l_dense's attention distribution
 *   fdl_block_means       (4) mean key per prompt block (keys only: can run ahead)
 *   fdl_block_score_topc  (4) relevance R_b of the active queries, top-C blocks
 *   fdl_sparse_attention  (5) attention of the active queries over I_p only
 *   fdl_block_score_topc_ex, fdl_sparse_attention_ex   per-KV-head block sets and the
 *                         max-over-queries relevance
 *   fdl_kv_refresh        approximate KV cache: the rows of U(t) take new K/V (Prerequisites)
 *   fdl_block_means_refresh  (4) the means of the blocks a refresh touched
 *   fdl_kv_refresh_means     both in one launch
 *   fdl_confidence_unmask    confidence of the masked positions, unmasking of n(t) of them
 *   fdl_dcu_select           per-layer cache update sets of the dynamic cache update (DCU)
 *   fdl_calibrate_read, fdl_calibrate_mfma   achievable read and MFMA rates (measurement)
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates device memory, never frees, never synchronises the stream
 *     and never throws or aborts: it validates what the host can see, enqueues
 *     its kernels on `stream` (NULL = the default stream) and returns a status.
 *     Kernels read device-side counts (n_focus, n_active) themselves, so a whole
 *     step runs without a host round trip.
 *   - Entry points that need temporary device memory take a caller-owned
 *     workspace (`ws`, `ws_bytes`); the matching *_workspace_bytes function
 *     returns the size needed.  The workspace holds no state between calls.
 *   - dtype (fdl_dtype) is shared by Q, K, V and O: FDL_F32, or FDL_BF16 with fp32
 *     accumulation.  Head dim d is 64 or 128 and is contiguous in memory.
 *     Q, K, V and O are addressed as base + b*s.b + h*s.h + row*s.r (element
 *     strides, fdl_strides); each row must start on a 16-byte boundary, and the
 *     row stride must lie below 2^31 elements in magnitude (FDL_ERR_SHAPE).
 *   - Query rows: the logical query row r of sequence b reads the physical row
 *     q_idx[b*nq_max + r] of Q when q_idx is non-NULL (e.g. the active_idx output
 *     of fdl_pcgi_select), else row r.  Rows r >= n_q[b] are padding (n_q NULL:
 *     all nq_max rows are valid); padding rows of O are written as 0 and their
 *     log-sum-exp as -inf.  Physical rows and indices must lie in [0, L); the
 *     host cannot check device-resident indices, and out-of-range values there
 *     give undefined results.
 *   - Grouped-query attention: query head h reads KV head floor(h*Hkv/Hq);
 *     Hq % Hkv == 0.  Scale: `scale` <= 0 selects 1/sqrt(d).  Attention has no
 *     mask (dLLM attention is bidirectional).
 *   - Index outputs are ascending and padded with -1.  Selections order by value,
 *     larger first, and take the lower index among equal values.
 *   - Calls are stream-ordered and reentrant; there is no global state.  Two
 *     calls that share a workspace must be ordered on one stream.
 */
#ifndef FDL_H
#define FDL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fdl_status {
    FDL_OK = 0,
    FDL_ERR_NULL = 1,        /* a required pointer is NULL */
    FDL_ERR_SHAPE = 2,       /* a size is negative, zero where it may not be, or inconsistent */
    FDL_ERR_DTYPE = 3,       /* dtype is not FDL_F32 or FDL_BF16 */
    FDL_ERR_ALIGN = 4,       /* a pointer or a row stride breaks the 16-byte row alignment */
    FDL_ERR_WORKSPACE = 5,   /* ws is NULL or ws_bytes is below the *_workspace_bytes size */
    FDL_ERR_HIP = 6,         /* a kernel launch failed; the HIP error is left for hipGetLastError */
    FDL_ERR_UNSUPPORTED = 7  /* a valid but unsupported configuration (head dim other than 64/128) */
} fdl_status;

typedef enum fdl_dtype { FDL_F32 = 0, FDL_BF16 = 1 } fdl_dtype;

/* Element strides of the batch, head and row axes; the head-dim axis is contiguous. */
typedef struct fdl_strides { int64_t b, h, r; } fdl_strides;

/* Static text for a status code (never NULL). */
const char* fdl_status_string(fdl_status status);

/* k = floor(rho * n_t), evaluated in double precision (negative results clamp to 0). */
int fdl_focus_count(int n_t, double rho);

/*
 * fdl_pcgi_select - past-confidence-guided focus selection and window expansion.
 * Summary page, "Core method" and "Method steps" (1)-(2): among the positions
 * still [MASK], keep the k = floor(rho*n_t) with the highest previous-step
 * confidence c_{t-1} (I_focus), then widen each focus position p to the window
 * [p - floor(w/2), p - floor(w/2) + w) clipped to [0, L); the union is I_active.
 *   conf       [B, L] fp32, previous-step confidence (compared exactly; NaN unsupported,
 *              -0.0 equals +0.0)
 *   mask       [B, L] uint8, non-zero where the slot is still [MASK]
 *   focus_idx  [B, k_cap] out, I_focus ascending, -1 padded; k_cap >= k
 *   n_focus    [B] out, min(k, #masked)
 *   active_idx [B, nq_max] out, I_active ascending, -1 padded; nq_max >= min(k*w, L)
 *   n_active   [B] out, |I_active|
 * Fewer masked slots than k: all of them are kept.  Errors: FDL_ERR_NULL,
 * FDL_ERR_SHAPE (B, L, w < 1, n_t < 0, rho < 0 or NaN, k_cap or nq_max too small).
 */
fdl_status fdl_pcgi_select(const float* conf, const uint8_t* mask, int B, int L,
                           int n_t, double rho, int w,
                           int32_t* focus_idx, int32_t* n_focus, int k_cap,
                           int32_t* active_idx, int32_t* n_active, int nq_max,
                           hipStream_t stream);

/*
 * fdl_dense_attention - full bidirectional attention of the given query rows over all L keys.
 * Summary page, "Method steps": the block-entry full refresh (use_sparse = False,
 * every row attends to every key) and the dense layers 1..l_dense of a sparse step
 * (step (3)), there for the active rows only (q_idx = active_idx, n_q = n_active).
 *   q       [B, Hq, *, d] with strides qs; q_idx [B, nq_max] or NULL; n_q [B] or NULL
 *   k, v    [B, Hkv, L, d] with strides ks, vs
 *   vt      NULL, or the same values as v laid out [B, Hkv, d, L] (keys contiguous) with
 *           strides vts = (b, h, d): read only by the bf16 d = 128 path, which then
 *           loads runs of 64 consecutive keys from it instead of transposing V rows
 *           on chip (used when L is a multiple of 8; in fdl_sparse_attention also
 *           bs a multiple of 64 and P a multiple of 8; otherwise ignored).  There the
 *           pointer must be 16-byte aligned and vts.b, vts.h, vts.r multiples of 8
 *           (FDL_ERR_ALIGN), with L <= vts.r < 2^24 (FDL_ERR_SHAPE).  The results are
 *           the same with or without it.  Keeping it current (e.g. for the rows an
 *           approximate KV cache refreshes) is the caller's part.
 *   o       [B, Hq, nq_max, d] out with strides os, in the input dtype
 *   lse     [B, Hq, nq_max] fp32 out (natural log of the softmax denominator) or NULL
 * Workspace: fdl_dense_attention_workspace_bytes (partial results of the key split).
 */
size_t fdl_dense_attention_workspace_bytes(fdl_dtype dtype, int B, int Hq, int Hkv, int L,
                                           int d, int nq_max);
fdl_status fdl_dense_attention(fdl_dtype dtype, int B, int Hq, int Hkv, int L, int d,
                               const void* q, fdl_strides qs, const int32_t* q_idx,
                               const int32_t* n_q, int nq_max,
                               const void* k, fdl_strides ks, const void* v, fdl_strides vs,
                               const void* vt, fdl_strides vts,
                               float scale, void* o, fdl_strides os, float* lse,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * fdl_sink_identify - attention-sink positions from layer l_dense.
 * Summary page, "Prerequisites" (attention sinks) and "Method steps" (3): layer
 * l_dense's attention distribution identifies the sinks, which every deeper layer
 * of the step reuses.  score_j = sum over query heads h and valid query rows i of
 * exp(q_{h,i} . k_{g(h),j} * scale - lse_{h,i}), for every key j in [0, L); the
 * n_sinks keys of highest score form I_sink.
 *   q, q_idx, n_q, nq_max, k, ks, scale   as in fdl_dense_attention (same layer)
 *   lse        [B, Hq, nq_max] fp32, the lse output of fdl_dense_attention for these rows,
 *              or NULL: the library then computes it with a dense attention pass over the
 *              same rows and keys (its outputs discarded) inside the workspace
 *   sink_idx   [B, n_sinks] out, ascending
 *   scores     [B, L] fp32 out, or NULL
 * Workspace: fdl_sink_identify_workspace_bytes, a size that covers lse = NULL (with lse
 * given, only its first part is used).
 * Errors as fdl_dense_attention; n_sinks must lie in [0, L].
 */
size_t fdl_sink_identify_workspace_bytes(fdl_dtype dtype, int B, int Hq, int Hkv, int L,
                                         int d, int nq_max);
fdl_status fdl_sink_identify(fdl_dtype dtype, int B, int Hq, int Hkv, int L, int d,
                             const void* q, fdl_strides qs, const int32_t* q_idx,
                             const int32_t* n_q, int nq_max,
                             const void* k, fdl_strides ks, float scale, const float* lse,
                             int n_sinks, int32_t* sink_idx, float* scores,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * fdl_block_means - the mean key of every prompt block.
 * Summary page, "Method steps" (4): split the P prompt keys into nb = ceil(P/bs)
 * contiguous blocks and represent each by the mean of its keys (a short last
 * block by the mean of its own keys).  The means depend on the keys only, so a
 * caller may compute them for every layer ahead of the layers that score them.
 *   k, ks   [B, Hkv, L, d] with strides ks (rows 0..P-1 are read)
 *   P, bs   prompt length (1 <= P <= L), block size (>= 1)
 *   kbar    [B, Hkv, nb, d] fp32 out, dense, 16-byte aligned (FDL_ERR_ALIGN); each mean is summed in fp64 and rounded
 *           once.  The sum is exact, hence the mean correctly rounded, while the binary
 *           exponents of a block's nonzero keys span at most 29 - log2(bs) (fp32) or
 *           45 - log2(bs) (bf16)
 * Errors: NULL pointers (FDL_ERR_NULL), bad shapes (FDL_ERR_SHAPE), as for the
 * other entry points.  No workspace.
 */
fdl_status fdl_block_means(fdl_dtype dtype, int B, int Hkv, int L, int P, int d,
                           const void* k, fdl_strides ks, int bs, float* kbar, hipStream_t stream);

/*
 * fdl_block_score_topc - prompt-block pruning.
 * Summary page, "Method steps" (4): score every prompt block by its relevance to
 * the candidate queries and keep the C best.
 * R_b = scale * sum over query heads h and valid query rows i of q_{h,i} . kbar_{g(h),b}
 * (one block set per sequence, shared by all heads), accumulated in fp64 from the
 * fp32 block means.
 *   q, q_idx, n_q, nq_max, scale   as in fdl_dense_attention
 *   k, ks   the keys: the block means are computed first (as fdl_block_means does),
 *           into kbar when kbar is non-NULL, else into the workspace.  k NULL: kbar
 *           must hold the means already (from fdl_block_means) and only the scoring
 *           runs.
 *   P, bs, C   prompt length (P <= L), block size (>= 1), blocks kept (>= 0)
 *   block_idx  [B, C] out, ascending, -1 padded when C > nb
 *   R          [B, nb] fp64 out, or NULL
 *   kbar       [B, Hkv, nb, d] fp32 block means: out (k given) or in (k NULL), or NULL;
 *              16-byte aligned when given (FDL_ERR_ALIGN)
 * The workspace holds each KV head's part of R, R, and the block means when k is
 * given and kbar is NULL; its size does not depend on nq_max.
 */
size_t fdl_block_score_topc_workspace_bytes(fdl_dtype dtype, int B, int Hq, int Hkv, int P,
                                            int d, int bs, int nq_max);
fdl_status fdl_block_score_topc(fdl_dtype dtype, int B, int Hq, int Hkv, int L, int P, int d,
                                const void* q, fdl_strides qs, const int32_t* q_idx,
                                const int32_t* n_q, int nq_max,
                                const void* k, fdl_strides ks, float scale, int bs, int C,
                                int32_t* block_idx, double* R, float* kbar,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * fdl_block_score_topc_ex - fdl_block_score_topc with the relevance variants.  Summary page,
 * "Independent weaknesses" (the block representative and the relevance may hide blocks that
 * matter to few queries; Dream-like models differ per layer) and "Method steps" (4).  mode is
 * a combination of:
 *   FDL_SCORE_PER_HEAD  every KV head g keeps its own top-C from its own part of the
 *                       relevance, R_{g,b} = scale * sum over the query heads h of g and the
 *                       valid rows i of q_{h,i} . kbar_{g,b}; block_idx is [B, Hkv, C] and R
 *                       [B, Hkv, nb]; pass the lists to fdl_sparse_attention_ex with
 *                       blocks_per_head = 1
 *   FDL_SCORE_MAX       a block scores by its strongest single query: the maximum over the
 *                       heads (of g, per head) and valid rows of q_{h,i} . kbar, each dot in
 *                       fp64, times scale; -inf for every block of a sequence without valid
 *                       rows (the lowest C block ids are then kept)
 * FDL_SCORE_SUM (0) is fdl_block_score_topc.  Other arguments, the workspace and the errors
 * as there; a mode outside these bits is FDL_ERR_SHAPE.
 */
typedef enum fdl_score_mode { FDL_SCORE_SUM = 0, FDL_SCORE_PER_HEAD = 1, FDL_SCORE_MAX = 2 } fdl_score_mode;
fdl_status fdl_block_score_topc_ex(fdl_dtype dtype, int B, int Hq, int Hkv, int L, int P, int d,
                                   const void* q, fdl_strides qs, const int32_t* q_idx,
                                   const int32_t* n_q, int nq_max,
                                   const void* k, fdl_strides ks, float scale, int bs, int C, int mode,
                                   int32_t* block_idx, double* R, float* kbar,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * fdl_block_score_topc_noalloc - fdl_block_score_topc for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, results and errors as fdl_block_score_topc, without ws and
 * ws_bytes: the workspace is a device array inside the library, one per GPU, of
 * fdl_block_score_topc_noalloc_max_bytes() bytes (8 MiB), held until the process ends.
 * A call whose fdl_block_score_topc_workspace_bytes exceeds it returns FDL_ERR_WORKSPACE;
 * a failed lookup of the array returns FDL_ERR_HIP.  It allocates nothing.  Every call on
 * one GPU uses that GPU's array: calls that overlap on one GPU (different streams, or
 * unordered host threads) race.
 */
size_t fdl_block_score_topc_noalloc_max_bytes(void);
fdl_status fdl_block_score_topc_noalloc(fdl_dtype dtype, int B, int Hq, int Hkv, int L, int P, int d,
                                        const void* q, fdl_strides qs, const int32_t* q_idx,
                                        const int32_t* n_q, int nq_max,
                                        const void* k, fdl_strides ks, float scale, int bs, int C,
                                        int32_t* block_idx, double* R, float* kbar, hipStream_t stream);

/*
 * fdl_sparse_attention - attention of the active queries over I_p only.
 * Summary page, "Method steps" (5): I_p is the union of the sinks and the
 * selected prompt blocks; this library also adds the generation region [P, L)
 * (without it, keeping every block could not reproduce dense attention).  Each
 * key of I_p is attended once, however many of the three sets hold it.
 *   q, q_idx, n_q, nq_max, k, ks, v, vs, vt, vts, scale, o, os, lse   as in fdl_dense_attention
 *   sink_idx   [B, n_sinks] positions (e.g. fdl_sink_identify output)
 *   block_idx  [B, C] prompt block ids (e.g. fdl_block_score_topc output)
 *              Each list is read as the set of its valid entries: positions in [0, L),
 *              block ids in [0, ceil(P/bs)).  Entries outside that range (-1 padding
 *              included) are ignored wherever they stand, repeated entries count once, and
 *              the order is free (ascending lists, as the selections write them, take the
 *              fast path; others are sorted on the device).
 *   P, bs      prompt length and block size used to select block_idx
 * n_sinks and C above 4096 give FDL_ERR_UNSUPPORTED.
 */
size_t fdl_sparse_attention_workspace_bytes(fdl_dtype dtype, int B, int Hq, int Hkv, int L,
                                            int P, int d, int nq_max, int n_sinks, int C,
                                            int bs);
fdl_status fdl_sparse_attention(fdl_dtype dtype, int B, int Hq, int Hkv, int L, int P, int d,
                                const void* q, fdl_strides qs, const int32_t* q_idx,
                                const int32_t* n_q, int nq_max,
                                const void* k, fdl_strides ks, const void* v, fdl_strides vs,
                                const void* vt, fdl_strides vts,
                                const int32_t* sink_idx, int n_sinks,
                                const int32_t* block_idx, int C, int bs,
                                float scale, void* o, fdl_strides os, float* lse,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * fdl_sparse_attention_ex - fdl_sparse_attention with one block list per KV head when
 * blocks_per_head is 1 (FDL_SCORE_PER_HEAD selections): block_idx is [B, Hkv, C], and the
 * query heads of KV head g attend over the sinks, the blocks of list (b, g) and [P, L).  The
 * sinks stay shared.  blocks_per_head 0 is fdl_sparse_attention; other values are
 * FDL_ERR_SHAPE.  Workspace: fdl_sparse_attention_ex_workspace_bytes (the key lists of
 * the list-building path are per (sequence, KV head)).
 */
size_t fdl_sparse_attention_ex_workspace_bytes(fdl_dtype dtype, int B, int Hq, int Hkv, int L,
                                               int P, int d, int nq_max, int n_sinks, int C,
                                               int bs, int blocks_per_head);
fdl_status fdl_sparse_attention_ex(fdl_dtype dtype, int B, int Hq, int Hkv, int L, int P, int d,
                                   const void* q, fdl_strides qs, const int32_t* q_idx,
                                   const int32_t* n_q, int nq_max,
                                   const void* k, fdl_strides ks, const void* v, fdl_strides vs,
                                   const void* vt, fdl_strides vts,
                                   const int32_t* sink_idx, int n_sinks,
                                   const int32_t* block_idx, int C, int blocks_per_head, int bs,
                                   float scale, void* o, fdl_strides os, float* lse,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * fdl_kv_refresh - the approximate KV cache refresh of one step.
 * Summary page, "Prerequisites" (approximate KV cache): the rows of the refresh set
 * U(t) take freshly computed keys and values, every other row keeps its cached ones.
 *   rows       [B, n_max] int32 positions of U(t) (distinct within a sequence; entries
 *              outside [0, L) are skipped), e.g. active_idx; n_rows [B] or NULL (all n_max)
 *   k_new, v_new  [B, Hkv, n_max, d] with strides kns, vns: row i belongs to rows[b][i]
 *   k, v       [B, Hkv, L, d] caches with strides ks, vs, updated in place
 *   vt, vts    NULL, or the caller's keys-contiguous copy of v (as in fdl_dense_attention),
 *              updated too (stride checks as there)
 * Pure data movement; rows repeated within a sequence race (which write lands is not
 * defined).  Errors: as fdl_dense_attention for dtype, sizes and alignment; rows NULL
 * with n_max > 0 is FDL_ERR_NULL.
 */
fdl_status fdl_kv_refresh(fdl_dtype dtype, int B, int Hkv, int L, int d, const int32_t* rows,
                          const int32_t* n_rows, int n_max, const void* k_new, fdl_strides kns,
                          const void* v_new, fdl_strides vns, void* k, fdl_strides ks, void* v,
                          fdl_strides vs, void* vt, fdl_strides vts, hipStream_t stream);

/*
 * fdl_block_means_refresh - the block means after a KV refresh.
 * Summary page, "Method steps" (4): a block's mean depends on its own keys only, so
 * after fdl_kv_refresh only the blocks holding a refreshed prompt row (< P) change.
 * This recomputes exactly those entries of kbar [B, Hkv, nb, d] (fp32) from the
 * refreshed k, and leaves the others as they are.  Within the exponent range stated at
 * fdl_block_means both passes sum exactly, so the entries equal what fdl_block_means
 * writes, bit for bit.  rows, n_rows, n_max as in fdl_kv_refresh; an ascending row list
 * recomputes each touched block once (any order gives the same result).
 * Errors: dtype, sizes, alignment as fdl_block_means; kbar NULL, or rows NULL with
 * n_max > 0, is FDL_ERR_NULL.
 */
fdl_status fdl_block_means_refresh(fdl_dtype dtype, int B, int Hkv, int L, int P, int d,
                                   const void* k, fdl_strides ks, int bs, const int32_t* rows,
                                   const int32_t* n_rows, int n_max, float* kbar,
                                   hipStream_t stream);

/*
 * fdl_kv_refresh_means - fdl_kv_refresh and fdl_block_means_refresh of the same rows in
 * one launch, with the same results (Summary page, "Prerequisites" (approximate KV cache)
 * and "Method steps" (4)).  The touched blocks' means take their refreshed rows from
 * k_new and the other rows from k, so they need not wait for the scatter.
 *   arguments as in fdl_kv_refresh, plus P, bs and kbar as in fdl_block_means_refresh;
 *   rows distinct within a sequence (as the means read one new row per position).
 * bs above 2048 is FDL_ERR_UNSUPPORTED; other errors as the two calls it replaces.
 */
fdl_status fdl_kv_refresh_means(fdl_dtype dtype, int B, int Hkv, int L, int P, int d, int bs,
                                const int32_t* rows, const int32_t* n_rows, int n_max, const void* k_new,
                                fdl_strides kns, const void* v_new, fdl_strides vns, void* k, fdl_strides ks,
                                void* v, fdl_strides vs, void* vt, fdl_strides vts, float* kbar,
                                hipStream_t stream);

/*
 * fdl_confidence_unmask - the confidence of the masked positions and the unmasking of
 * step t (the step that produces the c_t fdl_pcgi_select reads at step t+1).
 * Summary page, "Prerequisites" (dLLMs: every [MASK] position gets a distribution over
 * the vocabulary; positions are unmasked by confidence) and "Core method" (n(t) tokens
 * are decoded at step t).  For each listed row r of sequence b, with logits z over the V
 * tokens: c_r = max_v softmax(z)_v = 1 / sum_v exp(z_v - max z) (fp32), and its token is
 * the argmax (the lowest id among equal maxima).  Among the rows whose position is still
 * masked, the n_t of highest c (the lower position first among equal c) are unmasked.
 *   logits     [B, m_max, V] (dtype FDL_F32 or FDL_BF16): row r of sequence b at
 *              logits + b*ls.b + r*ls.r (elements; ls.h unused), the V logits contiguous,
 *              rows 16-byte aligned, ls.r >= V
 *   pos        [B, m_max] int32: the position of each row, ascending within a sequence;
 *              rows r >= n_rows[b] (n_rows NULL: none) and positions outside [0, L) are
 *              ignored
 *   n_t        tokens to unmask per sequence (fewer candidates: all of them)
 *   mask       [B, L] uint8, in/out: the unmasked positions are cleared
 *   conf       [B, L] fp32, out at the listed positions: c for rows that stay masked, 0 for
 *              the rows unmasked now and for rows whose position was not masked; other
 *              positions untouched
 *   tokens     [B, L] int32 out at the unmasked positions (the argmax), or NULL
 *   unmasked   [B, n_t] int32 out, the unmasked positions ascending, -1 padded, or NULL
 * m_max above 4096 is FDL_ERR_UNSUPPORTED.  Workspace: fdl_confidence_unmask_workspace_bytes.
 */
size_t fdl_confidence_unmask_workspace_bytes(int B, int V, int m_max);
fdl_status fdl_confidence_unmask(fdl_dtype dtype, int B, int L, int V, const void* logits, fdl_strides ls,
                                 const int32_t* pos, const int32_t* n_rows, int m_max, int n_t,
                                 uint8_t* mask, float* conf, int32_t* tokens, int32_t* unmasked,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * fdl_dcu_select - the dynamic cache update (DCU) of Dynamic-dLLM: which tokens each layer
 * refreshes.  Dynamic-dLLM article, section "DCU：动态缓存更新": the change of a token's
 * normalised layer input between adjacent steps is its cosine distance, a layer's activity
 * is the sum of its tokens' changes, the total update budget goes to the layers in proportion
 * to their activity, and a mandatory window around each key token is always refreshed.
 * For sequence b and layer l, with x = x_now[b, l, i] and y = x_prev[b, l, i] (H values):
 *   dist[b, l, i]   d = 1 - x.y / (|x| |y|) (0 where a norm is 0), computed in fp32 as
 *                   (|x - y|^2 - (|x| - |y|)^2) / (2 |x| |y|), clamped at +0
 *   activity[b, l]  the fp64 sum of dist[b, l, :] (in a fixed order: the same on every run)
 *   budgets[b, l]   floor(total a_l / sum_m a_m), plus one for the total - sum of floors
 *                   layers of largest fractional part (the lower layer first among equal
 *                   parts); total / NL shares when every activity is 0
 *   upd_idx[b, l, :n_upd[b, l]]  ascending: every position within a mandatory window
 *                   [c - floor(w_m/2), c - floor(w_m/2) + w_m) of a key token c (clipped to
 *                   [0, L)), and the budgets[b, l] other positions of largest d (the lower
 *                   position first among equal d; all of them when there are fewer)
 *   x_now, x_prev   [B, NL, L, H] (dtype FDL_F32 or FDL_BF16): token i of layer l of sequence
 *                   b at x + b*s.b + l*s.h + i*s.r (elements), H values contiguous, every
 *                   token's row 16-byte aligned; inputs finite (NaN distances come out 0)
 *   key_tokens      [B, n_keys] int32, entries outside [0, L) ignored (may be NULL when
 *                   n_keys is 0); w_m >= 1 when n_keys > 0
 *   total           update budget of each sequence, shared by its NL layers (>= 0)
 *   dist [B, NL, L] fp32, activity [B, NL] fp64, budgets [B, NL] int32, upd_idx [B, NL, L]
 *   int32 (entries past n_upd untouched), n_upd [B, NL] int32: all outputs, all required.
 * A caller that walks the layers one at a time passes NL = 1 and the layer's own budget as
 * total.  L above 262144 or NL above 1024 is FDL_ERR_UNSUPPORTED.
 * Workspace: fdl_dcu_select_workspace_bytes.
 */
size_t fdl_dcu_select_workspace_bytes(int B, int NL, int L);
fdl_status fdl_dcu_select(fdl_dtype dtype, int B, int NL, int L, int H, const void* x_now, fdl_strides xns,
                          const void* x_prev, fdl_strides xps, const int32_t* key_tokens, int n_keys, int w_m,
                          int total, float* dist, double* activity, int32_t* budgets, int32_t* upd_idx,
                          int32_t* n_upd, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Measurement helpers (not steps of the method): what plain kernels reach on this GPU,
 * so that a kernel's share of the published peaks (8 TB/s HBM, 2.5 PFLOP/s dense bf16
 * MFMA on MI355X) can be read beside its share of what the part sustains.
 *
 * fdl_calibrate_read streams `bytes` (a positive multiple of 16) from the device buffer
 *   `src` once with non-temporal 16-byte loads, `workgroups` (>= 1) workgroups of 256
 *   threads each taking 64 KB a round.  sink [workgroups] uint32 receives the XOR of the
 *   32-bit words each workgroup read; the XOR of all entries is the XOR of the buffer.
 *   src must be 16-byte aligned (FDL_ERR_ALIGN).
 * fdl_calibrate_mfma runs `workgroups` (>= 1) workgroups of 4 waves; every wave issues
 *   iters (>= 1) rounds of 8 independent v_mfma_f32_32x32x16_bf16 on operands held in
 *   registers (every element a_val resp. b_val, rounded to bf16): 262144 flop per wave
 *   and round.  sink [workgroups * 4 * 2] fp32: per wave an accumulator element, which is
 *   16 * a * b * iters (a, b the bf16 operands; exact while that stays below 2^24), and the
 *   largest deviation of any of its elements from it.
 */
fdl_status fdl_calibrate_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream);
fdl_status fdl_calibrate_mfma(int workgroups, int iters, float a_val, float b_val, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FDL_H */
