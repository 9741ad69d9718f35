/*
 * vws.h -- C ABI of libvws, the MI355X (gfx950) vocab-wide softmax reductions.
 *
 * The operations are the per-row reductions of DeepSpeed PR #8838 "Add Triton
 * kernels for vocab-parallel logprobs, entropy and KL" (first and second commit
 * messages, PR description) and the fused linear-logp of RL-Kernel PR #208
 * "[Feat][Kernel] Add TP Fused linear logp Triton" (PR body, "Implementation").
 * Each row of logits z (length V) is reduced in one read to the online
 * statistics m = max z, S = sum e^(z-m), and a max-centred weighted sum W, from
 * which the per-token result is formed (second commit message of PR #8838):
 *
 *   log-probability   logp = (z_t - m) - log S
 *   entropy           H    = log S - W_H / S,   W_H = sum e^(z-m) (z-m)
 *   KL(A||B)          KL   = W_K / S_A - log S_A + log S_B,
 *                     W_K  = sum e^(a-m_a) ((a-m_a) - (b-m_b)),
 *                     and +inf when B is -inf on a column where A is not
 *                     (support flag decided on the logits).
 *
 * Forward KL(B||A) is the same call with the arguments swapped.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All data pointers are DEVICE pointers on the current HIP device; the
 *   caller owns every buffer. Work is enqueued on `stream` (a hipStream_t; NULL
 *   is the null stream). No call synchronises, allocates device memory or
 *   keeps state between calls; calls are reentrant. (The one exception is
 *   vws_kl_fwd_noalloc, which uses a static per-GPU buffer in place of a
 *   workspace argument; see there.)
 * - Return value: VWS_OK (0) or a negative vws_status. Argument and layout
 *   errors are detected on the host before anything is launched; VWS_EHIP
 *   reports a failed launch. Data-dependent conditions never produce a status
 *   (that would need a host synchronisation); they produce the values below.
 * - N = 0 is a no-op returning VWS_OK. V must be >= 1.
 * - Outputs (logp, H, kl) are fp32 [N]; `stats` is fp32 [N, 2] holding
 *   (m, log S) per row, or [N, 4] holding (m_a, log S_A, m_b, log S_B) for KL.
 *   The backward recomputes p = exp((z - m) - log S) from these, so it needs
 *   exactly the stats its forward wrote (max-centred: m and log S are kept as
 *   two numbers, never folded into one log-sum-exp).
 * - Gradients are written contiguous [N, V] in the input dtype; a bf16 gradient
 *   is its fp32 value rounded to nearest, ties to even (review comment on
 *   PR #8838). `g` is the fp32 upstream gradient, element r at g[r * g_stride]
 *   (g_stride = 0 broadcasts one value, as an expanded scalar does).
 * - Outputs must not alias inputs.
 *
 * Values for degenerate rows (readings of the pages; the pages list these
 * cases but not their values):
 * - a -inf entry has probability 0, adds nothing, and gets gradient 0
 *   (zero-weight rule: the "0 x inf" review thread of PR #8838 and its fix);
 * - a row with no entry above -inf, or with a NaN or +inf entry, gives NaN
 *   outputs and NaN gradients;
 * - logprobs: t == ignore_index gives 0 and a zero gradient row; any other t
 *   outside [0, V) gives NaN and a NaN gradient row;
 * - KL rows with the support flag set give +inf; their gradient w.r.t. A is
 *   NaN in every column and their gradient w.r.t. B is g (p_B - p_A).
 */
#ifndef VWS_H
#define VWS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(_WIN32)
#define VWS_API
#else
#define VWS_API __attribute__((visibility("default")))
#endif

typedef enum vws_status {
  VWS_OK = 0,
  VWS_EINVAL = -1,     /* null pointer, negative or inconsistent size, bad op code */
  VWS_EDTYPE = -2,     /* unknown dtype, or A and B of different dtypes */
  VWS_ELAYOUT = -3,    /* col_stride != 1, negative stride, misaligned pointer, address overflow */
  VWS_EWORKSPACE = -4, /* workspace smaller than vws_workspace_bytes() */
  VWS_EHIP = -5,       /* a HIP launch failed */
  VWS_ESCRATCH = -6    /* vws_kl_fwd_noalloc: the split needs more than VWS_NOALLOC_SCRATCH_BYTES */
} vws_status;

typedef enum vws_dtype { VWS_F32 = 0, VWS_BF16 = 1, VWS_F16 = 2 } vws_dtype;

enum { VWS_SPLIT_INVARIANT = -1 };

typedef enum vws_op { VWS_OP_LOGPROBS = 0, VWS_OP_ENTROPY = 1, VWS_OP_KL = 2, VWS_OP_JSD = 3 } vws_op;

/*
 * A logical [N, V] matrix of logits. Row addresses take an outer and an inner
 * stride, which lets a causal-shift view like logits[:, :-1, :] be read where it
 * lies, without a copy (second commit message of PR #8838). Row r = r_o * n_inner + r_i (0 <= r_i < n_inner)
 * starts at element  r_o * s_outer + r_i * s_inner  of `data`; columns are
 * contiguous (col_stride must be 1; other layouts are copied by the caller).
 * Strides are in elements and must be >= 0. `data` must be aligned to the
 * element size. N = n_outer * n_inner. Rows hold 1 <= V <= INT32_MAX - 4096
 * columns (column and group indexes are 32-bit); V = 0 is VWS_EINVAL: on one
 * GPU a row without columns has no entry above -inf, and an empty vocabulary
 * shard of a tensor-parallel split is the caller's neutral partial (m = -inf,
 * S = 0), not a call into this library.
 */
typedef struct vws_rows {
  const void* data;
  int32_t dtype; /* vws_dtype */
  int64_t n_outer, n_inner;
  int64_t s_outer, s_inner;
  int64_t V;
  int64_t col_stride;
} vws_rows;

/* int64 target ids with the same row decomposition: id of row r at
 * data[r_o * s_outer + r_i * s_inner]. */
typedef struct vws_ids {
  const int64_t* data;
  int64_t s_outer, s_inner;
} vws_ids;

/* K ids per row for the multi-id logprobs: slot k of row r = r_o * n_inner + r_i
 * at data[r_o * s_outer + r_i * s_inner + k * s_k]; 1 <= K <= 2048. */
typedef struct vws_ids_k {
  const int64_t* data;
  int64_t s_outer, s_inner, s_k;
  int64_t K;
} vws_ids_k;

/*
 * Bytes of workspace the forward of `op` needs for N rows of V columns with the
 * given split_hint. The forward splits each row's vocabulary over P workgroups
 * when N is small (the pages' cross-shard combine -- MAX of m, re-centring of
 * S and W on it, SUM -- done inside one GPU); the partial statistics go to
 * the workspace and a second kernel merges them. split_hint:
 *   0 = automatic (P = ceil(768 / N): about three workgroups per CU, each part at
 *       least 4096 columns; unsplit from 768 rows; a row's rounding may then depend on N),
 *   1 = never split, P > 1 = split into P parts (capped at ceil(V/8)),
 *   VWS_SPLIT_INVARIANT (-1) = fixed segments of 32768 columns, so P and every
 *       row's reduction order depend on V alone: a row's outputs are bitwise
 *       the same whatever the batch it is in (the batch-invariance remark on
 *       PR #8838). Any fixed split_hint >= 1 is batch invariant too; the
 *       backward passes are per element and never depend on the batch.
 * Returns 0 when no workspace is needed, (size_t)-1 for invalid arguments.
 */
VWS_API size_t vws_workspace_bytes(int op, int64_t N, int64_t V, int split_hint);

/* Number of vocabulary parts the forward uses for these sizes (1 = no split). */
VWS_API int vws_split_parts(int op, int64_t N, int64_t V, int split_hint);

/*
 * Per-token log-probability of the target (first commit message of PR #8838;
 * RL-Kernel PR #208 returns (logp, lse) from its forward).
 *   z       logits [N, V]
 *   t       target ids (same row decomposition as z)
 *   logp    out fp32 [N]
 *   stats   out fp32 [N, 2] = (m, log S)
 *   ws      workspace of ws_bytes >= vws_workspace_bytes(VWS_OP_LOGPROBS, ...)
 */
VWS_API int vws_logprobs_fwd(const vws_rows* z, const vws_ids* t, int64_t ignore_index, float* logp,
                             float* stats, void* ws, size_t ws_bytes, int split_hint, void* stream);

/*
 * dz_j = g (1[j = t] - p_j) (RL-Kernel PR #208, review nitpick on the chunked
 * backward: the negated probabilities, one added at the target, scaled by g).
 *   stats   the [N, 2] stats written by vws_logprobs_fwd on the same z
 *   dz      out [N, V] contiguous, dtype of z
 */
VWS_API int vws_logprobs_bwd(const vws_rows* z, const vws_ids* t, int64_t ignore_index, const float* stats,
                             const float* g, int64_t g_stride, void* dz, void* stream);

/*
 * Multi-id (top-k) log-probabilities: K target ids per row (the logprobs test
 * cases of PR #8838 include repeated ids, ignored ids and rows whose ids are all
 * ignored).
 *   ids     K ids per row (vws_ids_k); a slot equal to ignore_index gives 0,
 *           any other slot outside [0, V) gives NaN
 *   logp    out fp32 [N, K] contiguous: logp[r, k] = (z_id - m) - log S
 *   stats   out fp32 [N, 2] = (m, log S);  ws as for vws_logprobs_fwd
 *           (vws_workspace_bytes(VWS_OP_LOGPROBS, ...))
 */
VWS_API int vws_logprobs_topk_fwd(const vws_rows* z, const vws_ids_k* ids, int64_t ignore_index, float* logp,
                                  float* stats, void* ws, size_t ws_bytes, int split_hint, void* stream);

/*
 * Gradient of sum_k g[r, k] logp[r, k]:  dz_j = h_j - G p_j, where h_j sums
 * g[r, k] over the live slots whose id is j (duplicate ids add) and G sums g
 * over all live slots. A row whose slots are all ignored gets a zero gradient
 * row; a row with a live slot outside [0, V) a NaN row.
 *   g       fp32 upstream gradient, element (r, k) at g[r * g_s_row + k * g_s_k]
 *           (zero strides broadcast)
 *   stats   as written by vws_logprobs_topk_fwd;  dz out [N, V] contiguous, dtype of z
 */
VWS_API int vws_logprobs_topk_bwd(const vws_rows* z, const vws_ids_k* ids, int64_t ignore_index, const float* stats,
                                  const float* g, int64_t g_s_row, int64_t g_s_k, void* dz, void* stream);

/*
 * Entropy H = -sum p log p = log S - W_H / S in one read (second commit
 * message of PR #8838).
 *   H       out fp32 [N];   stats out fp32 [N, 2] = (m, log S)
 */
VWS_API int vws_entropy_fwd(const vws_rows* z, float* H, float* stats, void* ws, size_t ws_bytes, int split_hint,
                            void* stream);

/*
 * dz_j = -g p_j (log p_j + H), derived from the definition of H (the pages do
 * not print it); 0 where z_j = -inf.
 *   stats, H   as written by vws_entropy_fwd;   dz out [N, V] contiguous
 */
VWS_API int vws_entropy_bwd(const vws_rows* z, const float* stats, const float* H, const float* g, int64_t g_stride,
                            void* dz, void* stream);

/*
 * KL(A||B) = W_K / S_A - log S_A + log S_B in one read of both inputs, +inf
 * when B masks a column that A supports (second commit message and review
 * comment of PR #8838). A and B must have equal N, V and dtype; their strides
 * may differ.
 *   kl      out fp32 [N];   stats out fp32 [N, 4] = (m_a, log S_A, m_b, log S_B)
 */
VWS_API int vws_kl_fwd(const vws_rows* a, const vws_rows* b, float* kl, float* stats, void* ws, size_t ws_bytes,
                       int split_hint, void* stream);

/*
 * vws_kl_fwd without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. It
 * computes exactly what vws_kl_fwd computes with the same split_hint (same kernels, same
 * bits), taking the split path's partial states from a static device buffer of
 * VWS_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until the process
 * ends; it calls no allocating routine. A split needing more than that (N * P * 24 bytes for
 * P > 1 vocabulary parts) returns VWS_ESCRATCH before anything is launched. Every call on one
 * GPU shares that GPU's buffer, and the buffer keeps the last call's contents (each call writes
 * every partial state it reads, so nothing needs clearing): calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race and must not be made.
 */
#define VWS_NOALLOC_SCRATCH_BYTES (8u << 20)

VWS_API int vws_kl_fwd_noalloc(const vws_rows* a, const vws_rows* b, float* kl, float* stats, int split_hint,
                               void* stream);

/*
 * da_j = g p_A,j (log p_A,j - log p_B,j - KL)  (0 where a_j = -inf),
 * db_j = g (p_B,j - p_A,j); derived from the definition of KL (not printed on
 * the pages). da or db may be NULL to skip that gradient (e.g. a frozen
 * teacher).
 *   stats, kl  as written by vws_kl_fwd;   da, db out [N, V] contiguous
 */
VWS_API int vws_kl_bwd(const vws_rows* a, const vws_rows* b, const float* stats, const float* kl, const float* g,
                       int64_t g_stride, void* da, void* db, void* stream);

/*
 * Generalized Jensen-Shannon divergence of student S and teacher T (the JSD
 * pull request pasted into PR #8838: "Changes", "Scope and limitations"), with
 * the GKD-style mixture M = (1 - beta) p_S + beta p_T:
 *   JSD = beta KL(T||M) + (1 - beta) KL(S||M)      for 0 < beta < 1,
 * and, as explicit endpoint branches, beta = 0 gives forward KL(T||S) and
 * beta = 1 reverse KL(S||T) (the KL entry points with the arguments in that
 * order). The interior takes two reads of both inputs: the single-read KL
 * statistics pass for (m, log S) of S and T, then a divergence pass that forms
 * K_S = KL(S||M) and K_T = KL(T||M). Disjoint supports are finite inside; a row
 * where either input is undefined gives NaN.
 *   s, t    logits [N, V] (equal N, V, dtype; strides may differ)
 *   beta    in [0, 1]
 *   jsd     out fp32 [N]
 *   stats   out fp32 [N, 6]; opaque, pass it unchanged to vws_jsd_bwd with the
 *           same beta (interior: m_S, log S_S, m_T, log S_T, K_S, K_T per row;
 *           endpoints: the KL statistics, [N, 4] packed at its start)
 *   ws      workspace of vws_workspace_bytes(VWS_OP_JSD, N, V, split_hint) bytes
 */
VWS_API int vws_jsd_fwd(const vws_rows* s, const vws_rows* t, float beta, float* jsd, float* stats, void* ws,
                        size_t ws_bytes, int split_hint, void* stream);

/*
 * Gradients of g * JSD (interior, derived from the definition; the page does not
 * print them):
 *   ds_j = g (1 - beta) p_S,j ((log p_S,j - log M_j) - K_S)
 *   dt_j = g beta p_T,j ((log p_T,j - log M_j) - K_T)
 * 0 where the input is -inf; the endpoints are the KL gradients. ds or dt may be
 * NULL (a detached teacher, a frozen student).
 *   stats, jsd   as written by vws_jsd_fwd with the same beta
 *   ds, dt       out [N, V] contiguous, dtype of the inputs
 */
VWS_API int vws_jsd_bwd(const vws_rows* s, const vws_rows* t, float beta, const float* stats, const float* jsd,
                        const float* g, int64_t g_stride, void* ds, void* dt, void* stream);

/*
 * Fused linear-logp (RL-Kernel PR #208, PR body "Implementation"): the per-row
 * log-probability of the target under logits z = h W^T, computed on MFMA in
 * vocabulary tiles whose (m, S) feed the online log-sum-exp, so the [N, V]
 * logits are never written. The forward returns logp = z_t - lse and the
 * per-row (m, log S); the backward goes over the vocabulary in chunks (the
 * chunked backward of the pages' review nitpick): for each chunk it recomputes
 * the logits tile by tile, forms dz = g (onehot(t) - p) in fp32, keeps it in the
 * workspace as a bf16 pair (hi = rne(dz), lo = rne(dz - hi), about 2^-17
 * relative), and contracts both parts into dW of the chunk's vocabulary rows
 * = dz^T h and into dh += dz W_chunk (fp32 accumulation, dh summed in fp32 over
 * the chunks; bf16 round-to-nearest-even outputs).
 *
 *   h       bf16 [N, H], row stride ldh (elements, >= H, multiple of 8)
 *   W       bf16 [V, H], row stride ldw (>= H, multiple of 8)
 *   t       int64 [N] contiguous target ids; ignore_index gives logp 0 and zero
 *           gradient rows; any other id outside [0, V) gives NaN
 *   logp    out fp32 [N];  stats out fp32 [N, 2] = (m, log S) of each row's logits
 *   dh      out bf16 [N, H] contiguous, may be NULL
 *   dW      out bf16 [V, H] contiguous, may be NULL
 *   ws      workspace of vws_linear_workspace_bytes(pass, N, H, V, split_hint) bytes
 *           (pass 0: forward, 1: backward), 256-byte aligned. The backward's holds one
 *           chunk's dz pair, 2 x N x chunk x 2 bytes, plus the fp32 sum of dh, N x H x 4
 *           bytes, when V spans more than one chunk (0.40 GB at 8192 x 4096 x 151936).
 *   split_hint  forward: vocabulary chunking as for the logits ops: 0 automatic (the
 *           chunking that spreads the (token tile, vocabulary tile) products most evenly
 *           over the CUs for this N; the order in which a token's chunk partials merge
 *           then follows the batch size), k >= 1 k chunks, VWS_SPLIT_INVARIANT
 *           chunks of 1024 columns. The last two depend on V alone: a token's logp and
 *           stats are then the same bits in every batch (batch invariance); < -1 is
 *           VWS_EINVAL.
 *           backward: 0 or VWS_SPLIT_INVARIANT chunks of 8192 columns, k >= 1 k chunks.
 *           Every choice depends on V alone and reduces each dz and dh entry in an order
 *           fixed by V, H and the chunking, so dh is batch invariant when the stats it is
 *           given are (dW sums over the batch by definition).
 * H must be a multiple of 8. h, W, dh, dW must be 16-byte aligned. dtype must be VWS_BF16.
 * Sizes: N <= 2^31, H and V <= INT32_MAX, and with T(x) = ceil(x / 256) each of
 * T(N) T(V), T(N) T(H) and T(V) T(H) below 2^23 (one 512-thread workgroup per 256 x 256
 * tile, fewer than 2^32 work-items per launch); larger shapes give VWS_EINVAL.
 */
VWS_API size_t vws_linear_workspace_bytes(int pass, int64_t N, int64_t H, int64_t V, int split_hint);

VWS_API int vws_linear_logp_fwd(const void* h, int64_t ldh, const void* W, int64_t ldw, int dtype, int64_t N,
                                int64_t H, int64_t V, const int64_t* t, int64_t ignore_index, float* logp,
                                float* stats, void* ws, size_t ws_bytes, int split_hint, void* stream);

VWS_API int vws_linear_logp_bwd(const void* h, int64_t ldh, const void* W, int64_t ldw, int dtype, int64_t N,
                                int64_t H, int64_t V, const int64_t* t, int64_t ignore_index, const float* stats,
                                const float* g, int64_t g_stride, void* dh, void* dW, void* ws, size_t ws_bytes,
                                int split_hint, void* stream);

/* Static description of a status code. */
VWS_API const char* vws_strerror(int status);

/* ABI version (major * 100 + minor). */
VWS_API int vws_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VWS_H */
