/*
 * psgd.h — C ABI of the MI355X PowerSGD gradient-compression library (libpsgd.so).
 *
 * The operation. Data-parallel training of the DALL·E 12B transformer averages gradients across
 * machines by all-reducing low-rank factors instead of the full gradient matrices. Each GPU
 * compresses its own parameter shard at rank 112 (total rank 896). An error buffer carries what
 * the factors miss. Finite-value checks guard the step, and the decompressed gradient is formed
 * with 32-bit products. Gains, biases, embeddings and unembeddings are reduced uncompressed in
 * 32-bit. Sources: "Zero-Shot Text-to-Image Generation — 中文验证版" (ai-papers.xuzou.cn reading
 * card), sections 方法适配 and 证据; the Korean summary of the same paper (only-wanna.tistory.com),
 * section "Distributed Optimization".
 *
 * Per gradient matrix i (m x n, row-major) with per-resblock scale s_b, error buffer E (m x n,
 * fp32) and warm start Q (n x r, fp32), one step computes
 *     M  = s_b * G + E
 *     P  = orthonormalise(M Q)          thin-QR factor with positive R diagonal
 *     Q' = M^T P                        next warm start
 *     D  = P Q'^T                       decompressed gradient
 *     E  = M - D
 * On one GPU the two factor all-reduces of the multi-GPU method (of M Q and of Q') are the
 * identity, so this library computes the whole step locally.
 *
 * Call order per step, all asynchronous on the caller's stream:
 *     psgd_compress            -> P (orthonormal), q_next, per-matrix non-finite flags
 *     psgd_check_finite        -> skip word (device; optional host copy, the only host sync)
 *     psgd_decompress_update   -> not skipped: E = M - D, optional D out, q <- q_next
 *                                 skipped:     E = 0 for every matrix, q kept, D not written
 *
 * Conventions
 *  - All data pointers are device memory owned by the caller (torch tensors, hipMalloc, ...).
 *    The library owns only its context, its plans and the plan workspace.
 *  - Every call is asynchronous on `stream`. Only psgd_check_finite with a non-NULL skip_host
 *    synchronises the stream.
 *  - Errors are status codes; nothing is thrown across the ABI. psgd_last_error gives the
 *    message of the last failure on a context. There is no CPU fallback: a failure is reported,
 *    never hidden.
 *  - Non-finite data is not an error: it is reported through the flags and the skip word.
 *  - A context and its plans are not thread-safe. Calls that overlap on one plan race.
 */
#ifndef PSGD_H
#define PSGD_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PSGD_ABI_VERSION 1

typedef enum psgd_status {
  PSGD_OK = 0,
  PSGD_EINVAL = 1,        /* bad argument: null pointer, shape, leading dimension, alignment */
  PSGD_EDTYPE = 2,        /* unknown gradient dtype */
  PSGD_ENOMEM = 3,        /* workspace allocation failed */
  PSGD_EHIP = 4,          /* a HIP runtime call or kernel launch failed */
  PSGD_EUNSUPPORTED = 5   /* valid request the library does not implement (rank above 1024) */
} psgd_status;

typedef enum psgd_dtype {
  PSGD_F16 = 1,           /* IEEE binary16 gradients */
  PSGD_BF16 = 2,          /* bfloat16 gradients */
  PSGD_F32 = 3            /* float32 gradients */
} psgd_dtype;

/*
 * One gradient matrix and its state. Row-major, element (i, j) of G at grad[i * ld_grad + j].
 *  grad    m x n gradient, dtype of the plan (read only). ld_grad >= n, ld_grad % 8 == 0.
 *          NULL selects the in-place form: the caller has already accumulated s_b * G into
 *          the error buffer, so err holds M; s_b is not applied to the matrix and no gradient
 *          is read (4 bytes per element per pass instead of 6 for an fp16 gradient). ld_grad
 *          is then ignored, and the flag reports a non-finite element of M.
 *  err     m x n fp32 error buffer E (read and written by psgd_decompress_update; read by
 *          psgd_compress). ld_err >= n, ld_err % 4 == 0.
 *  q       n x r fp32 warm start (row-major, leading dimension r). Read by psgd_compress,
 *          overwritten with q_next by a non-skipped psgd_decompress_update.
 *  q_next  n x r fp32, written by psgd_compress.
 *  p       m x r fp32, written by psgd_compress with the orthonormal factor.
 *  out     m x n fp32 decompressed gradient D, or NULL to skip writing it. ld_out >= n,
 *          ld_out % 4 == 0.
 *  m, n    shape; n % 8 == 0; 1 <= r <= min(m, n).
 *  block   index into the per-resblock scale array (0 <= block < n_blocks).
 * Every pointer must be 16-byte aligned. Buffers of different matrices must not overlap. The
 * byte span of each of G, E and out ((m - 1) * ld + n elements), and of q and p (n * r and
 * m * r elements), must be below 2 GiB.
 */
typedef struct psgd_matrix {
  const void* grad;   int64_t ld_grad;
  float* err;         int64_t ld_err;
  float* q;
  float* q_next;
  float* p;
  float* out;         int64_t ld_out;
  int64_t m, n;
  int32_t block;
  int32_t reserved;   /* must be 0 */
} psgd_matrix;

/* An uncompressed fp32 tensor (gain, bias, embedding, unembedding): only finite-checked here;
 * its 32-bit reduction is the identity on one GPU. */
typedef struct psgd_tensor {
  const float* data;
  int64_t numel;
} psgd_tensor;

typedef struct psgd_ctx psgd_ctx;
typedef struct psgd_plan psgd_plan;

/* Library ABI version (PSGD_ABI_VERSION). */
int psgd_version(void);

/* Create a context on HIP device `device` for compression rank `rank` (1..1024). Ranks above
 * 128 form M once per step as bf16 halves in the plan workspace (4 bytes per element of each
 * matrix, row-major; M^T P reads them transposed) for the two factor products, which then run
 * as GEMMs, and are orthonormalised by 128-column blocks.
 * Writes *ctx; on failure *ctx is NULL (rank above 1024: PSGD_EUNSUPPORTED). */
psgd_status psgd_create(psgd_ctx** ctx, int device, int rank);

/* Destroy a context. Plans created on it must be destroyed first. NULL is accepted. */
psgd_status psgd_destroy(psgd_ctx* ctx);

/*
 * Describe a group of gradient matrices that are compressed together in grouped launches
 * (the grouped all-reduce of "Zero-Shot Text-to-Image Generation — 中文验证版", section 证据).
 * Validates every matrix, allocates and zeroes the plan workspace (about 16 bytes per element
 * of the m x r factors, plus 4 per gradient element and 4 per factor element when the rank is
 * above 128), and uploads the descriptor tables once (synchronously, on the null stream). The
 * pointers in `mats` are captured: the same buffers are used by every later call on the plan.
 * n_blocks is the length of the scale array later calls pass.
 */
psgd_status psgd_plan_create(psgd_ctx* ctx, const psgd_matrix* mats, int n_mats,
                             psgd_dtype grad_dtype, int n_blocks, psgd_plan** plan);

/* Free a plan and its workspace (synchronises the device). NULL is accepted. */
psgd_status psgd_plan_destroy(psgd_plan* plan);

/*
 * Compression: for every matrix, M = s_b G + E, P = orthonormalise(M q), q_next = M^T P.
 * This is the low-rank factorisation of the gradient with an error buffer and a warm-started
 * factor ("Zero-Shot Text-to-Image Generation — 中文验证版", section 方法适配; Korean summary
 * of the paper, section "Distributed Optimization"), at the rank of the plan.
 * Writes p, q_next and flags[i] = 1 when any element of G_i or E_i is +-inf or NaN (else 0).
 * Reads E and q without modifying them.
 *  scale  device fp32[n_blocks], the per-resblock multipliers s_b.
 *  flags  device uint8[n_mats].
 */
psgd_status psgd_compress(psgd_ctx* ctx, psgd_plan* plan, const float* scale, uint8_t* flags,
                          hipStream_t stream);

/*
 * The same compression split at the two points where a data-parallel group exchanges factors
 * (the all-reduce of the low-rank factors instead of the gradients: "Zero-Shot Text-to-Image
 * Generation — 中文验证版", sections 方法适配 and 证据). psgd_compress is exactly
 * psgd_compress_p, psgd_orthogonalize and psgd_compress_q in a row. On several GPUs a step is
 *     psgd_compress_p      -> raw factors M q of every matrix in the plan's factor buffer
 *     all-reduce (mean) of the factor buffer across the group
 *     psgd_orthogonalize   -> P (identical on every rank)
 *     psgd_compress_q      -> q_next = M^T P of the local M
 *     all-reduce (mean) of every q_next, then psgd_refresh_q
 *     psgd_check_finite, all-reduce (max) of the skip word
 *     psgd_decompress_update -> D = P q_next^T (identical on every rank), E = M_local - D
 * The library issues no collective; on one GPU the exchanges are the identity.
 *
 * psgd_compress_p: clears flags, computes M q (and the flags).
 * psgd_orthogonalize: orthonormalises the factor buffer's contents into p.
 * psgd_compress_q: q_next = M^T p, and the row scales the decompression applies to it.
 * psgd_refresh_q: recomputes those row scales from q_next (after q_next was reduced).
 */
psgd_status psgd_compress_p(psgd_ctx* ctx, psgd_plan* plan, const float* scale, uint8_t* flags,
                            hipStream_t stream);
psgd_status psgd_orthogonalize(psgd_ctx* ctx, psgd_plan* plan, hipStream_t stream);
psgd_status psgd_compress_q(psgd_ctx* ctx, psgd_plan* plan, const float* scale, hipStream_t stream);
psgd_status psgd_refresh_q(psgd_ctx* ctx, psgd_plan* plan, hipStream_t stream);

/*
 * The plan's factor buffer: one contiguous fp32 region holding M q of every matrix, matrix i
 * row-major m_i x rpad at offset sum_{j<i} m_j * rpad (columns at or beyond r are zero).
 * *count receives the number of floats, *rpad the padded rank. The buffer is owned by the plan
 * and valid until psgd_plan_destroy.
 */
psgd_status psgd_factor_buffer(psgd_plan* plan, void** ptr, int64_t* count, int32_t* rpad);

/*
 * Skip decision ("Zero-Shot Text-to-Image Generation — 中文验证版", section 方法适配: the
 * skip-update rule for non-finite values). *skip_dev = 1 when any flags[i] is set, any element
 * of the pass-through tensors is non-finite, or any of scale[0..n_blocks) is non-finite;
 * otherwise 0.
 *  pass/n_pass  host array of fp32 device tensors (n_pass may be 0, pass may then be NULL).
 *  skip_dev     device int32, written.
 *  skip_host    NULL, or a host int32 that receives the skip word; the call then synchronises
 *               the stream.
 */
psgd_status psgd_check_finite(psgd_ctx* ctx, psgd_plan* plan, const uint8_t* flags,
                              const psgd_tensor* pass, int n_pass, const float* scale,
                              int32_t* skip_dev, int32_t* skip_host, hipStream_t stream);

/*
 * Decompression and error feedback, gated on the device-side skip word (no host sync).
 *  not skipped: D = P q_next^T formed with fp32-accurate products; E = M - D; out = D when the
 *               matrix has an out buffer; q <- q_next.
 *  skipped:     E = 0 for every matrix of the plan; q unchanged; out untouched
 *               (the error buffer is zeroed on non-finite values: Korean summary, section
 *               "Distributed Optimization").
 * Must follow psgd_compress on the same plan with the same scale array.
 */
psgd_status psgd_decompress_update(psgd_ctx* ctx, psgd_plan* plan, const float* scale,
                                   const int32_t* skip_dev, hipStream_t stream);

/*
 * Zero the error buffer of every matrix of the plan: the restart case of the rule that the
 * error buffer is zeroed as rarely as possible, on non-finite values from mixed-precision
 * backprop and when training restarts from a checkpoint (Korean summary of the paper, section
 * "Distributed Optimization"). Error buffers are not checkpointed; a caller resuming a run
 * calls this once before the first step and restores q (the warm starts) itself.
 * It is the skipped form of psgd_decompress_update with no skip word: E = 0 over m x n of
 * every matrix (in-place matrices included), nothing else is written, q and out are untouched.
 * Asynchronous on stream; PSGD_EINVAL for a plan of another context. Traced in slot 8.
 */
psgd_status psgd_reset_errors(psgd_ctx* ctx, psgd_plan* plan, hipStream_t stream);

/*
 * Per-resblock gradient scaling at the boundaries of backprop, the step that produces a
 * block's gradients and its multiplier s_b = 1 / S_b for the calls above. Every resblock has
 * its own scale factor S_b ("Zero-Shot Text-to-Image Generation — 中文验证版", section
 * 方法适配); the gradient is multiplied by S_b when backprop enters the block and divided by
 * it when backprop leaves, where Inf/NaN values become 0 so that they do not reach other
 * blocks (Korean summary, section "Mixed-Precision Training"). The gradient between blocks
 * (the residual stream) is fp32 in true units; inside the block it is fp16 or bf16.
 *
 * psgd_block_grad_enter: out[i] = to16(fp32(S_b * dx[i])), round to nearest even (fp16 keeps
 *   subnormals, overflow gives inf).
 *     dx     n fp32 (device, read), 16-byte aligned
 *     scale  one fp32 on the device: S_b, finite and > 0 (not checked: it stays on the device)
 *     out    n 16-bit values of out_dtype (device, written), 16-byte aligned
 * psgd_block_grad_exit: dx[i] += fp32(g[i] / S_b) for each finite g[i] (IEEE division and
 *   addition, each rounded once); a g[i] that is inf or NaN adds 0. *flag is set to 1 when any
 *   g[i] was inf or NaN and left as it is otherwise, so one flag can gather several calls (the
 *   caller clears it). flag may be NULL.
 *     dx     n fp32 (device, read and written), 16-byte aligned
 *     g      n 16-bit values of g_dtype (device, read): the block's output gradient, scaled
 * Both: n >= 0 (0 is a no-op), dtype PSGD_F16 or PSGD_BF16 (else PSGD_EDTYPE), asynchronous on
 * stream, PSGD_EINVAL for NULL or misaligned pointers. The ctx gives the device and the
 * error message; no plan is involved.
 */
psgd_status psgd_block_grad_enter(psgd_ctx* ctx, const float* dx, int64_t n, const float* scale,
                                  void* out, psgd_dtype out_dtype, hipStream_t stream);
psgd_status psgd_block_grad_exit(psgd_ctx* ctx, float* dx, const void* g, int64_t n,
                                 const float* scale, psgd_dtype g_dtype, uint8_t* flag,
                                 hipStream_t stream);
/*
 * The boundary between block b and block b - 1 in one pass: psgd_block_grad_exit with S_b
 * (scale_exit) on dx and g, then psgd_block_grad_enter with S_{b-1} (scale_enter) from the
 * updated dx into out (same 16-bit dtype as g). Results equal the two calls in sequence; dx,
 * g and out are read or written once (12 bytes per element instead of 16). dx, g and out
 * 16-byte aligned; out must not overlap g. Errors as for the two calls.
 */
psgd_status psgd_block_grad_exit_enter(psgd_ctx* ctx, float* dx, const void* g, int64_t n,
                                       const float* scale_exit, const float* scale_enter, void* out,
                                       psgd_dtype dtype, uint8_t* flag, hipStream_t stream);

/*
 * The optimizer that consumes the decompressed gradient: Adam with most moments in a custom
 * 16-bit format, gradient clipping, and the skip rule for non-finite values ("Zero-Shot
 * Text-to-Image Generation — 中文验证版", section 方法适配); gains, biases, embeddings and
 * unembeddings keep 32-bit parameters, gradients and moments (Korean summary of the paper,
 * section "Mixed-Precision Training"). The update is AdamW ("AIGC 基本功|混合精度与数值稳定性-
 * AMP", section 6.1), after a global-norm clip of every gradient of the step (section 6.2):
 *     t <- t + 1;  N = ||all gradients||;  c = min(1, max_norm / N)  (1 when max_norm <= 0)
 *     g' = c g;  m1 <- b1 m1 + (1 - b1) g';  m2 <- b2 m2 + (1 - b2) g'^2
 *     theta <- theta - lr ((m1 / (1 - b1^t)) / (sqrt(m2 / (1 - b2^t)) + eps) + wd theta)
 * using the new moments before they are stored. A skipped step changes nothing (t included).
 * Storage of a compressed matrix's state: theta in the attached parameter type (fp16, bf16 or
 * fp32); m1 bfloat16; m2 "ue8m8", a 16-bit code holding bits 30..15 of a non-negative float32
 * (8 exponent bits, 8 fraction bits: the second moment never needs a sign); every stored
 * value rounds to nearest even from its float32 value.
 *
 * Call order per step (all on one stream, no host sync):
 *     psgd_compress -> psgd_check_finite -> psgd_adam_prepare
 *     -> psgd_decompress_adam (instead of psgd_decompress_update) -> psgd_adam_update
 */
typedef struct psgd_adam_hparams {
  float lr, beta1, beta2, eps, weight_decay;   /* 0 <= beta < 1; lr, eps, weight_decay >= 0 */
} psgd_adam_hparams;

/* Optimizer state of one plan matrix (m x n, row-major): param with leading dimension
 * ld_param (>= n, multiple of 8), m1 and m2 with leading dimension n. Caller-owned device
 * memory, 16-byte aligned, each span below 2 GiB; updated in place. */
typedef struct psgd_adam_matrix {
  void* param;       int64_t ld_param;
  uint16_t* m1;      uint16_t* m2;
} psgd_adam_matrix;

/* A 32-bit pass-through tensor: fp32 param, moments and gradient of numel elements
 * (device memory; the gradient alone suffices for psgd_adam_prepare). */
typedef struct psgd_adam_tensor {
  float* param;  float* m1;  float* m2;  const float* grad;
  int64_t numel;
} psgd_adam_tensor;

/* Attach optimizer state to every matrix of the plan (opt has n_mats entries, in plan order);
 * param_dtype PSGD_F16, PSGD_BF16 or PSGD_F32. Allocates the plan's norm-reduction buffer and
 * re-uploads its descriptors (synchronises the device). A second call replaces the first. */
psgd_status psgd_adam_attach(psgd_ctx* ctx, psgd_plan* plan, const psgd_adam_matrix* opt,
                             psgd_dtype param_dtype);

/* The scalars of a step, after psgd_check_finite and before the updates. Not skipped:
 * *step_dev += 1, norm_dev[0] = N, norm_dev[1] = c. Skipped: nothing is written.
 * N covers the decompressed gradient of every plan matrix and the pass-through gradients
 * (pass[i].grad, numel; at most 8192 * 65536 elements in all). For a plan matrix ||D||_F is
 * taken as ||q_next||_F, equal to it because P has orthonormal columns, so N is known before
 * D is formed. Sums run in fp64 in a fixed order (bit-reproducible).
 *  step_dev  device int32: the optimizer's step count t (caller-owned, checkpointed with the
 *            moments; 0 before the first step)
 *  norm_dev  device fp32[2], written */
psgd_status psgd_adam_prepare(psgd_ctx* ctx, psgd_plan* plan, const psgd_adam_tensor* pass, int n_pass,
                              float max_norm, const int32_t* skip_dev, int32_t* step_dev,
                              float* norm_dev, hipStream_t stream);

/* psgd_decompress_update with the Adam update fused in: not skipped, E = M - D, q <- q_next,
 * and every matrix's param, m1 and m2 take one step on c D (D itself is not written, the
 * matrices' out buffers are ignored); skipped, E = 0 and nothing else changes. */
psgd_status psgd_decompress_adam(psgd_ctx* ctx, psgd_plan* plan, const float* scale, const int32_t* skip_dev,
                                 const int32_t* step_dev, const float* norm_dev,
                                 const psgd_adam_hparams* hp, hipStream_t stream);

/* The same fp32 step on pass-through tensors (param, m1, m2 fp32, gradient pass[i].grad),
 * with the scalars psgd_adam_prepare wrote; a skipped step changes nothing. No plan needed. */
psgd_status psgd_adam_update(psgd_ctx* ctx, const psgd_adam_tensor* pass, int n_pass, const int32_t* skip_dev,
                             const int32_t* step_dev, const float* norm_dev, const psgd_adam_hparams* hp,
                             hipStream_t stream);

/*
 * One whole step (psgd_compress, psgd_check_finite without the host copy, then
 * psgd_decompress_update) on a group given by its descriptors, with no plan and no device
 * allocation: for callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). The results equal those of a plan made from the
 * same descriptors and the three calls in a row.
 *  The plan's workspace, descriptor table and work lists are placed in the library's static
 *  scratch array of 32 MiB per device (held from the first psgd_create on that device until
 *  the process ends). A group that needs more (about 12 bytes per element of the m x r
 *  factors plus 8 r^2 bytes per 256 rows at r <= 128: one 3968-wide resblock shard at rank
 *  112 takes about 19 MiB; ranks above 128 add 4 bytes per gradient element and 4 per factor
 *  element) is rejected with PSGD_EINVAL before anything is launched.
 *  The call launches kernels only (a fill, uploads of the tables as kernel arguments, then the
 *  step's kernels), all on `stream`, and returns without synchronising. Every call on a device
 *  shares that device's array and overwrites the previous call's contents: calls on one
 *  stream are ordered, but calls that overlap on one device (other streams, other threads,
 *  other contexts) race and corrupt each other's results.
 *  Arguments as for psgd_plan_create (mats, n_mats, grad_dtype, n_blocks), psgd_compress
 *  (scale, flags) and psgd_check_finite (pass, n_pass, skip_dev). The caller owns every
 *  buffer; the descriptors are read during the call only.
 */
psgd_status psgd_step_noalloc(psgd_ctx* ctx, const psgd_matrix* mats, int n_mats,
                              psgd_dtype grad_dtype, const float* scale, int n_blocks,
                              const psgd_tensor* pass, int n_pass, uint8_t* flags,
                              int32_t* skip_dev, hipStream_t stream);

/*
 * Step counters of a plan, for monitoring (the skip count is the figure a mixed-precision run
 * is watched by: "AIGC 基本功|混合精度与数值稳定性-AMP", section 6.5). *counters receives the
 * device address of two int64: [0] steps decompressed (psgd_decompress_update or
 * psgd_decompress_adam calls that ran), [1] of those, steps skipped on non-finite values. The
 * decompression kernel updates them on the device in stream order (no host sync); they start
 * at 0 when the plan is made and psgd_reset_errors does not count. Owned by the plan.
 */
psgd_status psgd_plan_counters(psgd_plan* plan, const int64_t** counters);

/*
 * Tracing hook. Install an array of n HIP events created by the caller with timing enabled.
 * While installed, the launch of each kernel in slot k is bracketed by hipEventRecord of
 * events[2k] (before) and events[2k+1] (after) on the call's stream; elapsed times between the
 * pair give that kernel's duration. Slots: 0 flag clear, 1 M Q with error feedback, 2 Gram
 * partials, 3 Gram-Schmidt, 4 orthonormal P, 5 M^T P, 6 skip clear, 7 finite check,
 * 8 decompression + error update + q commit, 9 Gram sum (rank > 128 only), 10 decompression
 * row scales (rank > 128 only, and psgd_refresh_q), 11 second orthonormalisation pass (all
 * four of its launches; they return at once for matrices whose first pass was well
 * conditioned), 12 global gradient norm of psgd_adam_prepare, 13 decompression with the Adam
 * update, 14 pass-through Adam. Slots a call does not launch keep their events unrecorded.
 * n must be at least 30.
 * events == NULL (n ignored) removes the hook. The events stay owned by the caller.
 */
psgd_status psgd_profile_events(psgd_ctx* ctx, hipEvent_t* events, int n);

/* Message of the last failed call on ctx ("" if none). Valid until the next call on ctx. */
const char* psgd_last_error(const psgd_ctx* ctx);

/*
 * Diagnostics for tests: device address and byte size of an internal per-matrix buffer of a
 * plan. which: 0 = raw factor M q (m x rpad fp32, before orthonormalisation),
 * 1 = orthonormalising coefficient matrix T of the last pass (rpad x rpad fp64, upper
 * triangular; P = (M q) T after one pass, P = ((M q) T1) T after two).
 * *rpad receives the padded rank: a multiple of 16 that is at least r (ranks above 128 are padded
 * to whole rank chunks).
 */
psgd_status psgd_debug_buffer(psgd_plan* plan, int which, int mat, void** ptr, int64_t* bytes,
                              int32_t* rpad);

#ifdef __cplusplus
}
#endif
#endif /* PSGD_H */
