/*
 * lce.h -- fused linear + cross-entropy over a large vocabulary, forward and
 * backward, for AMD Instinct MI355X (gfx950).  C ABI, no C++ or torch types.
 *
 * The operation (for every row n of H that is not ignored):
 *
 *     z[n, v]  = sum_k H[n, k] W[v, k]
 *     lse[n]   = log sum_v exp(z[n, v])
 *     loss[n]  = lse[n] - z[n, labels[n]]
 *
 * and its gradient with respect to H and W for the mean (or sum) of loss over
 * the valid rows.  The projection and the loss are computed in streaming
 * tiles and never stored as an [N, V] logits table ("OjasX 0.6.1", section
 * 核心技术 / Core Technology: zero-byte vocabulary logits table, chunked
 * streaming projection + loss that skips padding tokens); the running max and
 * normaliser are merged tile by tile (same page, Online Softmax paragraph);
 * the backward pass recomputes the logits per chunk instead of saving them
 * ("6GB显卡预训练11亿参数模型", sections 内存实际花在哪里 and 关键参数说明,
 * --chunked-loss 512); rows are selected by a device-side valid-token index
 * built without a host round trip (MaximusLLM page, section 2.3).
 *
 * Conventions shared by every entry point
 *   - H is [N, d], W is [V, d], both row-major and contiguous, same dtype:
 *     LCE_BF16 (bfloat16, fp32 accumulation) or LCE_F32.  W is the layout of
 *     nn.Linear(d, V).weight and of nn.Embedding(V, d).weight, so a tied
 *     embedding table is passed as is.
 *   - labels is int64 [N].  A row is valid when labels[n] != ignore_index.  A
 *     valid label must lie in [0, V); one that does not is reported through
 *     err_flag (see lce_forward) and its row is treated as ignored.
 *   - Every pointer argument is DEVICE memory owned by the caller, except
 *     where noted.  The library allocates no device memory: scratch space is
 *     the caller's `workspace` of at least lce_workspace_bytes(...) bytes,
 *     256-byte aligned.  Its size does not depend on N beyond O(N) per-token
 *     vectors and never on N * V.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every kernel is
 *     launched on it and the calls return without synchronising (except
 *     lce_check_error and lce_timing_query).
 *   - Requirements: N >= 0, d > 0 with d % 64 == 0 and d below 2^22, V > 0,
 *     N and V below 2^31, N * d * (element size) below 4 GiB.  Outputs must
 *     not alias inputs.
 *   - No state is kept between calls (besides the optional timing registry);
 *     calls on different streams may run concurrently if they use different
 *     workspaces and outputs.
 *   - Errors are returned as lce_status; a host-checkable problem returns
 *     before anything is launched.  lce_last_error() gives a message.
 */
#ifndef LCE_H
#define LCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LCE_OK = 0,
  LCE_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad enum value   */
  LCE_ERR_UNSUPPORTED = 2,  /* shape outside the supported range (d % 64)     */
  LCE_ERR_WORKSPACE = 3,    /* workspace smaller than lce_workspace_bytes     */
  LCE_ERR_LABEL_RANGE = 4,  /* a valid label was outside [0, V) (from flag)   */
  LCE_ERR_HIP = 5           /* a HIP runtime call or kernel launch failed      */
} lce_status;

typedef enum { LCE_F32 = 0, LCE_BF16 = 1 } lce_dtype;
typedef enum { LCE_MEAN = 0, LCE_SUM = 1 } lce_reduction;

/* Bytes of device workspace that lce_forward and lce_backward need for these
 * sizes (the larger of the two; the calls may share one buffer).  Returns 0
 * for invalid sizes.  Bounded by the token chunk (8192 rows), the vocabulary
 * block (16384 entries) and d, plus O(N) per-token vectors: for bf16 the
 * bounded G block (bf16 [8192, 16384]) and the chunk's transposed H rows
 * (bf16 [d, 8192]); fp32 adds the transposed G and W blocks (fp32
 * [16384, 8192] and [d, 16384]).  It never grows with N * V. */
size_t lce_workspace_bytes(int64_t N, int64_t d, int64_t V, int dtype);

/* Forward pass.
 *
 *  H, W, labels   inputs as above.
 *  ignore_index   label value of rows that take no part (PyTorch default -100;
 *                 it may also be a class id inside [0, V)).
 *  loss  [N] f32  per-row loss; 0 on ignored rows.
 *  lse   [N] f32  per-row logsumexp; 0 on ignored rows.  Needed by backward.
 *  valid_idx [N] int32   ascending original row numbers of the valid rows;
 *                 the first *valid_count entries are meaningful.
 *  valid_count [1] int32 number of valid rows.
 *  loss_sum [1] f64      sum of loss over valid rows, summed in a fixed order
 *                 (bitwise reproducible).
 *  loss_mean [1] f32     loss_sum / valid_count, NaN when valid_count == 0;
 *                 may be NULL.
 *  err_flag [1] int32    set to 1 when a valid label lies outside [0, V),
 *                 else 0; the call never reads W out of bounds.  Turn it into
 *                 a status with lce_check_error.
 */
lce_status lce_forward(const void* H, const void* W, const int64_t* labels, int64_t ignore_index,
                       int64_t N, int64_t d, int64_t V, int dtype, float* loss, float* lse,
                       int32_t* valid_idx, int32_t* valid_count, double* loss_sum,
                       float* loss_mean, int32_t* err_flag, void* workspace,
                       size_t workspace_bytes, void* stream);

/* lce_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, outputs, kernels and
 * results as lce_forward (bit for bit).  The forward's scratch (its
 * per-vocabulary-chunk partials: (3 J + 1) * N' * 4 bytes with J <= 64
 * vocabulary chunks and N' = N rounded up to 256) lives in a static 16 MiB
 * device array inside the library, one per GPU, held until the process ends.
 * Every V fits up to N = 21504 rows (fewer vocabulary chunks, V < 16129,
 * allow more); larger sizes return LCE_ERR_UNSUPPORTED before any launch.
 * Every call on one GPU uses that GPU's array: calls that overlap in time on
 * one GPU (different streams or threads) race and must be serialised by the
 * caller.  Calls no hipMalloc / hipFree. */
lce_status lce_forward_noalloc(const void* H, const void* W, const int64_t* labels,
                               int64_t ignore_index, int64_t N, int64_t d, int64_t V, int dtype,
                               float* loss, float* lse, int32_t* valid_idx, int32_t* valid_count,
                               double* loss_sum, float* loss_mean, int32_t* err_flag,
                               void* stream);

/* Backward pass: dH = dL/dH [N, d] f32 and dW = dL/dW [V, d] f32 for
 * L = mean (reduction LCE_MEAN) or sum (LCE_SUM) of loss over valid rows,
 * scaled by the upstream gradient *grad_out (a device f32 scalar).
 *
 *  lse, valid_idx, valid_count  exactly as produced by lce_forward for the
 *                 same H, W, labels and ignore_index.
 *  dH             fully written: rows of ignored tokens are 0.
 *  dW             overwritten when accumulate_dW == 0, added to otherwise
 *                 (for a weight that also receives other gradients);
 *                 16-byte aligned (stored as 4-float vectors), else
 *                 LCE_ERR_INVALID_ARG before any launch.
 * The logits are recomputed chunk by chunk; nothing of size N * V is stored.
 * No floating-point atomics are used: results are bitwise reproducible.
 */
lce_status lce_backward(const void* H, const void* W, const int64_t* labels, int64_t ignore_index,
                        const float* lse, const int32_t* valid_idx, const int32_t* valid_count,
                        int64_t N, int64_t d, int64_t V, int dtype, const float* grad_out,
                        int reduction, float* dH, float* dW, int accumulate_dW, void* workspace,
                        size_t workspace_bytes, void* stream);

/* fp32 -> bf16 copy of n values (e.g. dH or dW for a bf16 parameter):
 * dst[i] = src[i] rounded to the nearest bfloat16, ties to even; NaN stays
 * NaN, values beyond the bf16 range become +-inf.  src (f32 [n]) and dst
 * (bf16 bits [n]) are device memory, 16-byte aligned, not overlapping, else
 * LCE_ERR_INVALID_ARG before any launch.  One HBM-bound kernel on `stream`
 * (the optional output cast after the dH zero-fill of ignored rows). */
lce_status lce_cast_bf16(const float* src, void* dst, int64_t n, void* stream);

/* ------------------------------------------ fused optimizer update
 *
 * The backward pass with the optimizer applied to each dW tile as it is
 * produced, so no dW table is ever stored: updating the weights inside the
 * backward pass and keeping no persistent gradient buffers ("OjasX 0.6.1",
 * section 核心技术 / Core Technology, zero-byte .grad buffers).
 */
typedef enum { LCE_OPT_SGD = 1, LCE_OPT_ADAMW = 2 } lce_opt_kind;

typedef struct {
  int kind;             /* LCE_OPT_SGD or LCE_OPT_ADAMW */
  float lr;             /* >= 0 */
  float weight_decay;   /* >= 0: SGD adds wd * p to the gradient, AdamW decays p by lr * wd */
  float beta1, beta2;   /* AdamW, in [0, 1) */
  float eps;            /* AdamW, > 0 */
  int64_t step;         /* AdamW step number t >= 1 (bias correction 1 - beta^t) */
} lce_optimizer;

/* lce_backward (same inputs, same dH) whose dW goes straight into the
 * optimizer, PyTorch's formulas, in fp32:
 *   SGD    p -= lr (g + wd p)
 *   AdamW  p *= 1 - lr wd;  m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
 *          p -= lr / (1 - b1^t) * m / (sqrt(v) / sqrt(1 - b2^t) + eps)
 * p is W_master (fp32 [V, d]); for bf16 W the updated p is written back to W
 * rounded to nearest even, and W_master is required; for fp32 W, W_master may
 * be NULL and W itself is updated.  exp_avg / exp_avg_sq: fp32 [V, d] AdamW
 * state, updated in place (NULL for SGD).  Every row of W is updated (g = 0
 * for rows no valid token touches).  Any N: the vocabulary is walked block by
 * block, and a block's dW, summed over the token chunks in an fp32
 * accumulator inside the workspace, is applied by the last chunk that holds
 * valid rows.  A W row is rewritten only after its last read in this pass;
 * dH uses the weights from before the update.  Workspace: at least
 * lce_step_workspace_bytes(N, d, V, dtype) bytes (also enough for
 * lce_forward), 256-byte aligned, else LCE_ERR_WORKSPACE.
 */
/* Bytes of device workspace lce_backward_step needs: lce_workspace_bytes plus
 * the transposed W block (dH keeps reading the block's old weights while the
 * update rewrites them) and either, when every valid row lies in one token
 * chunk (8192 rows), the transposed G block the optimizer epilogue reads
 * ([16384, 8192]), or else the fp32 dW block accumulator ([16384, d]).
 * Independent of N beyond that and of V.  Returns 0 for invalid sizes. */
size_t lce_step_workspace_bytes(int64_t N, int64_t d, int64_t V, int dtype);

lce_status lce_backward_step(const void* H, void* W, const int64_t* labels, int64_t ignore_index,
                             const float* lse, const int32_t* valid_idx, const int32_t* valid_count,
                             int64_t N, int64_t d, int64_t V, int dtype, const float* grad_out,
                             int reduction, float* dH, float* W_master, float* exp_avg,
                             float* exp_avg_sq, const lce_optimizer* opt, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------------- vocabulary shards
 *
 * The vocabulary [0, V_total) split into contiguous shards, each with its own
 * rows of W ("MaximusLLM" page, section 2.1: the vocabulary table cut into
 * contiguous sub-tables).  Shard k covers [v_begin, v_begin + V_shard) and
 * W_shard [V_shard, d] holds exactly those rows.  The shards' forward
 * partials merge with the online-softmax rescale step ("OjasX 0.6.1", Online
 * Softmax paragraph) into the same loss and lse as lce_forward over the
 * whole table; each shard's backward gives its own dW rows and a share of dH.
 * This is the single-device half of splitting the vocabulary across GPUs
 * (between GPUs the partials travel through one all-reduce, and the dH shares
 * through a reduce-scatter).  Workspace: lce_workspace_bytes(N, d, V_shard,
 * dtype).  Labels are global ids in [0, V_total).
 */

/* Forward of one shard.  Per row n (f32 [N] each, original row order):
 *  part_max[n]     largest logit of the row over the shard
 *  part_sum[n]     sum over the shard of exp(logit - part_max[n])  (>= 1)
 *  part_target[n]  the target logit if labels[n] lies in the shard, else -inf
 * Ignored rows: part_max = part_sum = 0, part_target unspecified.
 * valid_idx, valid_count and err_flag as in lce_forward (identical for every
 * shard; the label range check is against V_total).  Returns
 * LCE_ERR_INVALID_ARG when the shard does not lie in [0, V_total).
 */
lce_status lce_forward_shard(const void* H, const void* W_shard, const int64_t* labels,
                             int64_t ignore_index, int64_t N, int64_t d, int64_t V_total,
                             int64_t v_begin, int64_t V_shard, int dtype, float* part_max,
                             float* part_sum, float* part_target, int32_t* valid_idx,
                             int32_t* valid_count, int32_t* err_flag, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Merges the partials of n_shards shards that together cover [0, V_total)
 * exactly once; shard k's three arrays start at part_* + k * shard_stride
 * (elements, >= N when n_shards > 1).  Writes loss, lse (f32 [N], ignored rows
 * 0), loss_sum (f64, fixed-order sum over valid rows) and loss_mean (nullable;
 * NaN when no row is valid), as lce_forward does.  No workspace.
 */
lce_status lce_lse_merge(const float* part_max, const float* part_sum, const float* part_target,
                         int64_t n_shards, int64_t shard_stride, int64_t N,
                         const int32_t* valid_idx, const int32_t* valid_count, float* loss,
                         float* lse, double* loss_sum, float* loss_mean, void* stream);

/* Backward of one shard, given the merged lse.  dW_shard [V_shard, d] f32 as
 * dW in lce_backward (16-byte aligned).  dH receives this shard's share: overwritten (ignored
 * rows set to 0) when accumulate_dH == 0, added to otherwise; summing the
 * shares of every shard gives lce_backward's dH.
 */
lce_status lce_backward_shard(const void* H, const void* W_shard, const int64_t* labels,
                              int64_t ignore_index, const float* lse, const int32_t* valid_idx,
                              const int32_t* valid_count, int64_t N, int64_t d, int64_t V_total,
                              int64_t v_begin, int64_t V_shard, int dtype, const float* grad_out,
                              int reduction, float* dH, int accumulate_dH, float* dW_shard,
                              int accumulate_dW, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ------------------------------------------- tied table: input side
 *
 * The same table W [V, d] read as the input embedding ("6GB显卡预训练11亿参数模型",
 * section 使用的预训练配置: tied embeddings).  Only positions whose id is not
 * pad_id are looked up; the others get a zero vector, and the valid index is
 * built on the device in the same launch sequence, with no host round trip
 * ("MaximusLLM" page, section 2.3: padding-aware sparse index engine).
 */

/* X [N, d] (dtype of W) = W[input_ids[n]] for valid n, 0 elsewhere.  valid_idx
 * (int32 [N], ascending), valid_count and err_flag as lce_forward builds them
 * from labels, with pad_id in place of ignore_index: an id outside [0, V)
 * that is not pad_id sets err_flag and the row is treated as padding. */
lce_status lce_embed_forward(const void* W, const int64_t* input_ids, int64_t pad_id, int64_t N,
                             int64_t d, int64_t V, int dtype, void* X, int32_t* valid_idx,
                             int32_t* valid_count, int32_t* err_flag, void* stream);

/* Bytes of device workspace lce_embed_backward needs (0 for unsupported
 * sizes).  O(N + N * d / 32): sort keys, segment lists and chunk partials. */
size_t lce_embed_workspace_bytes(int64_t N, int64_t d, int64_t V);

/* dW [V, d] f32 += sum of dX [N, d] f32 rows over valid positions with that
 * id (accumulate_dW != 0: add to dW, e.g. after lce_backward filled in the
 * output side of a tied table; 0: rows with no occurrence become 0).  The
 * valid rows are stably sorted by id, rows sharing an id are summed in a
 * fixed order (ascending position inside 64-row chunks, then the chunks in
 * order): results are bitwise reproducible, no floating-point atomics. */
lce_status lce_embed_backward(const float* dX, const int64_t* input_ids, const int32_t* valid_idx,
                              const int32_t* valid_count, int64_t N, int64_t d, int64_t V,
                              float* dW, int accumulate_dW, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Synchronises `stream` and returns LCE_ERR_LABEL_RANGE when *err_flag is set
 * (a valid label outside [0, V) -- the out-of-range index failure described
 * in "6GB显卡预训练11亿参数模型", section 可证伪测试抓到的8个静默bug, #155),
 * LCE_OK otherwise.  err_flag is device memory. */
lce_status lce_check_error(const int32_t* err_flag, void* stream);

/* Static description of a status code. */
const char* lce_status_string(lce_status s);

/* Message of the last failure on the calling thread ("" if none). */
const char* lce_last_error(void);

/* ------------------------------------------------ online-softmax attention
 *
 * O = softmax(scale * Q K^T) V over the keys of each query, with an optional
 * causal mask (query i attends to keys 0..i), and the natural-log
 * logsumexp of each row of masked, scaled scores.  The [B, H, S, S] score
 * matrix is never stored: score tiles stream through registers and LDS with
 * the running max / normaliser recurrence ("OjasX 0.6.1", section 核心技术 /
 * "Core Technology", zero-byte attention score matrix, and its Online Softmax
 * paragraph).  The operation is the one the KV-cache page writes (section
 * KV Cache基础): softmax(Q K^T / sqrt(d_k)) V.
 *
 * Q, K, V: device pointers, bf16, layout [B, H, S, D] (D contiguous), read
 *          only.  D must be 64 or 128 (else LCE_ERR_UNSUPPORTED).
 * causal:  0 or 1.
 * scale:   > 0, or 0 for 1 / sqrt(D); negative or non-finite is
 *          LCE_ERR_INVALID_ARG.
 * O:       device, f32 [B, H, S, D], written.
 * lse:     device, f32 [B, H, S], written (the backward pass recomputes the
 *          probabilities from it).
 * B, H, S >= 0; nothing is launched when any of them is 0.  Accumulation in
 * f32; the probabilities enter the second product rounded to bf16 and the
 * normaliser sums those rounded values.  Allocates nothing; launches on
 * `stream` only. */
lce_status lce_attention_forward(const void* Q, const void* K, const void* V, int64_t B, int64_t H,
                                 int64_t S, int64_t D, int causal, float scale, float* O,
                                 float* lse, void* stream);

/* Gradient of lce_attention_forward for an upstream dO: dQ, dK, dV.  The
 * probabilities are recomputed tile by tile from Q, K and the forward's lse
 * (the [S, S] matrix is not stored in the backward pass either; same
 * passages as lce_attention_forward):
 *   dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),  D = rowsum(dO * O),
 *   dQ = scale dS K,  dK = scale dS^T Q.
 *
 * Q, K, V: as for lce_attention_forward (bf16 [B, H, S, D], D = 64 or 128).
 * O, lse:  the forward's outputs (f32), read only.
 * dO:      device, bf16 [B, H, S, D], read only.
 * dQ, dK, dV: device, f32 [B, H, S, D], written (not accumulated).
 * delta:   device scratch, f32 [B, H, S], overwritten with D.
 * causal, scale: as for the forward (and must match it).
 * Two kernels on `stream`, no atomics: results are deterministic.  The
 * probabilities and dS enter the products rounded to bf16.  Allocates
 * nothing; errors as for the forward. */
lce_status lce_attention_backward(const void* Q, const void* K, const void* V, const float* O,
                                  const float* lse, const void* dO, int64_t B, int64_t H,
                                  int64_t S, int64_t D, int causal, float scale, float* dQ,
                                  float* dK, float* dV, float* delta, void* stream);

/* ---------------------------------------------------------- measurement */

/* C[M, N] = A[M, K] B[N, K]^T with the same MFMA tile engine as the path
 * (f32 output, row-major; K % 64 == 0).  Used to measure the engine's bare
 * GEMM rate at the path's shapes and to check its layout in isolation. */
lce_status lce_gemm_nt(const void* A, const void* B, float* C, int64_t M, int64_t N, int64_t K,
                       int dtype, void* stream);

/* MFMA calibration: 1024 workgroups x 512 threads, each thread issuing
 * 4 * iters bf16 32x32x16 MFMAs (32768 FLOPs each) on register operands with
 * no memory traffic, then storing one float to out (device, >= 1024 * 512
 * floats).  Total FLOPs = 1024 * 8 * 4 * iters * 32768.  The rate (and, under
 * a counter run, the clock) the chip sustains when only the matrix cores
 * work: the reference the path's kernels are measured against ("6GB显卡预训练
 * 11亿参数模型", section 为什么是375天: time the hardware's matrix rate before
 * judging the model's).  iters in [1, 2^24]. */
lce_status lce_mfma_peak(float* out, int64_t n_out, int64_t iters, void* stream);

/* Kernel classes for the optional timing registry. */
typedef enum {
  LCE_K_COMPACT = 0,   /* valid-token compaction                         */
  LCE_K_FWD = 1,       /* fused projection + online logsumexp            */
  LCE_K_MERGE = 2,     /* merge of vocabulary-chunk partials             */
  LCE_K_REDUCE = 3,    /* loss reduction                                 */
  LCE_K_ZERO = 4,      /* zeroing dH rows of ignored tokens              */
  LCE_K_TRANSPOSE = 5, /* W / H^T operand layout for backward            */
  LCE_K_BWD_G = 6,     /* logit recompute + G tile                       */
  LCE_K_DH = 7,        /* not launched: dH runs in LCE_K_DH_DW           */
  LCE_K_DW = 8,        /* not launched: dW runs in LCE_K_DH_DW           */
  LCE_K_GEMM = 9,      /* lce_gemm_nt                                    */
  LCE_K_EMBED = 10,    /* embedding gather / gradient scatter-sum        */
  LCE_K_ATTN = 11,     /* online-softmax attention forward               */
  LCE_K_ATTN_DQ = 12,  /* attention backward, dQ pass (and rowsum(dO O)) */
  LCE_K_ATTN_DKV = 13, /* attention backward, dK / dV pass               */
  LCE_K_DH_DW = 14,    /* dH and dW of one vocabulary block, one launch   */
  LCE_K_CAST = 15,     /* fp32 -> bf16 output cast                        */
  LCE_K_MFMA = 16,     /* lce_mfma_peak                                   */
  LCE_K_OPT = 17,      /* optimizer update of a vocabulary block (the fused
                          step beyond one token chunk)                     */
  LCE_K_COUNT = 18
} lce_kernel_class;

/* When enabled, every launch is bracketed by HIP events recorded on the
 * launch stream (host-side registry, process-wide).  The events are created
 * with hipEventDisableSystemFence: they time the launches and order nothing
 * (a caller synchronises its stream or device before reading results). */
lce_status lce_timing_enable(int on);
/* Clears the registry. */
lce_status lce_timing_reset(void);
/* Synchronises on the recorded events and returns, for one kernel class, the
 * summed device time in milliseconds and the number of launches (both host
 * pointers). */
lce_status lce_timing_query(int kernel_class, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* LCE_H */
