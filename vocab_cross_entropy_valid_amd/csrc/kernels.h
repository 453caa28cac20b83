// Host-side launchers of the HIP kernels (internal to liblce).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

struct FwdArgs {
  const void* H;
  const void* W;
  const int64_t* labels;
  const int32_t* valid_idx;
  const int32_t* valid_count;
  int64_t N, d, V;
  int64_t y_off;  // label of vocabulary row v of W is y_off + v (a shard's first entry)
  int n_vtiles;  // ceil(V / 256)
  int tpc;       // vocabulary tiles per chunk
  int J;         // chunks: ceil(n_vtiles / tpc)
  int64_t Nb;    // row stride of the partial arrays (multiple of 256, >= N)
  float* pm;     // [J][Nb] running max, log2 units
  float* ps;     // [J][Nb] running sum of 2^(u - m)
  float* pz;     // [J][Nb] target logit if it lies in the chunk, else -inf
};

struct BwdGArgs {
  const void* H;
  const void* W;
  const int64_t* labels;
  const float* lse;
  const int32_t* valid_idx;
  const int32_t* valid_count;
  const float* grad_out;
  int reduction;  // 0 mean, 1 sum
  int64_t N, d, V;
  int64_t y_off;   // label of vocabulary row v of W is y_off + v (a shard's first entry)
  int64_t c0, C;   // token chunk of the compact index
  int64_t v0, Vs;  // vocabulary block
  void* G;         // [C][ldG]
  void* GT;        // [Vs][ldGT]
  int64_t ldG, ldGT;  // row strides in elements (padded off powers of two)
  int nslots;      // tile slots, one workgroup each
};

struct DhArgs {
  const void* G;   // [C][ldG]
  const void* WT;  // [d][ldWT] (when W is null)
  const void* W;   // [V][d] bf16 read directly (K-major B operand), or null
  int64_t C, Vs, d;
  int64_t ldG, ldWT;
  const int32_t* valid_idx;
  const int32_t* valid_count;
  int64_t c0, v0, V;
  float* dH;  // [N][d]
  int64_t N;
  int beta;
};

struct DwArgs {
  const void* GT;  // [Vs][ldGT]: fp32, and the bf16 optimizer epilogue
  const void* HT;  // [d][ldHT]
  int64_t C, Vs, d;
  int64_t ldGT, ldHT;
  const void* G;   // [C][ldG]: the bf16 plain store reads G K-major instead of G^T
  int64_t ldG;
  const int32_t* valid_count;
  int64_t c0, v0, V;
  float* dW;
  int accumulate;
  int nslots;      // tile slots (the launch walks them persistently)
  // optimizer epilogue (opt_kind > 0): the dW tile is applied here and never
  // stored.  bc1 = 1 - beta1^t, bc2s = sqrt(1 - beta2^t).
  int opt_kind;  // 0 none (the zero-initialised default), 1 SGD, 2 AdamW
  float lr, wd, beta1, beta2, eps, bc1, bc2s;
  float* master;      // fp32 [V, d] weights the update applies to
  float* exp_avg;     // fp32 [V, d] (AdamW)
  float* exp_avg_sq;  // fp32 [V, d] (AdamW)
  uint16_t* w16;      // bf16 [V, d] operand copy refreshed from master (nullable)
  // apply_opt_kernel only: fp32 [Vs][d] sum of the block's dW over the token
  // chunks (the plain store writes it when the rows span several chunks)
  float* acc;
};

struct TransposeArgs {
  const void* src;
  int64_t ld_src;          // elements
  const int32_t* gather;   // nullable: physical row = gather[row0 + i]
  int64_t row0;
  const int32_t* count;    // nullable: rows available = *count - row0 (clamped)
  int64_t nrows_static;    // used when count is null: rows available = nrows_static - row0
  void* dst;               // [K][ld_dst]
  int64_t ncols;           // columns of dst written (multiple of 64)
  int64_t ld_dst;          // row stride of dst in elements
  int64_t K;               // rows of dst = columns read from src (multiple of 64)
  const int32_t* active_count;  // nullable: skip the whole launch when *active_count <= active_c0
  int64_t active_c0;
};

hipError_t launch_compact(const int64_t* labels, int64_t N, int64_t ignore_index, int64_t V,
                          int32_t* valid_idx, int32_t* valid_count, int32_t* err_flag, float* loss,
                          float* lse, hipStream_t s);
hipError_t launch_fwd(const FwdArgs& a, int dtype, int grid, hipStream_t s);
hipError_t launch_fwd_merge(const FwdArgs& a, float* loss, float* lse, float* loss_c,
                            int64_t N, hipStream_t s);
hipError_t launch_fwd_part(const FwdArgs& a, float* part_max, float* part_sum, float* part_target,
                           int64_t N, hipStream_t s);
hipError_t launch_shard_merge(const float* part_max, const float* part_sum, const float* part_target,
                              int64_t n_shards, int64_t stride, int64_t N, float* loss, float* lse,
                              hipStream_t s);
// gather == nullptr: sums loss[0 .. count); else sums loss[gather[i]], i < count
hipError_t launch_loss_reduce(const float* loss, const int32_t* gather, const int32_t* valid_count,
                              double* loss_sum, float* loss_mean, hipStream_t s);
hipError_t launch_zero_ignored(const int64_t* labels, int64_t N, int64_t ignore_index, int64_t V,
                               float* dH, int64_t d, hipStream_t s);
hipError_t launch_transpose(const TransposeArgs& a, int dtype, hipStream_t s);
hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s);
hipError_t launch_bwd_g(BwdGArgs a, int dtype, hipStream_t s);
// dH and dW of one vocabulary block in a single launch: the dH tiles first
// (long K), then one workgroup per dW tile, dispatched onto the CUs the dH
// tiles leave free.
hipError_t launch_dh_dw(const DhArgs& ha, DwArgs wa, int dtype, hipStream_t s);
// The optimizer over block [v0, v0 + nv) from the summed gradient in a.acc.
hipError_t launch_apply_opt(const DwArgs& a, hipStream_t s);
// Workspace layout of the embedding backward (byte offsets, 256-aligned).
struct EmbedPlan {
  int end_bit;  // sort key bits: 2^end_bit > V (V itself is the padding sentinel)
  int passes;   // radix passes of 9 bits
  int nblocks;  // sort tiles of 2048 pairs
  size_t off_key, off_val, off_key_s, off_val_s, off_seg_start, off_seg_chunk0, off_seg_part0;
  size_t off_chunk_seg, off_meta, off_hist, off_part;
  int64_t max_chunks, max_parts;
  size_t total;
};
EmbedPlan make_embed_plan(int64_t N, int64_t d, int64_t V);
hipError_t launch_embed_gather(const void* W, const int64_t* ids, int64_t pad_id, int64_t N,
                               int64_t V, int64_t row_bytes, void* X, hipStream_t s);
hipError_t launch_embed_backward(const EmbedPlan& p, const float* dX, const int64_t* ids,
                                 const int32_t* valid_idx, const int32_t* valid_count, int64_t N,
                                 int64_t d, int64_t V, float* dW, int accumulate, void* ws,
                                 int grid, hipStream_t s);
hipError_t launch_gemm_nt(const void* A, const void* B, float* C, int64_t M, int64_t N, int64_t K,
                          int dtype, hipStream_t s);
// blocks workgroups of 512 threads, each thread 4 * iters bf16 32x32x16 MFMAs;
// out holds blocks * 512 floats
hipError_t launch_mfma_peak(float* out, int blocks, int64_t iters, hipStream_t s);


// Online-softmax attention forward over [B*H, S, D] bf16 Q, K, V.
struct AttnArgs {
  const uint16_t* Q;  // bf16 bits
  const uint16_t* K;
  const uint16_t* V;
  float* O;          // [B*H, S, D]
  float* lse;        // [B*H, S], natural log
  int64_t BH;
  int S;
  int causal;
  float scale_log2;  // scale * log2(e)
};

hipError_t launch_attn_fwd(const AttnArgs& a, int D, hipStream_t s);


// Online-softmax attention backward (two passes; see kernels_attn.hip).
struct AttnBwdArgs {
  const uint16_t* Q;   // bf16 [B*H, S, D]
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* dO;  // bf16 [B*H, S, D]
  const float* O;      // f32 [B*H, S, D], the forward output
  const float* lse;    // f32 [B*H, S], natural log
  float* dQ;           // f32 [B*H, S, D]
  float* dK;
  float* dV;
  float* delta;        // f32 [B*H, S] scratch: rowsum(dO * O)
  int64_t BH;
  int S;
  int causal;
  float scale;
  float scale_log2;    // scale * log2(e)
};

// The two passes launch separately: dQ (which also writes delta) first, then
// dK / dV, which reads delta.
hipError_t launch_attn_bwd_dq(const AttnBwdArgs& a, int D, hipStream_t s);
hipError_t launch_attn_bwd_dkv(const AttnBwdArgs& a, int D, hipStream_t s);

}  // namespace lce
