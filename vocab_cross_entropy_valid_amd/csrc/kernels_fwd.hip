// Forward kernels: valid-token compaction, fused projection + online
// logsumexp over vocabulary tiles, merge of vocabulary chunks, and the
// deterministic loss reduction.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace lce {

// ------------------------------------------------------------ compaction
//
// Builds the ascending index of rows whose label is kept (label !=
// ignore_index) in one workgroup, with no host round trip: the MaximusLLM
// page (section 2.3, padding-aware sparse index engine) builds its valid mask
// and uses it inside the same kernel to avoid a host-device sync; the OjasX
// page (core technology) packs per-lane predicates into hardware ballot masks.
// Here each wave64 takes a 64-bit ballot of the predicate, a lane's slot is
// the popcount of the ballot bits below it (mbcnt), and the 16 wave totals
// are scanned in LDS.  A kept label outside [0, V) raises err_flag and the
// row is treated as ignored, so no later kernel indexes W with it.
// Ignored rows get loss = lse = 0 here (when loss is not null).
__global__ __launch_bounds__(1024) void compact_kernel(const int64_t* __restrict__ labels, int64_t N,
                                                       int64_t ignore_index, int64_t V,
                                                       int32_t* __restrict__ valid_idx,
                                                       int32_t* __restrict__ valid_count,
                                                       int32_t* __restrict__ err_flag,
                                                       float* __restrict__ loss,
                                                       float* __restrict__ lse) {
  __shared__ int wave_tot[16];
  __shared__ int wave_base[17];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  int base = 0;
  int err = 0;
  for (int64_t n0 = 0; n0 < N; n0 += 1024) {
    const int64_t n = n0 + tid;
    const bool in = n < N;
    const int64_t y = in ? labels[n] : ignore_index;
    const bool keep = in && (y != ignore_index);
    const bool in_range = (y >= 0) && (y < V);
    err |= (keep && !in_range) ? 1 : 0;
    const bool valid = keep && in_range;
    if (in && !valid && loss) {
      loss[n] = 0.f;
      lse[n] = 0.f;
    }
    const uint64_t m = __ballot(valid);
    const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (lane == 0) wave_tot[wv] = __popcll(m);
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      for (int w = 0; w < 16; ++w) {
        wave_base[w] = acc;
        acc += wave_tot[w];
      }
      wave_base[16] = acc;
    }
    __syncthreads();
    if (valid) valid_idx[base + wave_base[wv] + rank] = (int32_t)n;
    base += wave_base[16];
    __syncthreads();
  }
  const int any_err = __syncthreads_or(err);
  if (tid == 0) {
    *valid_count = base;
    *err_flag = any_err ? 1 : 0;
  }
}

hipError_t launch_compact(const int64_t* labels, int64_t N, int64_t ignore_index, int64_t V,
                          int32_t* valid_idx, int32_t* valid_count, int32_t* err_flag, float* loss,
                          float* lse, hipStream_t s) {
  hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(1024), 0, s, labels, N, ignore_index, V,
                     valid_idx, valid_count, err_flag, loss, lse);
  return hipGetLastError();
}

// -------------------------------------------- fused projection + logsumexp
//
// The output projection and the loss are computed tile by tile and never
// stored as a [N, V] table (OjasX page, core technology: zero-byte
// vocabulary logits table).  Per token the running (max, sum of
// exponentials) pair is updated tile after tile, which is the online
// softmax recurrence of the same page: after each tile the stored maximum is
// corrected and the sum rescaled, which gives exactly the full logsumexp.
//
// Work decomposition: vocabulary tiles of 256 entries are grouped into J
// chunks of tpc tiles; an item is (token tile of 256 compact rows, chunk).
// The kernel is persistent: each workgroup walks items in rounds.  Within a
// round the 32 workgroups on one XCD take a 4 x 8 block of (token tile,
// chunk) items, so that four H tiles and eight W streams are shared through
// that XCD's L2.  A item leaves per-token partials (m, s, z_target) for its
// chunk; fwd_merge_kernel combines the J chunks.
//
// MFMA operand order: A = W rows (vocabulary), B = H rows (tokens, gathered
// through valid_idx).  Each lane then holds 2 consecutive tokens x 64
// vocabulary entries per tile, so the max / sum reductions run inside the
// lane, and only once per item across the lane pair (l, l ^ 32) and across
// the two waves that split the tile's vocabulary.
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void fwd_lse_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kMainLds];
  // wave-pair merge area: used only after an item's last main loop, which
  // ends with a barrier, so it shares the stage buffers
  float* mg = (float*)lds;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wa = wave & 1;
  const int wb = wave >> 1;
  const int j = lane & 31;
  const int h = lane >> 5;

  const int count = *a.valid_count;
  const int R = (count + kTile - 1) / kTile;
  if (R == 0) return;
  const int GA = 4, GB = 8;
  const int nsb = ((R + GA - 1) / GA) * ((a.J + GB - 1) / GB);
  const int nstages = (int)(a.d / Elem<T>::kPerStage);
  const int64_t ldb = a.d * Elem<T>::kSize;

  for (int64_t ls = blockIdx.x;; ls += gridDim.x) {
    const int k = (int)(ls >> 3);
    const int sb = ((k >> 5) << 3) + (int)(ls & 7);
    if (sb >= nsb) break;
    int tt, ch;
    if (!xcd_tile((int)ls, R, a.J, GA, GB, tt, ch)) continue;

    RowSource bs{(const char*)a.H, ldb, a.valid_idx, (int64_t)tt * kTile, count, a.N};
    const RowPtrs pb = make_row_ptrs<true>(bs, tid);

    int y[kNT];
    float m[kNT], s[kNT], zy[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const int i = tt * kTile + wb * kWaveN + 2 * j + nt;
      // label relative to row 0 of W (outside [0, V) in a vocabulary shard
      // that does not hold it: then it never matches an entry)
      y[nt] = (i < count) ? (int)(a.labels[a.valid_idx[i]] - a.y_off) : -1;
      m[nt] = -INFINITY;
      s[nt] = 0.f;
      zy[nt] = -INFINITY;
    }

    const int vt0 = ch * a.tpc;
    const int vt1 = min(vt0 + a.tpc, a.n_vtiles);
    for (int vt = vt0; vt < vt1; ++vt) {
      RowSource as{(const char*)a.W, ldb, nullptr, (int64_t)vt * kVocabTile, a.V, 0};
      const RowPtrs pa = make_row_ptrs<false>(as, tid);
      Acc acc;
      zero_acc(acc);
      tile_mainloop<T>(acc, lds, pa, pb, nstages, tid);

      const int vw0 = vt * kVocabTile + wa * kHalf;  // first vocabulary entry of this wave
      // Entry (mt, i) of this lane sits at c(mt, i) + 4 h past vw0, with the
      // compile-time constant c = 32 mt + 8 (i / 4) + i % 4.  Comparing c with
      // per-lane bounds keeps the 64 positions out of registers.
      const int vlim_h = (int)min<int64_t>(a.V - vw0, (int64_t)kHalf) - 4 * h;  // c < vlim_h: < V
      int rel_h[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) rel_h[nt] = y[nt] - vw0 - 4 * h;  // label at c == rel_h
      // Target logit, taken from the same fp32 accumulator as the sum (a
      // label is always below V, so never a masked entry).  Only a wave in
      // which some lane's label falls in its 128 entries runs the compare.
      bool lab = false;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) lab |= (unsigned)(y[nt] - vw0) < (unsigned)kHalf;
      if (__ballot(lab)) {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (32 * mt + 8 * (i >> 2) + (i & 3) == rel_h[nt]) zy[nt] = acc[mt][nt][i];
      }
      // per token: online (max, sum) update over each 32-entry slice (mt), so
      // that only 16 accumulator values are live in VGPRs at a time.  The
      // bounds mask (entries at or beyond V drop out as -inf) runs only on a
      // wave whose entries reach past V (a wave-uniform branch).
      auto slices = [&](auto kMask) {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            float z[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int c = 32 * mt + 8 * (i >> 2) + (i & 3);
              z[i] = (!decltype(kMask)::value || c < vlim_h) ? acc[mt][nt][i] : -INFINITY;
            }
            float tmax = z[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, z[i]);
            if (!decltype(kMask)::value || tmax != -INFINITY) {  // else the slice is past V
              tmax *= kLog2e;
              if (tmax > m[nt]) {
                s[nt] *= fast_exp2(m[nt] - tmax);
                m[nt] = tmax;
              }
              const float mn = m[nt];
              float sum = 0.f;
#pragma unroll
              for (int i = 0; i < 16; ++i) sum += fast_exp2(fmaf(z[i], kLog2e, -mn));
              s[nt] += sum;
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      };
      typedef std::integral_constant<bool, true> kOn;
      typedef std::integral_constant<bool, false> kOff;
      if (vw0 + kHalf > a.V) {
        slices(kOn());
      } else {
        slices(kOff());
      }
    }

    // merge the lane pair (l, l ^ 32): same tokens, other vocabulary rows
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const float mo = __shfl_xor(m[nt], 32);
      const float so = __shfl_xor(s[nt], 32);
      const float zo = __shfl_xor(zy[nt], 32);
      const float M = fmaxf(m[nt], mo);
      s[nt] = (M == -INFINITY) ? 0.f : s[nt] * fast_exp2(m[nt] - M) + so * fast_exp2(mo - M);
      m[nt] = M;
      zy[nt] = fmaxf(zy[nt], zo);
    }
    // merge the two waves (wa = 0, 1) that split the tile's vocabulary
    if (wa == 1 && h == 0) {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        float* q = mg + (wb * kWaveN + 2 * j + nt) * 3;
        q[0] = m[nt];
        q[1] = s[nt];
        q[2] = zy[nt];
      }
    }
    __syncthreads();
    if (wa == 0 && h == 0) {
      f32x2 om, os, oz;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const float* q = mg + (wb * kWaveN + 2 * j + nt) * 3;
        const float M = fmaxf(m[nt], q[0]);
        om[nt] = M;
        os[nt] = (M == -INFINITY) ? 0.f : s[nt] * fast_exp2(m[nt] - M) + q[1] * fast_exp2(q[0] - M);
        oz[nt] = fmaxf(zy[nt], q[2]);
      }
      const int64_t off = (int64_t)ch * a.Nb + (int64_t)tt * kTile + wb * kWaveN + 2 * j;
      *(f32x2*)(a.pm + off) = om;
      *(f32x2*)(a.ps + off) = os;
      *(f32x2*)(a.pz + off) = oz;
    }
    __syncthreads();
  }
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int grid, hipStream_t s) {
  if (dtype == 1)
    hipLaunchKernelGGL(fwd_lse_kernel<bf16_t>, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(fwd_lse_kernel<float>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- merge
//
// (M, S) of compact row i over the J chunk partials: M = max of the chunk
// maxima, S = sum of each chunk's sum rescaled to M (log2 units).  The loads
// go out in batches of 16, one memory round trip per batch instead of one
// per chunk (the merge is latency-bound); the sum runs over the chunks in
// order.
// Offsets of the 16 chunks of a batch are 32-bit products b * Nb (Nb <
// 2^25: the sizes check keeps N * d * element size below 4 GiB with d >= 64):
// as 64-bit values they kept 16 scalar register pairs live and the SGPR
// spills reserved a private stack frame.
__device__ __forceinline__ void merge_chunks(const float* __restrict__ pm_base,
                                             const float* __restrict__ ps_base, int J, int64_t Nb,
                                             int64_t i, float& M, float& S) {
  constexpr int kB = 16;
  const float* pmi = pm_base + i;
  const float* psi = ps_base + i;
  const uint32_t nb = (uint32_t)Nb;
  M = -INFINITY;
  for (int c0 = 0; c0 < J; c0 += kB) {
    const float* q = pmi + (int64_t)c0 * Nb;
    float pm[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) pm[b] = (c0 + b < J) ? q[(uint64_t)(b * nb)] : -INFINITY;
#pragma unroll
    for (int b = 0; b < kB; ++b) M = fmaxf(M, pm[b]);
  }
  S = 0.f;
  for (int c0 = 0; c0 < J; c0 += kB) {
    const float* q = pmi + (int64_t)c0 * Nb;
    const float* r = psi + (int64_t)c0 * Nb;
    float pm[kB], ps[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const bool in = c0 + b < J;
      pm[b] = in ? q[(uint64_t)(b * nb)] : -INFINITY;
      ps[b] = in ? r[(uint64_t)(b * nb)] : 0.f;
    }
#pragma unroll
    for (int b = 0; b < kB; ++b)
      if (c0 + b < J) S += ps[b] * fast_exp2(pm[b] - M);
  }
}

// Combines the J chunk partials of each compact row with the same
// max-and-rescale step, then lse = (M + log2 S) ln 2 and
// loss = lse - z_target, written at the row's original position.
__global__ __launch_bounds__(256) void fwd_merge_kernel(FwdArgs a, float* __restrict__ loss,
                                                        float* __restrict__ lse,
                                                        float* __restrict__ loss_c) {
  const int count = *a.valid_count;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  float M, S;
  merge_chunks(a.pm, a.ps, a.J, a.Nb, i, M, S);
  const int r = a.valid_idx[i];
  const int64_t yv = a.labels[r];
  const int cy = (int)(yv / kVocabTile) / a.tpc;
  const float zt = a.pz[(int64_t)cy * a.Nb + i];
  const float l = (M + fast_log2(S)) * kLn2;
  const float lv = l - zt;
  lse[r] = l;
  loss[r] = lv;
  loss_c[i] = lv;
}

hipError_t launch_fwd_merge(const FwdArgs& a, float* loss, float* lse, float* loss_c, int64_t N,
                            hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const int grid = (int)((N + 255) / 256);
  hipLaunchKernelGGL(fwd_merge_kernel, dim3(grid), dim3(256), 0, s, a, loss, lse, loss_c);
  return hipGetLastError();
}

// ------------------------------------------------- vocabulary shards
//
// A shard is a contiguous slice [y_off, y_off + V) of the vocabulary, with its
// own rows of W (MaximusLLM page, section 2.1: the vocabulary table split into
// contiguous sub-tables).  Per valid row the shard exports its partial of the
// online-softmax state (OjasX page, core technology): m = the largest logit
// in the shard, s = sum over the shard of exp(logit - m), and the target
// logit when the label lies in the shard (-inf otherwise), in natural-log
// units, at the row's original position.
__global__ __launch_bounds__(256) void fwd_part_kernel(FwdArgs a, float* __restrict__ part_max,
                                                       float* __restrict__ part_sum,
                                                       float* __restrict__ part_target) {
  const int count = *a.valid_count;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  float M, S;
  merge_chunks(a.pm, a.ps, a.J, a.Nb, i, M, S);
  const int r = a.valid_idx[i];
  const int64_t yl = a.labels[r] - a.y_off;
  float zt = -INFINITY;
  if (yl >= 0 && yl < a.V) zt = a.pz[(int64_t)((int)(yl / kVocabTile) / a.tpc) * a.Nb + i];
  part_max[r] = M * kLn2;
  part_sum[r] = S;
  part_target[r] = zt;
}

hipError_t launch_fwd_part(const FwdArgs& a, float* part_max, float* part_sum, float* part_target,
                           int64_t N, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const int grid = (int)((N + 255) / 256);
  hipLaunchKernelGGL(fwd_part_kernel, dim3(grid), dim3(256), 0, s, a, part_max, part_sum,
                     part_target);
  return hipGetLastError();
}

// Merges the partials of n shards that together cover the vocabulary, with
// the same rescale step as the online softmax: M = max m_i,
// S = sum s_i exp(m_i - M), lse = M + log S, loss = lse - (the one finite
// target).  Shard i's arrays start at i * stride.  A row that every shard
// left with s = 0 is an ignored row: loss = lse = 0.
__global__ __launch_bounds__(256) void shard_merge_kernel(const float* __restrict__ part_max,
                                                          const float* __restrict__ part_sum,
                                                          const float* __restrict__ part_target,
                                                          int64_t n_shards, int64_t stride,
                                                          int64_t N, float* __restrict__ loss,
                                                          float* __restrict__ lse) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= N) return;
  float M = -INFINITY;
  for (int64_t k = 0; k < n_shards; ++k)
    if (part_sum[k * stride + r] > 0.f) M = fmaxf(M, part_max[k * stride + r]);
  if (M == -INFINITY) {
    loss[r] = 0.f;
    lse[r] = 0.f;
    return;
  }
  float S = 0.f, zt = -INFINITY;
  for (int64_t k = 0; k < n_shards; ++k) {
    const int64_t o = k * stride + r;
    S += part_sum[o] * fast_exp2((part_max[o] - M) * kLog2e);
    zt = fmaxf(zt, part_target[o]);
  }
  const float l = M + fast_log2(S) * kLn2;
  lse[r] = l;
  loss[r] = l - zt;
}

hipError_t launch_shard_merge(const float* part_max, const float* part_sum, const float* part_target,
                              int64_t n_shards, int64_t stride, int64_t N, float* loss, float* lse,
                              hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const int grid = (int)((N + 255) / 256);
  hipLaunchKernelGGL(shard_merge_kernel, dim3(grid), dim3(256), 0, s, part_max, part_sum,
                     part_target, n_shards, stride, N, loss, lse);
  return hipGetLastError();
}

// ------------------------------------------------------- loss reduction
//
// Sum of per-token losses over valid rows in a fixed order (strided fp64
// per-thread sums, then a fixed binary tree in LDS), so the result is
// bitwise reproducible.  Writes the sum and the mean over valid rows (NaN
// when no row is valid, as PyTorch's mean cross-entropy does).
__global__ __launch_bounds__(1024) void loss_reduce_kernel(const float* __restrict__ loss_c,
                                                           const int32_t* __restrict__ gather,
                                                           const int32_t* __restrict__ valid_count,
                                                           double* __restrict__ loss_sum,
                                                           float* __restrict__ loss_mean) {
  __shared__ double part[1024];
  const int tid = threadIdx.x;
  const int count = *valid_count;
  double acc = 0.0;
  for (int i = tid; i < count; i += 1024) acc += (double)loss_c[gather ? gather[i] : i];
  part[tid] = acc;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    *loss_sum = part[0];
    if (loss_mean) *loss_mean = count > 0 ? (float)(part[0] / (double)count) : __builtin_nanf("");
  }
}

hipError_t launch_loss_reduce(const float* loss, const int32_t* gather, const int32_t* valid_count,
                              double* loss_sum, float* loss_mean, hipStream_t s) {
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(1024), 0, s, loss, gather, valid_count,
                     loss_sum, loss_mean);
  return hipGetLastError();
}

}  // namespace lce
