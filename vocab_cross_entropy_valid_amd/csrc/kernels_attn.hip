// Attention forward through an online softmax: O = softmax(scale Q K^T) V
// with an optional causal mask, and the per-row logsumexp, without storing
// the [B, H, S, S] score matrix ("OjasX 0.6.1", section 核心技术 / "Core
// Technology": zero-byte attention score matrix; the same page's Online
// Softmax paragraph gives the running max / normaliser recurrence used
// here; softmax(Q K^T / sqrt(d_k)) V as the KV-cache page, section
// KV Cache基础, writes the operation).
//
// Work decomposition: a workgroup of 8 waves (D = 128; 4 waves for D = 64)
// takes 256 (128) queries of one (batch, head), 32 per wave, and streams the
// keys in blocks of 64.
//
//  * Scores are computed transposed, S^T = K Q^T (A = K rows, B = Q rows),
//    on v_mfma_f32_32x32x16_bf16: lane l owns query l % 32 and, for key
//    block half mt, keys 32 mt + 8 (i / 4) + 4 (l / 32) + i % 4 (i = 0..15).
//    The running max and sum of a query then stay in its lane, plus one
//    exchange with lane l ^ 32.
//  * The output is accumulated transposed too, O^T += V^T P^T, so that lane l
//    again owns query l % 32 and the rescale by exp(m_old - m_new) needs no
//    data from other lanes.  The probabilities go straight from the score
//    registers into the B operand: the 8 values lane (q, h) feeds to one
//    MFMA are keys 4h + {0..3, 8..11} of a 16-key slice, and V^T is laid out
//    in LDS so that the A operand reads exactly those keys in that order as
//    one 16-byte chunk (a product over K does not care in which order K is
//    enumerated, as long as A and B agree).
//  * Q stays in registers for the whole key loop (B operand of S^T).  K and
//    V of the next key block are loaded into registers while the current
//    block computes, then written to LDS: K row-major with 16-byte chunks
//    XOR-swizzled by the row, V transposed into [dim][key] rows of 128 bytes
//    with 16-byte chunks XOR-swizzled by (dim / 2) % 8, so that the fragment
//    reads of consecutive rows hit distinct banks.
//  * Scores past the sequence end, and for a causal mask past the query, are
//    -inf before the max; a key block that lies wholly after a wave's
//    queries is skipped by that wave.  exp2 with the scale folded into
//    log2(e) scale.
//  * The softmax is what bounds this kernel (VALU work per score next to
//    1/64 of an MFMA), so it is kept lean: probabilities are packed to bf16
//    by the hardware conversion, and the reference max of a query moves only
//    when a block exceeds it by more than 2^8 (the probabilities then stay
//    <= 256, harmless in bf16 and fp32), so the 64 output accumulators are
//    rescaled only in the rare blocks where some lane of the wave moved.
//    The result does not depend on the reference (it cancels in O / sum and
//    is added back to the logsumexp).
//  * K / V tiles are double buffered in LDS: one barrier per key block.
#include "device_common.h"
#include "kernels.h"

namespace lce {

namespace {

constexpr int kQBlock = 128;  // queries per workgroup of the dQ pass
constexpr int kKBlock = 64;   // keys per block

template <int D>
struct AttnLds {
  static constexpr int kChunks = D / 8;             // 16-byte chunks per K row
  static constexpr int kKBytes = kKBlock * D * 2;   // K block
  static constexpr int kVBytes = D * kKBlock * 2;   // V^T block: D rows of 128 B
  static constexpr int kBuf = kKBytes + kVBytes;     // one key block
  static constexpr int kBytes = 2 * kBuf;            // double buffered
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two fp32 values -> packed bf16 (round to nearest even): one vector
// conversion, so that the backend emits a single v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

constexpr float kRescaleSlack = 8.f;  // log2 units

__device__ __forceinline__ int k_offset(int row, int chunk, int chunks) {
  return row * chunks * 16 + ((chunk ^ (row & (chunks - 1))) << 4);
}

// Workgroup -> (block b of the sequence, head bh) for a grid of nblk x BH
// workgroups, b = 0 the heaviest block of a head.  Workgroups go to the 8
// XCDs round-robin (blockIdx % 8), so here the blocks of G heads run back to
// back on one XCD, heaviest first across the G heads (all G heads' block 0,
// then their block 1, ...): the rows those workgroups all read (K / V, or
// Q / dO) are fetched into that XCD's L2 once (A/B on one box: the attention
// step 1.69 -> 1.62 ms against head-minor order, with G = 1), and the mix of
// block lengths in flight evens out the end of the launch (G = 4 against
// G = 1: forward 393 -> 375 us, dQ 524 -> 505, dK / dV 690 -> 649; G = 16 or
// 32 lose the L2 sharing: dK / dV 680, 716; the forward takes G = 8: 375 ->
// 370 us).  G shrinks to the largest power
// of two dividing BH / 8; head-minor order when BH is not a multiple of 8.
template <int G>
__device__ __forceinline__ void xcd_head_block(int nblk, int64_t BH, int& b, int64_t& bh) {
  if (BH % 8 == 0) {
    int g = G;
    while ((BH / 8) % g != 0) g >>= 1;
    const int64_t slot = blockIdx.x >> 3;
    const int64_t grp = slot / (g * nblk);
    const int r = (int)(slot % (g * nblk));
    b = r / g;
    bh = (grp * g + r % g) * 8 + (blockIdx.x & 7);
  } else {
    b = (int)(blockIdx.x / BH);
    bh = blockIdx.x % BH;
  }
}

// V^T row dv holds the block's 64 keys as 16 units of 4 keys.  One MFMA
// A fragment needs units u0 and u0 + 2 (u0 = 8 mt + 4 g + h: keys 4 u0 + {0..3}
// and 4 u0 + {8..11}), so each such pair is one 16-byte chunk, numbered
// c = (u0 >> 1) | (u0 & 1), and the chunks are XOR-swizzled by (dv / 2) % 8:
// the fragment read is one ds_read_b128 and each 16 lanes of it (rows of one
// parity, 8 distinct chunks) hit distinct banks.
__device__ __forceinline__ int vt_chunk_offset(int dv, int c) {
  return dv * (kKBlock * 2) + ((c ^ ((dv >> 1) & 7)) << 4);
}

// byte offset of unit u of row dv
__device__ __forceinline__ int vt_unit_offset(int dv, int u) {
  const int u0 = u & ~2;  // first unit of its pair
  return vt_chunk_offset(dv, (u0 >> 1) | (u0 & 1)) + ((u >> 1) & 1) * 8;
}

template <int D, int NT>
struct BlockRegs {
  static constexpr int kKLoads = kKBlock * D / 8 / NT;              // 16-B K loads
  static constexpr int kVUnits = (D / 8) * (kKBlock / 4);                     // (dv group, key group)
  static constexpr int kVIters = (kVUnits + NT - 1) / NT;
  u32x4 k[kKLoads];
  u32x4 v[kVIters][4];
};

// Global -> registers for key block kb: buffer loads over the head's K and V
// rows (rk, rv: S rows), so rows past S read as zeros and no load waits on a
// branch.
template <int D, int NT>
__device__ __forceinline__ void load_block(BlockRegs<D, NT>& r, const __amdgpu_buffer_rsrc_t& rk,
                                           const __amdgpu_buffer_rsrc_t& rv, int kb, int tid) {
  constexpr int C = AttnLds<D>::kChunks;
  const uint32_t soff = (uint32_t)(kb * kKBlock) * (uint32_t)(D * 2);
#pragma unroll
  for (int j = 0; j < BlockRegs<D, NT>::kKLoads; ++j) {
    const int idx = j * NT + tid;
    const uint32_t off = (uint32_t)((idx / C) * D + 8 * (idx % C)) * 2u;
    r.k[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, soff, 0));
  }
#pragma unroll
  for (int it = 0; it < BlockRegs<D, NT>::kVIters; ++it) {
    const int unit = it * NT + tid;
    const int kg = unit & 15;  // keys 4 kg .. 4 kg + 3
    const int dg = unit >> 4;  // dims 8 dg .. 8 dg + 7
    if (unit < BlockRegs<D, NT>::kVUnits) {  // wave-uniform
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t off = (uint32_t)((4 * kg + q) * D + 8 * dg) * 2u;
        r.v[it][q] =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, soff, 0));
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) r.v[it][q] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Registers -> LDS: K as is (swizzled), V transposed into 4-key units.
template <int D, int NT>
__device__ __forceinline__ void store_block(const BlockRegs<D, NT>& r, char* lds, int tid) {
  constexpr int C = AttnLds<D>::kChunks;
#pragma unroll
  for (int j = 0; j < BlockRegs<D, NT>::kKLoads; ++j) {
    const int idx = j * NT + tid;
    *(u32x4*)(lds + k_offset(idx / C, idx % C, C)) = r.k[j];
  }
  char* vt = lds + AttnLds<D>::kKBytes;
#pragma unroll
  for (int it = 0; it < BlockRegs<D, NT>::kVIters; ++it) {
    const int unit = it * NT + tid;
    if (unit >= BlockRegs<D, NT>::kVUnits) continue;
    const int kg = unit & 15;
    const int dg = unit >> 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // element e (dim 8 dg + e) of the 4 key rows, two keys per word:
      // v_perm_b32 picks the low (even e) or high (odd e) halves of word
      // e / 2 of two rows (bytes 0-3 come from the second operand)
      const int w = e >> 1;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x2 u;
      u[0] = __builtin_amdgcn_perm(r.v[it][1][w], r.v[it][0][w], sel);
      u[1] = __builtin_amdgcn_perm(r.v[it][3][w], r.v[it][2][w], sel);
      *(u32x2*)(vt + vt_unit_offset(8 * dg + e, kg)) = u;
    }
  }
}

}  // namespace

template <int D, int NT>
__global__ __launch_bounds__(NT, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int QB = NT / 2;  // queries per workgroup: 32 per wave
  __shared__ __attribute__((aligned(16))) char lds[AttnLds<D>::kBytes];
  constexpr int C = AttnLds<D>::kChunks;
  constexpr int KS = D / 16;  // MFMA k-steps of the score product
  constexpr int MD = D / 32;  // 32-row blocks of O^T
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform in a scalar register, so that conditions on the wave's
  // queries (masking, skipping) become scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31;
  const int h = lane >> 5;
  const int S = a.S;
  const int nqb = (S + QB - 1) / QB;
  // heaviest (last) query blocks of every head first
  int qb;
  int64_t bh;
  xcd_head_block<8>(nqb, a.BH, qb, bh);
  qb = nqb - 1 - qb;
  const int64_t head = bh * (int64_t)S * D;
  const bf16_t* Qh = a.Q + head;
  const bf16_t* Kh = a.K + head;
  const bf16_t* Vh = a.V + head;

  const int q0 = qb * QB + 32 * wave;  // first query of this wave
  const int q = q0 + j;                     // this lane's query
  const int qc = q < S ? q : S - 1;
  u32x4 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s] = *(const u32x4*)(Qh + (int64_t)qc * D + 16 * s + 8 * h);

  const int kend = a.causal ? min(S, (qb + 1) * QB) : S;
  const int nkb = (kend + kKBlock - 1) / kKBlock;

  f32x16 o[MD];
#pragma unroll
  for (int m = 0; m < MD; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[m][i] = 0.f;
  float mrun = -INFINITY;  // running max, log2 units
  float lrun = 0.f;        // this lane's part of the running sum
  const float c = a.scale_log2;

  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)Kh, (int64_t)S * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char*)Vh, (int64_t)S * D * 2);
  BlockRegs<D, NT> r;
  load_block<D, NT>(r, rk, rv, 0, tid);
  store_block<D, NT>(r, lds, tid);
  __syncthreads();
  if (nkb > 1) load_block<D, NT>(r, rk, rv, 1, tid);
  for (int kb = 0; kb < nkb; ++kb) {
    const char* buf = lds + (kb & 1) * AttnLds<D>::kBuf;
    const int k0 = kb * kKBlock;
    // a block wholly after this wave's queries contributes nothing
    if (!(a.causal && k0 > q0 + 31)) {
      // S^T = K Q^T for the 64 keys of the block
      f32x16 sc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[mt][i] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const u32x4 af = *(const u32x4*)(buf + k_offset(32 * mt + j, 2 * s + h, C));
          Mma<bf16_t>::run(sc[mt], af, qf[s]);
        }
      }
      // the first 4 fragment reads go out together, then one read after each
      // MFMA (the compiler's order waits on each read right in front of its
      // MFMA)
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int q = 0; q < 2 * KS - 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_barrier(0);

      // mask: keys past the end, and past the query under a causal mask
      const bool tail = k0 + kKBlock > S;
      const bool diag = a.causal && k0 + kKBlock - 1 > q0;
      if (tail || diag) {
        const int lim = a.causal ? min(q, S - 1) : S - 1;  // last allowed key
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
            if (key > lim) sc[mt][i] = -INFINITY;
          }
      }

      // online softmax update (log2 domain, scale folded in); the reference
      // max moves only when the block exceeds it by more than the slack
      float bmax = sc[0][0];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) bmax = fmaxf(bmax, sc[mt][i]);
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32)) * c;
      const bool up = bmax > mrun + kRescaleSlack;  // also the first finite block
      float alpha = 1.f;
      if (up) {
        alpha = fast_exp2(mrun - bmax);  // 0 while mrun = -inf
        mrun = bmax;
      }
      // mrun = -inf only while every key so far is masked for this query
      // (never for a valid query: key 0 is always allowed); keep p = 0 then
      const float mref = mrun == -INFINITY ? 0.f : mrun;
      float psum = 0.f;
      const bf16x2_t kOnes = {(__bf16)1.f, (__bf16)1.f};
      u32x4 pf[2][2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float p0 = fast_exp2(fmaf(sc[mt][8 * g + 2 * w], c, -mref));
            const float p1 = fast_exp2(fmaf(sc[mt][8 * g + 2 * w + 1], c, -mref));
            const uint32_t pk = cvt_pk_bf16(p0, p1);
            // the normaliser sums the rounded values the MFMA multiplies:
            // one packed dot product with (1, 1)
            psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), kOnes, psum,
                                                   false);
            pf[mt][g][w] = pk;
          }
      lrun = lrun * alpha + psum;
      if (__ballot(up)) {
        // keeps the compiler from hoisting the 64 multiplies out of the
        // branch (alpha = 1 on lanes that did not move makes that legal)
        asm volatile("");
#pragma unroll
        for (int m = 0; m < MD; ++m)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[m][i] *= alpha;
      }

      // O^T += V^T P^T
      const char* vt = buf + AttnLds<D>::kKBytes;
#pragma unroll
      for (int m = 0; m < MD; ++m) {
        const int dv = 32 * m + j;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            // units u0 = 8 mt + 4 g + h and u0 + 2: chunk 4 mt + 2 g + h
            const u32x4 af = *(const u32x4*)(vt + vt_chunk_offset(dv, 4 * mt + 2 * g + h));
            Mma<bf16_t>::run(o[m], af, pf[mt][g]);
          }
      }
    }
    // next block into the other buffer (last read in block kb - 1, which
    // every wave finished before the previous barrier)
    if (kb + 1 < nkb) store_block<D, NT>(r, lds + ((kb + 1) & 1) * AttnLds<D>::kBuf, tid);
    __syncthreads();
    if (kb + 2 < nkb) load_block<D, NT>(r, rk, rv, kb + 2, tid);
  }

  const float ltot = lrun + __shfl_xor(lrun, 32);
  if (q >= S) return;
  const float inv = 1.f / ltot;
  float* Oq = a.O + head + (int64_t)q * D;
#pragma unroll
  for (int m = 0; m < MD; ++m)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 v = {o[m][4 * r4] * inv, o[m][4 * r4 + 1] * inv, o[m][4 * r4 + 2] * inv,
                 o[m][4 * r4 + 3] * inv};
      *(f32x4*)(Oq + 32 * m + 8 * r4 + 4 * h) = v;
    }
  if (h == 0) a.lse[bh * S + q] = (mrun + fast_log2(ltot)) * kLn2;
}

hipError_t launch_attn_fwd(const AttnArgs& a, int D, hipStream_t s) {
  if (a.S <= 0 || a.BH <= 0) return hipSuccess;
  // D = 128: 8 waves (256 queries) per workgroup, so that the staging of each
  // key block serves twice the queries (A/B on one box: 371 -> 358 us); D = 64:
  // 4 waves (8 waves measured 0.425 -> 0.465 ms)
  if (D == 128) {
    constexpr int NT = 512;
    const dim3 grid((unsigned)((a.S + NT / 2 - 1) / (NT / 2) * a.BH));
    hipLaunchKernelGGL((attn_fwd_kernel<128, NT>), grid, dim3(NT), 0, s, a);
  } else {
    constexpr int NT = 256;
    const dim3 grid((unsigned)((a.S + NT / 2 - 1) / (NT / 2) * a.BH));
    hipLaunchKernelGGL((attn_fwd_kernel<64, NT>), grid, dim3(NT), 0, s, a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ backward
//
// dV = P^T dO, dP = dO V^T, dS = P (dP - D), D = rowsum(dO O),
// dQ = scale dS K, dK = scale dS^T Q, with P = exp(scale Q K^T - lse)
// recomputed tile by tile from the forward's logsumexp: the [S, S]
// probabilities are never stored in the backward pass either.  Two passes,
// no atomics (results are deterministic):
//
//  * dQ pass (attn_bwd_dq16_kernel<D>): a workgroup of 8 waves takes 128
//    queries, 16 per wave, and streams the keys in blocks of 64: S^T = K Q^T
//    and dP^T = V dO^T on the 16 x 16 x 32 product (Q and dO fragments stay
//    in registers), dS formed in the lane, dQ += dS K.  It also writes D.
//  * dK / dV pass (attn_bwd_dkv_pair_kernel<4, D>): a workgroup of 8 waves
//    takes 128 keys as 4 pairs of 32 and streams the queries in blocks of 64:
//    per pair one wave computes S, P and dV^T += dO^T P^T, the other dP, dS
//    and dK^T += Q^T dS^T.
//
// Both read their transposed operands straight from row-major tiles
// (transposing LDS reads) and stage the streamed tiles through registers
// with buffer loads; two waves per SIMD for D = 128, four for D = 64.

namespace {

// rows [row0, row0 + R) of two [S, D] bf16 heads (K and V) into row-major
// swizzled tiles.  Buffer loads read rows past S as zeros, and every load is
// issued before the first LDS write, so the staging costs one memory round
// trip (loads issued before the call, e.g. the first query block, complete
// in the same wait).
template <int D, int R, int NT>
__device__ __forceinline__ void stage_rows2(char* dst0, const bf16_t* src0, char* dst1,
                                            const bf16_t* src1, int row0, int S, int tid) {
  constexpr int C = D / 8;
  constexpr int kIt = R * C / NT;
  static_assert(R * C % NT == 0, "whole 16-byte chunks per thread");
  const int64_t bytes = row0 < S ? (int64_t)(S - row0) * D * 2 : 0;
  const __amdgpu_buffer_rsrc_t r0 = make_rsrc((const char*)(src0 + (int64_t)row0 * D), bytes);
  const __amdgpu_buffer_rsrc_t r1 = make_rsrc((const char*)(src1 + (int64_t)row0 * D), bytes);
  u32x4 v0[kIt], v1[kIt];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const uint32_t off = (uint32_t)(it * NT + tid) * 16u;  // row idx / C, chunk idx % C
    v0[it] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r0, off, 0, 0));
    v1[it] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r1, off, 0, 0));
  }
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int idx = it * NT + tid;
    const int o = k_offset(idx / C, idx % C, C);
    *(u32x4*)(dst0 + o) = v0[it];
    *(u32x4*)(dst1 + o) = v1[it];
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace

// Shared by the backward passes: 8 waves on v_mfma_f32_16x16x32_bf16.  Operand layouts of the 16 x 16 x 32 product: A
// lane l holds row l % 16 with K entries 8 (l / 16) .. + 7, B lane l column
// l % 16 with the same K entries, the result lane l column l % 16 with rows
// 4 (l / 16) .. + 3.
namespace {
constexpr int k16Threads = 512;

__device__ __forceinline__ void mma16(f32x4& c, const u32x4& a, const u32x4& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                              __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Row-major tiles of the 16 x 16 x 32 passes (rows of D bf16 entries, D / 8
// sixteen-byte chunks): chunk c of row r sits at position c ^ swz(r), with
// swz(r) = 2 (r % 8) for 256-byte rows (D = 128) and r & 6 for 128-byte rows
// (D = 64).  The S / dP fragment reads (16 lanes: one chunk of 16
// consecutive rows; lane groups 16 g read chunk 4 s + g) and the transposing
// reads (32 lanes: chunks 2 m, 2 m + 1 of 8 consecutive rows) then run at
// the LDS rate of conflict-free reads on gfx950 (16-byte reads 4 clocks per
// wave, transposing reads 175-181 bytes per clock per CU, measured).  Any
// term that flips bit 0 of the position (e.g. adding (r / 8) % 2 for
// D = 128, which separates rows r and r + 8 but pairs the chunk of lane
// group g with that of group g ^ 1 in rows r ^ 8) halves the rate of the
// 16-byte reads.
template <int D>
__device__ __forceinline__ int swz_offset(int row, int chunk) {
  static_assert(D == 64 || D == 128, "D = 64 or 128");
  if constexpr (D == 128)
    return row * 256 + ((chunk ^ ((row & 7) << 1)) << 4);
  else
    return row * 128 + ((chunk ^ (row & 6)) << 4);
}

// A fragment of the transposed tile for the 16 x 16 x 32 product: operand row
// = tile column 16 m + lane % 16, K entries = tile rows 4 (lane / 16) + {0..3}
// and 16 + the same, from two ds_read_b64_tr_b16 at per-lane offset off (and
// off + 16 rows).  Within a group of 16 lanes, lane i receives as element e
// the element i % 4 of the 8 bytes that lane 4 e + i / 4 addressed; so lane L
// of group G addresses row 4 G + L / 4, columns 16 m + 4 (L % 4) .. + 3.
template <int D>
__device__ __forceinline__ u32x4 tr_frag16(const char* p) {
  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)LCE_LDS_PTR(p));
  const i16x4_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)LCE_LDS_PTR(p + 16 * 2 * D));
  const u32x2 x = __builtin_bit_cast(u32x2, lo);
  const u32x2 y = __builtin_bit_cast(u32x2, hi);
  u32x4 r = {x[0], x[1], y[0], y[1]};
  return r;
}
}  // namespace

// dK / dV pass (D = 64 or 128), split by gradient: a workgroup of 8 waves takes
// 128 keys as 4 pairs of 32 and streams the queries in blocks of 64 through
// two LDS slots (Q rows, dO rows in the swizzle of swz_offset, lse, D).
// Of the two waves of a pair, which share a SIMD (waves w and w + 4), the P
// wave computes S = Q K^T, the softmax P and dV^T += dO^T P^T, the dS wave
// dP = dO V^T, dS = P (dP - D) and dK^T += Q^T dS^T.  Against one wave per
// 16 keys doing all four products, every Q / dO fragment read from LDS
// feeds two MFMAs (the pair's two 16-key tiles) instead of one, and a
// SIMD's vector work (the exponentials in the first half of an iteration,
// dS in the second) sits next to the other wave's MFMAs.
//  * S and dP per key tile t and 16-query quarter h of the block: lane l
//    (g = l / 16) holds key 16 t + l % 16 and queries 16 h + 4 g + e
//    (e = 0..3); the K (or V) rows of the pair stay in registers as the B
//    operands.
//  * P goes from the P wave to the dS wave through LDS, rounded to bf16 as
//    the dV product takes it, in the lane / register order both waves
//    share; a second barrier in each iteration separates its writes from
//    the reads.  (Sending fp32 P, with dP - D formed while the P wave
//    exponentiates, measured 2-4% slower.)
//  * dV^T += dO^T P^T and dK^T += Q^T dS^T over K = 32 queries at a time:
//    the B operand is P (dS) of the lane's 8 queries of that half in the
//    order above, the A operand the matching dO^T (Q^T) entries, read
//    straight from the row-major tile with two transposing reads (queries
//    4 g .. 4 g + 3 and 16 + 4 g .. + 3 of the half); each such fragment
//    feeds both key tiles.
//  * Query blocks are loaded into registers (buffer loads: rows past S read
//    as zeros, and so add nothing) an iteration ahead and written to LDS at
//    the start of the iteration before their use, into the other slot, so
//    that the writes overlap that iteration's products.  The prologue is
//    one memory round trip: the first block's loads go out beside the K / V
//    staging loads.
//  * The causal blocks that overlap the workgroup's keys (the first two)
//    take the masked path, with the mask applied to S only (dS = P (dP - D)
//    is then 0); the main loop carries no mask.
//  * NP pairs per workgroup (32 NP keys).  NP = 4 is launched: NP = 2 (two
//    workgroups per CU, each staging every query block for its 64 keys) ran
//    15% slower.
// Launch bounds: D = 128 needs up to 256 VGPRs (two waves per SIMD, one
// workgroup per CU); D = 64 is held to 128 (four waves per SIMD: two
// workgroups per CU, 8% faster than one despite a few spilled registers).
template <int NP, int D>
__global__ __launch_bounds__(128 * NP, D == 64 ? 4 : 4 / NP) void attn_bwd_dkv_pair_kernel(AttnBwdArgs a) {
  constexpr int QB = 64;                  // queries per block
  constexpr int C = D / 8;                // 16-byte chunks per row
  constexpr int RB = 2 * D;               // bytes per row
  constexpr int KS = D / 32;              // K steps of the S / dP products
  constexpr int NT = 128 * NP;            // threads
  constexpr int KK = 32 * NP;             // keys of the workgroup
  constexpr int kKV = KK * D * 2;         // K (or V) rows of the workgroup
  constexpr int kQT = QB * D * 2;         // one block's Q (or dO) tile
  constexpr int kSlot = 2 * kQT + 512;    // Q, dO, lse[64], D[64]
  constexpr int kXch = NP * 4 * 64 * 16;  // P of the pairs: 4 fragments x 64 lanes x 16 B
  constexpr int kLds = 2 * kKV > 2 * kSlot + kXch ? 2 * kKV : 2 * kSlot + kXch;
  constexpr int kRows = NT / C;           // tile rows staged per pass
  constexpr int kPre = QB / kRows;        // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(1024))) char lds[kLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave % NP;
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const int S = a.S;
  int kblk;
  int64_t bh;
  xcd_head_block<4>((S + KK - 1) / KK, a.BH, kblk, bh);
  const int64_t head = bh * (int64_t)S * D;
  const int kbase = kblk * KK;
  const int k0p = kbase + 32 * pair;  // first key of this pair
  const float c = a.scale_log2;
  char* xch = lds + 2 * kSlot + pair * 4096 + lane * 16;  // this lane's P fragments

  const int nq = (S + QB - 1) / QB;
  const int qstart = a.causal ? kbase / QB : 0;
  // register-staged loads: thread t carries chunk t % C of rows t / C +
  // kRows i of the Q and the dO tile, stored at position t % C of its row,
  // i.e. chunk (t % C) ^ swz(row) of the source row; even waves
  // carry the block's lse values (times log2 e), odd waves its D values (the
  // waves of a parity write identical values)
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)(a.Q + head), (int64_t)S * D * 2);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc((const char*)(a.dO + head), (int64_t)S * D * 2);
  const __amdgpu_buffer_rsrc_t rv = (wave & 1)
      ? make_rsrc((const char*)(a.delta + bh * S), (int64_t)S * 4)
      : make_rsrc((const char*)(a.lse + bh * S), (int64_t)S * 4);
  const int srow = tid / C;
  const uint32_t gvoff = (uint32_t)swz_offset<D>(srow, tid % C);
  const int lvoff = srow * RB + ((tid % C) << 4);
  typedef u32x4 BlockRegs16[2 * kPre];
  BlockRegs16 pre;
  float pre_v;
  auto slot_of = [&](int qbk) { return lds + ((qbk - qstart) & 1) * kSlot; };
  auto load_into = [&](BlockRegs16& r, float& rv_, int qbk) {
    const uint32_t soff = (uint32_t)(qbk * QB) * (uint32_t)RB;
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      r[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, gvoff + RB * kRows * i, soff, 0));
      r[kPre + i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rdo, gvoff + RB * kRows * i, soff, 0));
    }
    rv_ = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                       rv, lane * 4, (uint32_t)(qbk * QB) * 4u, 0));
  };
  auto store_from = [&](const BlockRegs16& r, float rv_, int qbk) {
    char* sl = slot_of(qbk);
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      *(u32x4*)(sl + lvoff + RB * kRows * i) = r[i];
      *(u32x4*)(sl + kQT + lvoff + RB * kRows * i) = r[kPre + i];
    }
    // lse in log2 units (one multiply here instead of one per score)
    *(float*)(sl + 2 * kQT + (wave & 1) * 256 + lane * 4) = (wave & 1) ? rv_ : rv_ * kLog2e;
  };
  auto load_regs = [&](int qbk) { load_into(pre, pre_v, qbk); };
  auto store_regs = [&](int qbk) { store_from(pre, pre_v, qbk); };

  // per-lane LDS offsets: S / dP fragments (row i16 of a 16-query quarter,
  // chunk 4 s + g) and the transposing reads of the accumulation
  int aoff[KS], toff[D / 16];
#pragma unroll
  for (int s = 0; s < KS; ++s) aoff[s] = swz_offset<D>(i16, 4 * s + g);
#pragma unroll
  for (int m = 0; m < D / 16; ++m) {
    const int row = 4 * g + (i16 >> 2);
    const int dim = 16 * m + 4 * (lane & 3);
    toff[m] = swz_offset<D>(row, dim >> 3) + (dim & 7) * 2;
  }

  // The two roles take separate code paths, each with its own registers.
  auto run = [&](auto role) {
    constexpr bool kP = decltype(role)::value;
    // K (P wave) or V (dS wave) fragments of the pair's two 16-key tiles:
    // B operands of S and dP for the whole pass
    u32x4 bf[2][KS];
    f32x4 acc[2][D / 16];  // dV^T (P wave) or dK^T (dS wave) per key tile
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int m = 0; m < D / 16; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][m][e] = 0.f;

    // prologue in one memory round trip: the loads of query blocks qstart
    // (into a prologue register set) and qstart + 1 (into the loop's) go out
    // first, then the K / V rows are staged (their wait covers all of them);
    // block qstart then takes its slot (which reuses the K / V staging LDS),
    // and block qstart + 1 waits in registers for the first iteration
    {
      BlockRegs16 pre0;
      float pre0_v;
      load_into(pre0, pre0_v, qstart);
      if (qstart + 1 < nq) load_regs(qstart + 1);
      char* lk = lds;
      char* lv = lds + kKV;
      stage_rows2<D, KK, NT>(lk, a.K + head, lv, a.V + head, kbase, S, tid);
      __syncthreads();
      const char* lb = kP ? lk : lv;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s = 0; s < KS; ++s)
          bf[t][s] = *(const u32x4*)(lb + k_offset(32 * pair + 16 * t + i16, 4 * s + g, D / 8));
      __syncthreads();
      store_from(pre0, pre0_v, qstart);
      __syncthreads();
    }

    // one block: products, then (after the middle barrier) the accumulation
    auto block = [&](int qbk, const bool masked, const bool live) {
      const char* sl = slot_of(qbk);
      f32x4 sc[2][4];  // S (P wave) or dP (dS wave): key tile x 16-query quarter
      u32x4 pp[2][2];  // P (bf16) per key tile and 32-query half, B operand order
      if (live) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[t][h][e] = 0.f;
        const char* op = sl + (kP ? 0 : kQT);  // Q or dO tile
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const u32x4 af = *(const u32x4*)(op + aoff[s] + 16 * RB * h);
            mma16(sc[0][h], af, bf[0][s]);
            mma16(sc[1][h], af, bf[1][s]);
          }
        // the first fragment reads (6 of 16, 4 of 8) go out together, then
        // one read after every two MFMAs (the compiler's order waits on each
        // read right in front of its MFMAs)
        constexpr int kAhead = KS == 4 ? 6 : 4;
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int q = 0; q < 4 * KS - kAhead; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * kAhead, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (kP) {
          const float* lv = (const float*)(sl + 2 * kQT);
          f32x4 l4[4];
#pragma unroll
          for (int h = 0; h < 4; ++h) l4[h] = *(const f32x4*)(lv + 16 * h + 4 * g);
          if (masked) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int h = 0; h < 4; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  sc[t][h][e] = (qbk * QB + 16 * h + 4 * g + e < k0p + 16 * t + i16) ? -INFINITY
                                                                                      : sc[t][h][e];
          }
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
              float pv[2][4];
#pragma unroll
              for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  pv[hh][e] = fast_exp2(fmaf(sc[t][2 * n + hh][e], c, -l4[2 * n + hh][e]));
              pp[t][n][0] = cvt_pk_bf16(pv[0][0], pv[0][1]);
              pp[t][n][1] = cvt_pk_bf16(pv[0][2], pv[0][3]);
              pp[t][n][2] = cvt_pk_bf16(pv[1][0], pv[1][1]);
              pp[t][n][3] = cvt_pk_bf16(pv[1][2], pv[1][3]);
              *(u32x4*)(xch + (2 * t + n) * 1024) = pp[t][n];
            }
        }
      }
      __syncthreads();  // P written
      if (live) {
        if (!kP) {
          // dS = P (dP - D), P as the P wave rounded it for dV
          const float* dv4 = (const float*)(sl + 2 * kQT + 256);
          f32x4 d4[4];
#pragma unroll
          for (int h = 0; h < 4; ++h) d4[h] = *(const f32x4*)(dv4 + 16 * h + 4 * g);
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
              const u32x4 pw = *(const u32x4*)(xch + (2 * t + n) * 1024);
              float dsv[2][4];
#pragma unroll
              for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                  const uint32_t w = pw[2 * hh + e];
                  dsv[hh][2 * e] = bf16_lo(w) * (sc[t][2 * n + hh][2 * e] - d4[2 * n + hh][2 * e]);
                  dsv[hh][2 * e + 1] =
                      bf16_hi(w) * (sc[t][2 * n + hh][2 * e + 1] - d4[2 * n + hh][2 * e + 1]);
                }
              pp[t][n][0] = cvt_pk_bf16(dsv[0][0], dsv[0][1]);
              pp[t][n][1] = cvt_pk_bf16(dsv[0][2], dsv[0][3]);
              pp[t][n][2] = cvt_pk_bf16(dsv[1][0], dsv[1][1]);
              pp[t][n][3] = cvt_pk_bf16(dsv[1][2], dsv[1][3]);
            }
        }
        // dV^T += dO^T P^T (P wave) or dK^T += Q^T dS^T (dS wave), K = 32
        // queries per half; each transposed fragment feeds both key tiles
        const char* tp = sl + (kP ? kQT : 0);
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int m = 0; m < D / 16; ++m) {
            const u32x4 tf = tr_frag16<D>(tp + 32 * RB * n + toff[m]);
            mma16(acc[0][m], tf, pp[0][n]);
            mma16(acc[1][m], tf, pp[1][n]);
          }
      }
    };

    // iteration qbk: block qbk + 1 written to the other slot, block qbk + 2
    // loaded, block qbk computed.  kDiag: a causal block that overlaps the
    // workgroup's keys, skipped by the pairs whose keys all come after its
    // queries and masked for the others
    auto iter = [&](int qbk, auto diag) {
      constexpr bool kDiag = decltype(diag)::value;
      if (qbk + 1 < nq) store_regs(qbk + 1);
      if (qbk + 2 < nq) load_regs(qbk + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (kDiag)
        block(qbk, qbk * QB < k0p + 32, qbk * QB + QB - 1 >= k0p);
      else
        block(qbk, false, true);
      __syncthreads();
    };
    int qbk = qstart;
    if (a.causal) {
      const int qd = min(qstart + (KK + QB - 1) / QB, nq);
      for (; qbk < qd; ++qbk) iter(qbk, std::integral_constant<bool, true>{});
    }
    for (; qbk < nq; ++qbk) iter(qbk, std::integral_constant<bool, false>{});

    float* out = kP ? a.dV : a.dK;
    const float sc_out = kP ? 1.f : a.scale;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int kk = k0p + 16 * t + i16;
      if (kk < S) {
        float* row = out + head + (int64_t)kk * D;
#pragma unroll
        for (int m = 0; m < D / 16; ++m) {
          f32x4 v = {acc[t][m][0] * sc_out, acc[t][m][1] * sc_out, acc[t][m][2] * sc_out,
                     acc[t][m][3] * sc_out};
          *(f32x4*)(row + 16 * m + 4 * g) = v;
        }
      }
    }
  };
  if (wave < NP)
    run(std::integral_constant<bool, true>{});
  else
    run(std::integral_constant<bool, false>{});
}

// dQ pass (D = 64 or 128) on the 16 x 16 x 32 product, two waves per SIMD
// (four for D = 64): a workgroup of 8 waves takes 128 queries, 16 per wave,
// and streams the keys in blocks of 64 through two LDS slots (K rows, V
// rows, in the swizzle of swz_offset).
//  * S^T = K Q^T and dP^T = V dO^T per 16-key quarter of the block: lane l
//    (g = l / 16) holds query l % 16 and keys 16 kq + 4 g + e; the wave's Q
//    and dO rows stay in registers (the B operands), so lse and D are one
//    value per lane.
//  * dQ += dS K over K = 32 keys at a time: the A operand is dS of the
//    lane's query for keys 4 g .. 4 g + 3 and 16 + 4 g .. + 3 of the half
//    (the lane's own values), the B operand the matching K entries, read
//    straight from the row-major K tile with two transposing reads.
//  * Key blocks are loaded into registers (buffer loads: rows past S read as
//    zeros) two iterations ahead (two register sets) and written to LDS at
//    the start of the iteration before their use, into the other of two
//    slots, so that the writes overlap that iteration's products.  The last
//    two blocks (the causal diagonal, the sequence tail) take the masked
//    path.
//  * It also writes D = rowsum(dO O) for the dK / dV pass.
template <int D>
__global__ __launch_bounds__(k16Threads, 1) void attn_bwd_dq16_kernel(AttnBwdArgs a) {
  constexpr int KB = 64;               // keys per block
  constexpr int C = D / 8;             // 16-byte chunks per row
  constexpr int RB = 2 * D;            // bytes per row
  constexpr int KS = D / 32;           // K steps of the S / dP products
  constexpr int kRows = k16Threads / C;  // tile rows staged per pass
  constexpr int kPre = KB / kRows;       // 16-byte chunks per thread per tile
  constexpr int kT = KB * D * 2;       // one block's K (or V) tile
  constexpr int kSlot = 2 * kT;
  __shared__ __attribute__((aligned(1024))) char lds[2 * kSlot];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15;
  const int g = lane >> 4;
  const int S = a.S;
  const int nqb = (S + kQBlock - 1) / kQBlock;
  int qb;
  int64_t bh;
  xcd_head_block<4>(nqb, a.BH, qb, bh);
  qb = nqb - 1 - qb;  // heaviest first
  const int64_t head = bh * (int64_t)S * D;
  const int q0w = qb * kQBlock + 16 * wave;  // first query of this wave
  const int q = q0w + i16;                   // this lane's query
  const int qc = q < S ? q : S - 1;
  const float c = a.scale_log2;

  f32x4 dq[D / 16];
#pragma unroll
  for (int m = 0; m < D / 16; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) dq[m][e] = 0.f;

  const int kend = a.causal ? min(S, qb * kQBlock + kQBlock) : S;
  const int nkb = (kend + KB - 1) / KB;
  // register-staged loads: thread t carries chunk t % C of rows t / C +
  // kRows i of the K and the V tile (position t % C of the row in LDS); two
  // register sets by block parity, compile-time at every use
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)(a.K + head), (int64_t)S * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char*)(a.V + head), (int64_t)S * D * 2);
  const int srow = tid / C;
  const uint32_t gvoff = (uint32_t)swz_offset<D>(srow, tid % C);
  const int lvoff = srow * RB + ((tid % C) << 4);
  u32x4 pre[2][2 * kPre];
  auto slot_of = [&](int kb) { return lds + (kb & 1) * kSlot; };
  auto load_regs = [&](int kb, auto par) {
    constexpr int r = decltype(par)::value;
    const uint32_t soff = (uint32_t)(kb * KB) * (uint32_t)RB;
#pragma unroll
    for (int i = 0; i < kPre; ++i)
      pre[r][i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, gvoff + RB * kRows * i, soff, 0));
#pragma unroll
    for (int i = 0; i < kPre; ++i)
      pre[r][kPre + i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, gvoff + RB * kRows * i, soff, 0));
    __builtin_amdgcn_sched_barrier(0);  // issued first
  };
  auto store_regs = [&](int kb, auto par) {
    constexpr int r = decltype(par)::value;
    char* sl = slot_of(kb);
#pragma unroll
    for (int i = 0; i < kPre; ++i) *(u32x4*)(sl + lvoff + RB * kRows * i) = pre[r][i];
#pragma unroll
    for (int i = 0; i < kPre; ++i) *(u32x4*)(sl + kT + lvoff + RB * kRows * i) = pre[r][kPre + i];
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  // Prologue, one memory round trip: the loads of key blocks 0 and 1 go out
  // first, then the lane's Q, dO and O rows (their wait covers all of them);
  // block 0 then takes its slot, block 1 waits in registers for the first
  // iteration, and block 2 is loaded.
  load_regs(0, P0{});
  if (1 < nkb) load_regs(1, P1{});
  // the Q and dO fragments (B operands: query i16, dims 32 s + 8 g .. + 7), and
  // D = rowsum(dO O) of the lane's query (the four lanes of a query each sum
  // a quarter of the dims)
  u32x4 qf[KS], df[KS];
  f32x4 of[2 * KS];
  // lse of the lane's query (0 past S: buffer bounds)
  const float lse_q = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(
                 make_rsrc((const char*)(a.lse + bh * S), (int64_t)S * 4), (uint32_t)q * 4u, 0, 0));
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int64_t off = head + (int64_t)qc * D + 32 * s + 8 * g;
    qf[s] = *(const u32x4*)(a.Q + off);
    df[s] = *(const u32x4*)(a.dO + off);
    of[2 * s] = *(const f32x4*)(a.O + off);
    of[2 * s + 1] = *(const f32x4*)(a.O + off + 4);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first use
  float dpart = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const f32x4 o0 = of[2 * s], o1 = of[2 * s + 1];
    dpart += bf16_lo(df[s][0]) * o0[0] + bf16_hi(df[s][0]) * o0[1] + bf16_lo(df[s][1]) * o0[2] +
             bf16_hi(df[s][1]) * o0[3] + bf16_lo(df[s][2]) * o1[0] + bf16_hi(df[s][2]) * o1[1] +
             bf16_lo(df[s][3]) * o1[2] + bf16_hi(df[s][3]) * o1[3];
  }
  dpart += __shfl_xor(dpart, 16);
  const float Dq = dpart + __shfl_xor(dpart, 32);
  if (g == 0 && q < S) a.delta[bh * S + q] = Dq;
  const float lse2 = lse_q * kLog2e;

  int aoff[KS], toff[D / 16];
#pragma unroll
  for (int s = 0; s < KS; ++s) aoff[s] = swz_offset<D>(i16, 4 * s + g);
#pragma unroll
  for (int m = 0; m < D / 16; ++m) {
    const int row = 4 * g + (i16 >> 2);
    const int dim = 16 * m + 4 * (lane & 3);
    toff[m] = swz_offset<D>(row, dim >> 3) + (dim & 7) * 2;
  }
  const int lim = a.causal ? min(q, S - 1) : S - 1;  // last key this lane may see

  auto block = [&](int kb, const bool masked) {
    const char* sl = slot_of(kb);
    f32x4 sc[4], dp[4];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[kq][e] = 0.f;
        dp[kq][e] = 0.f;
      }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        mma16(sc[kq], *(const u32x4*)(sl + aoff[s] + 16 * RB * kq), qf[s]);
        mma16(dp[kq], *(const u32x4*)(sl + kT + aoff[s] + 16 * RB * kq), df[s]);
      }
    // the first 4 fragment reads go out together, then one read after each
    // MFMA (the compiler's order waits on each read right in front of its
    // MFMA; 5 or more reads ahead measured 6% slower)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int q = 0; q < 8 * KS - 4; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (masked) {
#pragma unroll
      for (int kq = 0; kq < 4; ++kq)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sc[kq][e] = (kb * KB + 16 * kq + 4 * g + e > lim) ? -INFINITY : sc[kq][e];
    }
    u32x4 dsf[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float ds[2][4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kq = 2 * j + hh;
          const float p = fast_exp2(fmaf(sc[kq][e], c, -lse2));
          ds[hh][e] = p * (dp[kq][e] - Dq);
        }
      dsf[j][0] = cvt_pk_bf16(ds[0][0], ds[0][1]);
      dsf[j][1] = cvt_pk_bf16(ds[0][2], ds[0][3]);
      dsf[j][2] = cvt_pk_bf16(ds[1][0], ds[1][1]);
      dsf[j][3] = cvt_pk_bf16(ds[1][2], ds[1][3]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int m = 0; m < D / 16; ++m)
        mma16(dq[m], dsf[j], tr_frag16<D>(sl + 32 * RB * j + toff[m]));
  };

  store_regs(0, P0{});
  if (2 < nkb) load_regs(2, P0{});
  __syncthreads();
  // iteration kb: block kb + 1 (loaded two iterations earlier) written to
  // the other slot (block kb - 1's, read in iteration kb - 1), block kb + 3
  // loaded into the register set it freed, block kb computed
  auto iter = [&](int kb, auto par, auto last) {
    constexpr int P = decltype(par)::value;  // parity of kb
    constexpr bool kMasked = decltype(last)::value;
    using Pn = std::integral_constant<int, 1 - P>;
    if (kb + 1 < nkb) store_regs(kb + 1, Pn{});
    if (kb + 3 < nkb) load_regs(kb + 3, Pn{});
    __builtin_amdgcn_sched_barrier(0);
    if (kMasked) {
      // every key of the block after the wave's queries: nothing to add
      if (!(a.causal && kb * KB > q0w + 15)) block(kb, true);
    } else {
      block(kb, false);
    }
    __syncthreads();
  };
  using Masked = std::integral_constant<bool, true>;
  using Plain = std::integral_constant<bool, false>;
  const int nplain = nkb >= 2 ? nkb - 2 : 0;  // the last two blocks take the mask
  int kb = 0;
  for (; kb + 1 < nplain; kb += 2) {
    iter(kb, P0{}, Plain{});
    iter(kb + 1, P1{}, Plain{});
  }
  if (kb < nplain) {
    iter(kb, P0{}, Plain{});
    ++kb;
    if (kb < nkb) iter(kb, P1{}, Masked{});
    ++kb;
    if (kb < nkb) iter(kb, P0{}, Masked{});
  } else {
    if (kb < nkb) iter(kb, P0{}, Masked{});
    ++kb;
    if (kb < nkb) iter(kb, P1{}, Masked{});
  }

#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int qq = q0w + 4 * g + e;
    if (qq < S) {
      float* dQq = a.dQ + head + (int64_t)qq * D + i16;
#pragma unroll
      for (int m = 0; m < D / 16; ++m) dQq[16 * m] = dq[m][e] * a.scale;
    }
  }
}

hipError_t launch_attn_bwd_dq(const AttnBwdArgs& a, int D, hipStream_t s) {
  if (a.S <= 0 || a.BH <= 0) return hipSuccess;
  const int64_t nqb = (a.S + kQBlock - 1) / kQBlock;
  const dim3 grid((unsigned)(nqb * a.BH));
  if (D == 128)
    hipLaunchKernelGGL(attn_bwd_dq16_kernel<128>, grid, dim3(k16Threads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_bwd_dq16_kernel<64>, grid, dim3(k16Threads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dkv(const AttnBwdArgs& a, int D, hipStream_t s) {
  if (a.S <= 0 || a.BH <= 0) return hipSuccess;
  constexpr int NP = 4;
  const int64_t nkb = (a.S + 32 * NP - 1) / (32 * NP);
  const dim3 grid((unsigned)(nkb * a.BH));
  if (D == 128)
    hipLaunchKernelGGL((attn_bwd_dkv_pair_kernel<NP, 128>), grid, dim3(128 * NP), 0, s, a);
  else
    hipLaunchKernelGGL((attn_bwd_dkv_pair_kernel<NP, 64>), grid, dim3(128 * NP), 0, s, a);
  return hipGetLastError();
}

}  // namespace lce
