// Backward kernels: recompute each logit tile and form
// G = (softmax - onehot) * w in registers, then the two contractions
// dH += G W and dW += G^T H over a bounded [C x Vs] block of G, plus the
// helpers that lay operands out K-contiguous for the tile engine.
//
// Recomputing the logits chunk by chunk in the backward pass instead of
// saving them is what "6GB显卡预训练11亿参数模型" describes for its chunked loss
// (sections 内存实际花在哪里 and 关键参数说明: --chunked-loss 512 recomputes the
// logits in backward).  Here the chunk is a C-row slice of the compact token
// index times a Vs-entry slice of the vocabulary, so the workspace is
// O((C + d) * (Vs + C)) and independent of N and V.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace lce {

// ------------------------------------------------ zero rows of ignored tokens
//
// Padding / ignored tokens take no part in the loss (OjasX page, core
// technology: padding tokens are skipped), so their dH rows are exactly 0.
__global__ __launch_bounds__(256) void zero_ignored_kernel(const int64_t* __restrict__ labels,
                                                           int64_t ignore_index, int64_t V,
                                                           float* __restrict__ dH, int64_t d) {
  const int64_t row = blockIdx.x;
  const int64_t y = labels[row];
  if (y != ignore_index && y >= 0 && y < V) return;
  f32x4* p = (f32x4*)(dH + row * d);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k = threadIdx.x; k < d / 4; k += 256) p[k] = z;
}

hipError_t launch_zero_ignored(const int64_t* labels, int64_t N, int64_t ignore_index, int64_t V,
                               float* dH, int64_t d, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_ignored_kernel, dim3((unsigned)N), dim3(256), 0, s, labels, ignore_index,
                     V, dH, d);
  return hipGetLastError();
}

// ---------------------------------------------- fp32 -> bf16 output cast
//
// The gradients leave the backward pass in fp32; a bf16 parameter takes them
// rounded to nearest, ties to even (NaN stays NaN, overflow becomes inf).
// HBM-bound: 8 values (32 bytes read, 16 written) per thread and step, the
// pairs converted by the hardware packing conversion; the n % 8 tail values
// are converted one by one by the first workgroup.
__global__ __launch_bounds__(256) void cast_bf16_kernel(const float* __restrict__ src,
                                                        uint16_t* __restrict__ dst, int64_t n) {
  const int64_t n8 = n / 8;
  const f32x4* s4 = (const f32x4*)src;
  u32x4* d4 = (u32x4*)dst;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * 256) {
    const f32x4 a = __builtin_nontemporal_load(s4 + 2 * i);
    const f32x4 b = __builtin_nontemporal_load(s4 + 2 * i + 1);
    const u32x4 o = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                     pack_bf16x2(b[2], b[3])};
    d4[i] = o;
  }
  const int64_t t = n8 * 8 + threadIdx.x;
  if (blockIdx.x == 0 && t < n) dst[t] = (uint16_t)(pack_bf16x2(src[t], 0.f) & 0xffffu);
}

hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t n8 = n / 8;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((n8 + 255) / 256, 8192));
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

// ------------------------------------------------------------- transpose
//
// dst[k][i] = src[row(row0 + i)][k] for i < rows available, 0 for the rest of
// the ncols columns.  64 x 64 element tiles through LDS; HBM-bound.  Reads
// and writes are 16-byte vectors (8 bf16 or 4 fp32 per access).
//
// bf16: a thread reads 8 consecutive columns k of two adjacent rows (2p,
// 2p + 1) and pairs them into 32-bit words {src[2p][k], src[2p + 1][k]},
// which is already the layout of dst row k at columns 2p, 2p + 1.  The words
// go to LDS as 64 rows (k) of 32 words (p) with a 33-word stride, so that
// the 64 lanes of a write (8 column vectors x 8 row pairs) hit distinct
// banks; each output vector is then 4 word reads instead of 8 two-byte ones.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(TransposeArgs a) {
  constexpr int kV = 16 / sizeof(T);  // elements per 16-byte vector
  const int tid = threadIdx.x;
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  const int64_t k0 = (int64_t)blockIdx.y * 64;
  if (a.active_count && (int64_t)(*a.active_count) <= a.active_c0) return;
  int64_t avail = a.count ? (int64_t)(*a.count) - a.row0 : a.nrows_static - a.row0;
  if (avail < 0) avail = 0;
  if (avail > a.ncols) avail = a.ncols;
  if constexpr (sizeof(T) == 2) {
    __shared__ uint32_t tw[64 * 33];
    const int kv = tid & 7;  // column vector: columns k0 + 8 kv .. + 7
    const int p = tid >> 3;  // row pair: rows i0 + 2p, i0 + 2p + 1
    u32x4 v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t i = i0 + 2 * p + h;
      v[h] = u32x4{0u, 0u, 0u, 0u};
      if (i < avail) {
        const int64_t r = a.row0 + i;
        const int64_t phys = a.gather ? (int64_t)a.gather[r] : r;
        v[h] = *(const u32x4*)((const T*)a.src + phys * a.ld_src + k0 + 8 * kv);
      }
    }
    // word q of a row holds columns 2q (low half) and 2q + 1 (high half)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t x = v[0][q], y = v[1][q];
      tw[(8 * kv + 2 * q) * 33 + p] = (x & 0xffffu) | (y << 16);
      tw[(8 * kv + 2 * q + 1) * 33 + p] = (x >> 16) | (y & 0xffff0000u);
    }
    __syncthreads();
    // dst row k, columns i0 + 8 g .. + 7 = words 4 g .. 4 g + 3 of LDS row k
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int idx = it * 256 + tid;
      const int k = idx >> 3;
      const int g = idx & 7;
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = tw[k * 33 + 4 * g + j];
      *(u32x4*)((T*)a.dst + (k0 + k) * a.ld_dst + i0 + 8 * g) = w;
    }
    return;
  }
  __shared__ T tile[64][64 + kV];
  // read: 64 rows x 64 elements = 64 * 64 / kV vectors; thread -> (row, vector)
  constexpr int kVecPerRow = 64 / kV;
#pragma unroll
  for (int it = 0; it < 64 * kVecPerRow / 256; ++it) {
    const int idx = it * 256 + tid;
    const int ii = idx / kVecPerRow;
    const int kk = (idx % kVecPerRow) * kV;
    const int64_t i = i0 + ii;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (i < avail) {
      const int64_t r = a.row0 + i;
      const int64_t phys = a.gather ? (int64_t)a.gather[r] : r;
      v = *(const u32x4*)((const T*)a.src + phys * a.ld_src + k0 + kk);
    }
    const T* e = (const T*)&v;
#pragma unroll
    for (int q = 0; q < kV; ++q) tile[ii][kk + q] = e[q];
  }
  __syncthreads();
  // write: dst row k, kV consecutive i per vector
#pragma unroll
  for (int it = 0; it < 64 * kVecPerRow / 256; ++it) {
    const int idx = it * 256 + tid;
    const int kk = idx / kVecPerRow;
    const int ii = (idx % kVecPerRow) * kV;
    u32x4 v;
    T* e = (T*)&v;
#pragma unroll
    for (int q = 0; q < kV; ++q) e[q] = tile[ii + q][kk];
    *(u32x4*)((T*)a.dst + (k0 + kk) * a.ld_dst + i0 + ii) = v;
  }
}

hipError_t launch_transpose(const TransposeArgs& a, int dtype, hipStream_t s) {
  const dim3 grid((unsigned)(a.ncols / 64), (unsigned)(a.K / 64));
  if (dtype == 1)
    hipLaunchKernelGGL(transpose_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// Two values as one non-temporal global store, for data that a later kernel
// reads once (the recomputed G^T blocks).
template <typename T> __device__ __forceinline__ void stream2(void* p, float a, float b);
template <> __device__ __forceinline__ void stream2<bf16_t>(void* p, float a, float b) {
  __builtin_nontemporal_store(pack_bf16x2(a, b), (uint32_t*)p);
}
template <> __device__ __forceinline__ void stream2<float>(void* p, float a, float b) {
  const f32x2 v = {a, b};
  __builtin_nontemporal_store(v, (f32x2*)p);
}

// --------------------------------------------------- recompute + G tile
//
// Same MFMA tile as the forward (A = W rows, B = gathered H rows, so each lane
// holds 2 consecutive tokens).  Epilogue: p = exp(z - lse), subtract 1 at the
// label, scale by w = grad / N_valid (mean) or grad (sum); entries past V or
// past the valid tokens are 0.  G is written row-major [token][vocab] for the
// dH contraction (and the bf16 dW store, which reads it K-major) and, where
// the dW contraction needs it (fp32, the bf16 optimizer epilogue), also
// transposed [vocab][token].
template <typename T>
__device__ __forceinline__ void bwd_g_tile(const BwdGArgs& a, int slot, char* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wa = wave & 1;
  const int wb = wave >> 1;
  const int j = lane & 31;
  const int h = lane >> 5;

  // tile grid of this block: vocabulary tiles x token tiles that hold valid
  // tokens (the count is read on the device, so the active tiles are mapped
  // first and spread over every XCD; surplus slots exit)
  const int count = *a.valid_count;
  const int64_t n_act = min((int64_t)count - a.c0, a.C);
  if (n_act <= 0) return;
  const int64_t nv = min(a.Vs, a.V - a.v0);
  const int TM = (int)((nv + kTile - 1) / kTile);
  const int TN = (int)((n_act + kTile - 1) / kTile);
  int tm, tn;
  if (!xcd_tile(slot, TM, TN, 8, 4, tm, tn)) return;

  const int64_t ld = a.d * Elem<T>::kSize;
  RowSource as{(const char*)a.W, ld, nullptr, a.v0 + (int64_t)tm * kTile, a.V, 0};
  RowSource bs{(const char*)a.H, ld, a.valid_idx, a.c0 + (int64_t)tn * kTile, count, a.N};
  const RowPtrs pa = make_row_ptrs<false>(as, tid);
  const RowPtrs pb = make_row_ptrs<true>(bs, tid);

  // per-token data (2 consecutive tokens per lane)
  float lse_t[kNT], w_t[kNT];
  int y[kNT];
  const float g = *a.grad_out;
  const float w = a.reduction == 0 ? g / (float)count : g;
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int64_t i = a.c0 + (int64_t)tn * kTile + wb * kWaveN + 2 * j + nt;
    if (i < count) {
      const int r = a.valid_idx[i];
      y[nt] = (int)(a.labels[r] - a.y_off);  // outside [0, V) in a shard without it
      lse_t[nt] = a.lse[r];
      w_t[nt] = w;
    } else {
      y[nt] = -1;
      lse_t[nt] = 0.f;
      w_t[nt] = 0.f;
    }
  }

  Acc acc;
  zero_acc(acc);
  tile_mainloop<T>(acc, lds, pa, pb, (int)(a.d / Elem<T>::kPerStage), tid);

  const int vl0 = tm * kTile + wa * kHalf;  // first local vocab entry of this wave
  // entry (mt, i) sits at c + 4 h past vl0, c = 32 mt + 8 (i / 4) + i % 4 a
  // compile-time constant; bounds are shifted instead of the positions
  int y_h[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) y_h[nt] = (int)(y[nt] - a.v0) - vl0 - 4 * h;  // label at c
  // G = (exp(z - lse) - [c == label]) w, one code path for every tile:
  //   G = sgn(w) exp2(z log2(e) + cw) - [c == label] w,  cw = log2|w| - lse log2(e),
  // i.e. one fma and one exp per entry, then a compare, a select and an fma.
  // A token past the count has w = 0, so cw = -inf and its entries are
  // exactly 0 (for finite z, without a product that could make NaN).
  // Entries past V only need to be finite: dH multiplies them by the zeroed
  // W^T columns past V, and dW never stores those rows.
  float cw[kNT], wneg[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    cw[nt] = fast_log2(fabsf(w_t[nt])) - lse_t[nt] * kLog2e;
    wneg[nt] = -w_t[nt];
  }
  const float sgn = w < 0.f ? -1.f : 1.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = 32 * mt + 8 * (i >> 2) + (i & 3);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const float e = fast_exp2(fmaf(acc[mt][nt][i], kLog2e, cw[nt]));
        acc[mt][nt][i] = fmaf(e, sgn, c == y_h[nt] ? wneg[nt] : 0.f);
      }
    }

  // G^T[vocab][token]: the lane's 2 consecutive tokens per store; for a fixed
  // accumulator register the 32 lanes of a half-wave cover 128 contiguous
  // bytes.  Non-temporal stores: 1% faster than ordinary ones on the Llama-3
  // head (dW reads the block once, after the whole recompute).
  // (only where a dW contraction reads it: fp32, and the bf16 optimizer
  // epilogue; the bf16 dW store reads G K-major)
  const int il0 = tn * kTile + wb * kWaveN + 2 * j;  // local token of nt = 0
  char* GT = (char*)a.GT;
  if (GT) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t vl = vl0 + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
        stream2<T>(GT + (vl * a.ldGT + il0) * Elem<T>::kSize, acc[mt][0][i], acc[mt][1][i]);
      }
  }

  char* G = (char*)a.G;
  if constexpr (sizeof(T) == 2) {
    // G[token][vocab] goes through LDS: a lane holds 2 tokens x 64 vocabulary
    // entries, so direct row-major stores would scatter.  The 256 x 256 bf16
    // tile (128 KB) is written to LDS as rows of 32 sixteen-byte slots, slot q
    // of row t at position q ^ ((t >> 1) & 31) (conflict-free for both the
    // scattered writes and the row reads), then streamed out row by row.
    // The main loop ended with a barrier, so its LDS buffers are free.
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const int row = wb * kWaveN + 2 * j + nt;
      const int f = (row >> 1) & 31;
      char* lrow = lds + row * 512;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int q = wa * 16 + 4 * mt + g4;
          Store4<T>::run(lrow + ((q ^ f) << 4) + 8 * h, acc[mt][nt][4 * g4],
                         acc[mt][nt][4 * g4 + 1], acc[mt][nt][4 * g4 + 2], acc[mt][nt][4 * g4 + 3]);
        }
    }
    __syncthreads();
    const int64_t grow0 = (int64_t)tn * kTile;
    const int64_t gcol0 = (int64_t)tm * kTile;
#pragma unroll 4
    for (int it = 0; it < kTile * 32 / kThreads; ++it) {
      const int idx = it * kThreads + tid;
      const int row = idx >> 5;
      const int q = idx & 31;
      const u32x4 v = *(const u32x4*)(lds + row * 512 + ((q ^ ((row >> 1) & 31)) << 4));
      *(u32x4*)(G + ((grow0 + row) * a.ldG + gcol0 + 8 * q) * 2) = v;
    }
  } else {
    // fp32 (small shapes only): direct 16-byte stores
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int64_t vl = vl0 + 32 * mt + 8 * g4 + 4 * h;
          Store4<T>::run(G + ((int64_t)(il0 + nt) * a.ldG + vl) * Elem<T>::kSize,
                         acc[mt][nt][4 * g4], acc[mt][nt][4 * g4 + 1], acc[mt][nt][4 * g4 + 2],
                         acc[mt][nt][4 * g4 + 3]);
        }
  }
}

// One tile per workgroup (a persistent loop here costs more than it saves:
// the loop pushes the kernel's register use into spills in the main loop).
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void bwd_g_kernel(BwdGArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kMainLds];
  bwd_g_tile<T>(a, blockIdx.x, lds);
}

hipError_t launch_bwd_g(BwdGArgs a, int dtype, hipStream_t s) {
  const int TM = (int)(a.Vs / kTile), TN = (int)(a.C / kTile);
  const int nsb = ((TM + 7) / 8) * ((TN + 3) / 4);
  a.nslots = 256 * ((nsb + 7) / 8);
  const int grid = a.nslots;  // one workgroup per slot
  if (dtype == 1)
    hipLaunchKernelGGL(bwd_g_kernel<bf16_t>, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_g_kernel<float>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// ----------------------------------------------------------- dH += G W
//
// C tile rows = tokens of the chunk (A = G rows), columns = hidden units;
// K runs over the vocabulary block.  B is either W itself, read K-major with
// the transposing LDS reads (kBT: bf16, W not updated during the launch), or
// the W^T rows of the transposed block.  Rows are scattered to the tokens'
// original positions through valid_idx.  beta = 0 on the first vocabulary
// block, 1 afterwards.
// (ga, gb): the block of tiles the 32 slots of one XCD take (ga * gb = 32)
template <typename T, bool kBT = false>
__device__ __forceinline__ void dh_tile(const DhArgs& a, int slot, char* lds, int ga, int gb) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wa = wave & 1;
  const int wb = wave >> 1;
  const int h = lane >> 5;

  // token tiles holding valid tokens x hidden tiles; active tiles map first
  const int count = *a.valid_count;
  const int64_t n_act = min((int64_t)count - a.c0, a.C);
  if (n_act <= 0) return;
  const int TM = (int)((n_act + kTile - 1) / kTile);
  const int TN = (int)((a.d + kTile - 1) / kTile);
  // ga == 0: the block of tiles per XCD is chosen from the active grid: 4 x 8
  // when that gives every XCD a block (each XCD then streams half the W
  // panels a 2 x 16 block needs), else 2 x 16 (spreads few token tiles over
  // all eight XCDs)
  if (ga == 0) {
    const bool wide = ((TM + 3) / 4) * ((TN + 7) / 8) >= 8;
    ga = wide ? 4 : 2;
    gb = wide ? 8 : 16;
  }
  int tm, tn;
  if (!xcd_tile(slot, TM, TN, ga, gb, tm, tn)) return;
  const int64_t nv = min(a.Vs, a.V - a.v0);
  const int nstages = (int)((nv + Elem<T>::kPerStage - 1) / Elem<T>::kPerStage);

  // rows past the valid count clamp to the last valid row (cache hits)
  // instead of streaming the block's unused rows
  RowSource as{(const char*)a.G, a.ldG * Elem<T>::kSize, nullptr, (int64_t)tm * kTile, n_act, 0};
  const RowPtrs pa = make_row_ptrs<false>(as, tid);
  RowPtrs pb;
  if constexpr (kBT) {
    // W rows v0 .. v0 + nv of the block (rows past V read as zeros)
    pb = make_kmajor_ptrs((const char*)a.W, a.d * Elem<T>::kSize, a.v0, nv, (int64_t)tn * kTile,
                          tid);
  } else {
    RowSource bs{(const char*)a.WT, a.ldWT * Elem<T>::kSize, nullptr, (int64_t)tn * kTile, a.d, 0};
    pb = make_row_ptrs<false>(bs, tid);
  }
  Acc acc;
  zero_acc(acc);
  tile_mainloop<T, kBT>(acc, lds, pa, pb, nstages, tid);  // ends with a barrier: LDS is free

  // destination rows of the tile's tokens, in the (now free) stage buffers
  int* rows = (int*)lds;
  if (tid < kTile) {
    const int64_t m = (int64_t)tm * kTile + tid;
    rows[tid] = m < n_act ? a.valid_idx[a.c0 + m] : -1;
  }
  __syncthreads();

  const int n_base = tn * kTile + wb * kWaveN + (lane & 31);
  // Read-modify-write in four batches (one per mt): all 32 loads of a batch
  // are in flight together, so the epilogue pays four memory latencies, not
  // one per element.  Through a buffer resource over dH, an element without a
  // destination (no valid row, or a column past d) takes an offset past the
  // end, where the load reads 0 and the store is dropped: no element needs a
  // branch.  (With a branch per element the compiler waited for every
  // outstanding memory operation, stores included, in front of each store.)
  const int64_t hbytes = a.N * a.d * 4;
  if (hbytes < 0xFFFFFFFFll) {
    const __amdgpu_buffer_rsrc_t rh = make_rsrc((const char*)a.dH, hbytes);
    const uint32_t oob = (uint32_t)hbytes;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      float old[16][kNT];
      uint32_t off[16][kNT];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = rows[wa * kHalf + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3)];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          const int n = n_base + 32 * nt;
          off[i][nt] = (r >= 0 && n < a.d) ? (uint32_t)(((int64_t)r * a.d + n) * 4) : oob;
          old[i][nt] = a.beta ? __builtin_bit_cast(
                                    float, __builtin_amdgcn_raw_buffer_load_b32(rh, off[i][nt], 0, 0))
                              : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          __builtin_amdgcn_raw_buffer_store_b32(
              __builtin_bit_cast(uint32_t, old[i][nt] + acc[mt][nt][i]), rh, off[i][nt], 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
  // dH of 4 GB or more: 64-bit addresses
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    float old[16][kNT];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = rows[wa * kHalf + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3)];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const int n = n_base + 32 * nt;
        old[i][nt] = (a.beta && r >= 0 && n < a.d) ? a.dH[(int64_t)r * a.d + n] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = rows[wa * kHalf + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3)];
      if (r < 0) continue;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const int n = n_base + 32 * nt;
        if (n < a.d) a.dH[(int64_t)r * a.d + n] = old[i][nt] + acc[mt][nt][i];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------- dW += G^T H
//
// K runs over the chunk's valid tokens only (the count is read on the
// device).  Each workgroup owns its dW tile, so no atomics are needed and
// the result is deterministic.  The plain store computes the tile as dW^T
// (rows = hidden units from H^T, columns = vocabulary entries from G^T): a
// lane then holds four consecutive hidden units of one dW row and writes
// them as one 16-byte vector (2% faster than four 4-byte stores on the
// Llama-3 head).  The optimizer epilogue keeps rows = vocabulary entries, so
// that each of its load / store instructions covers two whole 128-byte rows
// of the weights and moments (with the dW^T layout, 32-byte pieces of 32 rows
// per instruction made the AdamW epilogue 26% slower on the Llama-3 head).
// It applies the update from the tile itself, so it serves the case where
// every valid row lies in one token chunk; otherwise the plain store sums the
// chunks into the block accumulator and apply_opt_kernel updates the block.
template <typename T, int kStep>  // 0: store dW; 1: SGD; 2: AdamW
__device__ __forceinline__ void dw_tile(const DwArgs& a, int slot, char* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wa = wave & 1;
  const int wb = wave >> 1;
  const int h = lane >> 5;

  const int64_t nv = min(a.Vs, a.V - a.v0);
  const int TM = (int)((nv + kTile - 1) / kTile);
  const int TN = (int)((a.d + kTile - 1) / kTile);
  int tm, tn;  // vocabulary and hidden tile
  if (kStep == 0 ? !xcd_tile(slot, TN, TM, 4, 8, tn, tm) : !xcd_tile(slot, TM, TN, 4, 8, tm, tn))
    return;
  const int count = *a.valid_count;
  int64_t kact = (int64_t)count - a.c0;
  if (kact < 0) kact = 0;
  if (kact > a.C) kact = a.C;
  const int nstages = (int)((kact + Elem<T>::kPerStage - 1) / Elem<T>::kPerStage);
  if (nstages == 0 && a.accumulate) return;

  RowSource as{(const char*)a.GT, a.ldGT * Elem<T>::kSize, nullptr, (int64_t)tm * kTile, a.Vs, 0};
  RowSource bs{(const char*)a.HT, a.ldHT * Elem<T>::kSize, nullptr, (int64_t)tn * kTile, a.d, 0};
  Acc acc;
  zero_acc(acc);
  if constexpr (kStep == 0) {
    if constexpr (sizeof(T) == 2) {
      // B = the block's G rows, K-major (token rows past the chunk's valid
      // count read as zeros): no G^T copy
      const RowPtrs pg = make_kmajor_ptrs((const char*)a.G, a.ldG * 2, 0, kact,
                                          (int64_t)tm * kTile, tid);
      tile_mainloop<T, true>(acc, lds, make_row_ptrs<false>(bs, tid), pg, nstages, tid);
    } else {
      tile_mainloop<T>(acc, lds, make_row_ptrs<false>(bs, tid), make_row_ptrs<false>(as, tid),
                       nstages, tid);
    }
    // acc[mt][nt][4 g + e] is dW[v_base + 32 nt][k_base + 32 mt + 8 g + e]
    // Through a buffer resource over the block's rows [v0, v0 + nv): rows
    // past nv fall outside it (loads read 0, stores are dropped), columns
    // past d take the offset past its end; no element needs a branch.
    const int64_t wbytes = nv * a.d * 4;
    const __amdgpu_buffer_rsrc_t rdw = make_rsrc((const char*)(a.dW + a.v0 * a.d), wbytes);
    const uint32_t oob = (uint32_t)wbytes;
    const int v_base = tm * kTile + wb * kWaveN + (lane & 31);
    const int k_base = tn * kTile + wa * kHalf + 4 * h;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // read-modify-write (accumulate) in two batches of 64 values
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const int v = v_base + 32 * nt;
      f32x4 old[4][4];
      uint32_t off[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int k = k_base + 32 * mt + 8 * g;  // d is a multiple of 64: all four in range
          off[mt][g] = k < a.d ? (uint32_t)(((int64_t)v * a.d + k) * 4) : oob;
          old[mt][g] = a.accumulate ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                    rdw, off[mt][g], 0, 0))
                                    : zero;
        }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = old[mt][g][e] + acc[mt][nt][4 * g + e];
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, r), rdw, off[mt][g], 0, 0);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    tile_mainloop<T>(acc, lds, make_row_ptrs<false>(as, tid), make_row_ptrs<false>(bs, tid),
                     nstages, tid);
    const int n_base = tn * kTile + wb * kWaveN + (lane & 31);
    const int m_base = tm * kTile + wa * kHalf + 4 * h;
    // The gradient tile goes straight into the optimizer (no dW table; OjasX
    // page, core technology: no persistent .grad buffers).  PyTorch's
    // formulas: SGD p -= lr (g + wd p); AdamW p *= 1 - lr wd, m = b1 m +
    // (1 - b1) g, v = b2 v + (1 - b2) g^2, p -= (lr / bc1) m / (sqrt(v) / bc2s
    // + eps).  Batches of 16 values per lane keep the loads in flight together.
    // State and weights through buffer resources over the block's rows
    // [v0, v0 + nv): loads past them read 0 and stores past them are dropped,
    // so no element needs a branch.  (With a branch per element the compiler
    // waited for all outstanding memory operations, stores included, in front
    // of each update.)  Columns past d (d not a multiple of the tile) stay
    // behind one per-lane condition.
    const char* mbase = (const char*)(a.master + a.v0 * a.d);
    const int64_t nbytes = nv * a.d * 4;
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(mbase, nbytes);
    const __amdgpu_buffer_rsrc_t rm1 =
        make_rsrc((const char*)(kStep == 2 ? a.exp_avg + a.v0 * a.d : nullptr), kStep == 2 ? nbytes : 0);
    const __amdgpu_buffer_rsrc_t rm2 = make_rsrc(
        (const char*)(kStep == 2 ? a.exp_avg_sq + a.v0 * a.d : nullptr), kStep == 2 ? nbytes : 0);
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc((const char*)(a.w16 ? a.w16 + a.v0 * a.d : nullptr), a.w16 ? nv * a.d * 2 : 0);
    // values per lane in flight (AdamW holds three arrays; 16 fp32 values
    // for SGD spilled)
    constexpr int kB = (kStep == 2 || sizeof(T) == 4) ? 8 : 16;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int i0 = 0; i0 < 16; i0 += kB) {
          const int n = n_base + 32 * nt;
          float p[kB], m[kB], v[kB];
          uint32_t off[kB];  // element offset from the block's first row
#pragma unroll
          for (int b = 0; b < kB; ++b) {
            const int i = i0 + b;
            const int ml = m_base + 32 * mt + 8 * (i >> 2) + (i & 3);
            off[b] = (uint32_t)((int64_t)ml * a.d + n);
            p[b] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, off[b] * 4u, 0, 0));
            if constexpr (kStep == 2) {
              m[b] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rm1, off[b] * 4u, 0, 0));
              v[b] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rm2, off[b] * 4u, 0, 0));
            }
          }
          if (n < a.d) {
#pragma unroll
            for (int b = 0; b < kB; ++b) {
              const float g = acc[mt][nt][i0 + b];
              float q;
              if constexpr (kStep == 1) {
                q = p[b] - a.lr * (g + a.wd * p[b]);
              } else {
                const float pd = p[b] * (1.f - a.lr * a.wd);
                const float m1 = a.beta1 * m[b] + (1.f - a.beta1) * g;
                const float v1 = a.beta2 * v[b] + (1.f - a.beta2) * g * g;
                q = pd - (a.lr / a.bc1) * m1 / (__builtin_sqrtf(v1) / a.bc2s + a.eps);
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, m1), rm1, off[b] * 4u, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v1), rm2, off[b] * 4u, 0, 0);
              }
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, q), rp, off[b] * 4u, 0, 0);
              if (a.w16)
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)bf16_bits(q), rw, off[b] * 2u, 0, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
  }
}

// ------------------------------------------- optimizer over a whole block
//
// When the valid rows span several token chunks, the plain dW store sums the
// block's gradient over the chunks in the fp32 accumulator acc ([Vs][d],
// row-major), and this kernel then applies the update to the block's rows
// [v0, v0 + nv): the same formulas as the fused epilogue, one thread per
// four consecutive values (16-byte vectors), grid-stride.  No dW table
// beyond the one block is ever held.
template <int kOpt>
__global__ __launch_bounds__(256) void apply_opt_kernel(DwArgs a) {
  const int64_t nv = min(a.Vs, a.V - a.v0);
  const int64_t n4 = nv * a.d / 4;
  const int64_t base = a.v0 * a.d;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * 256) {
    const int64_t o = base + 4 * i;
    const f32x4 g = ((const f32x4*)a.acc)[i];
    const f32x4 p = *(const f32x4*)(a.master + o);
    f32x4 m, v, q;
    if constexpr (kOpt == 2) {
      m = *(const f32x4*)(a.exp_avg + o);
      v = *(const f32x4*)(a.exp_avg_sq + o);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (kOpt == 1) {
        q[e] = p[e] - a.lr * (g[e] + a.wd * p[e]);
      } else {
        const float pd = p[e] * (1.f - a.lr * a.wd);
        m[e] = a.beta1 * m[e] + (1.f - a.beta1) * g[e];
        v[e] = a.beta2 * v[e] + (1.f - a.beta2) * g[e] * g[e];
        q[e] = pd - (a.lr / a.bc1) * m[e] / (__builtin_sqrtf(v[e]) / a.bc2s + a.eps);
      }
    }
    *(f32x4*)(a.master + o) = q;
    if constexpr (kOpt == 2) {
      *(f32x4*)(a.exp_avg + o) = m;
      *(f32x4*)(a.exp_avg_sq + o) = v;
    }
    if (a.w16) {
      u32x2 w;
      w[0] = bf16_bits(q[0]) | (bf16_bits(q[1]) << 16);
      w[1] = bf16_bits(q[2]) | (bf16_bits(q[3]) << 16);
      *(u32x2*)(a.w16 + o) = w;
    }
  }
}

hipError_t launch_apply_opt(const DwArgs& a, hipStream_t s) {
  const int64_t nv = std::min<int64_t>(a.Vs, a.V - a.v0);
  const int64_t n4 = nv * a.d / 4;
  if (n4 <= 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((n4 + 255) / 256, 8192);
  if (a.opt_kind == 1)
    hipLaunchKernelGGL(apply_opt_kernel<1>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(apply_opt_kernel<2>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ launches

// dH and dW of one vocabulary block in one launch, one tile per workgroup:
// the dH tiles in slots [0, n_dh), the dW tiles after them (n_dh is a
// multiple of 256, so every slot keeps its XCD: slot % 8).  Workgroups are
// dispatched in slot order as CUs free up, so the short dW tiles fill the
// CUs that the long dH tiles (K = the vocabulary block) leave idle: a chunk
// of 6800 valid tokens has 27 x 16 = 432 dH tiles, 1.69 rounds of 256 CUs,
// and its dW tiles run in the gap.  Measured against separate dH and
// persistent dW launches (A/B on one box): config 4 51.5 -> 50.5 ms per step,
// the Llama-3 head 14.7 -> 14.5, the 64K context 222.5 -> 221.9.  The dH
// tiles choose their per-XCD block on the device (dh_tile with ga = 0).
// One LDS object only: with a second __shared__ array the compiler can no
// longer tell the direct-to-LDS loads of the next stage from the fragment
// reads of the current one and waits for every load right after issuing it.
template <typename T, int kOpt, bool kBT>
__global__ __launch_bounds__(kThreads, 1) void dh_dw_kernel(DhArgs ha, DwArgs wa, int n_dh) {
  __shared__ __attribute__((aligned(16))) char lds[kMainLds];
  const int b = (int)blockIdx.x;
  if (b < n_dh)
    dh_tile<T, kBT>(ha, b, lds, 0, 0);
  else
    dw_tile<T, kOpt>(wa, b - n_dh, lds);
}

// Slots for the dW tiles of one vocabulary block: 4 x 8 blocks of tiles per
// XCD, over (hidden, vocabulary) tiles for the plain store and over
// (vocabulary, hidden) tiles for the optimizer epilogue (as dw_tile maps them).
int dw_slots(const DwArgs& a) {
  const int TV = (int)((a.Vs + kTile - 1) / kTile), TD = (int)((a.d + kTile - 1) / kTile);
  const int TM = a.opt_kind == 0 ? TD : TV, TN = a.opt_kind == 0 ? TV : TD;
  return 256 * ((((TM + 3) / 4) * ((TN + 7) / 8) + 7) / 8);
}

hipError_t launch_dh_dw(const DhArgs& ha, DwArgs wa, int dtype, hipStream_t s) {
  const int TMh = (int)(ha.C / kTile), TNh = (int)((ha.d + kTile - 1) / kTile);
  // slots for either block of tiles dh_tile may choose (a multiple of 256)
  const int n_dh = 256 * std::max(((((TMh + 1) / 2) * ((TNh + 15) / 16) + 7) / 8),
                                  ((((TMh + 3) / 4) * ((TNh + 7) / 8) + 7) / 8));
  wa.nslots = dw_slots(wa);
  const dim3 grid((unsigned)(n_dh + wa.nslots));
  // the optimizer epilogues rewrite W's rows while dH tiles run: they keep
  // dH on the transposed copy (ha.W null)
  if (dtype == 1) {
    if (wa.opt_kind == 1)
      hipLaunchKernelGGL((dh_dw_kernel<bf16_t, 1, false>), grid, dim3(kThreads), 0, s, ha, wa, n_dh);
    else if (wa.opt_kind == 2)
      hipLaunchKernelGGL((dh_dw_kernel<bf16_t, 2, false>), grid, dim3(kThreads), 0, s, ha, wa, n_dh);
    else if (ha.W)
      hipLaunchKernelGGL((dh_dw_kernel<bf16_t, 0, true>), grid, dim3(kThreads), 0, s, ha, wa, n_dh);
    else
      hipLaunchKernelGGL((dh_dw_kernel<bf16_t, 0, false>), grid, dim3(kThreads), 0, s, ha, wa, n_dh);
  } else {
    if (wa.opt_kind == 1)
      hipLaunchKernelGGL((dh_dw_kernel<float, 1, false>), grid, dim3(kThreads), 0, s, ha, wa, n_dh);
    else if (wa.opt_kind == 2)
      hipLaunchKernelGGL((dh_dw_kernel<float, 2, false>), grid, dim3(kThreads), 0, s, ha, wa, n_dh);
    else
      hipLaunchKernelGGL((dh_dw_kernel<float, 0, false>), grid, dim3(kThreads), 0, s, ha, wa, n_dh);
  }
  return hipGetLastError();
}

// ------------------------------------------------------- plain NT GEMM
//
// C[M][N] = A[M][K] B[N][K]^T in fp32: the same tile engine with a plain
// store, used to measure what this MFMA engine reaches on a bare GEMM of the
// path's shapes and to check the engine's layout in isolation.
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(const void* A, const void* B, float* C,
                                                              int64_t M, int64_t N, int64_t K) {
  __shared__ __attribute__((aligned(16))) char lds[kMainLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wa = wave & 1;
  const int wb = wave >> 1;
  const int h = lane >> 5;
  const int TM = (int)((M + kTile - 1) / kTile);
  const int TN = (int)((N + kTile - 1) / kTile);
  int tm, tn;
  if (!xcd_tile(blockIdx.x, TM, TN, 4, 8, tm, tn)) return;
  const int64_t ld = K * Elem<T>::kSize;
  RowSource as{(const char*)A, ld, nullptr, (int64_t)tm * kTile, M, 0};
  RowSource bs{(const char*)B, ld, nullptr, (int64_t)tn * kTile, N, 0};
  const RowPtrs pa = make_row_ptrs<false>(as, tid);
  const RowPtrs pb = make_row_ptrs<false>(bs, tid);
  Acc acc;
  zero_acc(acc);
  tile_mainloop<T>(acc, lds, pa, pb, (int)(K / Elem<T>::kPerStage), tid);
  const int64_t n_base = (int64_t)tn * kTile + wb * kWaveN + (lane & 31);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t m = (int64_t)tm * kTile + wa * kHalf + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
      if (m >= M) continue;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const int64_t n = n_base + 32 * nt;
        if (n < N) C[m * N + n] = acc[mt][nt][i];
      }
    }
}

// ----------------------------------------------------- MFMA calibration
//
// The matrix cores alone: four independent chains of the bf16 32x32x16 MFMA
// on register operands, no memory traffic inside the loop.  It gives the
// MFMA rate (and, under a counter run, the clock) the chip sustains when
// only the matrix cores work, the reference the fused kernels are held
// against.  Each thread stores one float (so the loop is not removed).
__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(float* __restrict__ out,
                                                             int64_t iters) {
  u32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = 0x3c003c00u + (uint32_t)i + ((threadIdx.x & 7) << 4);  // small finite bf16 values
    b[i] = 0x3c003c00u - (uint32_t)i;
  }
  f32x16 c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[j][i] = 0.f;
  for (int64_t it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < 4; ++j) Mma<bf16_t>::run(c[j], a, b);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += c[j][i];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = sum;
}

hipError_t launch_mfma_peak(float* out, int blocks, int64_t iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(kThreads), 0, s, out, iters);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(const void* A, const void* B, float* C, int64_t M, int64_t N, int64_t K,
                          int dtype, hipStream_t s) {
  const int TM = (int)((M + kTile - 1) / kTile), TN = (int)((N + kTile - 1) / kTile);
  const int nsb = ((TM + 3) / 4) * ((TN + 7) / 8);
  const int grid = 256 * ((nsb + 7) / 8);
  if (dtype == 1)
    hipLaunchKernelGGL(gemm_nt_kernel<bf16_t>, dim3(grid), dim3(kThreads), 0, s, A, B, C, M, N, K);
  else
    hipLaunchKernelGGL(gemm_nt_kernel<float>, dim3(grid), dim3(kThreads), 0, s, A, B, C, M, N, K);
  return hipGetLastError();
}

}  // namespace lce
