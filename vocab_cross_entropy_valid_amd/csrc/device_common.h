// Device-side building blocks shared by every kernel of the fused
// linear + cross-entropy path on gfx950 (CDNA4, wave64, MFMA, 160 KB LDS).
//
// The tile engine computes a 256 x 256 fp32 block C = A * B^T where both
// operands are "K-contiguous" (each logical row holds its K elements
// contiguously): that is how H [N, d] and W [V, d] are stored, and how the
// backward pass lays out its bounded G / G^T / W^T / H^T buffers.
//
//  * 256 threads = 4 waves in a 2 x 2 arrangement; wave (wa, wb) owns A rows
//    [128 wa, 128 wa + 128) and B rows [128 wb, 128 wb + 128) of the tile,
//    held as 4 x 4 accumulators of the 32x32 MFMA (16 fp32 per lane each,
//    256 accumulator registers per lane).
//  * K advances 128 bytes per pipeline stage (64 bf16 or 32 fp32).  In LDS
//    one operand stage is split by K into four sub-buffers of 256 rows x 32 B
//    (one per MFMA step); a lane's 16-byte fragment of row r sits at
//    r * 32 + 16 * (h ^ g(r)) with g(r) = bit 2 ^ bit 3 of r, so that any 8 or
//    16 consecutive lanes read distinct banks, and the sub-buffers are 32 B
//    apart modulo 256 so that the loader's 16-byte writes do not collide.
//    With this layout every LDS address of the main loop is one per-lane
//    register plus a compile-time offset.  Two operands, double buffered,
//    take 2 x 2 x 32.1 KB of the 160 KB per CU.
//  * bf16 uses v_mfma_f32_32x32x16_bf16 (one per 16-byte fragment pair);
//    fp32 uses four v_mfma_f32_32x32x2_f32, one per float of the fragment.
//    Lanes 0-31 and 32-63 hold the two halves of a 32-byte K slice.  A and B
//    use the same K assignment, so the product is exact regardless of how
//    the hardware orders K inside one instruction.
//  * Accumulator layout (32x32 MFMA): lane l holds column n = l % 32 (a B
//    row) and rows m = 8 (i / 4) + 4 (l / 32) + (i % 4), i = 0..15 (A rows).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

constexpr int kThreads = 256;
constexpr int kTile = 256;                     // rows of A and of B per tile
constexpr int kHalf = 128;                     // rows per wave along A or B
constexpr int kRowBytes = 128;                 // K bytes per row per stage
constexpr int kSubBytes = kTile * 32 + 32;     // one K sub-buffer (+32 B bank shift)
constexpr int kOpBytes = 4 * kSubBytes;        // one operand, one stage
constexpr int kStageBytes = 2 * kOpBytes;      // A + B
constexpr int kMainLds = 2 * kStageBytes;      // double buffered
constexpr int kVocabTile = kTile;              // vocabulary entries per tile

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int kPerStage = 64;  // elements of K per stage
  static constexpr int kSize = 2;
};
template <> struct Elem<float> {
  static constexpr int kPerStage = 32;
  static constexpr int kSize = 4;
};

// ---------------------------------------------------------------- LDS layout

__device__ __forceinline__ int lds_g(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }

// Row of the loader: thread t moves 16-byte chunk t % 8 of tile rows
// row_base(t) + 32 i, i = 0..7.  Inside a wave the eight row groups are
// ordered 0,4,1,5,2,6,3,7 so that lanes t and t + 8 write rows 4 apart
// (different banks for 16-lane write groups).
__device__ __forceinline__ int loader_row_base(int tid) {
  const int q = (tid >> 3) & 7;
  return ((tid >> 6) << 3) + (((q & 1) << 2) | (q >> 1));
}
__device__ __forceinline__ int loader_lds_off(int tid) {
  const int r = loader_row_base(tid);
  const int kc = tid & 7;
  return (kc >> 1) * kSubBytes + r * 32 + (((kc & 1) ^ lds_g(r)) << 4);
}
// Per-lane part of a fragment read: row lane % 32 of a 32-row block.
__device__ __forceinline__ int frag_lds_off(int lane) {
  const int r = lane & 31;
  const int h = lane >> 5;
  return r * 32 + ((h ^ lds_g(r)) << 4);
}

// Token permutation used when B holds tokens: within each 128-row wave half,
// MFMA column (nt, j) (nt = 0..3 the accumulator index, j = lane % 32) reads
// LDS row 32 nt + j, which is loaded with token 4 j + nt, so that one lane owns
// four consecutive tokens.  tok_of_lds_row maps an LDS row to its token.
__device__ __forceinline__ int tok_of_lds_row(int r) {
  return (r & kHalf) | (((r & 31) << 2) + ((r & (kHalf - 1)) >> 5));
}

// ------------------------------------------------------------------- MFMA

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
  __device__ __forceinline__ static void run(f32x16& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  __device__ __forceinline__ static void run(f32x16& c, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[j]), __uint_as_float(b[j]),
                                               c, 0, 0, 0);
  }
};

// ------------------------------------------------------- operand row source

// Where the 256 rows of one operand tile come from.  Logical row r of the
// tile is row0 + r; rows at or beyond nrows are clamped to nrows - 1 (their
// results are never stored); with a gather list the physical row is
// gather[logical].  With perm_tokens, LDS row R holds logical row
// tok_of_lds_row(R).
struct RowSource {
  const char* base;
  int64_t ld;              // row stride in bytes
  const int32_t* gather;   // nullable
  int64_t row0;
  int64_t nrows;           // >= 1
};

struct RowPtrs {
  const char* p[8];
};

template <bool kPerm>
__device__ __forceinline__ RowPtrs make_row_ptrs(const RowSource& s, int tid) {
  RowPtrs rp;
  const int kc = tid & 7;
  const int rb = loader_row_base(tid);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int lr = kPerm ? tok_of_lds_row(rb + 32 * i) : rb + 32 * i;
    int64_t r = s.row0 + lr;
    if (r >= s.nrows) r = s.nrows - 1;
    const int64_t phys = s.gather ? (int64_t)s.gather[r] : r;
    rp.p[i] = s.base + phys * s.ld + kc * 16;
  }
  return rp;
}

struct Staged {
  u32x4 a[8];
  u32x4 b[8];
};

__device__ __forceinline__ void load_stage(Staged& st, const RowPtrs& pa, const RowPtrs& pb,
                                           int64_t kbyte) {
#pragma unroll
  for (int i = 0; i < 8; ++i) st.a[i] = *(const u32x4*)(pa.p[i] + kbyte);
#pragma unroll
  for (int i = 0; i < 8; ++i) st.b[i] = *(const u32x4*)(pb.p[i] + kbyte);
}

// wr = lds stage base + loader_lds_off(tid)
__device__ __forceinline__ void store_stage(char* wr, const Staged& st) {
#pragma unroll
  for (int i = 0; i < 8; ++i) *(u32x4*)(wr + i * 1024) = st.a[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) *(u32x4*)(wr + kOpBytes + i * 1024) = st.b[i];
}

// rd_a / rd_b = lds stage base + operand offset + wave-half rows + frag_lds_off
template <typename T>
__device__ __forceinline__ void compute_stage(f32x16 (&acc)[4][4], const char* rd_a,
                                              const char* rd_b) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 fa[4], fb[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) fa[mt] = *(const u32x4*)(rd_a + s * kSubBytes + mt * 32 * 32);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) fb[nt] = *(const u32x4*)(rd_b + s * kSubBytes + nt * 32 * 32);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) Mma<T>::run(acc[mt][nt], fa[mt], fb[nt]);
  }
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;
}

// acc += A_tile(256 x K) * B_tile(256 x K)^T over nstages stages of 128 bytes.
// Double-buffered LDS with register staging: the global loads of stage k + 1
// are in flight while stage k feeds the MFMAs.  Ends with a barrier, so the
// caller may reuse LDS afterwards.
template <typename T>
__device__ __forceinline__ void tile_mainloop(f32x16 (&acc)[4][4], char* lds, const RowPtrs& pa,
                                              const RowPtrs& pb, int nstages, int tid) {
  if (nstages <= 0) return;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wa = wave & 1;
  const int wb = wave >> 1;
  const int wr_off = loader_lds_off(tid);
  const int rd_off = frag_lds_off(lane);
  const int rd_a = rd_off + wa * kHalf * 32;
  const int rd_b = kOpBytes + rd_off + wb * kHalf * 32;
  Staged st;
  load_stage(st, pa, pb, 0);
  store_stage(lds + wr_off, st);
  __syncthreads();
  for (int k = 0; k < nstages; ++k) {
    char* cur = lds + (k & 1) * kStageBytes;
    char* nxt = lds + ((k + 1) & 1) * kStageBytes;
    const bool more = k + 1 < nstages;
    if (more) load_stage(st, pa, pb, (int64_t)(k + 1) * kRowBytes);
    compute_stage<T>(acc, cur + rd_a, cur + rd_b);
    if (more) store_stage(nxt + wr_off, st);
    __syncthreads();
  }
}

// ------------------------------------------------------- XCD-aware mapping

// Workgroups are dispatched round-robin over the 8 XCDs (slot s lands on XCD
// s % 8), and each XCD has its own L2.  This maps slot s to a tile of a
// TM x TN grid so that the 32 slots that run together on one XCD form a
// GA x GB block of tiles (GA * GB = 32): they then share GA A-tiles and GB
// B-tiles through that XCD's L2 while they step through K in lockstep.
// Returns false for slots that fall outside the grid.
__device__ __forceinline__ bool xcd_tile(int slot, int TM, int TN, int GA, int GB, int& tm,
                                         int& tn) {
  const int x = slot & 7;
  const int k = slot >> 3;
  const int sb = ((k >> 5) << 3) + x;
  const int e = k & 31;
  const int sbn_count = (TN + GB - 1) / GB;
  const int sbm = sb / sbn_count;
  const int sbn = sb - sbm * sbn_count;
  tm = sbm * GA + (e % GA);
  tn = sbn * GB + (e / GA);
  return tm < TM && tn < TN;
}

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite here).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

template <typename T> struct Store4;
template <> struct Store4<bf16_t> {
  __device__ __forceinline__ static void run(void* p, float a, float b, float c, float d) {
    u32x2 v;
    v[0] = bf16_bits(a) | (bf16_bits(b) << 16);
    v[1] = bf16_bits(c) | (bf16_bits(d) << 16);
    *(u32x2*)p = v;
  }
};
template <> struct Store4<float> {
  __device__ __forceinline__ static void run(void* p, float a, float b, float c, float d) {
    f32x4 v = {a, b, c, d};
    *(f32x4*)p = v;
  }
};

}  // namespace lce
