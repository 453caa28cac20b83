// Device-side building blocks shared by every kernel of the fused
// linear + cross-entropy path on gfx950 (CDNA4, wave64, MFMA, 160 KB LDS).
//
// The tile engine computes a 256 x 256 fp32 block C = A * B^T where both
// operands are "K-contiguous" (each logical row holds its K elements
// contiguously): that is how H [N, d] and W [V, d] are stored, and how the
// backward pass lays out its bounded G / G^T / W^T / H^T buffers.
//
//  * 512 threads = 8 waves, two per SIMD, in a 2 x 4 arrangement: wave
//    (wa, wb) owns A rows [128 wa, 128 wa + 128) and B rows [64 wb, 64 wb +
//    64) of the tile, held as 4 x 2 accumulators of the 32x32 MFMA (16 fp32
//    per lane each, 128 accumulator registers per lane).  Two waves per SIMD
//    let one wave's MFMAs run while the other waits on a barrier or on LDS.
//  * K advances 128 bytes per pipeline stage (64 bf16 or 32 fp32).  An
//    operand stage is 256 rows x 128 B = 32 KB of LDS.  A has three stage
//    buffers and B two (160 KB, all of a CU's LDS): A is loaded two stages
//    ahead, B one.  A stage then only has to wait for its 32 KB of B to
//    stream in, not for all 64 KB (measured 5-10% faster than double
//    buffering both operands).  The eight 16-byte chunks of
//    row r are XOR-swizzled (chunk c sits at position c ^ swz(r), swz(r) =
//    (r ^ (r >> 3)) & 7) so that the fragment reads of 8 or 16 consecutive
//    rows hit distinct banks.
//  * Global -> LDS moves use the gfx950 direct-to-LDS 16-byte load
//    (buffer_load_dwordx4 ... lds): each wave instruction fills 1 KB of LDS
//    (8 swizzled rows), each lane fetching the chunk that lands at its slot,
//    so the 8 lanes of a row read its 128 contiguous bytes.  No staging
//    registers.  Stage k issues B(k + 1), then A(k + 2), and closes with one
//    wait that leaves only A(k + 2) in flight, and one barrier.
//  * Fragment reads are double buffered in registers: the 8 fragments of
//    MFMA step s + 1 are requested before the 16 MFMAs of step s issue.  A
//    lane's fragment address is one base register XOR a compile-time
//    constant plus an immediate offset.
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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

constexpr int kThreads = 512;
constexpr int kTile = 256;                     // rows of A and of B per tile
constexpr int kHalf = 128;                     // rows per wave along A
constexpr int kWaveN = 64;                     // rows per wave along B
constexpr int kNT = 2;                         // 32-row MFMA blocks per wave along B
constexpr int kRowBytes = 128;                 // K bytes per row per stage
constexpr int kOpBytes = kTile * kRowBytes;    // 32 KB: one operand, one stage
constexpr int kLdsA = 0;                       // A stage buffers 0..2
constexpr int kLdsB = 3 * kOpBytes;            // B stage buffers 0..1
constexpr int kMainLds = 5 * kOpBytes;         // 160 KB
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

__device__ __forceinline__ int lds_swz(int row) { return (row ^ (row >> 3)) & 7; }

// Token permutation used when B holds tokens: within each 64-row wave slice,
// MFMA column (nt, j) (nt = 0..1 the accumulator index, j = lane % 32) reads
// LDS row 32 nt + j, which is loaded with token 2 j + nt, so that one lane owns
// two consecutive tokens.  tok_of_lds_row maps an LDS row to its token.
__device__ __forceinline__ int tok_of_lds_row(int r) {
  return (r & ~(kWaveN - 1)) | ((r & 31) << 1) | ((r >> 5) & 1);
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
// gather[logical].
struct RowSource {
  const char* base;
  int64_t ld;              // row stride in bytes
  const int32_t* gather;   // nullable
  int64_t row0;
  int64_t nrows;           // >= 1
  int64_t phys_rows;       // rows of the source tensor (bounds of the gathered rows)
};

// Sources of the 4 direct-to-LDS loads one wave issues per operand and
// stage: a buffer resource (wave-uniform, in SGPRs) and 32-bit per-lane byte
// offsets; the stage advance goes in the scalar soffset, so the loop carries
// no per-lane address arithmetic (buffer_load_dwordx4 ... offen lds).  The
// resource covers exactly the source tensor: an offset past its end reads
// zeros instead of faulting.  Load i of wave w fills LDS rows 8 b .. 8 b + 7
// with b = 8 i + w; lane L covers row 8 b + L / 8 at slot L % 8, which must
// hold chunk (L % 8) ^ swz(row).  With kPerm (B holding tokens) LDS row R
// holds logical row tok_of_lds_row(R).  Offsets stay below 4 GB (the host
// checks the tensor sizes).
constexpr int kBufferFlags = 0x00020000;  // raw 32-bit buffer, gfx9 family

struct RowPtrs {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[4];
  uint32_t stride;  // bytes the source advances per stage
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int64_t bytes) {
  const int64_t lim = 0xFFFFFFFFll;
  const uint32_t n = (uint32_t)(bytes < lim ? bytes : lim);
  // Base and size are wave-uniform, but where the compiler cannot prove it
  // the resource stays in VGPRs and every load becomes a readfirstlane /
  // compare / exec-mask loop.  readfirstlane states the uniformity.
  const uint64_t p = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint32_t nu = __builtin_amdgcn_readfirstlane(n);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, (int)nu,
                                           kBufferFlags);
}

template <bool kPerm>
__device__ __forceinline__ RowPtrs make_row_ptrs(const RowSource& s, int tid) {
  RowPtrs rp;
  const int w = tid >> 6;
  const int L = tid & 63;
  // direct rows: the resource starts at row0; gathered rows: at row 0
  const int64_t first = s.gather ? 0 : s.row0;
  const int64_t rows = s.gather ? s.phys_rows : s.nrows - s.row0;
  rp.rsrc = make_rsrc(s.base + first * s.ld, rows * s.ld);
  // Row numbers stay 32-bit (every size is below 2^31): as 64-bit values the
  // compiler hoisted the four per-lane rows out of the persistent item loop
  // and spilled them.
  const int row0 = (int)s.row0;
  const int last = (int)s.nrows - 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (8 * i + w) + (L >> 3);
    const int chunk = (L & 7) ^ lds_swz(row);
    const int lr = kPerm ? tok_of_lds_row(row) : row;
    const int r = min(row0 + lr, last);
    const int rel = s.gather ? s.gather[r] : r - row0;
    rp.off[i] = (uint32_t)rel * (uint32_t)s.ld + chunk * 16;
  }
  rp.stride = kRowBytes;
  return rp;
}

// K-major B operand: the source is row-major [K][n] (each K row holds the
// tile's 256 operand rows contiguously, e.g. W [vocabulary][hidden] when K
// runs over the vocabulary), so a stage is 64 K rows x 256 operand rows of
// bf16, 512 bytes per K row.  LDS row v (0..63) holds K row k0 + 64 s + v;
// its sixteen-byte chunk c sits at position c ^ (4 (v % 4)), so that the
// transposing fragment reads below (8 K rows x 64 bytes per instruction)
// hit each bank group exactly twice.  Load i of wave w fills LDS rows
// 2 (8 i + w) and 2 (8 i + w) + 1, lane L the chunk at position L % 32 of
// row 2 (8 i + w) + L / 32.  The resource covers K rows [k0, k0 + krows):
// rows past it read as zeros.
__device__ __forceinline__ RowPtrs make_kmajor_ptrs(const char* base, int64_t ld, int64_t k0,
                                                    int64_t krows, int64_t n0, int tid) {
  RowPtrs rp;
  const int w = tid >> 6;
  const int L = tid & 63;
  rp.rsrc = make_rsrc(base + k0 * ld, (krows > 0 ? krows : 0) * ld);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = 2 * (8 * i + w) + (L >> 5);
    const int c = (L & 31) ^ (4 * (v & 3));
    rp.off[i] = (uint32_t)(v * ld + (n0 + 8 * c) * 2);
  }
  rp.stride = (uint32_t)(64 * ld);
  return rp;
}

#define LCE_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Issue the 4 direct-to-LDS loads of one wave for one operand stage.
__device__ __forceinline__ void load_op(char* buf, const RowPtrs& p, uint32_t kbyte, int wave_u) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(p.rsrc, LCE_LDS_PTR(buf + (8 * i + wave_u) * 1024), 16,
                                             p.off[i], kbyte, 0, 0);
}

// Fragment reads of MFMA step s (32 bytes of K): 4 A fragments (32-row
// blocks mt) and 2 B fragments.  a_base / b_base = per-lane offset of row
// (wave slice + lane % 32), slot bits holding h ^ (r & 7) ^ (r >> 3); step s
// XORs 2 s into the slot, a 32-row block adds 4 KB and XORs 4 into the slot
// for odd blocks (slot bits are byte-offset bits 4..6, hence XOR, not add).
// Issued in the order the MFMAs consume them (mma_step runs (mt, nt) =
// (0,0) (0,1) (1,0) (1,1) ...): the first MFMA of a step then waits for 2 of
// the 6 reads instead of 5 (1.5-6% faster).
__device__ __forceinline__ void load_frags_ab(u32x4 (&fa)[4], u32x4 (&fb)[kNT], const char* ca,
                                              const char* cb, int a_base, int b_base, int s) {
  const int ea = a_base ^ (32 * s), oa = a_base ^ ((32 * s) ^ 64);
  const int eb = b_base ^ (32 * s), ob = b_base ^ ((32 * s) ^ 64);
  fa[0] = *(const u32x4*)(ca + ea);
  fb[0] = *(const u32x4*)(cb + eb);
  fb[1] = *(const u32x4*)(cb + ob + 4096);
  fa[1] = *(const u32x4*)(ca + oa + 4096);
  fa[2] = *(const u32x4*)(ca + ea + 8192);
  fa[3] = *(const u32x4*)(ca + oa + 12288);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// One B fragment (32 operand rows x 16 K) from a K-major stage with the
// gfx950 transposing LDS read ds_read_b64_tr_b16: within each group of 16
// lanes, lane i receives, as element e of its result, element i % 4 of the
// 8 bytes lane 4 e + i / 4 addressed.  Lane l addresses K row kb + 8 (l / 32)
// + (l % 16) / 4 (+ 4 for the second read) at operand row nb + 16 ((l / 16)
// % 2) + 4 (l % 4), so that it receives operand row nb + l % 32 at K rows
// kb + 8 (l / 32) + 0..7: the layout of a row-major fragment.  bt_base is
// that lane's byte address of K row kb = 0 (swizzle included).
__device__ __forceinline__ u32x4 load_frag_bt(const char* cb, int bt_base, int s) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const char* p = cb + bt_base + s * (16 * 512);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)LCE_LDS_PTR(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)LCE_LDS_PTR(p + 4 * 512));
  const u32x2 a = __builtin_bit_cast(u32x2, lo);
  const u32x2 b = __builtin_bit_cast(u32x2, hi);
  u32x4 r = {a[0], a[1], b[0], b[1]};
  return r;
}

// Byte address of lane l's first transposed read for 32-row block nt of the
// wave's 64 operand rows (see load_frag_bt).
__device__ __forceinline__ int bt_lane_base(int wb, int nt, int lane) {
  const int v = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int n = wb * kWaveN + 32 * nt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int pos = (n >> 3) ^ (4 * (v & 3));
  return v * 512 + pos * 16 + (n & 7) * 2;
}

// Fragment reads of MFMA step s with a K-major B (two transposing reads per
// B fragment, eight reads per step), in the order the MFMAs consume them.
__device__ __forceinline__ void load_frags_abt(u32x4 (&fa)[4], u32x4 (&fb)[kNT], const char* ca,
                                               const char* cb, int a_base, int bt0, int bt1,
                                               int s) {
  const int ea = a_base ^ (32 * s), oa = a_base ^ ((32 * s) ^ 64);
  fa[0] = *(const u32x4*)(ca + ea);
  fb[0] = load_frag_bt(cb, bt0, s);
  fb[1] = load_frag_bt(cb, bt1, s);
  fa[1] = *(const u32x4*)(ca + oa + 4096);
  fa[2] = *(const u32x4*)(ca + ea + 8192);
  fa[3] = *(const u32x4*)(ca + oa + 12288);
}

typedef f32x16 Acc[4][kNT];

template <typename T>
__device__ __forceinline__ void mma_step(Acc& acc, const u32x4 (&fa)[4], const u32x4 (&fb)[kNT]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) Mma<T>::run(acc[mt][nt], fa[mt], fb[nt]);
}

__device__ __forceinline__ void zero_acc(Acc& acc) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;
}

// Instruction order of one stage body (bf16; sched_group_barrier masks:
// 0x008 MFMA, 0x020 VMEM read, 0x100 DS read).  Left alone, the compiler
// funnels every A fragment through one register quad and waits on each LDS
// read right in front of its two MFMAs.  Here: the 6 fragment reads of step
// 0 go first; the previous stage's step-3 MFMAs (kPrev) cover their latency
// and carry the nl direct-to-LDS loads of this stage; then each step's 8
// MFMAs alternate with the 6 fragment reads of the following step.
template <bool kPrev, int nl, int kReads = 6>
__device__ __forceinline__ void schedule_body() {
  __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
  if (kPrev) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (q < nl) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  } else if (nl) {
    __builtin_amdgcn_sched_group_barrier(0x020, nl, 0);
  }
#pragma unroll
  for (int s = 0; s < 3; ++s) {
#pragma unroll
    for (int q = 0; q < kReads; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if (kReads < 8) __builtin_amdgcn_sched_group_barrier(0x008, 8 - kReads, 0);
  }
}

// End of a stage: wait until this wave's loads for the next stage have
// landed (all but the newest kInFlight load instructions: loads complete in
// issue order) and its fragment reads have returned, then meet the other
// waves.  The barrier is issued directly: __syncthreads() would add a release
// fence, i.e. wait for every load, including A(k + 2), which is meant to stay
// in flight.  sched_barrier keeps the compiler from moving work across.
template <int kInFlight>
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  // s_waitcnt: vmcnt in bits 3:0, expcnt 6:4 (7 = no wait), lgkmcnt 11:8
  __builtin_amdgcn_s_waitcnt(0x0070 | kInFlight);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Stage k of the main loop, software-pipelined across the barrier: MFMA
// steps 0-2 of stage k run here, while step 3's fragments are read into f3a /
// f3b and their MFMAs run at the start of the next body (kPrev), after the
// barrier, where they hide the barrier skew and the next stage's first LDS
// reads.  Reads A buffer sa and B buffer k & 1.  Loads B(k + 1) (kLB) into
// the B buffer read by stage k - 1, then A(k + 2) (kLA) into A buffer sa2,
// also last read by stage k - 1: both were free at the previous barrier.
// kBT: B is K-major (make_kmajor_ptrs) and its fragments come from the
// transposing reads; b_base then holds the lane's base for block nt = 0 and
// b_base1 the one for nt = 1.
template <bool kBT>
__device__ __forceinline__ void load_frags(u32x4 (&fa)[4], u32x4 (&fb)[kNT], const char* ca,
                                           const char* cb, int a_base, int b_base, int b_base1,
                                           int s) {
  if constexpr (kBT)
    load_frags_abt(fa, fb, ca, cb, a_base, b_base, b_base1, s);
  else
    load_frags_ab(fa, fb, ca, cb, a_base, b_base, s);
}

// Stage body with a K-major B (kBT).  The compiler puts a full vmcnt(0) in
// front of any transposing LDS read that follows a direct-to-LDS load still
// in flight (it does not for ordinary LDS reads), so all 16 transposing reads
// of the stage (4 steps x 2 blocks x 2 halves) are issued before the stage's
// loads; the wait then falls on the next stage's first read, by which time
// only A(k + 2), issued a stage earlier, can still be outstanding.
template <typename T, bool kPrev, bool kLB, bool kLA>
__device__ __forceinline__ void stage_body_bt(Acc& acc, char* lds, int k, int sa, int sa2,
                                              int a_base, int b_base, int b_base1,
                                              const RowPtrs& pa, const RowPtrs& pb, int wave_u,
                                              u32x4 (&f3a)[4], u32x4 (&f3b)[kNT]) {
  const char* ca = lds + kLdsA + sa * kOpBytes;
  const char* cb = lds + kLdsB + (k & 1) * kOpBytes;
  u32x4 fa[3][4], fb[3][kNT];
  auto a_frags = [&](u32x4 (&f)[4], int s) {
    const int ea = a_base ^ (32 * s), oa = a_base ^ ((32 * s) ^ 64);
    f[0] = *(const u32x4*)(ca + ea);
    f[1] = *(const u32x4*)(ca + oa + 4096);
    f[2] = *(const u32x4*)(ca + ea + 8192);
    f[3] = *(const u32x4*)(ca + oa + 12288);
  };
  a_frags(fa[0], 0);
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    fb[s][0] = load_frag_bt(cb, b_base, s);
    fb[s][1] = load_frag_bt(cb, b_base1, s);
  }
  u32x4 nb0 = load_frag_bt(cb, b_base, 3), nb1 = load_frag_bt(cb, b_base1, 3);
  if (kLB) load_op(lds + kLdsB + ((k + 1) & 1) * kOpBytes, pb, (uint32_t)(k + 1) * pb.stride, wave_u);
  if (kLA) load_op(lds + kLdsA + sa2 * kOpBytes, pa, (uint32_t)((k + 2) * kRowBytes), wave_u);
  if (kPrev) mma_step<T>(acc, f3a, f3b);
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if (s < 2) a_frags(fa[s + 1], s + 1);
    else a_frags(f3a, 3);
    mma_step<T>(acc, fa[s], fb[s]);
  }
  f3b[0] = nb0;
  f3b[1] = nb1;
  // reads: the 4 A fragments of step 0 and the 16 transposing reads first;
  // then the previous stage's step-3 MFMAs carry the loads; then each step's
  // 8 MFMAs alternate with the following step's 4 A reads
  __builtin_amdgcn_sched_group_barrier(0x100, 20, 0);
  if (kPrev) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (q < (kLB ? 4 : 0) + (kLA ? 4 : 0)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  } else if (kLB || kLA) {
    __builtin_amdgcn_sched_group_barrier(0x020, (kLB ? 4 : 0) + (kLA ? 4 : 0), 0);
  }
#pragma unroll
  for (int s = 0; s < 3; ++s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  }
  if (kLB) stage_barrier<kLA ? 4 : 0>();
}

template <typename T, bool kPrev, bool kLB, bool kLA, bool kBT = false>
__device__ __forceinline__ void stage_body(Acc& acc, char* lds, int k, int sa, int sa2, int a_base,
                                           int b_base, int b_base1, const RowPtrs& pa,
                                           const RowPtrs& pb, int wave_u, u32x4 (&f3a)[4],
                                           u32x4 (&f3b)[kNT]) {
  if constexpr (kBT) {
    stage_body_bt<T, kPrev, kLB, kLA>(acc, lds, k, sa, sa2, a_base, b_base, b_base1, pa, pb,
                                      wave_u, f3a, f3b);
    return;
  }
  const char* ca = lds + kLdsA + sa * kOpBytes;
  const char* cb = lds + kLdsB + (k & 1) * kOpBytes;
  const uint32_t bstride = kBT ? pb.stride : (uint32_t)kRowBytes;
  u32x4 fa[3][4], fb[3][kNT];
  load_frags<kBT>(fa[0], fb[0], ca, cb, a_base, b_base, b_base1, 0);
  if (kLB) load_op(lds + kLdsB + ((k + 1) & 1) * kOpBytes, pb, (uint32_t)(k + 1) * bstride, wave_u);
  if (kLA) load_op(lds + kLdsA + sa2 * kOpBytes, pa, (uint32_t)((k + 2) * kRowBytes), wave_u);
  if (kPrev) mma_step<T>(acc, f3a, f3b);
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if (s < 2) load_frags<kBT>(fa[s + 1], fb[s + 1], ca, cb, a_base, b_base, b_base1, s + 1);
    else load_frags<kBT>(f3a, f3b, ca, cb, a_base, b_base, b_base1, 3);
    mma_step<T>(acc, fa[s], fb[s]);
  }
  if constexpr (sizeof(T) == 2)
    schedule_body<kPrev, (kLB ? 4 : 0) + (kLA ? 4 : 0), kBT ? 8 : 6>();
  // B(k + 1) and A(k + 1) must have landed; A(k + 2), issued last, may not
  if (kLB) stage_barrier<kLA ? 4 : 0>();
}

__device__ __forceinline__ int next3(int b) { return b == 2 ? 0 : b + 1; }

// acc += A_tile(256 x K) * B_tile(256 x K)^T over nstages stages of 128 bytes.
// Ends with a barrier, so the caller may reuse LDS afterwards.  Stage j of A
// lives in A buffer j % 3, stage j of B in B buffer j % 2.
// kBT: B is a K-major operand (make_kmajor_ptrs), read with the transposing
// fragment reads (bf16 only).
template <typename T, bool kBT = false>
__device__ __forceinline__ void tile_mainloop(Acc& acc, char* lds, const RowPtrs& pa,
                                              const RowPtrs& pb, int nstages, int tid) {
  static_assert(!kBT || sizeof(T) == 2, "the transposing B path is bf16 only");
  if (nstages <= 0) return;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wa = wave & 1;
  const int wb = wave >> 1;
  const int r = lane & 31;
  const int x = ((lane >> 5) ^ (r & 7) ^ (r >> 3)) << 4;
  const int a_base = (wa * kHalf + r) * kRowBytes + x;
  const int b_base = kBT ? bt_lane_base(wb, 0, lane) : (wb * kWaveN + r) * kRowBytes + x;
  const int b_base1 = kBT ? bt_lane_base(wb, 1, lane) : 0;
  // prologue: A(0), B(0), A(1); stage 0 needs the first two
  load_op(lds + kLdsA, pa, 0, wave_u);
  load_op(lds + kLdsB, pb, 0, wave_u);
  if (nstages > 1) {
    load_op(lds + kLdsA + kOpBytes, pa, kRowBytes, wave_u);
    stage_barrier<4>();
  } else {
    stage_barrier<0>();
  }
  u32x4 f3a[4], f3b[kNT];
  if (nstages == 1) {
    stage_body<T, false, false, false, kBT>(acc, lds, 0, 0, 2, a_base, b_base, b_base1, pa, pb,
                                            wave_u, f3a, f3b);
  } else if (nstages == 2) {
    stage_body<T, false, true, false, kBT>(acc, lds, 0, 0, 2, a_base, b_base, b_base1, pa, pb,
                                           wave_u, f3a, f3b);
    stage_body<T, true, false, false, kBT>(acc, lds, 1, 1, 0, a_base, b_base, b_base1, pa, pb,
                                           wave_u, f3a, f3b);
  } else {
    stage_body<T, false, true, true, kBT>(acc, lds, 0, 0, 2, a_base, b_base, b_base1, pa, pb,
                                          wave_u, f3a, f3b);
    int sa = 1, sa2 = 0;  // k % 3 and (k + 2) % 3
    int k = 1;
    for (; k + 2 < nstages; ++k) {
      stage_body<T, true, true, true, kBT>(acc, lds, k, sa, sa2, a_base, b_base, b_base1, pa, pb,
                                           wave_u, f3a, f3b);
      sa = next3(sa);
      sa2 = next3(sa2);
    }
    stage_body<T, true, true, false, kBT>(acc, lds, k, sa, sa2, a_base, b_base, b_base1, pa, pb,
                                          wave_u, f3a, f3b);
    stage_body<T, true, false, false, kBT>(acc, lds, k + 1, next3(sa), sa2, a_base, b_base,
                                           b_base1, pa, pb, wave_u, f3a, f3b);
  }
  mma_step<T>(acc, f3a, f3b);
  __syncthreads();
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

// Two fp32 values -> packed bf16, round to nearest even: one vector
// conversion, which the backend emits as a single v_cvt_pk_bf16_f32 (the
// same rounding as bf16_bits for finite values, at one instruction per pair
// instead of four per value).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

template <typename T> struct Store2;
template <> struct Store2<bf16_t> {
  __device__ __forceinline__ static void run(void* p, float a, float b) {
    *(uint32_t*)p = pack_bf16x2(a, b);
  }
};
template <> struct Store2<float> {
  __device__ __forceinline__ static void run(void* p, float a, float b) {
    f32x2 v = {a, b};
    *(f32x2*)p = v;
  }
};

template <typename T> struct Store4;
template <> struct Store4<bf16_t> {
  __device__ __forceinline__ static void run(void* p, float a, float b, float c, float d) {
    u32x2 v;
    v[0] = pack_bf16x2(a, b);
    v[1] = pack_bf16x2(c, d);
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
