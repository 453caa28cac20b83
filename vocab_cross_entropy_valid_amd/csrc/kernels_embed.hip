// Input side of a tied table: the masked embedding gather and the
// deterministic scatter-sum of its gradient into dW.
//
// MaximusLLM page, section 2.3 (padding-aware sparse index engine): only
// positions whose id is not the padding id are looked up, the others get a
// zero vector, and the valid mask is built on the device with no host
// round trip.  The valid index comes from the same compaction kernel as the
// loss's (with pad_id in place of ignore_index).  The gradient of the lookup
// is dW[v] += sum of dX[n] over valid n with id[n] = v; rows sharing an id
// are summed in a fixed order (ascending position inside fixed 64-row
// chunks, then the chunks in order) so the result is bitwise reproducible.
// The rows are grouped by id with a stable least-significant-digit radix
// sort written here (8-bit digits, wave ballots for the ranks of equal
// digits), so the whole pass is this file's kernels.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace lce {

// ----------------------------------------------------------------- gather
// One thread per 16-byte chunk of X (row bytes are a multiple of 16).
__global__ __launch_bounds__(256) void embed_gather_kernel(const char* __restrict__ W,
                                                           const int64_t* __restrict__ ids,
                                                           int64_t pad_id, int64_t N, int64_t V,
                                                           int64_t row_bytes,
                                                           char* __restrict__ X) {
  const int64_t cpr = row_bytes / 16;
  const int64_t total = N * cpr;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * 256) {
    const int64_t n = q / cpr;
    const int64_t c = q - n * cpr;
    const int64_t id = ids[n];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (id != pad_id && id >= 0 && id < V) v = *(const u32x4*)(W + id * row_bytes + 16 * c);
    *(u32x4*)(X + n * row_bytes + 16 * c) = v;
  }
}

hipError_t launch_embed_gather(const void* W, const int64_t* ids, int64_t pad_id, int64_t N,
                               int64_t V, int64_t row_bytes, void* X, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const int64_t total = N * (row_bytes / 16);
  const int grid = (int)std::min<int64_t>((total + 255) / 256, 1 << 16);
  hipLaunchKernelGGL(embed_gather_kernel, dim3(grid), dim3(256), 0, s, (const char*)W, ids,
                     pad_id, N, V, row_bytes, (char*)X);
  return hipGetLastError();
}

// ------------------------------------------------------ backward: keys
// key[i] = id of the i-th valid row (valid_idx ascending), val[i] = its
// position; entries past the valid count get the sentinel key V (they sort
// last and are never summed).
__global__ __launch_bounds__(256) void embed_keys_kernel(const int64_t* __restrict__ ids,
                                                         const int32_t* __restrict__ valid_idx,
                                                         const int32_t* __restrict__ valid_count,
                                                         int64_t N, int64_t V,
                                                         uint32_t* __restrict__ key,
                                                         int32_t* __restrict__ val) {
  const int count = *valid_count;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  if (i < count) {
    const int r = valid_idx[i];
    key[i] = (uint32_t)ids[r];
    val[i] = r;
  } else {
    key[i] = (uint32_t)V;
    val[i] = 0;
  }
}

// ---------------------------------------------- backward: radix sort
//
// Stable sort of (key, value) pairs by key, least significant 9-bit digit
// first (two passes cover every vocabulary below 2^18).  A pass over n pairs
// runs two kernels:
//   hist     block b counts the digits of its tile of kSortTile pairs (LDS
//            integer atomics: exact counts, order-free) into
//            hist[digit * nblocks + b];
//   scatter  block b first derives where its run of each digit starts in the
//            output (the pairs of smaller digits, plus those of the same
//            digit in earlier tiles), then walks its tile in order, 1024
//            pairs at a time: a lane's rank among the lanes of its wave with
//            the same digit comes from nine ballots (one per digit bit) and a
//            popcount, the waves' digit counts are scanned in wave order, and
//            the pair lands after every pair of that digit already placed by
//            earlier rows, waves and lanes.
// Equal keys keep their input order (tiles, rows, waves and lanes are all
// taken in ascending input position), which is what makes the sort stable
// and the later sums bitwise reproducible.
constexpr int kSortThreads = 1024;
constexpr int kSortTile = 2048;  // pairs per block and pass: 2 rows of 1024
constexpr int kRadixBits = 9;
constexpr int kRadix = 1 << kRadixBits;
constexpr int kSortWaves = kSortThreads / 64;

__global__ __launch_bounds__(kSortThreads) void radix_hist_kernel(const uint32_t* __restrict__ key,
                                                                  int64_t n, int shift,
                                                                  int32_t* __restrict__ hist,
                                                                  int nblocks) {
  __shared__ int h[kRadix];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  if (tid < kRadix) h[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSortTile / kSortThreads; ++r) {
    const int64_t i = (int64_t)b * kSortTile + r * kSortThreads + tid;
    if (i < n) atomicAdd(&h[(key[i] >> shift) & (kRadix - 1)], 1);
  }
  __syncthreads();
  if (tid < kRadix) hist[(int64_t)tid * nblocks + b] = h[tid];
}

__device__ __forceinline__ int wg_exclusive_scan(int v, int* wtot, int* wbase, int& total);

__global__ __launch_bounds__(kSortThreads) void radix_scatter_kernel(
    const uint32_t* __restrict__ key_in, const int32_t* __restrict__ val_in,
    uint32_t* __restrict__ key_out, int32_t* __restrict__ val_out, int64_t n, int shift,
    const int32_t* __restrict__ hist, int nblocks) {
  __shared__ int cnt[kSortWaves][kRadix];  // per wave: pairs of each digit in this row
  __shared__ int run[kRadix];              // next output slot of each digit
  __shared__ int wtot[16];
  __shared__ int wbase[17];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.x;
  // output start of this block's run of digit tid: every pair of a smaller
  // digit (exclusive scan of the digit totals) plus the pairs of the same
  // digit in earlier tiles
  int total = 0, before = 0;
  if (tid < kRadix)
    for (int q = 0; q < nblocks; ++q) {
      const int c = hist[(int64_t)tid * nblocks + q];
      total += c;
      before += q < b ? c : 0;
    }
  int all;
  const int start = wg_exclusive_scan(tid < kRadix ? total : 0, wtot, wbase, all);
  if (tid < kRadix) run[tid] = start + before;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes below this one
#pragma unroll 1
  for (int r = 0; r < kSortTile / kSortThreads; ++r) {
    const int64_t i = (int64_t)b * kSortTile + r * kSortThreads + tid;
    const bool valid = i < n;
    const uint32_t k = valid ? key_in[i] : 0u;
    const int32_t v = valid ? val_in[i] : 0;
    const int d = (int)((k >> shift) & (kRadix - 1));
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < kRadixBits; ++bit) {
      const uint64_t m = __ballot((d >> bit) & 1);
      peers &= ((d >> bit) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
#pragma unroll
    for (int q = 0; q < kSortWaves * kRadix / kSortThreads; ++q)
      (&cnt[0][0])[q * kSortThreads + tid] = 0;
    __syncthreads();
    if (valid && rank == 0) cnt[wave][d] = __popcll(peers);  // the group's first lane
    __syncthreads();
    if (tid < kRadix) {  // digit tid: exclusive scan over the waves, in order
      int acc = run[tid];
#pragma unroll
      for (int w = 0; w < kSortWaves; ++w) {
        const int c = cnt[w][tid];
        cnt[w][tid] = acc;
        acc += c;
      }
      run[tid] = acc;
    }
    __syncthreads();
    if (valid) {
      const int pos = cnt[wave][d] + rank;
      key_out[pos] = k;
      val_out[pos] = v;
    }
    __syncthreads();
  }
}

// ------------------------------------------------ backward: segments
// One workgroup of 1024 threads.  Over the sorted keys of the valid rows it
// lists the segments (runs of one id) in order and cuts each into chunks of
// kChunkRows rows:
//   seg_start[j]   first sorted position of segment j (seg_start[nseg] = count)
//   chunk_seg[c]   segment of chunk c, chunks numbered segment by segment
//   seg_chunk0[j]  first chunk of segment j
//   seg_part0[j]   first partial slot of segment j (segments of one chunk
//                  take none: their chunk adds straight into dW)
//   meta[0..2]     number of segments, chunks and partial slots
constexpr int kChunkRows = 64;

__device__ __forceinline__ int wg_exclusive_scan(int v, int* wtot, int* wbase, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // inclusive scan inside the wave
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wtot[wv] = x;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int w = 0; w < 16; ++w) {
      wbase[w] = acc;
      acc += wtot[w];
    }
    wbase[16] = acc;
  }
  __syncthreads();
  total = wbase[16];
  const int r = wbase[wv] + x - v;
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void embed_segments_kernel(const uint32_t* __restrict__ key_s,
                                                              const int32_t* __restrict__ valid_count,
                                                              int32_t* __restrict__ seg_start,
                                                              int32_t* __restrict__ seg_chunk0,
                                                              int32_t* __restrict__ seg_part0,
                                                              int32_t* __restrict__ chunk_seg,
                                                              int32_t* __restrict__ meta) {
  __shared__ int wtot[16];
  __shared__ int wbase[17];
  const int tid = threadIdx.x;
  const int count = *valid_count;
  // pass 1: segment heads, in order
  int nseg = 0;
  for (int i0 = 0; i0 < count; i0 += 1024) {
    const int i = i0 + tid;
    const int head = (i < count && (i == 0 || key_s[i] != key_s[i - 1])) ? 1 : 0;
    int tot;
    const int pos = wg_exclusive_scan(head, wtot, wbase, tot);
    if (head) seg_start[nseg + pos] = i;
    nseg += tot;
  }
  if (tid == 0) seg_start[nseg] = count;
  __syncthreads();
  // pass 2: chunks and partial slots per segment, in order
  int nchunk = 0, npart = 0;
  for (int j0 = 0; j0 < nseg; j0 += 1024) {
    const int j = j0 + tid;
    int ch = 0;
    if (j < nseg) ch = (seg_start[j + 1] - seg_start[j] + kChunkRows - 1) / kChunkRows;
    int tot_c, tot_p;
    const int c0 = wg_exclusive_scan(ch, wtot, wbase, tot_c);
    const int p0 = wg_exclusive_scan(ch > 1 ? ch : 0, wtot, wbase, tot_p);
    if (j < nseg) {
      seg_chunk0[j] = nchunk + c0;
      seg_part0[j] = npart + p0;
      for (int c = 0; c < ch; ++c) chunk_seg[nchunk + c0 + c] = j;
    }
    nchunk += tot_c;
    npart += tot_p;
  }
  if (tid == 0) {
    meta[0] = nseg;
    meta[1] = nchunk;
    meta[2] = npart;
  }
}

// -------------------------------------------- backward: level-1 sums
// Work item = (chunk, 1024-column slice); 256 threads x 4 columns.  A chunk
// sums its rows in sorted (= ascending position) order.  The only chunk of
// a segment adds into dW[id]; chunks of longer segments store a partial.
__global__ __launch_bounds__(256) void embed_chunk_sum_kernel(
    const float* __restrict__ dX, const uint32_t* __restrict__ key_s,
    const int32_t* __restrict__ val_s, const int32_t* __restrict__ seg_start,
    const int32_t* __restrict__ seg_chunk0, const int32_t* __restrict__ seg_part0,
    const int32_t* __restrict__ chunk_seg, const int32_t* __restrict__ meta, int64_t d,
    float* __restrict__ part, float* __restrict__ dW) {
  const int nchunk = meta[1];
  const int nslice = (int)((d + 1023) / 1024);
  const int64_t items = (int64_t)nchunk * nslice;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int c = (int)(it / nslice);
    const int sl = (int)(it - (int64_t)c * nslice);
    const int64_t col = (int64_t)sl * 1024 + 4 * threadIdx.x;
    const int j = chunk_seg[c];
    const int k = c - seg_chunk0[j];
    const int b = seg_start[j] + k * kChunkRows;
    const int e = min(b + kChunkRows, seg_start[j + 1]);
    const int nch = (seg_start[j + 1] - seg_start[j] + kChunkRows - 1) / kChunkRows;
    if (col >= d) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int p = b; p < e; ++p) acc += *(const f32x4*)(dX + (int64_t)val_s[p] * d + col);
    if (nch == 1) {
      float* o = dW + (int64_t)key_s[b] * d + col;
      *(f32x4*)o = *(const f32x4*)o + acc;
    } else {
      *(f32x4*)(part + (int64_t)(seg_part0[j] + k) * d + col) = acc;
    }
  }
}

// -------------------------------------------- backward: level-2 sums
// Work item = (segment, slice); segments of more than one chunk add the sum
// of their partials, taken in chunk order, into dW[id].
__global__ __launch_bounds__(256) void embed_seg_sum_kernel(
    const uint32_t* __restrict__ key_s, const int32_t* __restrict__ seg_start,
    const int32_t* __restrict__ seg_part0, const int32_t* __restrict__ meta, int64_t d,
    const float* __restrict__ part, float* __restrict__ dW) {
  const int nseg = meta[0];
  const int nslice = (int)((d + 1023) / 1024);
  const int64_t items = (int64_t)nseg * nslice;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int j = (int)(it / nslice);
    const int sl = (int)(it - (int64_t)j * nslice);
    const int nch = (seg_start[j + 1] - seg_start[j] + kChunkRows - 1) / kChunkRows;
    const int64_t col = (int64_t)sl * 1024 + 4 * threadIdx.x;
    if (nch < 2 || col >= d) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < nch; ++k) acc += *(const f32x4*)(part + (int64_t)(seg_part0[j] + k) * d + col);
    float* o = dW + (int64_t)key_s[seg_start[j]] * d + col;
    *(f32x4*)o = *(const f32x4*)o + acc;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(f32x4* __restrict__ p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ----------------------------------------------------- host-side plan
EmbedPlan make_embed_plan(int64_t N, int64_t d, int64_t V) {
  EmbedPlan p{};
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t n = (size_t)std::max<int64_t>(N, 1);
  p.end_bit = 1;
  while (p.end_bit < 32 && ((uint64_t)1 << p.end_bit) <= (uint64_t)V) ++p.end_bit;
  p.passes = (p.end_bit + kRadixBits - 1) / kRadixBits;
  p.nblocks = (int)((n + kSortTile - 1) / kSortTile);
  size_t o = 0;
  p.off_key = o; o += al(n * 4);
  p.off_val = o; o += al(n * 4);
  p.off_key_s = o; o += al(n * 4);
  p.off_val_s = o; o += al(n * 4);
  p.off_seg_start = o; o += al((n + 1) * 4);
  p.off_seg_chunk0 = o; o += al(n * 4);
  p.off_seg_part0 = o; o += al(n * 4);
  // chunks: at most count / 64 full ones plus one partial per segment
  p.max_chunks = (int64_t)n / kChunkRows + (int64_t)n;
  p.off_chunk_seg = o; o += al((size_t)p.max_chunks * 4);
  p.off_meta = o; o += al(16);
  p.off_hist = o; o += al((size_t)kRadix * p.nblocks * 4);
  // partial slots: only segments longer than one chunk, at most 2 count / 64
  p.max_parts = 2 * (int64_t)n / kChunkRows + 1;
  p.off_part = o; o += al((size_t)p.max_parts * (size_t)d * 4);
  p.total = o;
  return p;
}

hipError_t launch_embed_backward(const EmbedPlan& p, const float* dX, const int64_t* ids,
                                 const int32_t* valid_idx, const int32_t* valid_count, int64_t N,
                                 int64_t d, int64_t V, float* dW, int accumulate, void* ws,
                                 int grid, hipStream_t s) {
  char* w = (char*)ws;
  uint32_t* key = (uint32_t*)(w + p.off_key);
  int32_t* val = (int32_t*)(w + p.off_val);
  uint32_t* key_s = (uint32_t*)(w + p.off_key_s);
  int32_t* val_s = (int32_t*)(w + p.off_val_s);
  int32_t* seg_start = (int32_t*)(w + p.off_seg_start);
  int32_t* seg_chunk0 = (int32_t*)(w + p.off_seg_chunk0);
  int32_t* seg_part0 = (int32_t*)(w + p.off_seg_part0);
  int32_t* chunk_seg = (int32_t*)(w + p.off_chunk_seg);
  int32_t* meta = (int32_t*)(w + p.off_meta);
  float* part = (float*)(w + p.off_part);
  if (!accumulate) {
    const int64_t n4 = V * d / 4;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((int)std::min<int64_t>((n4 + 255) / 256, 1 << 16)),
                       dim3(256), 0, s, (f32x4*)dW, n4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (N <= 0) return hipSuccess;
  // The keys start in the buffer pair that makes the last pass land in
  // (key_s, val_s): each pass moves them to the other pair.
  uint32_t* kbuf[2] = {key, key_s};
  int32_t* vbuf[2] = {val, val_s};
  int cur = (p.passes % 2 == 0) ? 1 : 0;
  hipLaunchKernelGGL(embed_keys_kernel, dim3((int)((N + 255) / 256)), dim3(256), 0, s, ids,
                     valid_idx, valid_count, N, V, kbuf[cur], vbuf[cur]);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int32_t* hist = (int32_t*)(w + p.off_hist);
  for (int pass = 0; pass < p.passes; ++pass) {
    const int shift = kRadixBits * pass;
    hipLaunchKernelGGL(radix_hist_kernel, dim3(p.nblocks), dim3(kSortThreads), 0, s, kbuf[cur], N,
                       shift, hist, p.nblocks);
    hipLaunchKernelGGL(radix_scatter_kernel, dim3(p.nblocks), dim3(kSortThreads), 0, s, kbuf[cur],
                       vbuf[cur], kbuf[1 - cur], vbuf[1 - cur], N, shift, hist, p.nblocks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    cur = 1 - cur;
  }
  hipLaunchKernelGGL(embed_segments_kernel, dim3(1), dim3(1024), 0, s, key_s, valid_count,
                     seg_start, seg_chunk0, seg_part0, chunk_seg, meta);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(embed_chunk_sum_kernel, dim3(grid), dim3(256), 0, s, dX, key_s, val_s,
                     seg_start, seg_chunk0, seg_part0, chunk_seg, meta, d, part, dW);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(embed_seg_sum_kernel, dim3(grid), dim3(256), 0, s, key_s, seg_start,
                     seg_part0, meta, d, part, dW);
  return hipGetLastError();
}

}  // namespace lce
