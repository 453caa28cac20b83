// C-ABI of liblce: argument checks, workspace plan, launch sequence and the
// optional event-timing registry.  Every kernel runs on the caller's stream;
// nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cmath>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "kernels.h"
#include "lce.h"

// -------------------------------------------- forward without a workspace
//
// Scratch of lce_forward_noalloc: the forward's per-chunk partials (running
// max, sum and target logit of every vocabulary chunk, and the compact loss
// vector) live in this file-scope device array instead of a caller
// workspace.  Every GPU the library runs on holds its own copy until the
// process ends.  In host code the array's name is a host-side stand-in, not
// a device address: each device's copy is resolved once, with that device
// current, by hipGetSymbolAddress, and only that pointer is handed to the
// kernels.  The forward writes every partial it later reads, so nothing has
// to start at zero.
static constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

thread_local std::string g_err;

lce_status fail(lce_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

lce_status hip_fail(hipError_t e, const char* what) {
  return fail(LCE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Token chunk C (rows of the compact index) and vocabulary block Vs of the
// backward pass.  G and G^T hold C * Vs elements each; with C = Vs = 8192 the
// backward workspace is fixed once N and V exceed the block sizes.
constexpr int64_t kChunkMax = 8192;
constexpr int64_t kVocabBlockMax = 16384;
constexpr int64_t kTargetChunks = 64;  // vocabulary chunks of the forward
constexpr int64_t kStridePad = 64;     // elements added to workspace row strides
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct Plan {
  int64_t N, d, V;
  int dtype;
  size_t esz;
  // forward
  int n_vtiles, tpc, J;
  int64_t Nb;
  size_t off_pm, off_ps, off_pz, off_lossc, fwd_bytes;
  // backward
  int64_t C, Vs;
  int64_t ldG, ldGT, ldHT, ldWT;  // padded row strides (elements)
  size_t off_G, off_GT, off_HT, off_WT, off_D, bwd_bytes;
  bool has_gt;  // G^T block: fp32 and the one-chunk fused step (bf16 dW reads G K-major)
  bool has_wt;  // W^T block: fp32 (no transposing LDS read) and the fused step
  bool has_d;   // fp32 dW block accumulator: fused step over several token chunks
  size_t total;
};

// step: the plan of lce_backward_step, which keeps dH on a W^T copy of each
// vocabulary block (the block's rows of W are rewritten by the update while
// dH tiles may still read them) and, when the rows span several token
// chunks, sums a block's dW over the chunks in an fp32 [Vs][d] accumulator
// before the update consumes it.
Plan make_plan(int64_t N, int64_t d, int64_t V, int dtype, bool step = false) {
  Plan p{};
  p.N = N;
  p.d = d;
  p.V = V;
  p.dtype = dtype;
  p.esz = dtype == LCE_BF16 ? 2 : 4;
  p.n_vtiles = (int)((V + 255) / 256);
  p.tpc = (int)std::max<int64_t>(1, (p.n_vtiles + kTargetChunks - 1) / kTargetChunks);
  p.J = (p.n_vtiles + p.tpc - 1) / p.tpc;
  p.Nb = round_up(std::max<int64_t>(N, 1), 256);
  size_t o = 0;
  const size_t part = align_up((size_t)p.J * (size_t)p.Nb * sizeof(float));
  p.off_pm = o; o += part;
  p.off_ps = o; o += part;
  p.off_pz = o; o += part;
  p.off_lossc = o; o += align_up((size_t)p.Nb * sizeof(float));
  p.fwd_bytes = o;
  p.C = std::min<int64_t>(kChunkMax, round_up(std::max<int64_t>(N, 1), 256));
  p.Vs = std::min<int64_t>(kVocabBlockMax, round_up(V, 256));
  // fp32 rows of a vocabulary block (dW, optimizer state) are addressed by
  // 32-bit byte offsets: Vs * d * 4 stays below 4 GiB
  p.Vs = std::min<int64_t>(p.Vs, (((int64_t)1 << 32) - 1) / (d * 4) / 256 * 256);
  // Row strides of the K-contiguous backward buffers are padded by 64
  // elements: with power-of-two strides the 256 rows of a tile all start on
  // the same memory channel at every K step.
  p.ldG = p.Vs + kStridePad;
  p.ldGT = p.C + kStridePad;
  p.ldHT = p.C + kStridePad;
  p.ldWT = p.Vs + kStridePad;
  p.has_wt = dtype != LCE_BF16 || step;
  p.has_d = step && N > p.C;
  // the optimizer epilogue (one chunk) reads G^T; the plain bf16 dW store
  // (also the fused step's accumulation over several chunks) reads G K-major
  p.has_gt = dtype != LCE_BF16 || (step && !p.has_d);
  o = 0;
  p.off_G = o; o += align_up((size_t)p.C * (size_t)p.ldG * p.esz);
  p.off_GT = o;
  if (p.has_gt) o += align_up((size_t)p.Vs * (size_t)p.ldGT * p.esz);
  p.off_HT = o; o += align_up((size_t)d * (size_t)p.ldHT * p.esz);
  p.off_WT = o;
  if (p.has_wt) o += align_up((size_t)d * (size_t)p.ldWT * p.esz);
  p.off_D = o;
  if (p.has_d) o += align_up((size_t)p.Vs * (size_t)d * sizeof(float));
  p.bwd_bytes = o;
  p.total = std::max(p.fwd_bytes, p.bwd_bytes);
  return p;
}

lce_status check_sizes(int64_t N, int64_t d, int64_t V, int dtype) {
  if (dtype != LCE_F32 && dtype != LCE_BF16)
    return fail(LCE_ERR_INVALID_ARG, "dtype must be LCE_F32 (0) or LCE_BF16 (1)");
  if (N < 0) return fail(LCE_ERR_INVALID_ARG, "N must be >= 0");
  if (d <= 0) return fail(LCE_ERR_INVALID_ARG, "d must be > 0");
  if (V <= 0) return fail(LCE_ERR_INVALID_ARG, "V must be > 0");
  const int64_t lim = (int64_t)1 << 31;
  if (N >= lim || d >= lim || V >= lim)
    return fail(LCE_ERR_UNSUPPORTED, "N, d and V must be below 2^31");
  if (d % 64 != 0) return fail(LCE_ERR_UNSUPPORTED, "d must be a multiple of 64");
  if (d * 4 * 256 >= ((int64_t)1 << 32))
    return fail(LCE_ERR_UNSUPPORTED, "d must be below 2^22");
  // gathered token rows are addressed by 32-bit byte offsets from H
  const int64_t esz = dtype == LCE_BF16 ? 2 : 4;
  if (N * d * esz >= ((int64_t)1 << 32))
    return fail(LCE_ERR_UNSUPPORTED, "N * d * element size must stay below 4 GiB");
  return LCE_OK;
}

lce_status check_workspace(const Plan& p, const void* ws, size_t bytes) {
  if (bytes < p.total)
    return fail(LCE_ERR_WORKSPACE, "workspace of " + std::to_string(bytes) +
                                       " bytes is smaller than the required " +
                                       std::to_string(p.total));
  if (p.total && !ws) return fail(LCE_ERR_INVALID_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
    return fail(LCE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return LCE_OK;
}

int grid_persistent() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  static std::mutex mu;
  static std::vector<int> cache;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (!cache[dev]) {
    int cus = 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    cache[dev] = std::max(8, cus / 8 * 8);
  }
  return cache[dev];
}

// ------------------------------------------------------------ timing registry
struct Timing {
  std::atomic<bool> on{false};
  std::mutex mu;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[LCE_K_COUNT];
  std::vector<hipEvent_t> pool;
};
Timing& timing() {
  static Timing t;
  return t;
}

hipEvent_t take_event() {
  Timing& t = timing();
  {
    std::lock_guard<std::mutex> lk(t.mu);
    if (!t.pool.empty()) {
      hipEvent_t e = t.pool.back();
      t.pool.pop_back();
      return e;
    }
  }
  // Timing-only events: without the system-scope fence that a default event
  // performs when it completes, recording one writes back and invalidates no
  // cache, so the instrumented launches run as they would without it.
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

template <class F>
hipError_t run(int kid, hipStream_t s, F&& launch) {
  Timing& t = timing();
  if (!t.on.load(std::memory_order_relaxed)) return launch();
  hipEvent_t a = take_event(), b = take_event();
  const bool ok_a = a && hipEventRecord(a, s) == hipSuccess;
  const hipError_t e = launch();
  const bool ok_b = b && hipEventRecord(b, s) == hipSuccess;
  if (ok_a && ok_b) {
    std::lock_guard<std::mutex> lk(t.mu);
    t.ev[kid].emplace_back(a, b);
  }
  return e;
}

}  // namespace

extern "C" {

size_t lce_workspace_bytes(int64_t N, int64_t d, int64_t V, int dtype) {
  if (check_sizes(N, d, V, dtype) != LCE_OK) return 0;
  return make_plan(N, d, V, dtype).total;
}

size_t lce_step_workspace_bytes(int64_t N, int64_t d, int64_t V, int dtype) {
  if (check_sizes(N, d, V, dtype) != LCE_OK) return 0;
  return make_plan(N, d, V, dtype, true).total;
}

}  // extern "C"

namespace {

// Forward over vocabulary rows [y_off, y_off + V) held by W (the whole
// vocabulary when y_off = 0 and V = V_total).  In shard mode, writes the
// shard partials instead of loss / lse and skips the reduction (loss_sum is
// then NULL).  The mode is passed, not inferred from part_max: with N = 0 the
// partial arrays may legitimately be NULL.
lce_status forward_impl(bool shard, const void* H, const void* W, const int64_t* labels,
                        int64_t ignore_index, int64_t N, int64_t d, int64_t V_total, int64_t y_off,
                        int64_t V, int dtype, float* loss, float* lse, float* part_max, float* part_sum,
                        float* part_target, int32_t* valid_idx, int32_t* valid_count,
                        double* loss_sum, float* loss_mean, int32_t* err_flag, void* workspace,
                        size_t workspace_bytes, hipStream_t s, bool forward_bytes_only = false) {
  Plan p = make_plan(N, d, V, dtype);
  if (forward_bytes_only) p.total = p.fwd_bytes;  // the caller's scratch serves the forward only
  lce_status st = check_workspace(p, workspace, workspace_bytes);
  if (st != LCE_OK) return st;
  char* ws = (char*)workspace;

  // ignored rows: loss = lse = 0, or part_max = part_sum = 0 for a shard
  hipError_t e = run(LCE_K_COMPACT, s, [&] {
    return lce::launch_compact(labels, N, ignore_index, V_total, valid_idx, valid_count, err_flag,
                               shard ? part_max : loss, shard ? part_sum : lse, s);
  });
  if (e != hipSuccess) return hip_fail(e, "compaction launch");

  lce::FwdArgs fa{};
  fa.H = H;
  fa.W = W;
  fa.labels = labels;
  fa.valid_idx = valid_idx;
  fa.valid_count = valid_count;
  fa.N = N;
  fa.d = d;
  fa.V = V;
  fa.y_off = y_off;
  fa.n_vtiles = p.n_vtiles;
  fa.tpc = p.tpc;
  fa.J = p.J;
  fa.Nb = p.Nb;
  fa.pm = (float*)(ws + p.off_pm);
  fa.ps = (float*)(ws + p.off_ps);
  fa.pz = (float*)(ws + p.off_pz);
  float* loss_c = (float*)(ws + p.off_lossc);
  if (N > 0) {
    e = run(LCE_K_FWD, s, [&] { return lce::launch_fwd(fa, dtype, grid_persistent(), s); });
    if (e != hipSuccess) return hip_fail(e, "forward launch");
    e = run(LCE_K_MERGE, s, [&] {
      return shard ? lce::launch_fwd_part(fa, part_max, part_sum, part_target, N, s)
                   : lce::launch_fwd_merge(fa, loss, lse, loss_c, N, s);
    });
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  if (shard) return LCE_OK;
  e = run(LCE_K_REDUCE, s, [&] {
    return lce::launch_loss_reduce(loss_c, nullptr, valid_count, loss_sum, loss_mean, s);
  });
  if (e != hipSuccess) return hip_fail(e, "reduction launch");
  return LCE_OK;
}

lce_status scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  static std::mutex mu;
  static std::vector<void*> ptrs;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the static scratch");
    if (!p) return fail(LCE_ERR_HIP, "hipGetSymbolAddress of the static scratch returned NULL");
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return LCE_OK;
}

lce_status check_shard(int64_t V_total, int64_t v_begin, int64_t V_shard) {
  if (V_total <= 0 || V_total >= ((int64_t)1 << 31))
    return fail(LCE_ERR_INVALID_ARG, "V_total must be in [1, 2^31)");
  if (v_begin < 0 || V_shard <= 0 || v_begin + V_shard > V_total)
    return fail(LCE_ERR_INVALID_ARG, "the shard [v_begin, v_begin + V_shard) must lie in [0, V_total)");
  return LCE_OK;
}

}  // namespace

extern "C" {

lce_status lce_forward(const void* H, const void* W, const int64_t* labels, int64_t ignore_index,
                       int64_t N, int64_t d, int64_t V, int dtype, float* loss, float* lse,
                       int32_t* valid_idx, int32_t* valid_count, double* loss_sum,
                       float* loss_mean, int32_t* err_flag, void* workspace,
                       size_t workspace_bytes, void* stream) {
  g_err.clear();
  lce_status st = check_sizes(N, d, V, dtype);
  if (st != LCE_OK) return st;
  if (!W || !valid_count || !loss_sum || !err_flag)
    return fail(LCE_ERR_INVALID_ARG, "W, valid_count, loss_sum and err_flag must not be NULL");
  if (N > 0 && (!H || !labels || !loss || !lse || !valid_idx))
    return fail(LCE_ERR_INVALID_ARG, "H, labels, loss, lse and valid_idx must not be NULL");
  return forward_impl(false, H, W, labels, ignore_index, N, d, V, 0, V, dtype, loss, lse, nullptr,
                      nullptr, nullptr, valid_idx, valid_count, loss_sum, loss_mean, err_flag,
                      workspace, workspace_bytes, (hipStream_t)stream);
}

lce_status lce_forward_noalloc(const void* H, const void* W, const int64_t* labels,
                               int64_t ignore_index, int64_t N, int64_t d, int64_t V, int dtype,
                               float* loss, float* lse, int32_t* valid_idx, int32_t* valid_count,
                               double* loss_sum, float* loss_mean, int32_t* err_flag,
                               void* stream) {
  g_err.clear();
  lce_status st = check_sizes(N, d, V, dtype);
  if (st != LCE_OK) return st;
  if (!W || !valid_count || !loss_sum || !err_flag)
    return fail(LCE_ERR_INVALID_ARG, "W, valid_count, loss_sum and err_flag must not be NULL");
  if (N > 0 && (!H || !labels || !loss || !lse || !valid_idx))
    return fail(LCE_ERR_INVALID_ARG, "H, labels, loss, lse and valid_idx must not be NULL");
  const size_t need = make_plan(N, d, V, dtype).fwd_bytes;
  if (need > kScratchBytes)
    return fail(LCE_ERR_UNSUPPORTED,
                "lce_forward_noalloc: these sizes need " + std::to_string(need) +
                    " bytes of scratch and the static scratch holds " +
                    std::to_string(kScratchBytes) + " (use lce_forward with a workspace)");
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != LCE_OK) return st;
  return forward_impl(false, H, W, labels, ignore_index, N, d, V, 0, V, dtype, loss, lse, nullptr,
                      nullptr, nullptr, valid_idx, valid_count, loss_sum, loss_mean, err_flag, ws,
                      kScratchBytes, (hipStream_t)stream, true);
}

lce_status lce_forward_shard(const void* H, const void* W_shard, const int64_t* labels,
                             int64_t ignore_index, int64_t N, int64_t d, int64_t V_total,
                             int64_t v_begin, int64_t V_shard, int dtype, float* part_max,
                             float* part_sum, float* part_target, int32_t* valid_idx,
                             int32_t* valid_count, int32_t* err_flag, void* workspace,
                             size_t workspace_bytes, void* stream) {
  g_err.clear();
  lce_status st = check_sizes(N, d, V_shard, dtype);
  if (st != LCE_OK) return st;
  st = check_shard(V_total, v_begin, V_shard);
  if (st != LCE_OK) return st;
  if (!W_shard || !valid_count || !err_flag)
    return fail(LCE_ERR_INVALID_ARG, "W_shard, valid_count and err_flag must not be NULL");
  if (N > 0 && (!H || !labels || !part_max || !part_sum || !part_target || !valid_idx))
    return fail(LCE_ERR_INVALID_ARG,
                "H, labels, part_max, part_sum, part_target and valid_idx must not be NULL");
  return forward_impl(true, H, W_shard, labels, ignore_index, N, d, V_total, v_begin, V_shard, dtype,
                      nullptr, nullptr, part_max, part_sum, part_target, valid_idx, valid_count,
                      nullptr, nullptr, err_flag, workspace, workspace_bytes, (hipStream_t)stream);
}

lce_status lce_lse_merge(const float* part_max, const float* part_sum, const float* part_target,
                         int64_t n_shards, int64_t shard_stride, int64_t N,
                         const int32_t* valid_idx, const int32_t* valid_count, float* loss,
                         float* lse, double* loss_sum, float* loss_mean, void* stream) {
  g_err.clear();
  if (N < 0 || N >= ((int64_t)1 << 31)) return fail(LCE_ERR_INVALID_ARG, "N must be in [0, 2^31)");
  if (n_shards < 1) return fail(LCE_ERR_INVALID_ARG, "n_shards must be >= 1");
  if (n_shards > 1 && shard_stride < N)
    return fail(LCE_ERR_INVALID_ARG, "shard_stride must be >= N");
  if (!valid_count || !loss_sum)
    return fail(LCE_ERR_INVALID_ARG, "valid_count and loss_sum must not be NULL");
  if (N > 0 && (!part_max || !part_sum || !part_target || !valid_idx || !loss || !lse))
    return fail(LCE_ERR_INVALID_ARG,
                "part_max, part_sum, part_target, valid_idx, loss and lse must not be NULL");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = run(LCE_K_MERGE, s, [&] {
    return lce::launch_shard_merge(part_max, part_sum, part_target, n_shards, shard_stride, N,
                                   loss, lse, s);
  });
  if (e != hipSuccess) return hip_fail(e, "shard merge launch");
  e = run(LCE_K_REDUCE, s, [&] {
    return lce::launch_loss_reduce(loss, valid_idx, valid_count, loss_sum, loss_mean, s);
  });
  if (e != hipSuccess) return hip_fail(e, "reduction launch");
  return LCE_OK;
}

}  // extern "C"

namespace {

// Backward over vocabulary rows [y_off, y_off + V) held by W (the whole
// vocabulary when y_off = 0 and V = V_total).  accumulate_dH adds this
// shard's dH contribution instead of overwriting (ignored rows are then left
// as they are: the first shard zeroed them).
lce_status backward_impl(const void* H, const void* W, const int64_t* labels, int64_t ignore_index,
                         const float* lse, const int32_t* valid_idx, const int32_t* valid_count,
                         int64_t N, int64_t d, int64_t V_total, int64_t y_off, int64_t V, int dtype,
                         const float* grad_out, int reduction, float* dH, int accumulate_dH,
                         float* dW, int accumulate_dW, void* workspace, size_t workspace_bytes,
                         hipStream_t s, const lce::DwArgs* step = nullptr) {
  const Plan p = make_plan(N, d, V, dtype, step != nullptr);
  lce_status st = check_workspace(p, workspace, workspace_bytes);
  if (st != LCE_OK) return st;
  char* ws = (char*)workspace;
  void* G = ws + p.off_G;
  void* GT = p.has_gt ? ws + p.off_GT : nullptr;
  void* HT = ws + p.off_HT;
  void* WT = p.has_wt ? ws + p.off_WT : nullptr;
  float* Dacc = p.has_d ? (float*)(ws + p.off_D) : nullptr;

  hipError_t e = hipSuccess;
  if (!accumulate_dH) {
    e = run(LCE_K_ZERO, s, [&] {
      return lce::launch_zero_ignored(labels, N, ignore_index, V_total, dH, d, s);
    });
    if (e != hipSuccess) return hip_fail(e, "zero-rows launch");
  }

  // bf16 without an optimizer step: dH reads each W block directly (K-major,
  // transposing LDS reads), so no W^T copy is built.  The optimizer step
  // rewrites W's rows in its dW epilogue while dH may still run (the merged
  // dH + dW launch), so it keeps dH on the copy; fp32 has no transposing read.
  const bool w_direct = !p.has_wt;

  // H^T of token chunk c0 (the chunk's gathered valid rows, transposed);
  // skipped on the device when the chunk holds no valid row
  auto transpose_h = [&](int64_t c0) -> hipError_t {
    lce::TransposeArgs th{};
    th.src = H;
    th.ld_src = d;
    th.gather = valid_idx;
    th.row0 = c0;
    th.count = valid_count;
    th.dst = HT;
    th.ncols = p.C;
    th.ld_dst = p.ldHT;
    th.K = d;
    th.active_count = c0 > 0 ? valid_count : nullptr;
    th.active_c0 = c0;
    return run(LCE_K_TRANSPOSE, s, [&] { return lce::launch_transpose(th, dtype, s); });
  };
  // W^T of vocabulary block v0 (skipped when chunk c0 holds no valid row)
  auto transpose_w = [&](int64_t v0, int64_t c0) -> hipError_t {
    lce::TransposeArgs tw{};
    tw.src = W;
    tw.ld_src = d;
    tw.gather = nullptr;
    tw.row0 = v0;
    tw.count = nullptr;
    tw.nrows_static = V;
    tw.dst = WT;
    tw.ncols = p.Vs;
    tw.ld_dst = p.ldWT;
    tw.K = d;
    tw.active_count = c0 > 0 ? valid_count : nullptr;
    tw.active_c0 = c0;
    return run(LCE_K_TRANSPOSE, s, [&] { return lce::launch_transpose(tw, dtype, s); });
  };
  // recompute + G, dH and dW of token chunk c0 x vocabulary block v0
  auto block = [&](int64_t c0, int64_t v0) -> lce_status {
    lce::BwdGArgs ga{};
    ga.H = H;
    ga.W = W;
    ga.labels = labels;
    ga.lse = lse;
    ga.valid_idx = valid_idx;
    ga.valid_count = valid_count;
    ga.grad_out = grad_out;
    ga.reduction = reduction;
    ga.N = N;
    ga.d = d;
    ga.V = V;
    ga.y_off = y_off;
    ga.c0 = c0;
    ga.C = p.C;
    ga.v0 = v0;
    ga.Vs = p.Vs;
    ga.G = G;
    ga.GT = GT;
    ga.ldG = p.ldG;
    ga.ldGT = p.ldGT;
    hipError_t err = run(LCE_K_BWD_G, s, [&] { return lce::launch_bwd_g(ga, dtype, s); });
    if (err != hipSuccess) return hip_fail(err, "recompute launch");

    lce::DhArgs ha{};
    ha.G = G;
    ha.WT = WT;
    ha.W = w_direct ? W : nullptr;
    ha.ldG = p.ldG;
    ha.ldWT = p.ldWT;
    ha.C = p.C;
    ha.Vs = p.Vs;
    ha.d = d;
    ha.valid_idx = valid_idx;
    ha.valid_count = valid_count;
    ha.c0 = c0;
    ha.v0 = v0;
    ha.V = V;
    ha.dH = dH;
    ha.N = p.N;
    ha.beta = (v0 > 0 || accumulate_dH) ? 1 : 0;
    lce::DwArgs wa{};
    wa.GT = GT;
    wa.HT = HT;
    wa.ldGT = p.ldGT;
    wa.G = G;
    wa.ldG = p.ldG;
    wa.ldHT = p.ldHT;
    wa.C = p.C;
    wa.Vs = p.Vs;
    wa.d = d;
    wa.valid_count = valid_count;
    wa.c0 = c0;
    wa.v0 = v0;
    wa.V = V;
    wa.dW = dW;
    wa.accumulate = (c0 > 0 || accumulate_dW) ? 1 : 0;
    if (step && Dacc) {
      // rows over several chunks: the plain store sums the block's dW over
      // the chunks into the accumulator (addressed as rows v0.. of a dW table)
      wa.dW = (float*)((uintptr_t)Dacc - (uintptr_t)(v0 * d * sizeof(float)));
      wa.accumulate = c0 > 0 ? 1 : 0;
    } else if (step) {  // one chunk: the optimizer epilogue instead of the dW store
      wa.opt_kind = step->opt_kind;
      wa.lr = step->lr;
      wa.wd = step->wd;
      wa.beta1 = step->beta1;
      wa.beta2 = step->beta2;
      wa.eps = step->eps;
      wa.bc1 = step->bc1;
      wa.bc2s = step->bc2s;
      wa.master = step->master;
      wa.exp_avg = step->exp_avg;
      wa.exp_avg_sq = step->exp_avg_sq;
      wa.w16 = step->w16;
    }
    // dH and dW share one launch: the dH tiles (long K) are dispatched first,
    // right after the recompute while the G block is still largely in the
    // Infinity Cache, and the short dW tiles fill the CUs they leave idle
    err = run(LCE_K_DH_DW, s, [&] { return lce::launch_dh_dw(ha, wa, dtype, s); });
    if (err != hipSuccess) return hip_fail(err, "dH + dW launch");
    return LCE_OK;
  };

  if (!step) {
    // Token chunks outside, vocabulary blocks inside: each chunk's H^T is
    // built once.  At least one chunk, so that dW is written even when N == 0.
    for (int64_t c0 = 0; c0 == 0 || c0 < N; c0 += p.C) {
      e = transpose_h(c0);
      if (e != hipSuccess) return hip_fail(e, "transpose launch");
      for (int64_t v0 = 0; v0 < V; v0 += p.Vs) {
        if (!w_direct) {
          e = transpose_w(v0, c0);
          if (e != hipSuccess) return hip_fail(e, "transpose launch");
        }
        st = block(c0, v0);
        if (st != LCE_OK) return st;
      }
    }
    return LCE_OK;
  }
  // Fused update: vocabulary blocks outside, token chunks inside.  With one
  // token chunk (N <= C) the dW epilogue applies the update to each tile as
  // it is produced.  Beyond that, a block's dW is summed over the chunks in
  // the accumulator and the update is applied to the whole block after its
  // last chunk.  The W^T copy of a block is taken before any chunk (dH keeps
  // reading the old weights), and H^T is rebuilt per chunk.
  for (int64_t v0 = 0; v0 < V; v0 += p.Vs) {
    e = transpose_w(v0, 0);
    if (e != hipSuccess) return hip_fail(e, "transpose launch");
    for (int64_t c0 = 0; c0 == 0 || c0 < N; c0 += p.C) {
      e = transpose_h(c0);
      if (e != hipSuccess) return hip_fail(e, "transpose launch");
      st = block(c0, v0);
      if (st != LCE_OK) return st;
    }
    if (Dacc) {
      lce::DwArgs oa = *step;
      oa.acc = Dacc;
      oa.v0 = v0;
      oa.Vs = p.Vs;
      oa.V = V;
      oa.d = d;
      e = run(LCE_K_OPT, s, [&] { return lce::launch_apply_opt(oa, s); });
      if (e != hipSuccess) return hip_fail(e, "optimizer launch");
    }
  }
  return LCE_OK;
}

}  // namespace

extern "C" {

lce_status lce_backward(const void* H, const void* W, const int64_t* labels, int64_t ignore_index,
                        const float* lse, const int32_t* valid_idx, const int32_t* valid_count,
                        int64_t N, int64_t d, int64_t V, int dtype, const float* grad_out,
                        int reduction, float* dH, float* dW, int accumulate_dW, void* workspace,
                        size_t workspace_bytes, void* stream) {
  g_err.clear();
  lce_status st = check_sizes(N, d, V, dtype);
  if (st != LCE_OK) return st;
  if (reduction != LCE_MEAN && reduction != LCE_SUM)
    return fail(LCE_ERR_INVALID_ARG, "reduction must be LCE_MEAN (0) or LCE_SUM (1)");
  if (!W || !valid_count || !grad_out || !dW)
    return fail(LCE_ERR_INVALID_ARG, "W, valid_count, grad_out and dW must not be NULL");
  if ((reinterpret_cast<uintptr_t>(dW) & 15) != 0)
    return fail(LCE_ERR_INVALID_ARG, "dW must be 16-byte aligned");
  if (N > 0 && (!H || !labels || !lse || !valid_idx || !dH))
    return fail(LCE_ERR_INVALID_ARG, "H, labels, lse, valid_idx and dH must not be NULL");
  return backward_impl(H, W, labels, ignore_index, lse, valid_idx, valid_count, N, d, V, 0, V,
                       dtype, grad_out, reduction, dH, 0, dW, accumulate_dW, workspace,
                       workspace_bytes, (hipStream_t)stream);
}

lce_status lce_backward_step(const void* H, void* W, const int64_t* labels, int64_t ignore_index,
                             const float* lse, const int32_t* valid_idx, const int32_t* valid_count,
                             int64_t N, int64_t d, int64_t V, int dtype, const float* grad_out,
                             int reduction, float* dH, float* W_master, float* exp_avg,
                             float* exp_avg_sq, const lce_optimizer* opt, void* workspace,
                             size_t workspace_bytes, void* stream) {
  g_err.clear();
  lce_status st = check_sizes(N, d, V, dtype);
  if (st != LCE_OK) return st;
  if (reduction != LCE_MEAN && reduction != LCE_SUM)
    return fail(LCE_ERR_INVALID_ARG, "reduction must be LCE_MEAN (0) or LCE_SUM (1)");
  if (!W || !valid_count || !grad_out || !opt)
    return fail(LCE_ERR_INVALID_ARG, "W, valid_count, grad_out and opt must not be NULL");
  if (N > 0 && (!H || !labels || !lse || !valid_idx || !dH))
    return fail(LCE_ERR_INVALID_ARG, "H, labels, lse, valid_idx and dH must not be NULL");
  if (dtype == LCE_BF16 && !W_master)
    return fail(LCE_ERR_INVALID_ARG, "bf16 weights need fp32 master weights (W_master)");
  // the block update moves 16-byte vectors of the fp32 arrays and 8-byte
  // vectors of a bf16 W
  for (const void* q : {(const void*)W_master, (const void*)exp_avg, (const void*)exp_avg_sq})
    if ((reinterpret_cast<uintptr_t>(q) & 15) != 0)
      return fail(LCE_ERR_INVALID_ARG, "W_master, exp_avg and exp_avg_sq must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(W) & (dtype == LCE_BF16 ? 7 : 15)) != 0)
    return fail(LCE_ERR_INVALID_ARG, "W must be 8-byte (bf16) or 16-byte (fp32) aligned");
  if (!(opt->lr >= 0.f) || !(opt->weight_decay >= 0.f))
    return fail(LCE_ERR_INVALID_ARG, "lr and weight_decay must be >= 0");
  lce::DwArgs step{};
  if (opt->kind == LCE_OPT_SGD) {
    step.opt_kind = 1;
  } else if (opt->kind == LCE_OPT_ADAMW) {
    if (!exp_avg || !exp_avg_sq)
      return fail(LCE_ERR_INVALID_ARG, "AdamW needs exp_avg and exp_avg_sq");
    if (opt->step < 1) return fail(LCE_ERR_INVALID_ARG, "AdamW step must be >= 1");
    if (!(opt->beta1 >= 0.f && opt->beta1 < 1.f && opt->beta2 >= 0.f && opt->beta2 < 1.f) ||
        !(opt->eps > 0.f))
      return fail(LCE_ERR_INVALID_ARG, "AdamW needs betas in [0, 1) and eps > 0");
    step.opt_kind = 2;
    step.beta1 = opt->beta1;
    step.beta2 = opt->beta2;
    step.eps = opt->eps;
    step.bc1 = (float)(1.0 - std::pow((double)opt->beta1, (double)opt->step));
    step.bc2s = (float)std::sqrt(1.0 - std::pow((double)opt->beta2, (double)opt->step));
    step.exp_avg = exp_avg;
    step.exp_avg_sq = exp_avg_sq;
  } else {
    return fail(LCE_ERR_INVALID_ARG, "opt->kind must be LCE_OPT_SGD or LCE_OPT_ADAMW");
  }
  step.lr = opt->lr;
  step.wd = opt->weight_decay;
  step.master = W_master ? W_master : (float*)W;
  step.w16 = dtype == LCE_BF16 ? (uint16_t*)W : nullptr;
  return backward_impl(H, W, labels, ignore_index, lse, valid_idx, valid_count, N, d, V, 0, V,
                       dtype, grad_out, reduction, dH, 0, nullptr, 0, workspace, workspace_bytes,
                       (hipStream_t)stream, &step);
}

lce_status lce_backward_shard(const void* H, const void* W_shard, const int64_t* labels,
                              int64_t ignore_index, const float* lse, const int32_t* valid_idx,
                              const int32_t* valid_count, int64_t N, int64_t d, int64_t V_total,
                              int64_t v_begin, int64_t V_shard, int dtype, const float* grad_out,
                              int reduction, float* dH, int accumulate_dH, float* dW_shard,
                              int accumulate_dW, void* workspace, size_t workspace_bytes,
                              void* stream) {
  g_err.clear();
  lce_status st = check_sizes(N, d, V_shard, dtype);
  if (st != LCE_OK) return st;
  st = check_shard(V_total, v_begin, V_shard);
  if (st != LCE_OK) return st;
  if (reduction != LCE_MEAN && reduction != LCE_SUM)
    return fail(LCE_ERR_INVALID_ARG, "reduction must be LCE_MEAN (0) or LCE_SUM (1)");
  if (!W_shard || !valid_count || !grad_out || !dW_shard)
    return fail(LCE_ERR_INVALID_ARG, "W_shard, valid_count, grad_out and dW_shard must not be NULL");
  if ((reinterpret_cast<uintptr_t>(dW_shard) & 15) != 0)
    return fail(LCE_ERR_INVALID_ARG, "dW_shard must be 16-byte aligned");
  if (N > 0 && (!H || !labels || !lse || !valid_idx || !dH))
    return fail(LCE_ERR_INVALID_ARG, "H, labels, lse, valid_idx and dH must not be NULL");
  return backward_impl(H, W_shard, labels, ignore_index, lse, valid_idx, valid_count, N, d, V_total,
                       v_begin, V_shard, dtype, grad_out, reduction, dH, accumulate_dH ? 1 : 0,
                       dW_shard, accumulate_dW, workspace, workspace_bytes, (hipStream_t)stream);
}

lce_status lce_cast_bf16(const float* src, void* dst, int64_t n, void* stream) {
  g_err.clear();
  if (n < 0) return fail(LCE_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return LCE_OK;
  if (!src || !dst) return fail(LCE_ERR_INVALID_ARG, "src and dst must not be NULL");
  if ((reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) != 0)
    return fail(LCE_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
  const char* a = (const char*)src;
  const char* b = (const char*)dst;
  if (a < b + 2 * n && b < a + 4 * n) return fail(LCE_ERR_INVALID_ARG, "src and dst overlap");
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e =
      run(LCE_K_CAST, s, [&] { return lce::launch_cast_bf16(src, (uint16_t*)dst, n, s); });
  if (e != hipSuccess) return hip_fail(e, "cast launch");
  return LCE_OK;
}

size_t lce_embed_workspace_bytes(int64_t N, int64_t d, int64_t V) {
  if (check_sizes(N, d, V, LCE_F32) != LCE_OK) return 0;
  return lce::make_embed_plan(N, d, V).total;
}

lce_status lce_embed_forward(const void* W, const int64_t* input_ids, int64_t pad_id, int64_t N,
                             int64_t d, int64_t V, int dtype, void* X, int32_t* valid_idx,
                             int32_t* valid_count, int32_t* err_flag, void* stream) {
  g_err.clear();
  lce_status st = check_sizes(N, d, V, dtype);
  if (st != LCE_OK) return st;
  if (!W || !valid_count || !err_flag)
    return fail(LCE_ERR_INVALID_ARG, "W, valid_count and err_flag must not be NULL");
  if (N > 0 && (!input_ids || !X || !valid_idx))
    return fail(LCE_ERR_INVALID_ARG, "input_ids, X and valid_idx must not be NULL");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = run(LCE_K_COMPACT, s, [&] {
    return lce::launch_compact(input_ids, N, pad_id, V, valid_idx, valid_count, err_flag, nullptr,
                               nullptr, s);
  });
  if (e != hipSuccess) return hip_fail(e, "compaction launch");
  const int64_t esz = dtype == LCE_BF16 ? 2 : 4;
  e = run(LCE_K_EMBED, s,
          [&] { return lce::launch_embed_gather(W, input_ids, pad_id, N, V, d * esz, X, s); });
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return LCE_OK;
}

lce_status lce_embed_backward(const float* dX, const int64_t* input_ids, const int32_t* valid_idx,
                              const int32_t* valid_count, int64_t N, int64_t d, int64_t V,
                              float* dW, int accumulate_dW, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_err.clear();
  lce_status st = check_sizes(N, d, V, LCE_F32);
  if (st != LCE_OK) return st;
  if (!valid_count || !dW) return fail(LCE_ERR_INVALID_ARG, "valid_count and dW must not be NULL");
  if (N > 0 && (!dX || !input_ids || !valid_idx))
    return fail(LCE_ERR_INVALID_ARG, "dX, input_ids and valid_idx must not be NULL");
  const lce::EmbedPlan p = lce::make_embed_plan(N, d, V);
  if (workspace_bytes < p.total)
    return fail(LCE_ERR_WORKSPACE, "workspace of " + std::to_string(workspace_bytes) +
                                       " bytes is smaller than the required " +
                                       std::to_string(p.total));
  if (!workspace) return fail(LCE_ERR_INVALID_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return fail(LCE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = run(LCE_K_EMBED, s, [&] {
    return lce::launch_embed_backward(p, dX, input_ids, valid_idx, valid_count, N, d, V, dW,
                                      accumulate_dW ? 1 : 0, workspace, 4 * grid_persistent(), s);
  });
  if (e != hipSuccess) return hip_fail(e, "embedding backward launch");
  return LCE_OK;
}

lce_status lce_attention_forward(const void* Q, const void* K, const void* V, int64_t B, int64_t H,
                                 int64_t S, int64_t D, int causal, float scale, float* O,
                                 float* lse, void* stream) {
  g_err.clear();
  if (B < 0 || H < 0 || S < 0) return fail(LCE_ERR_INVALID_ARG, "B, H and S must be >= 0");
  if (D != 64 && D != 128) return fail(LCE_ERR_UNSUPPORTED, "head dimension D must be 64 or 128");
  if (causal != 0 && causal != 1) return fail(LCE_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(LCE_ERR_INVALID_ARG, "scale must be finite and >= 0 (0 selects 1 / sqrt(D))");
  const int64_t BH = B * H;
  if (BH == 0 || S == 0) return LCE_OK;
  const int64_t lim = (int64_t)1 << 31;
  if (S >= lim || BH >= lim || ((S + 127) / 128) * BH >= lim)
    return fail(LCE_ERR_UNSUPPORTED, "B * H * ceil(S / 128) and S must be below 2^31");
  if (!Q || !K || !V || !O || !lse)
    return fail(LCE_ERR_INVALID_ARG, "Q, K, V, O and lse must not be NULL");
  lce::AttnArgs a{};
  a.Q = (const uint16_t*)Q;
  a.K = (const uint16_t*)K;
  a.V = (const uint16_t*)V;
  a.O = O;
  a.lse = lse;
  a.BH = BH;
  a.S = (int)S;
  a.causal = causal;
  const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)D);
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = run(LCE_K_ATTN, s, [&] { return lce::launch_attn_fwd(a, (int)D, s); });
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return LCE_OK;
}

lce_status lce_attention_backward(const void* Q, const void* K, const void* V, const float* O,
                                  const float* lse, const void* dO, int64_t B, int64_t H,
                                  int64_t S, int64_t D, int causal, float scale, float* dQ,
                                  float* dK, float* dV, float* delta, void* stream) {
  g_err.clear();
  if (B < 0 || H < 0 || S < 0) return fail(LCE_ERR_INVALID_ARG, "B, H and S must be >= 0");
  if (D != 64 && D != 128) return fail(LCE_ERR_UNSUPPORTED, "head dimension D must be 64 or 128");
  if (causal != 0 && causal != 1) return fail(LCE_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(LCE_ERR_INVALID_ARG, "scale must be finite and >= 0 (0 selects 1 / sqrt(D))");
  const int64_t BH = B * H;
  if (BH == 0 || S == 0) return LCE_OK;
  const int64_t lim = (int64_t)1 << 31;
  if (S >= lim || BH >= lim || ((S + 127) / 128) * BH >= lim)
    return fail(LCE_ERR_UNSUPPORTED, "B * H * ceil(S / 128) and S must be below 2^31");
  if (!Q || !K || !V || !O || !lse || !dO || !dQ || !dK || !dV || !delta)
    return fail(LCE_ERR_INVALID_ARG,
                "Q, K, V, O, lse, dO, dQ, dK, dV and delta must not be NULL");
  lce::AttnBwdArgs a{};
  a.Q = (const uint16_t*)Q;
  a.K = (const uint16_t*)K;
  a.V = (const uint16_t*)V;
  a.dO = (const uint16_t*)dO;
  a.O = O;
  a.lse = lse;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.delta = delta;
  a.BH = BH;
  a.S = (int)S;
  a.causal = causal;
  const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)D);
  a.scale = (float)sc;
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = run(LCE_K_ATTN_DQ, s, [&] { return lce::launch_attn_bwd_dq(a, (int)D, s); });
  if (e != hipSuccess) return hip_fail(e, "attention backward (dQ pass) launch");
  e = run(LCE_K_ATTN_DKV, s, [&] { return lce::launch_attn_bwd_dkv(a, (int)D, s); });
  if (e != hipSuccess) return hip_fail(e, "attention backward (dK/dV pass) launch");
  return LCE_OK;
}

lce_status lce_check_error(const int32_t* err_flag, void* stream) {
  g_err.clear();
  if (!err_flag) return fail(LCE_ERR_INVALID_ARG, "err_flag is NULL");
  int32_t h = 0;
  hipError_t e = hipMemcpyAsync(&h, err_flag, sizeof(h), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "reading err_flag");
  if (h) return fail(LCE_ERR_LABEL_RANGE, "a label that is not ignore_index lies outside [0, V)");
  return LCE_OK;
}

const char* lce_status_string(lce_status s) {
  switch (s) {
    case LCE_OK: return "ok";
    case LCE_ERR_INVALID_ARG: return "invalid argument";
    case LCE_ERR_UNSUPPORTED: return "unsupported shape";
    case LCE_ERR_WORKSPACE: return "workspace too small";
    case LCE_ERR_LABEL_RANGE: return "label outside [0, V)";
    case LCE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* lce_last_error(void) { return g_err.c_str(); }

lce_status lce_gemm_nt(const void* A, const void* B, float* C, int64_t M, int64_t N, int64_t K,
                       int dtype, void* stream) {
  g_err.clear();
  if (dtype != LCE_F32 && dtype != LCE_BF16) return fail(LCE_ERR_INVALID_ARG, "bad dtype");
  if (M <= 0 || N <= 0 || K <= 0) return fail(LCE_ERR_INVALID_ARG, "M, N, K must be > 0");
  if (K % 64 != 0) return fail(LCE_ERR_UNSUPPORTED, "K must be a multiple of 64");
  if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31))
    return fail(LCE_ERR_UNSUPPORTED, "M and N must be below 2^31");
  if (!A || !B || !C) return fail(LCE_ERR_INVALID_ARG, "NULL pointer");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = run(LCE_K_GEMM, s, [&] { return lce::launch_gemm_nt(A, B, C, M, N, K, dtype, s); });
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return LCE_OK;
}

lce_status lce_mfma_peak(float* out, int64_t n_out, int64_t iters, void* stream) {
  g_err.clear();
  constexpr int64_t kBlocks = 1024, kThreadsPer = 512;
  if (!out) return fail(LCE_ERR_INVALID_ARG, "out must not be NULL");
  if (n_out < kBlocks * kThreadsPer)
    return fail(LCE_ERR_INVALID_ARG, "out must hold 1024 * 512 floats");
  if (iters < 1 || iters > ((int64_t)1 << 24))
    return fail(LCE_ERR_INVALID_ARG, "iters must be in [1, 2^24]");
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e =
      run(LCE_K_MFMA, s, [&] { return lce::launch_mfma_peak(out, (int)kBlocks, iters, s); });
  if (e != hipSuccess) return hip_fail(e, "mfma calibration launch");
  return LCE_OK;
}

lce_status lce_timing_enable(int on) {
  timing().on.store(on != 0);
  return LCE_OK;
}

lce_status lce_timing_reset(void) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  for (auto& v : t.ev) {
    for (auto& pr : v) {
      t.pool.push_back(pr.first);
      t.pool.push_back(pr.second);
    }
    v.clear();
  }
  return LCE_OK;
}

lce_status lce_timing_query(int kernel_class, double* total_ms, int64_t* launches) {
  g_err.clear();
  if (kernel_class < 0 || kernel_class >= LCE_K_COUNT || !total_ms || !launches)
    return fail(LCE_ERR_INVALID_ARG, "bad kernel class or NULL output");
  Timing& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  double sum = 0.0;
  for (auto& pr : t.ev[kernel_class]) {
    hipError_t e = hipEventSynchronize(pr.second);
    if (e != hipSuccess) return hip_fail(e, "event synchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) return hip_fail(e, "event elapsed time");
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int64_t)t.ev[kernel_class].size();
  return LCE_OK;
}

}  // extern "C"
