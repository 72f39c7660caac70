// C ABI front end of libattn.so (declared in include/attn.h): argument checks,
// kernel choice, stream-ordered workspace, HIP error mapping.  Argument checks
// run before any HIP call, so an invalid call neither touches the device nor
// needs one.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <vector>

#include <hip/hip_runtime.h>

#include "attn.h"
#include "attn_launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return ATTN_ERR_HIP;
}

bool dims_ok(int B, int H, int Tq, int Tk, int d, int dv) {
  if (B < 1 || H < 1 || Tq < 1 || Tk < 1 || d < 1 || dv < 1) return false;
  // element counts of every tensor must fit the 64-bit offsets used inside,
  // and B*H and the workgroup counts must fit an int
  const int64_t bh = (int64_t)B * H;
  if (bh > (int64_t)INT32_MAX / 8) return false;
  if (bh * Tq > (int64_t)INT32_MAX || bh * Tk > (int64_t)INT32_MAX) return false;
  return true;
}

bool scale_ok(float s) { return isfinite(s) && s >= 0.f; }

int check_common(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int H, int Tq,
                 int Tk, int d, int dv, float scale) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID_ARG;
  if (!dims_ok(B, H, Tq, Tk, d, dv)) return ATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

bool bf16_dims_supported(int d, int dv) { return d == dv && (d == 64 || d == 128); }

// Workspace memory.  Every call takes its workspace stream-ordered from a
// memory pool that the library creates per device and that keeps up to
// kPoolKeepBytes of freed memory across synchronisations.  (The device's
// default pool hands freed memory back to the driver whenever the device
// synchronises, and the next allocation maps fresh memory: with the device
// synchronised after every call, a backward of B=2 H=32 L=8192 took about
// 75 us longer than back to back; from this pool, about 10 us.)  Pools live
// until the process ends.
constexpr uint64_t kPoolKeepBytes = 256ull << 20;
std::mutex g_pool_mu;
std::vector<hipMemPool_t> g_pools;  // by device ordinal, null until first use

hipError_t ws_pool(hipMemPool_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if ((int)g_pools.size() <= dev) g_pools.resize(dev + 1, nullptr);
  if (!g_pools[dev]) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = kPoolKeepBytes;
    e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return e;
    }
    g_pools[dev] = pool;
  }
  *out = g_pools[dev];
  return hipSuccess;
}

hipError_t ws_alloc(void** ptr, size_t bytes, hipStream_t s) {
  hipMemPool_t pool = nullptr;
  hipError_t e = ws_pool(&pool);
  if (e != hipSuccess) return e;
  return hipMallocFromPoolAsync(ptr, bytes, pool, s);
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Tq, int Tk, int d,
             int dv, float scale, int causal, int num_splits, void* stream) {
  int rc = check_common(q, k, v, o, lse, B, H, Tq, Tk, d, dv, scale);
  if (rc != ATTN_OK) return rc;
  if (num_splits < 0) return ATTN_ERR_INVALID_ARG;
  if (!bf16_dims_supported(d, dv)) return ATTN_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int BH = B * H;
  const int splits = attn::fwd_bf16_num_splits(BH, Tq, Tk, causal, num_splits);
  const size_t ws_bytes = attn::fwd_bf16_workspace_bytes(BH, Tq, Tk, d, splits);
  void* ws = nullptr;
  if (ws_bytes) {
    hipError_t e = ws_alloc(&ws, ws_bytes, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  hipError_t e = attn::fwd_bf16_launch(q, k, v, o, lse, BH, Tq, Tk, d, scale, causal, splits, ws, s);
  if (ws) {
    hipError_t f = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = f;
  }
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse, const float* dlse,
             const void* dout, void* dq, void* dk, void* dv_grad, int B, int H, int Tq, int Tk, int d, int dv,
             float scale, int causal, void* stream) {
  int rc = check_common(q, k, v, o, lse, B, H, Tq, Tk, d, dv, scale);
  if (rc != ATTN_OK) return rc;
  if (!dout || !dq || !dk || !dv_grad) return ATTN_ERR_INVALID_ARG;
  if (!bf16_dims_supported(d, dv)) return ATTN_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int BH = B * H;
  const int splits = attn::bwd_bf16_dq_splits(BH, Tq, Tk, d, SIZE_MAX);
  void* ws = nullptr;
  hipError_t e = ws_alloc(&ws, attn::bwd_bf16_workspace_bytes(BH, Tq, Tk, d, splits), s);
  if (e != hipSuccess) return hip_fail(e);
  e = attn::bwd_bf16_launch(q, k, v, o, lse, dlse, dout, dq, dk, dv_grad, BH, Tq, Tk, d, scale, causal, splits, ws,
                            s);
  hipError_t f = hipFreeAsync(ws, s);
  if (e == hipSuccess) e = f;
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

// The backward with its workspace in the library's static scratch array: no
// allocation of any kind.  Sizes are checked before any HIP call.
int bwd_noalloc_impl(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv_grad, int B, int H, int Tq, int Tk, int d, int dv, float scale,
                     int causal, void* stream) {
  int rc = check_common(q, k, v, o, lse, B, H, Tq, Tk, d, dv, scale);
  if (rc != ATTN_OK) return rc;
  if (!dout || !dq || !dk || !dv_grad) return ATTN_ERR_INVALID_ARG;
  if (!bf16_dims_supported(d, dv)) return ATTN_ERR_UNSUPPORTED;
  const int BH = B * H;
  const int splits = attn::bwd_bf16_dq_splits(BH, Tq, Tk, d, ATTN_NOALLOC_SCRATCH_BYTES);
  if (splits < 1) return ATTN_ERR_TOO_LARGE;
  void* scratch = nullptr;
  hipError_t e = attn::bwd_bf16_noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e);
  e = attn::bwd_bf16_launch(q, k, v, o, lse, nullptr, dout, dq, dk, dv_grad, BH, Tq, Tk, d, scale, causal, splits,
                            scratch, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int decode_impl(const void* q, const void* k, const void* v, const int* kv_lens, void* o, float* lse, int B, int H,
                int Tq, int Tk, int d, int dv, float scale, int causal, int num_splits, void* stream) {
  int rc = check_common(q, k, v, o, lse, B, H, Tq, Tk, d, dv, scale);
  if (rc != ATTN_OK) return rc;
  if (num_splits < 0) return ATTN_ERR_INVALID_ARG;
  if (!bf16_dims_supported(d, dv) || Tq > ATTN_DECODE_MAX_QUERIES) return ATTN_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int BH = B * H;
  const int splits = attn::decode_bf16_num_splits(BH, Tk, d, num_splits);
  const size_t ws_bytes = attn::decode_bf16_workspace_bytes(BH, Tq, d, splits);
  void* ws = nullptr;
  if (ws_bytes) {
    hipError_t e = ws_alloc(&ws, ws_bytes, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  hipError_t e = attn::decode_bf16_launch(q, k, v, kv_lens, o, lse, B, H, Tq, Tk, d, scale, causal, splits, ws, s);
  if (ws) {
    hipError_t f = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = f;
  }
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

// ---- event profiler ----------------------------------------------------------
struct Prof {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<hipEvent_t> pool;                       // free events
  std::vector<hipEvent_t> open[ATTN_KERNEL_KINDS];     // begin event of the launch in flight (per kind)
  std::vector<std::pair<hipEvent_t, hipEvent_t>> done[ATTN_KERNEL_KINDS];
  double total_ms[ATTN_KERNEL_KINDS] = {};
  int launches[ATTN_KERNEL_KINDS] = {};
};
Prof& prof() {
  static Prof* p = new Prof();  // never destroyed: events may outlive static teardown
  return *p;
}

hipEvent_t prof_event(Prof& p) {
  if (!p.pool.empty()) {
    hipEvent_t e = p.pool.back();
    p.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace attn {

void prof_begin(int kind, hipStream_t stream) {
  Prof& p = prof();
  if (!p.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> g(p.mu);
  hipEvent_t e = prof_event(p);
  if (!e) return;
  if (hipEventRecord(e, stream) != hipSuccess) {
    p.pool.push_back(e);
    return;
  }
  p.open[kind].push_back(e);
}

void prof_end(int kind, hipStream_t stream) {
  Prof& p = prof();
  if (!p.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> g(p.mu);
  if (p.open[kind].empty()) return;
  hipEvent_t b = p.open[kind].back();
  p.open[kind].pop_back();
  hipEvent_t e = prof_event(p);
  if (!e || hipEventRecord(e, stream) != hipSuccess) {
    p.pool.push_back(b);
    if (e) p.pool.push_back(e);
    return;
  }
  p.done[kind].emplace_back(b, e);
}

}  // namespace attn

extern "C" {

int attn_profile_start(void) {
  Prof& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  for (int k = 0; k < ATTN_KERNEL_KINDS; ++k) {
    for (auto& be : p.done[k]) {
      p.pool.push_back(be.first);
      p.pool.push_back(be.second);
    }
    p.done[k].clear();
    p.total_ms[k] = 0.0;
    p.launches[k] = 0;
  }
  p.on.store(true);
  return ATTN_OK;
}

int attn_profile_stop(void) {
  prof().on.store(false);
  return ATTN_OK;
}

int attn_profile_query(int kind, double* total_ms, int* launches) {
  if (kind < 0 || kind >= ATTN_KERNEL_KINDS || !total_ms || !launches) return ATTN_ERR_INVALID_ARG;
  Prof& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  for (auto& be : p.done[kind]) {
    hipError_t e = hipEventSynchronize(be.second);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, be.first, be.second);
    if (e != hipSuccess) return hip_fail(e);
    p.total_ms[kind] += ms;
    p.launches[kind] += 1;
    p.pool.push_back(be.first);
    p.pool.push_back(be.second);
  }
  p.done[kind].clear();
  *total_ms = p.total_ms[kind];
  *launches = p.launches[kind];
  return ATTN_OK;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Tq, int Tk, int d,
             int dv, float scale, int causal, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, Tq, Tk, d, dv, scale, causal, 0, stream);
}

int attn_fwd_splits(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Tq, int Tk,
                    int d, int dv, float scale, int causal, int num_splits, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, Tq, Tk, d, dv, scale, causal, num_splits, stream);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv_grad, int B, int H, int Tq, int Tk, int d, int dv, float scale, int causal,
             void* stream) {
  return bwd_impl(q, k, v, o, lse, nullptr, dout, dq, dk, dv_grad, B, H, Tq, Tk, d, dv, scale, causal, stream);
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv_grad, int B, int H, int Tq, int Tk, int d, int dv, float scale,
                     int causal, void* stream) {
  return bwd_noalloc_impl(q, k, v, o, lse, dout, dq, dk, dv_grad, B, H, Tq, Tk, d, dv, scale, causal, stream);
}

int attn_bwd_dlse(const void* q, const void* k, const void* v, const void* o, const float* lse, const float* dlse,
                  const void* dout, void* dq, void* dk, void* dv_grad, int B, int H, int Tq, int Tk, int d, int dv,
                  float scale, int causal, void* stream) {
  if (!dlse) return ATTN_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, o, lse, dlse, dout, dq, dk, dv_grad, B, H, Tq, Tk, d, dv, scale, causal, stream);
}

int attn_fwd_state(const void* q, const void* k, const void* v, float* acc, float* m, float* l, int B, int H, int Tq,
                   int Tk, int d, int dv, float scale, int causal, int q_offset, int k_offset, void* stream) {
  if (!q || !k || !v || !acc || !m || !l) return ATTN_ERR_INVALID_ARG;
  if (!dims_ok(B, H, Tq, Tk, d, dv) || !scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (q_offset < 0 || k_offset < 0) return ATTN_ERR_INVALID_ARG;
  if (!bf16_dims_supported(d, dv)) return ATTN_ERR_UNSUPPORTED;
  // blocked iff k_offset + j > q_offset + i, i.e. j > i + diag
  const long long diag = (long long)q_offset - (long long)k_offset;
  const long long lim = 1LL << 30;
  const int diag_c = (int)(diag > lim ? lim : (diag < -lim ? -lim : diag));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int BH = B * H;
  const int splits = attn::fwd_bf16_state_splits(BH, Tq, Tk, causal);
  void* ws = nullptr;
  if (splits > 1) {
    hipError_t e = ws_alloc(&ws, attn::fwd_bf16_workspace_bytes(BH, Tq, Tk, d, splits), s);
    if (e != hipSuccess) return hip_fail(e);
  }
  hipError_t e = attn::fwd_bf16_state_launch(q, k, v, acc, m, l, BH, Tq, Tk, d, scale, causal, diag_c, splits, ws, s);
  if (ws) {
    hipError_t f = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = f;
  }
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int attn_merge_states(const float* acc, const float* m, const float* l, int n, void* o, float* lse, int B, int H,
                      int Tq, int dv, void* stream) {
  if (!acc || !m || !l || !o || !lse) return ATTN_ERR_INVALID_ARG;
  if (n < 1 || !dims_ok(B, H, Tq, 1, dv, dv)) return ATTN_ERR_INVALID_ARG;
  if ((long long)n * B * H * Tq * dv > (1LL << 40)) return ATTN_ERR_INVALID_ARG;
  if (dv != 64 && dv != 128) return ATTN_ERR_UNSUPPORTED;
  hipError_t e = attn::merge_states_launch(acc, m, l, n, o, lse, B * H, Tq, dv, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int attn_fwd_standard(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Tq, int Tk,
                      int d, int dv, float scale, int causal, void* stream) {
  int rc = check_common(q, k, v, o, lse, B, H, Tq, Tk, d, dv, scale);
  if (rc != ATTN_OK) return rc;
  if (!bf16_dims_supported(d, dv)) return ATTN_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int BH = B * H;
  void* ws = nullptr;
  hipError_t e = ws_alloc(&ws, attn::std_bf16_workspace_bytes(BH, Tq, Tk, d), s);
  if (e != hipSuccess) return hip_fail(e);
  e = attn::std_bf16_launch(q, k, v, o, lse, BH, Tq, Tk, d, scale, causal, ws, s);
  hipError_t f = hipFreeAsync(ws, s);
  if (e == hipSuccess) e = f;
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int attn_decode(const void* q, const void* k, const void* v, const int* kv_lens, void* o, float* lse, int B, int H,
                int Tq, int Tk, int d, int dv, float scale, int causal, void* stream) {
  return decode_impl(q, k, v, kv_lens, o, lse, B, H, Tq, Tk, d, dv, scale, causal, 0, stream);
}

int attn_decode_splits(const void* q, const void* k, const void* v, const int* kv_lens, void* o, float* lse, int B,
                       int H, int Tq, int Tk, int d, int dv, float scale, int causal, int num_splits, void* stream) {
  return decode_impl(q, k, v, kv_lens, o, lse, B, H, Tq, Tk, d, dv, scale, causal, num_splits, stream);
}

namespace {
int fwd_f32_impl(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int Tq, int Tk,
                 int d, int dv, float scale, int causal, int block_n, int rescale, void* stream) {
  int rc = check_common(q, k, v, o, lse, B, H, Tq, Tk, d, dv, scale);
  if (rc != ATTN_OK) return rc;
  if (d > 128 || dv > 128) return ATTN_ERR_UNSUPPORTED;
  if (block_n < 0 || block_n > 1024) return ATTN_ERR_INVALID_ARG;
  if (block_n == 0) block_n = 64;
  hipError_t e = attn::fwd_f32_launch(q, k, v, o, lse, B * H, Tq, Tk, d, dv, scale, causal, block_n, rescale,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}
}  // namespace

int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int Tq, int Tk,
                 int d, int dv, float scale, int causal, int block_n, void* stream) {
  return fwd_f32_impl(q, k, v, o, lse, B, H, Tq, Tk, d, dv, scale, causal, block_n, 1, stream);
}

int attn_fwd_f32_unrescaled(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int Tq,
                            int Tk, int d, int dv, float scale, int causal, int block_n, void* stream) {
  return fwd_f32_impl(q, k, v, o, lse, B, H, Tq, Tk, d, dv, scale, causal, block_n, 0, stream);
}

int attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* lse, const float* dout,
                 float* dq, float* dk, float* dv_grad, int B, int H, int Tq, int Tk, int d, int dv, float scale,
                 int causal, void* stream) {
  int rc = check_common(q, k, v, o, lse, B, H, Tq, Tk, d, dv, scale);
  if (rc != ATTN_OK) return rc;
  if (!dout || !dq || !dk || !dv_grad) return ATTN_ERR_INVALID_ARG;
  if (d > 128 || dv > 128) return ATTN_ERR_UNSUPPORTED;
  hipError_t e = attn::bwd_f32_launch(q, k, v, o, lse, dout, dq, dk, dv_grad, B * H, Tq, Tk, d, dv, scale, causal,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK:
      return "success";
    case ATTN_ERR_INVALID_ARG:
      return "invalid argument (null pointer, dimension < 1, non-finite or negative scale, or bad block size)";
    case ATTN_ERR_UNSUPPORTED:
      return "unsupported head dimensions for this entry point";
    case ATTN_ERR_HIP:
      return "a HIP launch or allocation failed (see attn_last_hip_error)";
    case ATTN_ERR_TOO_LARGE:
      return "the problem needs more scratch memory than the no-allocation entry point holds "
             "(ATTN_NOALLOC_SCRATCH_BYTES)";
    default:
      return "unknown error code";
  }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
