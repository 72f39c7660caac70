// Host-side launchers of the attention kernels (internal; the public ABI is
// include/attn.h).  Each launcher only enqueues kernels on `stream` and returns
// the launch status; argument checking is done by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <algorithm>
#include <atomic>

namespace attn {

// Workgroups of kernel K (`threads` per workgroup, static LDS only) that the
// current device holds at once: CUs x workgroups per CU, the grid of a
// persistent launch; 0 when the device cannot be queried.  Cached per device.
template <auto K>
int resident_workgroups(int threads) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, K, threads, 0) != hipSuccess) return 0;
  v = cus * std::max(per, 1);
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Event profiler hooks (defined in api.cpp).  When profiling is off these are
// a single relaxed load each.
void prof_begin(int kind, hipStream_t stream);
void prof_end(int kind, hipStream_t stream);

// Heads whose blocks a launch dispatches interleaved (work_item).  With fewer
// than eight workgroups per CU, a head-major order leaves the heavy causal
// blocks of an XCD's last head to run after the light blocks of its first
// ones (at B=2, H=16, L=4096 the dQ and forward launches finish at about 1.5x
// their balanced time), so the BH / 8 heads that one XCD holds are
// interleaved block-major instead.  Only when BH is a multiple of 8, so that
// each group fills exactly one XCD's range of xcd_remap; with more
// workgroups per CU the head-major order keeps one head per XCD (its K/V
// stay in that XCD's L2) and already balances.
inline int head_group(int BH, int items_per_head) {
  const long long items = (long long)BH * items_per_head;
  if (items >= 8LL * 256 || BH % 8 != 0 || BH < 16) return 1;
  return BH / 8;
}

// ---- bf16 forward ---------------------------------------------------------------
// Number of key splits to use (requested <= 0: heuristic), clamped to the number
// of 64-key blocks.
int fwd_bf16_num_splits(int BH, int Tq, int Tk, int causal, int requested);
size_t fwd_bf16_workspace_bytes(int BH, int Tq, int Tk, int d, int num_splits);
hipError_t fwd_bf16_launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Tq,
                           int Tk, int d, float scale, int causal, int num_splits, void* workspace,
                           hipStream_t stream);
// Partial state (acc, m, l) of one key range; causal blocks key j for query i
// when j > i + diag.  m in natural-log units.  With num_splits > 1 the range
// is computed in key splits (workspace of fwd_bf16_workspace_bytes) whose
// states are merged into acc, m, l; fwd_bf16_state_splits gives the count.
int fwd_bf16_state_splits(int BH, int Tq, int Tk, int causal);
hipError_t fwd_bf16_state_launch(const void* q, const void* k, const void* v, float* acc, float* m, float* l, int BH,
                                 int Tq, int Tk, int d, float scale, int causal, int diag, int num_splits,
                                 void* workspace, hipStream_t stream);
// Merge of n partial states [n][BH][Tq](x d) into O (bf16) and LSE.
hipError_t merge_states_launch(const float* acc, const float* m, const float* l, int n, void* o, float* lse, int BH,
                               int Tq, int d, hipStream_t stream);

// ---- bf16 backward --------------------------------------------------------------
// Key-range splits of the dQ kernel for a workspace of at most ws_cap bytes:
// the default plan when it fits, else the most splits that fit (1 = no fp32
// partials), 0 if not even the row statistics fit.
int bwd_bf16_dq_splits(int BH, int Tq, int Tk, int d, size_t ws_cap);
size_t bwd_bf16_workspace_bytes(int BH, int Tq, int Tk, int d, int dq_splits);
// dlse (may be null): upstream gradient of the loss with respect to LSE [BH][Tq].
hipError_t bwd_bf16_launch(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const float* dlse, const void* dout, void* dq, void* dk, void* dv, int BH, int Tq, int Tk,
                           int d, float scale, int causal, int dq_splits, void* workspace, hipStream_t stream);
// Device address of this device's copy of the library's static scratch array
// (ATTN_NOALLOC_SCRATCH_BYTES bytes), looked up once per device.
hipError_t bwd_bf16_noalloc_scratch(void** ptr);

// ---- bf16 decode (newest 1..4 queries against a key cache) -----------------------
int decode_bf16_num_splits(int BH, int Tk, int d, int requested);
size_t decode_bf16_workspace_bytes(int BH, int Tq, int d, int num_splits);
// kv_lens: device int32 [B] or null; query i of sequence b sits at position
// len_b - Tq + i.
hipError_t decode_bf16_launch(const void* q, const void* k, const void* v, const int* kv_lens, void* o, float* lse,
                              int B, int H, int Tq, int Tk, int d, float scale, int causal, int num_splits,
                              void* workspace, hipStream_t stream);

// ---- bf16 standard (materialised) attention, for the IO comparison -------------
size_t std_bf16_workspace_bytes(int BH, int Tq, int Tk, int d);
hipError_t std_bf16_launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Tq, int Tk,
                           int d, float scale, int causal, void* workspace, hipStream_t stream);

// ---- fp32 path (block-size faithful forward, deterministic backward) -------------
// rescale == 0: the chunk-wise mode without the running max (overflows for
// large scores; a negative control).
hipError_t fwd_f32_launch(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int Tq,
                          int Tk, int d, int dv, float scale, int causal, int block_n, int rescale,
                          hipStream_t stream);
hipError_t bwd_f32_launch(const float* q, const float* k, const float* v, const float* o, const float* lse,
                          const float* dout, float* dq, float* dk, float* dv_grad, int BH, int Tq, int Tk, int d,
                          int dv, float scale, int causal, hipStream_t stream);

}  // namespace attn
