// Decode: the newest Tq (1..4) queries of each sequence against its key/value
// cache, bf16 inputs, fp32 arithmetic.
//
// This is the recurrent mode of "The Hidden Recurrence in Softmax Attention"
// (section "Recurrent mode": the query of step t sees the keys of steps up to
// t, and the state (l, a) is updated key by key), kept numerically safe with
// the running max of "Tiled attention with an online softmax" (section "Task")
// and split over key ranges whose states are merged by the rescale rule of
// the first page's section "Chunk-wise Mode with Online Softmax Re-scale".
//
// The work is a matrix-vector product per head: every cached key and value is
// read once and used for 2*(d + dv) flops per query, so the kernel is bound by
// HBM bandwidth, not by the matrix cores.  It runs on the vector ALUs:
//   * a group of LPK = D/8 lanes owns one key at a time; each lane loads 16
//     bytes (8 bf16) of the key row and of the value row, so a wave reads
//     64/LPK whole rows per load instruction and a workgroup 4*64/LPK
//     consecutive rows (4 KB of K and 4 KB of V at D = 128);
//   * q.k is 4 bf16 dot2 instructions per lane and a sum over the group by
//     DPP lane moves that leaves the same value in every lane of the group;
//   * each group keeps its own state (m, l, a) per query, with the lazy
//     reference max of the forward kernel (moved only when a score exceeds it
//     by more than 8 in log2 units), and each lane accumulates p*v for its 8
//     columns;
//   * the groups' states are merged through LDS at the end; with several key
//     splits per row the workgroup writes its merged state and a second
//     kernel merges the splits (one workgroup per query row, reading that
//     row's partial states, which lie next to each other).
// Each lane issues the 2*U 16-byte loads of a batch before using any of
// them; latency is hidden by the several workgroups resident per CU.  K and V
// rows are read once, with non-temporal loads.  Splits are short (256 rows by
// default) so that caches of mixed lengths still give every CU a similar
// share; splits that lie past a sequence's length exit at once, and the
// merge reads only the splits a sequence's length covers.
#include "attn_common.hpp"
#include "attn_launch.hpp"

namespace attn {
namespace {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeBatchSteps = 8;  // U: rows per group per batch
constexpr int kDecodeMaxSplits = 1024;
constexpr int kDecodeMinSplitRows = 256;
constexpr float kDecodeTau = 8.f;     // lazy rescale threshold, log2 units

struct DecodeArgs {
  const __bf16* q;      // [BH][Tq][D]
  const __bf16* k;      // [BH][Tk][D]
  const __bf16* v;      // [BH][Tk][D]
  const int* kv_lens;   // [B] or null (every sequence uses all Tk slots)
  __bf16* o;            // [BH][Tq][D]           (single split)
  float* lse;           // [BH][Tq]              (single split)
  float* part_acc;      // [BH][Tq][splits][D]   (several splits)
  float* part_m;        // [BH][Tq][splits]      natural-log units
  float* part_l;        // [BH][Tq][splits]
  int H, BH, Tq, Tk;
  int num_splits, keys_per_split;
  float scale_log2;
};

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over an aligned group of LPK (8 or 16) lanes.  Every step pairs lanes
// whose partial sums are equal as sets, so all lanes of the group end with
// bit-identical values (x + y == y + x in floating point).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_mov<0xB1>(x);  // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_mov<0x4E>(x);  // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LPK == 16) x += dpp_mov<0x140>(x);  // row_mirror: quad 0 <-> 3, 1 <-> 2
  x += dpp_mov<0x141>(x);  // row_half_mirror: the other quad of each 8
  return x;
}

__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // copy the element out first: a bit cast of a vector-element lvalue reads
    // element 0 with this compiler
    const unsigned x = a[e], y = b[e];
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), s, false);
  }
  return s;
}

__device__ __forceinline__ u32x4 ld_row16(const __bf16* p) { return *reinterpret_cast<const u32x4*>(p); }
// cache rows are used once: non-temporal
__device__ __forceinline__ u32x4 ld_stream16(const __bf16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <int D, int NQ, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kDecodeThreads) void decode_bf16_kernel(DecodeArgs a) {
  constexpr int LPK = D / 8;           // lanes per key row
  constexpr int KPW = 64 / LPK;        // rows per wave per load
  constexpr int G = 4 * KPW;           // lane groups per workgroup
  constexpr int U = kDecodeBatchSteps;
  constexpr int BATCH = U * G;         // rows per workgroup per batch
  __shared__ float red_m[NQ][G], red_l[NQ][G];
  __shared__ __attribute__((aligned(16))) float red_acc[NQ][G][D];

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int sub = lane % LPK, grp = wave * KPW + lane / LPK;
  const int split = blockIdx.x % a.num_splits;
  const int bh = blockIdx.x / a.num_splits;
  const int b = bh / a.H;

  int len = a.Tk;
  if (a.kv_lens) len = min(max(a.kv_lens[b], 0), a.Tk);
  const int kbeg = split * a.keys_per_split;
  const int kend = min(len, kbeg + a.keys_per_split);
  const int pos0 = len - a.Tq;  // cache position of query 0
  // the merge reads only the splits below the sequence's length
  if (SPLIT && kend <= kbeg) return;

  u32x4 qv[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) qv[i] = ld_row16(a.q + ((size_t)bh * a.Tq + min(i, a.Tq - 1)) * D + 8 * sub);

  float m[NQ], l[NQ], acc[NQ][8];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[i][c] = 0.f;
  }

  if (kend > kbeg) {
    const __bf16* Kh = a.k + (size_t)bh * a.Tk * D + 8 * sub;
    const __bf16* Vh = a.v + (size_t)bh * a.Tk * D + 8 * sub;
    const float c2 = a.scale_log2;
    // rows past the range are clamped to its last row (loaded, then ignored)
    auto load = [&](u32x4 (&kb)[U], u32x4 (&vb)[U], int base) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int key = min(base + u * G + grp, kend - 1);
        kb[u] = ld_stream16(Kh + (size_t)key * D);
        vb[u] = ld_stream16(Vh + (size_t)key * D);
      }
    };
    auto consume = [&](const u32x4 (&kb)[U], const u32x4 (&vb)[U], int base) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int key = base + u * G + grp;
        const bool valid = key < kend;
        float vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[2 * e] = __builtin_bit_cast(float, vb[u][e] << 16);
          vf[2 * e + 1] = __builtin_bit_cast(float, vb[u][e] & 0xFFFF0000u);
        }
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          // the lane-group sum runs with every lane active, outside any branch
          const float dot = group_sum<LPK>(dot8(kb[u], qv[i]));
          const bool ok = valid && (!CAUSAL || key <= pos0 + i);
          const float s = ok ? dot * c2 : -INFINITY;
          if (s > m[i] + kDecodeTau) {  // uniform over the lane group
            const float alpha = fast_exp2(m[i] - s);  // m = -inf -> 0
            l[i] *= alpha;
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[i][c] *= alpha;
            m[i] = s;
          }
          const float p = ok ? fast_exp2(s - m[i]) : 0.f;
          l[i] += p;
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[i][c] += p * vf[c];
        }
      }
    };
    // all 2*U loads of a batch are issued before its first use; the other
    // workgroups resident on the CU keep HBM busy meanwhile
    for (int base = kbeg; base < kend; base += BATCH) {
      u32x4 kb[U], vb[U];
      load(kb, vb, base);
      consume(kb, vb, base);
    }
  }

  // ---- merge the lane groups' states ---------------------------------------------
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    if (sub == 0) {
      red_m[i][grp] = m[i];
      red_l[i][grp] = l[i];
    }
    *reinterpret_cast<f32x4*>(&red_acc[i][grp][8 * sub]) = f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    *reinterpret_cast<f32x4*>(&red_acc[i][grp][8 * sub + 4]) = f32x4{acc[i][4], acc[i][5], acc[i][6], acc[i][7]};
  }
  __syncthreads();
  for (int idx = tid; idx < NQ * D; idx += kDecodeThreads) {
    const int i = idx / D, c = idx % D;
    if (i >= a.Tq) break;
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < G; ++g) M = fmaxf(M, red_m[i][g]);
    const float mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float w = fast_exp2(red_m[i][g] - mu);  // -inf -> 0
      L += w * red_l[i][g];
      A += w * red_acc[i][g][c];
    }
    const size_t row = (size_t)bh * a.Tq + i;
    if (SPLIT) {
      const size_t prow = row * a.num_splits + split;
      a.part_acc[prow * D + c] = A;
      if (c == 0) {
        a.part_m[prow] = M * kLn2;  // -inf stays -inf
        a.part_l[prow] = L;
      }
    } else {
      a.o[row * D + c] = to_bf16(L > 0.f ? A * (1.f / L) : 0.f);
      if (c == 0) a.lse[row] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
    }
  }
}

// Merge of one query row's split states (m natural log, l, a), the rescale
// rule of "The Hidden Recurrence in Softmax Attention", section "Chunk-wise
// Mode with Online Softmax Re-scale": M = max m_s, w_s = e^(m_s - M),
// O = sum w_s a_s / sum w_s l_s, LSE = M + ln(sum w_s l_s).  One workgroup per
// row; only the splits that the sequence's length reaches were written.
template <int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_merge_kernel(DecodeArgs a) {
  constexpr int CG = D / 4;                  // float4 column groups
  constexpr int PH = kDecodeThreads / CG;    // split phases
  __shared__ float w_s[kDecodeMaxSplits];
  __shared__ float red[kDecodeThreads];
  __shared__ __attribute__((aligned(16))) f32x4 part[PH][CG];
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;             // bh * Tq + i
  const int b = (int)(row / a.Tq) / a.H;
  int len = a.Tk;
  if (a.kv_lens) len = min(max(a.kv_lens[b], 0), a.Tk);
  const int n = min(a.num_splits, (len + a.keys_per_split - 1) / a.keys_per_split);
  const size_t base = row * a.num_splits;

  float mx = -INFINITY;
  for (int s = tid; s < n; s += kDecodeThreads) mx = fmaxf(mx, a.part_m[base + s]);
  red[tid] = mx;
  __syncthreads();
  for (int k = kDecodeThreads / 2; k > 0; k >>= 1) {
    if (tid < k) red[tid] = fmaxf(red[tid], red[tid + k]);
    __syncthreads();
  }
  const float M = red[0];
  const float mu = (M == -INFINITY) ? 0.f : M;
  __syncthreads();
  float lsum = 0.f;
  for (int s = tid; s < n; s += kDecodeThreads) {
    const float w = fast_exp2((a.part_m[base + s] - mu) * kLog2e);  // -inf -> 0
    w_s[s] = w;
    lsum += w * a.part_l[base + s];
  }
  red[tid] = lsum;
  __syncthreads();
  for (int k = kDecodeThreads / 2; k > 0; k >>= 1) {
    if (tid < k) red[tid] += red[tid + k];
    __syncthreads();
  }
  const float L = red[0];

  const int cg = tid % CG, ph = tid / CG;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const f32x4* pa = reinterpret_cast<const f32x4*>(a.part_acc + base * D) + cg;
#pragma unroll 8
  for (int s = ph; s < n; s += PH) acc += w_s[s] * pa[(size_t)s * CG];
  part[ph][cg] = acc;
  __syncthreads();
  if (tid < CG) {
    f32x4 t = part[0][tid];
#pragma unroll
    for (int p = 1; p < PH; ++p) t += part[p][tid];
    const float inv = L > 0.f ? 1.f / L : 0.f;
    u32x2 w2 = {pack_bf16x2(t[0] * inv, t[1] * inv), pack_bf16x2(t[2] * inv, t[3] * inv)};
    *reinterpret_cast<u32x2*>(a.o + row * D + 4 * tid) = w2;
    if (tid == 0) a.lse[row] = L > 0.f ? M + fast_log2(L) * kLn2 : -INFINITY;
  }
}

template <int D, int NQ, bool CAUSAL>
hipError_t launch_decode(const DecodeArgs& args, hipStream_t stream) {
  const dim3 grid((unsigned)args.BH * (unsigned)args.num_splits);
  prof_begin(5, stream);
  if (args.num_splits > 1)
    hipLaunchKernelGGL((decode_bf16_kernel<D, NQ, CAUSAL, true>), grid, dim3(kDecodeThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((decode_bf16_kernel<D, NQ, CAUSAL, false>), grid, dim3(kDecodeThreads), 0, stream, args);
  prof_end(5, stream);
  return hipGetLastError();
}

template <int D, int NQ>
hipError_t decode_causal(const DecodeArgs& args, bool causal, hipStream_t stream) {
  return causal ? launch_decode<D, NQ, true>(args, stream) : launch_decode<D, NQ, false>(args, stream);
}

template <int D>
hipError_t decode_dispatch(const DecodeArgs& args, bool causal, hipStream_t stream) {
  if (args.Tq == 1) return decode_causal<D, 1>(args, causal, stream);
  if (args.Tq == 2) return decode_causal<D, 2>(args, causal, stream);
  return decode_causal<D, 4>(args, causal, stream);
}

int decode_batch_rows(int d) { return kDecodeBatchSteps * 4 * (64 / (d / 8)); }

}  // namespace

int decode_bf16_num_splits(int BH, int Tk, int d, int requested) {
  const int batch = decode_batch_rows(d);
  const int max_splits = (Tk + batch - 1) / batch;  // at least one batch of rows per split
  int s = requested;
  if (s <= 0) {
    // about 32768 workgroups over the whole cache (so that caches filled to
    // mixed lengths still spread evenly), splits of at least 256 rows
    s = (32768 + BH - 1) / BH;
    const int by_len = (Tk + kDecodeMinSplitRows - 1) / kDecodeMinSplitRows;
    if (s > by_len) s = by_len;
  }
  if (s > max_splits) s = max_splits;
  if (s > kDecodeMaxSplits) s = kDecodeMaxSplits;
  if ((long long)s * BH > 2147483647LL) s = (int)(2147483647LL / BH);  // workgroup count fits an int
  if (s < 1) s = 1;
  return s;
}

size_t decode_bf16_workspace_bytes(int BH, int Tq, int d, int num_splits) {
  if (num_splits <= 1) return 0;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = (size_t)num_splits * BH * Tq;
  return up(rows * d * sizeof(float)) + 2 * up(rows * sizeof(float));
}

hipError_t decode_bf16_launch(const void* q, const void* k, const void* v, const int* kv_lens, void* o, float* lse,
                              int B, int H, int Tq, int Tk, int d, float scale, int causal, int num_splits,
                              void* workspace, hipStream_t stream) {
  DecodeArgs args;
  args.q = static_cast<const __bf16*>(q);
  args.k = static_cast<const __bf16*>(k);
  args.v = static_cast<const __bf16*>(v);
  args.kv_lens = kv_lens;
  args.o = static_cast<__bf16*>(o);
  args.lse = lse;
  args.part_acc = args.part_m = args.part_l = nullptr;
  args.H = H;
  args.BH = B * H;
  args.Tq = Tq;
  args.Tk = Tk;
  args.num_splits = num_splits;
  const int batch = decode_batch_rows(d);
  const int rows_per_split = (Tk + num_splits - 1) / num_splits;
  args.keys_per_split = (rows_per_split + batch - 1) / batch * batch;
  args.scale_log2 = scale * kLog2e;
  if (num_splits > 1) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t rows = (size_t)num_splits * args.BH * Tq;
    char* ws = static_cast<char*>(workspace);
    args.part_acc = reinterpret_cast<float*>(ws);
    args.part_m = reinterpret_cast<float*>(ws + up(rows * d * sizeof(float)));
    args.part_l = reinterpret_cast<float*>(ws + up(rows * d * sizeof(float)) + up(rows * sizeof(float)));
  }
  hipError_t e = (d == 128) ? decode_dispatch<128>(args, causal != 0, stream)
                            : decode_dispatch<64>(args, causal != 0, stream);
  if (e != hipSuccess || num_splits <= 1) return e;
  const dim3 grid((unsigned)((size_t)args.BH * Tq));
  prof_begin(1, stream);
  if (d == 128)
    hipLaunchKernelGGL(decode_merge_kernel<128>, grid, dim3(kDecodeThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(decode_merge_kernel<64>, grid, dim3(kDecodeThreads), 0, stream, args);
  prof_end(1, stream);
  return hipGetLastError();
}

}  // namespace attn
