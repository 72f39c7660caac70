// Forward pass of exact tiled-softmax attention, bf16 in / bf16 out, for
// gfx950 (MI355X).
//
// One workgroup of 8 waves owns a tile of 256 query rows of one (batch, head)
// (the "inner-outer loop exchange" of "The Hidden Recurrence in Softmax
// Attention", section "Chunk-wise Mode with Online Softmax Re-scale": query
// tiles outside, key tiles inside).  Each wave owns 32 rows and keeps, per
// row, the running max m, running sum l and accumulator a of "Tiled attention
// with an online softmax", section "Task", in registers.  K/V are streamed in
// tiles of 64 keys through double-buffered LDS; each tile is consumed as two
// 32-key online-softmax steps.
//
// Per 32-key step and wave:
//   S^T = K Q^T           32x32x16 bf16 MFMA, fp32 accumulators, keys on the
//                         M side so that every lane holds one query row's
//                         scores in registers (a row reduction is 16 registers
//                         plus one exchange between the lane halves)
//   mask                  causal (key > query) and ragged tails -> blocked
//   m  = max(m, rowmax)   scores in log2 units (multiplied by scale*log2(e))
//   P  = exp2(s - m), l += rowsum(P), a += V^T P^T  (P rounded to bf16)
// Epilogue: O = a / l, LSE = (m + log2 l) * ln 2.
//
// The reference max m used in the exponent is only moved when a row's block
// max exceeds it by more than kTau (log2 units); then l and a are rescaled by
// exp2(m_old - m_new) as in the page's recurrence.  Between moves P <= 2^kTau,
// and O = a / l and LSE = m + log2 l are the same quantities for any m (the
// result is exact; only fp32 rounding differs).  This keeps the 64-register
// rescale of a off the common path.  A row with no allowed key yet keeps
// m = -inf and uses 0 in its exponent (the page's guard).
//
// LDS layout per stage: K row-major [64][D+8] (MFMA A operand rows, 16-byte
// reads); V transposed, V^T[c][64 keys] with rows of 80 elements, the 4-key
// groups of each 16-key MFMA step ordered so that the 8 keys one lane feeds
// into an MFMA are contiguous, and the 16-byte units XOR-swizzled by (c >> 3)
// (conflict-free 16-byte reads and at most 2-way conflicts on the 8-byte
// transposing writes).
//
// With key splits, each workgroup covers one contiguous key range and stores
// its unnormalised state (m, l, a) in fp32; a second kernel merges the states
// of a row with the same rescale rule and writes O and LSE.
#include "attn_common.hpp"
#include "attn_launch.hpp"

namespace attn {

namespace {

constexpr int kFwdWaves = 8;
constexpr int kFwdThreads = kFwdWaves * 64;
constexpr int kBM = 32 * kFwdWaves;  // query rows per workgroup
constexpr int kBN = 64;              // keys per K/V tile
constexpr int kVtStr = 80;           // V^T row stride (elements)
constexpr float kTau = 8.f;          // lazy-rescale threshold (log2 units)

template <int D>
struct FwdCfg {
  static constexpr int KS = D / 16;                  // MFMA k-steps over the head dim
  static constexpr int CB = D / 32;                  // 32-wide blocks of the value dim
  static constexpr int KSTR = D + 8;                 // K row stride (elements)
  static constexpr int KTILE = kBN * KSTR;           // elements of a K stage
  static constexpr int VTILE = D * kVtStr;           // elements of a V^T stage
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int KCHUNKS = kBN * D / 8;        // 16-byte chunks of a K tile
  static constexpr int KPER = KCHUNKS / kFwdThreads;
  static constexpr int VTASKS = kBN * D / 16;        // 4 keys x 4 columns per task
  static_assert(KCHUNKS % kFwdThreads == 0, "K tile must split evenly over threads");
  static_assert(VTASKS <= kFwdThreads, "one V task per thread at most");
};

// position of 4-key group G (0..15) inside a V^T row: swap bits 0 and 1, so
// groups (8b+4u+h) and (8b+4u+2+h) become adjacent (one lane's 8 keys)
__device__ __forceinline__ int vt_group_pos(int g) { return (g & ~3) | ((g & 1) << 1) | ((g >> 1) & 1); }

// element offset of (column c, 16-byte unit U) in a V^T stage
__device__ __forceinline__ int vt_off(int c, int unit) { return c * kVtStr + ((unit ^ ((c >> 3) & 7)) << 3); }

template <int D>
struct TileRegs {
  u32x4 k[FwdCfg<D>::KPER];
  u32x2 v[4];
};

// Global -> registers for one K/V tile (keys >= key_lim read as zero).
template <int D>
__device__ __forceinline__ void load_tile(const __bf16* __restrict__ Kh, const __bf16* __restrict__ Vh, int key0,
                                          int key_lim, int tid, TileRegs<D>& r) {
  using C = FwdCfg<D>;
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < C::KPER; ++i) {
    const int c = tid + i * kFwdThreads;
    const int row = c / CPR, col = (c % CPR) * 8;
    const int key = key0 + row;
    r.k[i] = key < key_lim ? *reinterpret_cast<const u32x4*>(Kh + (size_t)key * D + col) : u32x4{0u, 0u, 0u, 0u};
  }
  if (tid < C::VTASKS) {
    constexpr int CG = D / 4;  // column groups
    const int kg = tid / CG, cg = tid % CG;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = key0 + 4 * kg + j;
      r.v[j] = key < key_lim ? *reinterpret_cast<const u32x2*>(Vh + (size_t)key * D + 4 * cg) : u32x2{0u, 0u};
    }
  }
}

// Registers -> LDS stage: K rows as is, V transposed into V^T.
template <int D>
__device__ __forceinline__ void store_tile(__bf16* stage, int tid, const TileRegs<D>& r) {
  using C = FwdCfg<D>;
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < C::KPER; ++i) {
    const int c = tid + i * kFwdThreads;
    const int row = c / CPR, col = (c % CPR) * 8;
    *reinterpret_cast<u32x4*>(stage + row * C::KSTR + col) = r.k[i];
  }
  if (tid < C::VTASKS) {
    constexpr int CG = D / 4;
    const int kg = tid / CG, cg = tid % CG;
    const int pos = vt_group_pos(kg);
    __bf16* vt = stage + C::KTILE;
    // r.v[j] = {c0 c1 | c2 c3} of key 4kg+j; write {k0 k1 | k2 k3} of each column
    const u32x2 w0 = {pack_lo16(r.v[0][0], r.v[1][0]), pack_lo16(r.v[2][0], r.v[3][0])};
    const u32x2 w1 = {pack_hi16(r.v[0][0], r.v[1][0]), pack_hi16(r.v[2][0], r.v[3][0])};
    const u32x2 w2 = {pack_lo16(r.v[0][1], r.v[1][1]), pack_lo16(r.v[2][1], r.v[3][1])};
    const u32x2 w3 = {pack_hi16(r.v[0][1], r.v[1][1]), pack_hi16(r.v[2][1], r.v[3][1])};
    const int c0 = 4 * cg, unit = pos >> 1, half = (pos & 1) * 4;
    *reinterpret_cast<u32x2*>(vt + vt_off(c0 + 0, unit) + half) = w0;
    *reinterpret_cast<u32x2*>(vt + vt_off(c0 + 1, unit) + half) = w1;
    *reinterpret_cast<u32x2*>(vt + vt_off(c0 + 2, unit) + half) = w2;
    *reinterpret_cast<u32x2*>(vt + vt_off(c0 + 3, unit) + half) = w3;
  }
}

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  float* part_acc;  // [splits][BH][Tq][D]   (split mode)
  float* part_ml;   // [splits][BH][Tq][2]   (split mode: m in log2 units, l)
  int BH, Tq, Tk;
  int num_qtiles, num_splits, keys_per_split;
  float scale_log2;  // scale * log2(e)
};

// One 64-key tile for one wave: S^T for both 32-key blocks, row max and
// reference-max update, then P and a += V^T P^T block by block.
//
// Blocked keys (need_mask: causal diagonal or ragged tail) are handled by
// scaling the scores in place and writing -inf for blocked ones, after which
// the shared code runs with a unit scale: exp2(-inf - mu) = 0 exactly, also
// when scale == 0.  A row with no allowed key yet (m_ref = -inf) uses mu = 0.
template <int D>
__device__ __forceinline__ void fwd_tile(const __bf16* Ks, const __bf16* Vt, const bf16x8 (&qf)[D / 16],
                                         f32x16 (&acc)[D / 32], float& m_ref, float& l_run, float c, int lr, int hf,
                                         bool need_mask, int key_r0, int kend, int row, bool causal) {
  using C = FwdCfg<D>;
  f32x16 s0 = f32x16{}, s1 = f32x16{};
  {
    bf16x8 kf[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      kf[ks] = *reinterpret_cast<const bf16x8*>(Ks + lr * C::KSTR + 16 * ks + 8 * hf);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) s0 = mfma32(kf[ks], qf[ks], s0);
  }
  {
    bf16x8 kf[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      kf[ks] = *reinterpret_cast<const bf16x8*>(Ks + (32 + lr) * C::KSTR + 16 * ks + 8 * hf);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) s1 = mfma32(kf[ks], qf[ks], s1);
  }
  bf16x8 vf[2][C::CB];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) vf[u][cb] = *reinterpret_cast<const bf16x8*>(Vt + vt_off(32 * cb + lr, 2 * u + hf));

  float cc = c;
  if (need_mask) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key_r0 + 8 * (r / 4) + (r % 4);
      s0[r] = (key >= kend || (causal && key > row)) ? -INFINITY : s0[r] * c;
      s1[r] = (key + 32 >= kend || (causal && key + 32 > row)) ? -INFINITY : s1[r] * c;
    }
    cc = 1.f;
  }
  // ---- row max and reference-max update -----------------------------------------
  float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
  mx = pair_max(mx);
  const float mt = (mx == -INFINITY) ? -INFINITY : mx * cc;
  const bool move = mt > m_ref + kTau;
  if (__builtin_amdgcn_ballot_w64(move)) {
    const float m_new = move ? mt : m_ref;
    const float alpha = move ? fast_exp2(m_ref - m_new) : 1.f;  // m_ref = -inf -> 0
    l_run *= alpha;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
    m_ref = m_new;
  }
  const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
  // ---- block 0: P, row sum, a += V^T P^T ------------------------------------------
  float psum = 0.f;
  bf16x8 p0, p1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = fast_exp2(__builtin_fmaf(s0[e], cc, -mu));
    const float y = fast_exp2(__builtin_fmaf(s0[8 + e], cc, -mu));
    psum += x + y;
    p0[e] = to_bf16(x);
    p1[e] = to_bf16(y);
  }
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) acc[cb] = mfma32(vf[0][cb], p0, acc[cb]);
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) acc[cb] = mfma32(vf[1][cb], p1, acc[cb]);
  // ---- block 1 --------------------------------------------------------------------
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
      vf[u][cb] = *reinterpret_cast<const bf16x8*>(Vt + vt_off(32 * cb + lr, 4 + 2 * u + hf));
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = fast_exp2(__builtin_fmaf(s1[e], cc, -mu));
    const float y = fast_exp2(__builtin_fmaf(s1[8 + e], cc, -mu));
    psum += x + y;
    p0[e] = to_bf16(x);
    p1[e] = to_bf16(y);
  }
  l_run += psum;
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) acc[cb] = mfma32(vf[0][cb], p0, acc[cb]);
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) acc[cb] = mfma32(vf[1][cb], p1, acc[cb]);
#if ATTN_FWD_SCHED
  // interleave the second block's exponentials (VALU) with the first block's
  // P V MFMAs
#pragma unroll
  for (int i = 0; i < 2 * C::CB; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
  }
#endif
}

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kFwdThreads, 1) void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int lr = lane % 32, hf = lane / 32;
  const int n_items = a.BH * a.num_qtiles * a.num_splits;
  const int item = xcd_remap(blockIdx.x, n_items);
  // item = (bh * num_qtiles + (num_qtiles-1-qt)) * num_splits + split: heads
  // outermost, heavier (later) causal query tiles first within a head.
  const int split = item % a.num_splits;
  const int qt = a.num_qtiles - 1 - (item / a.num_splits) % a.num_qtiles;
  const int bh = item / (a.num_splits * a.num_qtiles);

  const int q0 = qt * kBM;
  const int row = q0 + wave * 32 + lr;  // this lane's query row
  const __bf16* Qh = a.q + (size_t)bh * a.Tq * D;
  const __bf16* Kh = a.k + (size_t)bh * a.Tk * D;
  const __bf16* Vh = a.v + (size_t)bh * a.Tk * D;

  int kbeg = 0, kend = a.Tk;
  if (SPLIT) {
    kbeg = split * a.keys_per_split;
    kend = min(a.Tk, kbeg + a.keys_per_split);
  }
  if (CAUSAL) kend = min(kend, q0 + kBM);
  const int ntiles = kend > kbeg ? (kend - kbeg + kBN - 1) / kBN : 0;
  // end of the keys this wave's rows may see (causal): whole tiles past it are
  // skipped
  const int wave_kend = CAUSAL ? min(kend, q0 + wave * 32 + 32) : kend;
  const int wave_row0 = q0 + wave * 32;

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[row][16*ks + 8*hf + 0..7]
  bf16x8 qf[C::KS];
  {
    const bool ok = row < a.Tq;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 t = ok ? *reinterpret_cast<const u32x4*>(Qh + (size_t)row * D + 16 * ks + 8 * hf)
                   : u32x4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, t);
    }
  }

  f32x16 acc[C::CB];
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) acc[cb] = f32x16{};
  float m_ref = -INFINITY;  // reference max of scaled scores, log2 units
  float l_run = 0.f;        // this lane's share of the running sum
  const float c = a.scale_log2;

  TileRegs<D> tr;
  if (ntiles > 0) {
    load_tile<D>(Kh, Vh, kbeg, kend, tid, tr);
    store_tile<D>(lds, tid, tr);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int key0 = kbeg + t * kBN;
    const __bf16* Ks = lds + (t & 1) * C::STAGE;
    const __bf16* Vt = Ks + C::KTILE;
    const bool more = t + 1 < ntiles;
    if (more) load_tile<D>(Kh, Vh, key0 + kBN, kend, tid, tr);

    if (key0 < wave_kend) {
      const bool need_mask = (key0 + kBN > kend) || (CAUSAL && key0 + kBN - 1 > wave_row0);
      fwd_tile<D>(Ks, Vt, qf, acc, m_ref, l_run, c, lr, hf, need_mask, key0 + 4 * hf, kend, row, CAUSAL);
    }

    if (more) store_tile<D>(lds + ((t + 1) & 1) * C::STAGE, tid, tr);
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------------
  const float l_tot = pair_sum(l_run);
  if (SPLIT) {
    if (row < a.Tq) {
      const size_t prow = ((size_t)split * a.BH + bh) * a.Tq + row;
      float* pa = a.part_acc + prow * D;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int cc = 32 * cb + 8 * g + 4 * hf;
          *reinterpret_cast<f32x4*>(pa + cc) =
              f32x4{acc[cb][4 * g], acc[cb][4 * g + 1], acc[cb][4 * g + 2], acc[cb][4 * g + 3]};
        }
      if (hf == 0) {
        a.part_ml[prow * 2 + 0] = m_ref;
        a.part_ml[prow * 2 + 1] = l_tot;
      }
    }
    return;
  }
  if (row < a.Tq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* orow = a.o + ((size_t)bh * a.Tq + row) * D;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cc = 32 * cb + 8 * g + 4 * hf;
        u32x2 w = {pack_bf16x2(acc[cb][4 * g] * inv, acc[cb][4 * g + 1] * inv),
                   pack_bf16x2(acc[cb][4 * g + 2] * inv, acc[cb][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + cc) = w;
      }
    if (hf == 0) {
      a.lse[(size_t)bh * a.Tq + row] = l_tot > 0.f ? (m_ref + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

// Merge of split partial states (m_s, l_s, a_s) of one row:
//   M = max_s m_s, l = sum_s 2^(m_s - M) l_s, a = sum_s 2^(m_s - M) a_s,
//   O = a / l, LSE = (M + log2 l) ln 2.  One wave per row, D/64 columns per lane.
template <int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(const float* __restrict__ part_acc,
                                                          const float* __restrict__ part_ml,
                                                          __bf16* __restrict__ o, float* __restrict__ lse,
                                                          int BH, int Tq, int num_splits) {
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / 64;
  const int lane = threadIdx.x % 64;
  if (wave >= BH * Tq) return;
  const size_t rowid = wave;  // = bh * Tq + row
  const size_t stride = (size_t)BH * Tq;
  float M = -INFINITY;
  for (int s = 0; s < num_splits; ++s) M = fmaxf(M, part_ml[(s * stride + rowid) * 2]);
  const float mu = (M == -INFINITY) ? 0.f : M;
  float l = 0.f;
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  for (int s = 0; s < num_splits; ++s) {
    const float ms = part_ml[(s * stride + rowid) * 2];
    const float w = fast_exp2(ms - mu);
    l += w * part_ml[(s * stride + rowid) * 2 + 1];
    const float* pa = part_acc + (s * stride + rowid) * D;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] += w * pa[lane + 64 * j];
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) o[rowid * D + lane + 64 * j] = to_bf16(acc[j] * inv);
  if (lane == 0) lse[rowid] = l > 0.f ? (M + fast_log2(l)) * kLn2 : -INFINITY;
}

template <int D, bool CAUSAL, bool SPLIT>
hipError_t launch_fwd(const FwdArgs& args, hipStream_t stream) {
  const int n = args.BH * args.num_qtiles * args.num_splits;
  prof_begin(0, stream);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, SPLIT>), dim3(n), dim3(kFwdThreads), 0, stream, args);
  prof_end(0, stream);
  return hipGetLastError();
}

template <int D>
hipError_t fwd_dispatch(const FwdArgs& args, bool causal, bool split, hipStream_t stream) {
  if (causal) return split ? launch_fwd<D, true, true>(args, stream) : launch_fwd<D, true, false>(args, stream);
  return split ? launch_fwd<D, false, true>(args, stream) : launch_fwd<D, false, false>(args, stream);
}

}  // namespace

int fwd_bf16_num_splits(int BH, int Tq, int Tk, int causal, int requested) {
  const int qtiles = (Tq + kBM - 1) / kBM;
  const int kblocks = (Tk + kBN - 1) / kBN;
  int s = requested;
  if (s <= 0) {
    // Split the key range only when the query tiles alone leave the 256 CUs
    // under-filled and each split still streams a long key range.
    const int items = BH * qtiles;
    s = 1;
    if (!causal) {
      while (items * s < 2 * 256 && kblocks / (2 * s) >= 8) s *= 2;
    }
  }
  if (s > kblocks) s = kblocks;
  if (s < 1) s = 1;
  return s;
}

size_t fwd_bf16_workspace_bytes(int BH, int Tq, int d, int num_splits) {
  if (num_splits <= 1) return 0;
  return (size_t)num_splits * BH * Tq * (d + 2) * sizeof(float);
}

hipError_t fwd_bf16_launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Tq,
                           int Tk, int d, float scale, int causal, int num_splits, void* workspace,
                           hipStream_t stream) {
  FwdArgs args;
  args.q = static_cast<const __bf16*>(q);
  args.k = static_cast<const __bf16*>(k);
  args.v = static_cast<const __bf16*>(v);
  args.o = static_cast<__bf16*>(o);
  args.lse = lse;
  args.BH = BH;
  args.Tq = Tq;
  args.Tk = Tk;
  args.num_qtiles = (Tq + kBM - 1) / kBM;
  args.num_splits = num_splits;
  const int kblocks = (Tk + kBN - 1) / kBN;
  args.keys_per_split = ((kblocks + num_splits - 1) / num_splits) * kBN;
  args.scale_log2 = scale * kLog2e;
  const bool split = num_splits > 1;
  args.part_acc = split ? static_cast<float*>(workspace) : nullptr;
  args.part_ml = split ? args.part_acc + (size_t)num_splits * BH * Tq * d : nullptr;
  hipError_t e = (d == 128) ? fwd_dispatch<128>(args, causal != 0, split, stream)
                            : fwd_dispatch<64>(args, causal != 0, split, stream);
  if (e != hipSuccess || !split) return e;
  const int rows = BH * Tq;
  const int blocks = (rows + 3) / 4;
  prof_begin(1, stream);
  if (d == 128)
    hipLaunchKernelGGL(fwd_combine_kernel<128>, dim3(blocks), dim3(256), 0, stream, args.part_acc, args.part_ml,
                       args.o, lse, BH, Tq, num_splits);
  else
    hipLaunchKernelGGL(fwd_combine_kernel<64>, dim3(blocks), dim3(256), 0, stream, args.part_acc, args.part_ml,
                       args.o, lse, BH, Tq, num_splits);
  prof_end(1, stream);
  return hipGetLastError();
}

}  // namespace attn
