// Forward pass of exact tiled-softmax attention, bf16 in / bf16 out, for
// gfx950 (MI355X).
//
// One workgroup of 8 waves owns a tile of 256 query rows of one (batch, head)
// (the "inner-outer loop exchange" of "The Hidden Recurrence in Softmax
// Attention", section "Chunk-wise Mode with Online Softmax Re-scale": query
// tiles outside, key tiles inside).  Each wave owns 32 rows and keeps, per
// row, the running max m, running sum l and accumulator a of "Tiled attention
// with an online softmax", section "Task", entirely in registers.  K/V are
// streamed in tiles of 64 keys through double-buffered LDS.
//
// Per K/V tile and wave:
//   S^T = K Q^T           32x32x16 bf16 MFMA, fp32 accumulators, keys on the
//                         M side so that every lane holds one query row's
//                         scores in registers (row max/sum need only one
//                         exchange between the two lane halves)
//   mask                  causal (key > query) and ragged tails -> blocked
//   m' = max(m, rowmax)   log2 domain: scores are multiplied by scale*log2(e)
//   mu = (m' == -inf) ? 0 : m'      (the page's guard for rows with no key yet)
//   alpha = exp2(m - mu), P = exp2(s - mu), l = alpha*l + rowsum(P)
//   a = alpha*a + V^T P^T  P rounded to bf16; V read transposed from LDS
// Epilogue: O = a / l, LSE = (m + log2 l) * ln 2.
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

template <int D>
struct FwdCfg {
  static constexpr int KS = D / 16;                    // MFMA k-steps over the head dim
  static constexpr int CB = D / 32;                    // 32-wide blocks of the value dim
  static constexpr int STR = D + 8;                    // LDS row stride (elements)
  static constexpr int TILE = kBN * STR;               // elements per K or V tile
  static constexpr int CHUNKS = kBN * D / 8;           // 16-byte chunks per tile
  static constexpr int PER_THREAD = CHUNKS / kFwdThreads;
  static_assert(CHUNKS % kFwdThreads == 0, "tile must split evenly over threads");
};

template <int D>
__device__ __forceinline__ void load_tile_regs(const __bf16* __restrict__ base, int key0, int key_lim,
                                               int tid, u32x4 (&r)[FwdCfg<D>::PER_THREAD]) {
  constexpr int CPR = D / 8;  // chunks per row
#pragma unroll
  for (int i = 0; i < FwdCfg<D>::PER_THREAD; ++i) {
    const int c = tid + i * kFwdThreads;
    const int row = c / CPR, col = (c % CPR) * 8;
    const int key = key0 + row;
    if (key < key_lim) {
      r[i] = *reinterpret_cast<const u32x4*>(base + (size_t)key * D + col);
    } else {
      r[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile_lds(__bf16* lds, int tid, const u32x4 (&r)[FwdCfg<D>::PER_THREAD]) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < FwdCfg<D>::PER_THREAD; ++i) {
    const int c = tid + i * kFwdThreads;
    const int row = c / CPR, col = (c % CPR) * 8;
    *reinterpret_cast<u32x4*>(lds + row * FwdCfg<D>::STR + col) = r[i];
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

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kFwdThreads, 1) void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[4 * C::TILE];  // K0 V0 K1 V1

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
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
  // last key this wave's rows may see (causal), used to skip whole tiles
  const int wave_kend = CAUSAL ? min(kend, q0 + wave * 32 + 32) : kend;

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
  float m_run = -INFINITY;  // running max of scaled scores, log2 units
  float l_run = 0.f;        // this lane's share of the running sum

  u32x4 kr[C::PER_THREAD], vr[C::PER_THREAD];
  if (ntiles > 0) {
    load_tile_regs<D>(Kh, kbeg, kend, tid, kr);
    load_tile_regs<D>(Vh, kbeg, kend, tid, vr);
    store_tile_lds<D>(lds, tid, kr);
    store_tile_lds<D>(lds + C::TILE, tid, vr);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int key0 = kbeg + t * kBN;
    const __bf16* Ks = lds + (t & 1) * 2 * C::TILE;
    const __bf16* Vs = Ks + C::TILE;
    const bool more = t + 1 < ntiles;
    if (more) {
      load_tile_regs<D>(Kh, key0 + kBN, kend, tid, kr);
      load_tile_regs<D>(Vh, key0 + kBN, kend, tid, vr);
    }

    if (key0 < wave_kend) {
      // ---- S^T = K Q^T : two 32-key blocks -----------------------------------
      f32x16 s[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        s[blk] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (32 * blk + lr) * C::STR + 16 * ks + 8 * hf);
          s[blk] = mfma32(kf, qf[ks], s[blk]);
        }
      }
      // ---- mask: causal and ragged key tail ----------------------------------
      const bool need_mask = (key0 + kBN > kend) || (CAUSAL && key0 + kBN - 1 > q0 + wave * 32);
      if (need_mask) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * blk + 8 * (r / 4) + 4 * hf + (r % 4);
            const bool blocked = key >= kend || (CAUSAL && key > row);
            s[blk][r] = blocked ? -INFINITY : s[blk][r];
          }
      }
      // ---- running max -----------------------------------------------------------
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[blk][r]);
      mx = fmaxf(mx, swap_halves(mx));
      const float mt = (mx == -INFINITY) ? -INFINITY : mx * a.scale_log2;
      const float m_new = fmaxf(m_run, mt);
      const float mu = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - mu);
      m_run = m_new;
      // ---- P = exp2(s*scale*log2e - mu), row sum -------------------------------
      float psum = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[blk][r], a.scale_log2, -mu));
          s[blk][r] = p;
          psum += p;
        }
      if (need_mask) {  // blocked scores must contribute exactly zero (also when scale == 0)
        psum = 0.f;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * blk + 8 * (r / 4) + 4 * hf + (r % 4);
            const bool blocked = key >= kend || (CAUSAL && key > row);
            s[blk][r] = blocked ? 0.f : s[blk][r];
            psum += s[blk][r];
          }
      }
      l_run = l_run * alpha + psum;
      // rescale the accumulator only when some row of the wave changed its max
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
      }
      // ---- P^T as bf16 B operands: k-slot 8*hf+e of (blk,u) <-> key
      //      32*blk + 16*u + (e<4 ? 4*hf+e : 8+4*hf+e-4)
      bf16x8 pb[2][2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[blk][u][e] = to_bf16(s[blk][8 * u + e]);
      // ---- a += V^T P^T ----------------------------------------------------------
      const int g16 = lane % 16, csub = (lane / 16) % 2;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r0 = 32 * blk + 16 * u + 4 * hf + g16 / 4;
#pragma unroll
          for (int cb = 0; cb < C::CB; ++cb) {
            const int c0 = 32 * cb + 16 * csub + 4 * (g16 % 4);
            const i16x4 lo = lds_read_tr(Vs + r0 * C::STR + c0);
            const i16x4 hi = lds_read_tr(Vs + (r0 + 8) * C::STR + c0);
            acc[cb] = mfma32(join_tr(lo, hi), pb[blk][u], acc[cb]);
          }
        }
    }

    if (more) {
      __bf16* Kn = lds + ((t + 1) & 1) * 2 * C::TILE;
      store_tile_lds<D>(Kn, tid, kr);
      store_tile_lds<D>(Kn + C::TILE, tid, vr);
    }
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------------
  const float l_tot = l_run + swap_halves(l_run);
  if (SPLIT) {
    if (row < a.Tq) {
      const size_t prow = ((size_t)split * a.BH + bh) * a.Tq + row;
      float* pa = a.part_acc + prow * D;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = 32 * cb + 8 * g + 4 * hf;
          *reinterpret_cast<f32x4*>(pa + c) =
              f32x4{acc[cb][4 * g], acc[cb][4 * g + 1], acc[cb][4 * g + 2], acc[cb][4 * g + 3]};
        }
      if (hf == 0) {
        a.part_ml[prow * 2 + 0] = m_run;
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
        const int c = 32 * cb + 8 * g + 4 * hf;
        u32x2 w = {pack_bf16x2(acc[cb][4 * g] * inv, acc[cb][4 * g + 1] * inv),
                   pack_bf16x2(acc[cb][4 * g + 2] * inv, acc[cb][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + c) = w;
      }
    if (hf == 0) {
      a.lse[(size_t)bh * a.Tq + row] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
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
