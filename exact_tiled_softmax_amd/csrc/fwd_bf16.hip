// Forward pass of exact tiled-softmax attention, bf16 in / bf16 out, for
// gfx950 (MI355X).
//
// A workgroup of 8 waves owns a tile of 256 query rows of one (batch, head)
// at a time (at d = 128 a persistent workgroup runs a list of such tiles)
// (the "inner-outer loop exchange" of "The Hidden Recurrence in Softmax
// Attention", section "Chunk-wise Mode with Online Softmax Re-scale": query
// tiles outside, key tiles inside).  Each wave owns 32 rows and keeps, per
// row, the running max m, running sum l and accumulator a of "Tiled attention
// with an online softmax", section "Task", in registers; its Q rows stay in
// registers as MFMA operands.  K and V are streamed, row-major, in tiles of
// 64 keys through a 4-stage LDS ring filled by direct-to-LDS copies, three
// tiles ahead of the compute; the V operand of the PV product (V^T, keys
// along k) comes from transposing LDS reads (ds_read_b64_tr_b16), so no
// transposed copy of V is made in HBM.
//
// Per 64-key tile and wave:
//   S^T = K Q^T           32x32x16 bf16 MFMA, fp32 accumulators, keys on the
//                         M side so that every lane holds one query row's
//                         scores in registers (a row reduction is 32 registers
//                         plus one exchange between the lane halves)
//   mask                  causal (key > query) and ragged tails -> blocked
//                         (diagonal and tail tiles only)
//   m  = max(m, rowmax)   scores in log2 units (multiplied by scale*log2(e))
//   P  = exp2(s - m), l += rowsum(P), a += V^T P^T  (P rounded to bf16; V^T
//                         fragments by transposing reads of the V tile)
// Epilogue: O = a / l, LSE = (m + log2 l) * ln 2.
//
// The reference max m used in the exponent is only moved when a row's tile
// max exceeds it by more than kTau (log2 units); then l and a are rescaled by
// exp2(m_old - m_new) as in the page's recurrence.  O = a / l and LSE = m +
// log2 l are the same quantities for any m (the result is exact; only fp32
// rounding differs), so m only has to keep P bounded.  An unmasked tile
// (head dim 128) therefore takes no row max at all: its P is computed against
// the current m and kept when the tile's row sum is at most 2^16 (every
// value of P at most 2^16); only past that bound is the tile redone with its
// row max.  This keeps both the row max and the 64-register rescale of a off
// the common path.  A row with no allowed key yet keeps m = -inf and uses 0
// in its exponent (the page's guard).
//
// With key splits, each workgroup covers one contiguous key range and stores
// its unnormalised state (m, l, a) in fp32; a second kernel merges the states
// of a row with the same rescale rule and writes O and LSE.
#include <algorithm>
#include <type_traits>

#include "attn_common.hpp"
#include "attn_launch.hpp"
#include "tile_stream.hpp"

namespace attn {

namespace {

constexpr float kTau = 8.f;  // lazy-rescale threshold (log2 units)
// largest row sum of one tile's P accepted without a row max (every value of
// P is then at most 2^16)
constexpr float kFastSum = 65536.f;

template <int D>
struct FwdCfg {
  static constexpr int KS = D / 16;                      // MFMA k-steps over the head dim
  static constexpr int CB = D / 32;                      // 32-wide blocks of the value dim
  static constexpr int CPR = D / 8;                      // 16-byte chunks per K row
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 32 * WAVES;                  // query rows per workgroup
  static constexpr int BN = 64;                          // keys per tile
  static constexpr int TILE = BN * D;                    // bf16 elements of a K tile and of a V^T tile
  static constexpr int PER_TENSOR = TILE * 2 / 1024;     // wave copies per tensor and tile
  static constexpr int PER_WAVE = 2 * PER_TENSOR / WAVES;
  static constexpr int VM = PER_WAVE;                    // vector-memory ops per wave and tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int NSTAGE = 4;
  static constexpr int AHEAD = NSTAGE - 1;               // tiles in flight ahead of the compute
  // waves per SIMD the register budget is set for: two workgroups per CU at
  // d = 64 (64 KB of LDS each), one at d = 128
  static constexpr int WAVES_PER_SIMD = D == 64 ? 4 : 2;
  // d = 128: persistent workgroups, each running a list of items; d = 64:
  // one workgroup per item (two share a CU, hiding each other's fill and
  // drain, and the item loop would not fit the 128-register budget)
  static constexpr bool PERSIST = D == 128;
  static_assert(PER_WAVE >= 1 && 2 * PER_TENSOR == PER_WAVE * WAVES, "tile copy split");
  static_assert(PER_TENSOR % PER_WAVE == 0, "the copies of one wave belong to one tensor");
};

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;   // V [BH][Tk][D]: row-major tiles in LDS, read transposed
  __bf16* o;
  float* lse;
  float* part_acc;  // [splits][BH][Tq][D]   (split / state mode: unnormalised a)
  float* part_m;    // [splits][BH][Tq]      (split / state mode: reference max, natural log units)
  float* part_l;    // [splits][BH][Tq]      (split / state mode: l)
  int BH, Tq, Tk, Tk_pad;
  int diag;          // causal: key j is blocked for query i when j > i + diag
  int num_qtiles, num_splits, keys_per_split;
  int n_items;         // BH * num_qtiles * num_splits
  int n_items_paired;  // BH * ceil(num_qtiles / 2) * num_splits: pairs of query tiles
  int nwg;           // workgroups of the persistent launch
  float scale_log2;  // scale * log2(e)
};

// Copies of one K tile and one V tile (keys key0 .. key0+63, both row-major,
// 16-byte chunks swizzled per row) into a stage.
template <int D>
__device__ __forceinline__ void fwd_issue(const FwdArgs& a, int bh, int key0, __bf16* stg, int wave, int lane) {
  using C = FwdCfg<D>;
  // The lane index is made opaque here: otherwise the compiler hoists this
  // rare path's per-lane 64-bit addresses out of the tile loop and keeps them
  // in registers for the whole kernel (22 VGPRs at head dim 128).
  asm volatile("" : "+v"(lane));
  const __bf16* Kh = a.k + (size_t)bh * a.Tk * D;
  const __bf16* Vh = a.v + (size_t)bh * a.Tk * D;
#pragma unroll
  for (int n = 0; n < C::PER_WAVE; ++n) {
    const int cpy = wave * C::PER_WAVE + n;  // wave-uniform
    const int tensor = cpy / C::PER_TENSOR, i = cpy % C::PER_TENSOR;
    const int p = 64 * i + lane;
    __bf16* dst = stg + tensor * C::TILE + 512 * i;
    const int row = p / C::CPR, c = (p % C::CPR) ^ swz<C::CPR>(row);
    const int kk = min(key0 + row, a.Tk - 1);
    dma16((tensor == 0 ? Kh : Vh) + (size_t)kk * D + 8 * c, dst);
  }
}

// One 64-key tile for one wave: S^T for both 32-key blocks, row max and
// reference-max update, then P and a += V^T P^T.
//
// Blocked keys (need_mask: causal diagonal or ragged tail) are handled by
// scaling the scores in place and writing -inf for blocked ones, after which
// the shared code runs with a unit scale: exp2(-inf - mu) = 0 exactly, also
// when scale == 0.  A row with no allowed key yet (m_ref = -inf) uses mu = 0.
//
// LDS addresses are a per-lane byte offset, computed once per kernel
// (FwdLdsOffsets), plus a constant: the stage base is a compile-time constant
// (the tile loop is unrolled over the stages) and the rows of a fragment
// group differ from the first group's by whole 16-row blocks, which the
// swizzle leaves unchanged.
template <int D>
struct FwdLdsOffsets {
  uint32_t k[D / 16];          // K fragment of k-step ks, rows 0..31 (+32u rows for block u)
  uint32_t v[D / 32][2];       // V^T fragment of column block cb, rows 4hf..+3 (h = 0) and 8 more (h = 1)
};

template <int D>
__device__ __forceinline__ FwdLdsOffsets<D> fwd_lds_offsets(int lane) {
  using C = FwdCfg<D>;
  const int lr = lane % 32, hf = lane / 32, rsw = swz<C::CPR>(lr);
  const int g16 = lane % 16, csub = (lane / 16) % 2;
  auto at = [](int r, int cc) { return r * D + 8 * ((cc >> 3) ^ swz<C::CPR>(r)) + (cc & 7); };
  FwdLdsOffsets<D> o;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) o.k[ks] = (uint32_t)(lr * D + 8 * ((2 * ks + hf) ^ rsw)) * 2u;
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      o.v[cb][h] = (uint32_t)(C::TILE + at(4 * hf + g16 / 4 + 8 * h, 32 * cb + 16 * csub + 4 * (g16 % 4))) * 2u;
  // opaque to the compiler's known-bits analysis, so that base + constant
  // stays an add, which folds into the LDS instruction's offset field
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) asm volatile("" : "+v"(o.k[ks]));
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) asm volatile("" : "+v"(o.v[cb][0]), "+v"(o.v[cb][1]));
  return o;
}

template <int D>
__device__ __forceinline__ void fwd_tile(const char* stg, const FwdLdsOffsets<D>& lo, const bf16x8 (&qf)[8],
                                         f32x16 (&acc)[4], float& m_ref, float& l_run, float c, int lane,
                                         bool need_mask, int key0, int kend, int row, bool causal) {
  using C = FwdCfg<D>;
  const int hf = lane / 32;
  // the two 32-key score chains alternate; K fragments are read 4 k-steps
  // ahead of their MFMAs (each read issued after the MFMA that frees its
  // registers)
  constexpr int LA = C::KS < 4 ? C::KS : 4;
  bf16x8 kfr[C::KS][2];
  auto rd = [&](int ks) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      kfr[ks][u] = *reinterpret_cast<const bf16x8*>(stg + lo.k[ks] + 32 * u * D * 2);
  };
#pragma unroll
  for (int ks = 0; ks < LA; ++ks) rd(ks);
  f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 2; ++u) s[u] = mfma32(kfr[ks][u], qf[ks], s[u]);
    if (ks + LA < C::KS) rd(ks + LA);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- P (bf16 B operand: k-slot 8hf+e of step s2 = register 8*s2 + e) ------------
  float psum = 0.f;
  bf16x8 pb[2][2];
  auto make_p = [&](float cc, float mu) {
    psum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = fast_exp2(__builtin_fmaf(s[u][r], cc, -mu));
        psum += x;
        pb[u][r / 8][r % 8] = to_bf16(x);
      }
  };
  // Fast path (head dim 128, an unmasked tile, every row with a finite
  // reference): P against the current reference without a row max; the row
  // sum shows whether any value has grown past the bound, and only then the
  // tile is redone with the row max.  (At head dim 64 the branch costs more
  // than the maxima it saves.)
  bool redo = true;
  if (D == 128 && !need_mask && !__builtin_amdgcn_ballot_w64(m_ref == -INFINITY)) {
    make_p(c, m_ref);
    redo = __builtin_amdgcn_ballot_w64(!(psum <= kFastSum)) != 0;
  }
  if (redo) {
    // accumulator register r of block u: key key0 + 32u + 8(r/4) + 4hf + r%4
    float cc = c;
    if (need_mask) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * u + 8 * (r / 4) + 4 * hf + (r % 4);
          s[u][r] = (key >= kend || (causal && key > row)) ? -INFINITY : s[u][r] * c;  // row: i + diag
        }
      cc = 1.f;
    }
    // ---- row max and reference-max update ---------------------------------------
    // a chain of three-input maxima: two scores per instruction
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, s[0][r]), s[1][r]);
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
    make_p(cc, (m_ref == -INFINITY) ? 0.f : m_ref);
  }
  l_run += psum;
  // ---- a += V^T P^T -----------------------------------------------------------------
  // A operand (column 32cb + lane%32 of V, k-slots = the keys of P's k-slots)
  // by two transposing reads of the row-major V tile: rows 32u + 16s2 + 4hf
  // + 0..3 and the same + 8 (the order in which the score accumulator hands
  // its keys to P's k-slots)
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) {
        const char* vr = stg + (32 * u + 16 * s2) * D * 2;
        const bf16x8 va = join_tr(lds_read_tr(reinterpret_cast<const __bf16*>(vr + lo.v[cb][0])),
                                  lds_read_tr(reinterpret_cast<const __bf16*>(vr + lo.v[cb][1])));
        acc[cb] = mfma32(va, pb[u][s2], acc[cb]);
      }
}

// Work list of the forward launch.  At d = 128 the launch is persistent: a.nwg
// workgroups (as many as the chip holds at once) each run a fixed list of
// items (head, key split, query tile) one after the other, so that no
// workgroup waits on the dispatcher between items (with one workgroup per CU
// a CU idled about 6 us, median, between two workgroups), and the first tile
// copies of the next item are issued before the current item's outputs are
// written.  Items come in pairs (query tile nq-1-k, query tile k) of one
// (head, split), whose causal work adds up to the same total for every k,
// dealt round-robin over the workgroups (pair wg + r*nwg, head-major): one
// XCD's workgroups (consecutive logical ids, xcd_remap) hold the pairs of one
// or two heads in each round and share their K/V tiles in L2.  With no more
// items than workgroups, each workgroup takes one item.
struct FwdItem {
  int bh, qt, split;
  int kbeg, kend, ntiles;  // key range and its 64-key tiles
};

template <int D, bool CAUSAL, bool SPLIT>
__device__ __forceinline__ bool fwd_item(const FwdArgs& a, int wg, int m, FwdItem& it) {
  using C = FwdCfg<D>;
  const int nq = a.num_qtiles;
  int rest;
  if (a.nwg >= a.n_items) {
    // one item per workgroup, query tile fastest
    if (m > 0 || wg >= a.n_items) return false;
    rest = wg / nq;
    it.qt = wg % nq;
  } else {
    // pairs (query tile nq-1-k, query tile k) of one (head, split), dealt
    // round-robin; the middle tile of an odd count pairs with itself and is
    // run once
    const int npair = (nq + 1) >> 1;
    const int q = wg + (m >> 1) * a.nwg;
    if (q >= a.n_items_paired) return false;
    rest = q / npair;
    const int k = q - rest * npair;
    if ((m & 1) && nq - 1 - k == k) {
      it.ntiles = -1;  // the middle tile, already run
      return true;
    }
    it.qt = (m & 1) ? k : nq - 1 - k;
  }
  it.split = SPLIT ? rest % a.num_splits : 0;
  it.bh = SPLIT ? rest / a.num_splits : rest;
  int kbeg = 0, kend = a.Tk;
  if (SPLIT) {
    kbeg = it.split * a.keys_per_split;
    kend = min(a.Tk, kbeg + a.keys_per_split);
  }
  if (CAUSAL) kend = max(kbeg, min(kend, it.qt * C::BM + C::BM + a.diag));
  it.kbeg = kbeg;
  it.kend = kend;
  it.ntiles = kend > kbeg ? (kend - kbeg + C::BN - 1) / C::BN : 0;
  return true;
}

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(FwdCfg<D>::THREADS, FwdCfg<D>::WAVES_PER_SIMD) void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 stages[C::NSTAGE * C::STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int lr = lane % 32, hf = lane / 32;
  const int wg = xcd_remap(blockIdx.x, a.nwg);

  // Tile copies: a tile that lies inside [0, Tk) is copied from a
  // wave-uniform base with per-lane byte offsets computed here once (the
  // layout of fwd_issue); a tile that runs past Tk clamps its rows per lane.
  uint32_t voff[C::PER_WAVE];
#pragma unroll
  for (int n = 0; n < C::PER_WAVE; ++n) {
    const int i = (wave * C::PER_WAVE + n) % C::PER_TENSOR, p = 64 * i + lane;
    const int rr = p / C::CPR, cc = (p % C::CPR) ^ swz<C::CPR>(rr);
    voff[n] = (uint32_t)((rr * D + 8 * cc) * (int)sizeof(__bf16));
  }
  auto issue = [&](int bh, int key0, __bf16* stg) {
    if (key0 + C::BN <= a.Tk) {
      const int tensor = (wave * C::PER_WAVE) / C::PER_TENSOR;  // the same for all copies of a wave
      const __bf16* base = (tensor == 0 ? a.k : a.v) + ((size_t)bh * a.Tk + key0) * D;
#pragma unroll
      for (int n = 0; n < C::PER_WAVE; ++n) {
        const int i = (wave * C::PER_WAVE + n) % C::PER_TENSOR;
        dma16_sbase(base, voff[n], stg + tensor * C::TILE + 512 * i);
      }
    } else {
      fwd_issue<D>(a, bh, key0, stg, wave, lane);
    }
  };
  auto stage = [&](int t) { return stages + (t % C::NSTAGE) * C::STAGE; };
  auto prologue = [&](const FwdItem& it) {
    for (int t = 0; t < C::AHEAD && t < it.ntiles; ++t) issue(it.bh, it.kbeg + t * C::BN, stage(t));
  };
  const FwdLdsOffsets<D> lo = fwd_lds_offsets<D>(lane);
  const float c = a.scale_log2;

  // item m of the workgroup's list, or the first after it that is not a
  // repeated middle tile (m advances to it); false at the end of the list
  auto take = [&](int& m, FwdItem& it) {
    for (; fwd_item<D, CAUSAL, SPLIT>(a, wg, m, it); ++m)
      if (it.ntiles >= 0) return true;
    return false;
  };
  FwdItem it;
  int m = 0;
  bool have = take(m, it);
  if (have) prologue(it);
  while (have) {
    const int q0 = it.qt * C::BM;
    const int row = q0 + wave * 32 + lr;  // this lane's query row
    const int ntiles = it.ntiles, kbeg = it.kbeg, kend = it.kend;
    // end of the keys this wave's rows may see (causal): whole tiles past it are
    // skipped
    const int wave_kend = CAUSAL ? min(kend, q0 + wave * 32 + 32 + a.diag) : kend;
    const int wave_row0 = q0 + wave * 32;

    // Q fragments (B operand of S^T = K Q^T): lane holds Q[row][16*ks + 8*hf + 0..7]
    bf16x8 qf[8];
    {
      const __bf16* Qh = a.q + (size_t)it.bh * a.Tq * D;
      const int qr = min(row, a.Tq - 1);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) qf[ks] = ld16(Qh + (size_t)qr * D + 16 * ks + 8 * hf);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) settle(qf[ks]);
    }

    f32x16 acc[4];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) acc[cb] = f32x16{};
    float m_ref = -INFINITY;  // reference max of scaled scores, log2 units
    float l_run = 0.f;        // this lane's share of the running sum

    static_assert(C::AHEAD >= 1 && C::AHEAD <= 3, "the waits below cover up to 2 later tiles");
    static_assert(C::NSTAGE == 4, "the tile loop is unrolled over 4 stages");
    // tile t in stage S = t % NSTAGE, S a compile-time constant
    auto step = [&](int t, auto stage_c) {
      constexpr int S = decltype(stage_c)::value;
      // this wave's copies of tiles t+1 .. t+AHEAD-1 may still be in flight
      const int later = min(C::AHEAD - 1, ntiles - 1 - t);
      if (C::AHEAD >= 3 && later >= 2) wait_vm<2 * C::VM>();
      else if (C::AHEAD >= 2 && later == 1) wait_vm<C::VM>();
      else wait_vm<0>();
      barrier();
      if (t + C::AHEAD < ntiles)
        issue(it.bh, kbeg + (t + C::AHEAD) * C::BN, stages + ((S + C::AHEAD) % C::NSTAGE) * C::STAGE);
      const int key0 = kbeg + t * C::BN;
      if (key0 < wave_kend) {
        const bool need_mask = (key0 + C::BN > kend) || (CAUSAL && key0 + C::BN - 1 > wave_row0 + a.diag);
        fwd_tile<D>(reinterpret_cast<const char*>(stages + S * C::STAGE), lo, qf, acc, m_ref, l_run, c, lane,
                    need_mask, key0, kend, row + a.diag, CAUSAL);
      }
    };
    for (int t = 0; t < ntiles; t += C::NSTAGE) {
      step(t, std::integral_constant<int, 0>{});
      if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
      if (t + 2 < ntiles) step(t + 2, std::integral_constant<int, 2>{});
      if (t + 3 < ntiles) step(t + 3, std::integral_constant<int, 3>{});
    }

    // the next item's first tile copies go out before this item's outputs:
    // every wave is done with the stages once all have passed this barrier
    const FwdItem cur = it;
    if constexpr (C::PERSIST) {
      ++m;
      have = take(m, it);
      barrier();
      if (have) prologue(it);
    } else {
      have = false;
    }

    // ---- epilogue ------------------------------------------------------------------
    const float l_tot = pair_sum(l_run);
    if (SPLIT) {
      if (row < a.Tq) {
        const size_t prow = ((size_t)cur.split * a.BH + cur.bh) * a.Tq + row;
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
          a.part_m[prow] = m_ref * kLn2;  // -inf stays -inf
          a.part_l[prow] = l_tot;
        }
      }
    } else if (row < a.Tq) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      __bf16* orow = a.o + ((size_t)cur.bh * a.Tq + row) * D;
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
        a.lse[(size_t)cur.bh * a.Tq + row] = l_tot > 0.f ? (m_ref + fast_log2(l_tot)) * kLn2 : -INFINITY;
      }
    }
  }
}

// Merge of partial states (m_s, l_s, a_s) of one row, m in natural-log units
// ("The Hidden Recurrence in Softmax Attention", section "Chunk-wise Mode
// with Online Softmax Re-scale": states of key chunks combine by rescaling
// each to the common max):
//   M = max_s m_s, l = sum_s e^(m_s - M) l_s, a = sum_s e^(m_s - M) a_s,
//   O = a / l, LSE = M + ln l.  D/4 lanes per row, each with 4 consecutive
// columns, so that every partial accumulator is read with 16-byte loads (with
// one wave per row and 4-byte loads the merge ran at 3.3-3.6 TB/s).
// With STATE the merged state itself is written (acc = a, m = M, l) instead
// of O and LSE: a key-range state computed in splits.
template <int D, bool STATE>
__global__ __launch_bounds__(256) void fwd_combine_kernel(const float* __restrict__ part_acc,
                                                          const float* __restrict__ part_m,
                                                          const float* __restrict__ part_l,
                                                          __bf16* __restrict__ o, float* __restrict__ lse,
                                                          float* __restrict__ st_acc, float* __restrict__ st_m,
                                                          float* __restrict__ st_l, int BH, int Tq,
                                                          int num_splits) {
  constexpr int LPR = D / 4;  // lanes per row
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t rowid = t / LPR;
  const int c = (int)(t % LPR) * 4;  // this lane's first column
  if (rowid >= (size_t)BH * Tq) return;
  const size_t stride = (size_t)BH * Tq;
  float M = -INFINITY;
  for (int s = 0; s < num_splits; ++s) M = fmaxf(M, part_m[s * stride + rowid]);
  const float mu = (M == -INFINITY) ? 0.f : M;
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < num_splits; ++s) {
    const float w = fast_exp2((part_m[s * stride + rowid] - mu) * kLog2e);  // -inf -> 0
    l += w * part_l[s * stride + rowid];
    const f32x4 pa = *reinterpret_cast<const f32x4*>(part_acc + (s * stride + rowid) * D + c);
    acc += w * pa;
  }
  if constexpr (STATE) {
    *reinterpret_cast<f32x4*>(st_acc + rowid * D + c) = acc;
    if (c == 0) {
      st_m[rowid] = M;
      st_l[rowid] = l;
    }
  } else {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const u32x2 ov = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    *reinterpret_cast<u32x2*>(o + rowid * D + c) = ov;
    if (c == 0) lse[rowid] = l > 0.f ? M + fast_log2(l) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool SPLIT>
hipError_t launch_fwd(FwdArgs args, hipStream_t stream) {
  const int resident = resident_workgroups<fwd_bf16_kernel<D, CAUSAL, SPLIT>>(FwdCfg<D>::THREADS);
  if (resident <= 0) return hipErrorInvalidDevice;
  args.nwg = (FwdCfg<D>::PERSIST && args.n_items > resident) ? std::min(args.n_items_paired, resident) : args.n_items;
  prof_begin(0, stream);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, SPLIT>), dim3(args.nwg), dim3(FwdCfg<D>::THREADS), 0, stream, args);
  prof_end(0, stream);
  return hipGetLastError();
}

template <int D>
hipError_t fwd_dispatch(const FwdArgs& args, bool causal, bool split, hipStream_t stream) {
  if (causal) return split ? launch_fwd<D, true, true>(args, stream) : launch_fwd<D, true, false>(args, stream);
  return split ? launch_fwd<D, false, true>(args, stream) : launch_fwd<D, false, false>(args, stream);
}

constexpr int kBM = FwdCfg<128>::BM;  // the same for both head dims
constexpr int kBN = 64;
static_assert(FwdCfg<64>::BM == kBM && FwdCfg<128>::BM == kBM && FwdCfg<128>::BN == kBN, "tile sizes");

struct FwdLayout {
  size_t part_acc, part_m, part_l, total;
};

// workspace: the key-split partial states only (none without splits)
FwdLayout fwd_layout(int BH, int Tq, int Tk, int d, int num_splits) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  (void)Tk;
  FwdLayout L;
  L.part_acc = 0;
  L.part_m = L.part_l = L.total = L.part_acc;
  if (num_splits > 1) {
    L.part_m = up(L.part_acc + (size_t)num_splits * BH * Tq * d * sizeof(float));
    L.part_l = up(L.part_m + (size_t)num_splits * BH * Tq * sizeof(float));
    L.total = up(L.part_l + (size_t)num_splits * BH * Tq * sizeof(float));
  }
  return L;
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
  // the workgroup count BH * qtiles * s must fit an int
  const long long cap = 2147483647LL / ((long long)BH * qtiles);
  if (s > cap) s = (int)cap;
  if (s < 1) s = 1;
  return s;
}

size_t fwd_bf16_workspace_bytes(int BH, int Tq, int Tk, int d, int num_splits) {
  return fwd_layout(BH, Tq, Tk, d, num_splits).total;
}

namespace {

FwdArgs fwd_args(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Tq, int Tk,
                 float scale, int num_splits, int diag) {
  FwdArgs args;
  args.q = static_cast<const __bf16*>(q);
  args.k = static_cast<const __bf16*>(k);
  args.v = static_cast<const __bf16*>(v);
  args.o = static_cast<__bf16*>(o);
  args.lse = lse;
  args.part_acc = args.part_m = args.part_l = nullptr;
  args.BH = BH;
  args.Tq = Tq;
  args.Tk = Tk;
  args.Tk_pad = (Tk + kBN - 1) / kBN * kBN;
  args.diag = diag;
  args.num_qtiles = (Tq + kBM - 1) / kBM;
  args.num_splits = num_splits;
  const int kblocks = (Tk + kBN - 1) / kBN;
  args.keys_per_split = ((kblocks + num_splits - 1) / num_splits) * kBN;
  args.n_items = BH * args.num_qtiles * num_splits;
  args.n_items_paired = BH * ((args.num_qtiles + 1) / 2) * num_splits;
  args.scale_log2 = scale * kLog2e;
  return args;
}

hipError_t fwd_run(const FwdArgs& args, int d, bool causal, bool split, hipStream_t stream) {
  return (d == 128) ? fwd_dispatch<128>(args, causal, split, stream) : fwd_dispatch<64>(args, causal, split, stream);
}

}  // namespace

hipError_t merge_states_launch(const float* acc, const float* m, const float* l, int n, void* o, float* lse, int BH,
                               int Tq, int d, hipStream_t stream) {
  const unsigned blocks = (unsigned)(((size_t)BH * Tq * (d / 4) + 255) / 256);
  prof_begin(1, stream);
  if (d == 128)
    hipLaunchKernelGGL((fwd_combine_kernel<128, false>), dim3(blocks), dim3(256), 0, stream, acc, m, l,
                       static_cast<__bf16*>(o), lse, nullptr, nullptr, nullptr, BH, Tq, n);
  else
    hipLaunchKernelGGL((fwd_combine_kernel<64, false>), dim3(blocks), dim3(256), 0, stream, acc, m, l,
                       static_cast<__bf16*>(o), lse, nullptr, nullptr, nullptr, BH, Tq, n);
  prof_end(1, stream);
  return hipGetLastError();
}

hipError_t fwd_bf16_launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Tq,
                           int Tk, int d, float scale, int causal, int num_splits, void* workspace,
                           hipStream_t stream) {
  const FwdLayout L = fwd_layout(BH, Tq, Tk, d, num_splits);
  char* ws = static_cast<char*>(workspace);
  FwdArgs args = fwd_args(q, k, v, o, lse, BH, Tq, Tk, scale, num_splits, 0);
  const bool split = num_splits > 1;
  if (split) {
    args.part_acc = reinterpret_cast<float*>(ws + L.part_acc);
    args.part_m = reinterpret_cast<float*>(ws + L.part_m);
    args.part_l = reinterpret_cast<float*>(ws + L.part_l);
  }
  hipError_t e = fwd_run(args, d, causal != 0, split, stream);
  if (e != hipSuccess || !split) return e;
  return merge_states_launch(args.part_acc, args.part_m, args.part_l, num_splits, o, lse, BH, Tq, d, stream);
}

int fwd_bf16_state_splits(int BH, int Tq, int Tk, int causal) {
  // the forward's own rule (key splits only without the mask)
  return fwd_bf16_num_splits(BH, Tq, Tk, causal, 0);
}

hipError_t fwd_bf16_state_launch(const void* q, const void* k, const void* v, float* acc, float* m, float* l, int BH,
                                 int Tq, int Tk, int d, float scale, int causal, int diag, int num_splits,
                                 void* workspace, hipStream_t stream) {
  FwdArgs args = fwd_args(q, k, v, nullptr, nullptr, BH, Tq, Tk, scale, num_splits, diag);
  if (num_splits <= 1) {
    args.part_acc = acc;
    args.part_m = m;
    args.part_l = l;
    return fwd_run(args, d, causal != 0, true, stream);
  }
  // the key range in splits, then the split states merged into one state
  const FwdLayout L = fwd_layout(BH, Tq, Tk, d, num_splits);
  char* ws = static_cast<char*>(workspace);
  args.part_acc = reinterpret_cast<float*>(ws + L.part_acc);
  args.part_m = reinterpret_cast<float*>(ws + L.part_m);
  args.part_l = reinterpret_cast<float*>(ws + L.part_l);
  hipError_t e = fwd_run(args, d, causal != 0, true, stream);
  if (e != hipSuccess) return e;
  const unsigned blocks = (unsigned)(((size_t)BH * Tq * (d / 4) + 255) / 256);
  prof_begin(1, stream);
  if (d == 128)
    hipLaunchKernelGGL((fwd_combine_kernel<128, true>), dim3(blocks), dim3(256), 0, stream, args.part_acc,
                       args.part_m, args.part_l, nullptr, nullptr, acc, m, l, BH, Tq, num_splits);
  else
    hipLaunchKernelGGL((fwd_combine_kernel<64, true>), dim3(blocks), dim3(256), 0, stream, args.part_acc,
                       args.part_m, args.part_l, nullptr, nullptr, acc, m, l, BH, Tq, num_splits);
  prof_end(1, stream);
  return hipGetLastError();
}

}  // namespace attn
