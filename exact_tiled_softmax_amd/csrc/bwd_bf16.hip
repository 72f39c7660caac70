// Backward pass of exact tiled-softmax attention, bf16 in / bf16 out, for
// gfx950 (MI355X).
//
// P is recomputed tile by tile from the stored log-sum-exp instead of being
// kept from the forward ("The Hidden Recurrence in Softmax Attention",
// section "Flash Attention Backward Pass": store the row statistics, recompute
// the attention matrix per tile).  The gradients are those of "attention
// backprop": dV = P^T dO, dP = dO V^T ("Gradient of V and P"),
// dS = P o (dP - D) with D = ROW_SUM(dO o O) ("Gradient of S"), dQ = dS K and
// dK = dS^T Q ("Gradient of Q and K"), each of dQ and dK times `scale` because
// the scores are scale * Q K^T.
//
// dK/dV and dQ are reductions over different axes (over queries and over
// keys), so they come from two kernels that each keep their own accumulator
// in registers and write it once; no workgroup adds into another's output.
// Kernels, in launch order:
//   bwd_dq         one workgroup (8 waves) per 256 queries; each wave keeps
//                  its 32 queries' Q and dO rows as MFMA operands and dQ^T in
//                  registers and walks 64-key tiles streamed into LDS:
//                    S^T = K Q^T, dP^T = V dO^T, P^T = exp2(S^T*scale*log2e
//                    - LSE*log2e), dS^T = P^T o (dP^T - D),
//                    dQ^T += K^T dS^T (K^T fragments by transposing reads of
//                    the row-major K tile already in LDS)
//                  It first forms each row's statistics from the forward's
//                  LSE and O: D = sum_c dO_c O_c (with an upstream gradient
//                  dLSE on the log-sum-exp, dS gains dLSE_i P_ij: the row sum
//                  l is a smooth function of the inputs that gradients flow
//                  through, "The Hidden Recurrence in Softmax Attention",
//                  sections "Flash Attention Backward Pass" and "Gradient at
//                  the Output", i.e. D becomes D - dLSE), and writes -LSE/scale
//                  and -D for the dK/dV kernel.
//   bwd_dkdv       persistent: each workgroup (8 waves) runs a fixed list of
//                  128-key blocks back to back, walking 32-query tiles
//                  streamed into LDS (see the kernel's comment):
//                    S' = Q K^T - LSE/scale, dP' = dO V^T - D (both from the
//                    MFMA accumulators' start values), P = exp2(S'*scale*log2e),
//                    dS = P o dP', dV^T += dO^T P, dK^T += Q^T dS
// LDS tiles have their 16-byte chunks XOR-swizzled per row so that both
// 16-byte row reads and transposing reads are free of bank conflicts, and
// tiles are copied global -> LDS by the direct-to-LDS vector load, several
// tiles ahead of the compute.
#include <algorithm>
#include <mutex>

#include "attn.h"

#include "attn_common.hpp"
#include "attn_launch.hpp"
#include "tile_stream.hpp"

namespace attn {

namespace {

// Row statistics of one 32-row block, written by the dQ kernel and read by the
// dK/dV kernel: -LSE / scale and -D, the start values of the dK/dV kernel's
// MFMA accumulators (its MFMAs then produce S - LSE/scale and dP - D).
constexpr int kStatsPerBlock = 64;

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const __bf16* o;     // forward output O, for D = rowsum(dO o O)
  const float* lse;    // forward log-sum-exp [BH][Tq]
  const float* dlse;   // upstream gradient of the LSE [BH][Tq] (or null)
  float* stats;        // [BH][nqb32][kStatsPerBlock] per 32-row block: -LSE/scale x32, -D x32
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* dq_part;      // [dq_splits][BH][Tq][D] fp32 when the dQ key range is split
  int BH, Tq, Tk, nqb32;
  int dq_splits, dq_tiles_per_split;  // key-range split of the dQ kernel (64-key tiles per split)
  int dq_head_group;                  // heads whose query blocks the dQ kernel dispatches interleaved
  int kv_nwg, kv_nkb;                 // dK/dV: workgroups of the persistent launch, 128-key blocks per head
  int kv_zero_items;                  // dK/dV (causal): some key blocks are past every query
  float scale, scale_log2;
};

// ---------------------------------------------------------------------------------
// bwd_dkdv: workgroups of 8 waves, each owning 128 keys (an item) at a time
// and running its list of items back to back (KvItem below).  Waves w and w+4
// run on the same SIMD and share key group w (32 keys):
//   score wave (w < 4): holds its keys' K and V rows as MFMA operands; per
//     32-query tile computes S = Q K^T, dP = dO V^T, P and dS and hands P, dS
//     (bf16 MFMA operands, in the lane layout both waves use) to its partner
//     through LDS;
//   gradient wave (w >= 4): holds dK^T, dV^T for one 32-column block of d
//     and the key groups that go with it; one tile behind, adds dO^T P and
//     Q^T dS, reading its column block of dO and Q with transposing LDS reads
//     (shared by all its key groups) and P, dS from the score waves.
// The partner's MFMA work fills the SIMD while the score wave does its
// softmax, and neither role needs more than half the register file.  The
// score waves' chain sets the step time, so the gradient waves (which wait
// at the barrier for them) issue every tile copy.
constexpr int kKvBlock = 128;  // keys of one dK/dV item

template <int D>
struct KvCfg {
  static constexpr int KS = D / 16;                    // 16-wide k-steps over d
  static constexpr int CB = D / 32;                    // 32-row blocks of d
  static constexpr int CPR = D / 8;                    // 16-byte chunks per Q / dO row
  static constexpr int WAVES = 8;
  static constexpr int BK = kKvBlock;                  // keys per item (one workgroup's accumulators)
  static constexpr int TILE = 32 * D;                  // bf16 elements of one Q or dO tile
  static constexpr int PER_TENSOR = TILE * 2 / 1024;   // wave copies per tensor and tile
  static constexpr int PER_WAVE = 2 * PER_TENSOR / 4;  // copies per gradient wave (they issue all copies)
  static constexpr int VM = PER_WAVE + 1;              // vector-memory ops per gradient wave and tile (+ stats)
  static constexpr int STAGE = 2 * TILE + 128;         // bf16 elements per stage (-LSE/scale, -D: 64 floats)
  // Tiles j-1 .. j+2 resident, copies two tiles ahead.  With four tiles in
  // flight (six stages) the gradient waves' copy issue stalled behind the
  // copies still outstanding and the backward was 3-13% slower.
  static constexpr int NSTAGE = 4;
  static constexpr int AHEAD = NSTAGE - 2;             // copies in flight ahead of the score waves
  static constexpr int HAND_GRP = 64 * 4 * 8;          // bf16 elements of one group's P/dS hand-off (64 lanes x 4 x 8)
  static constexpr int HAND = 4 * HAND_GRP;            // all 4 key groups
  // gradient wave gw (0..3) owns column block gw % CB of d and key groups
  // kgroup(gw, 0..CB-1): the 4 * CB (block, group) pairs, CB per wave
  __host__ __device__ static constexpr int kgroup(int gw, int i) { return gw / CB + (4 / CB) * i; }
  static_assert(PER_WAVE >= 1 && 2 * PER_TENSOR == PER_WAVE * 4, "tile copy split");
};

// The gradient waves (gw = 0..3) issue every copy of a tile: the score
// waves, whose chain sets the step time, issue none.  Each copy takes a
// wave-uniform base (the tile's first row, in scalar registers) and a 32-bit
// per-lane byte offset; rows past Tq repeat the last query row.
template <int D>
__device__ __forceinline__ void dkdv_issue(const BwdArgs& a, int bh, int t, __bf16* stg, int gw, int lane) {
  using C = KvCfg<D>;
  const size_t row0 = (size_t)bh * a.Tq + 32 * t;
  const __bf16* Qt = a.q + row0 * D;
  const __bf16* dOt = a.dout + row0 * D;
  const int last = a.Tq - 1 - 32 * t;  // last row of the tile inside Tq (>= 0)
#pragma unroll
  for (int n = 0; n < C::PER_WAVE; ++n) {
    const int cpy = gw * C::PER_WAVE + n;  // wave-uniform
    const int tensor = cpy / C::PER_TENSOR, i = cpy % C::PER_TENSOR;
    const int p = 64 * i + lane;
    const int row = p / C::CPR, c = (p % C::CPR) ^ swz<C::CPR>(row);
    const uint32_t off = (uint32_t)(min(row, last) * D + 8 * c) * 2;
    dma16_sbase(tensor == 0 ? Qt : dOt, off, stg + tensor * C::TILE + 512 * i);
  }
  // 256 bytes of row statistics (-LSE/scale, -D): lanes 0..3 of every
  // gradient wave copy 64 of them
  if (lane < 4) {
    const float* src = a.stats + ((size_t)bh * a.nqb32 + t) * kStatsPerBlock + 16 * gw;
    dma16_sbase(src, (uint32_t)(16 * lane), stg + 2 * C::TILE + 32 * gw);
  }
}

// Score wave, one tile: P and dS as bf16 B operands (k-slot 8hf+e of k-step
// s2 = accumulator register 8*s2 + e), stored per lane into `hand`.  The
// accumulators start at -LSE/scale and -D of their rows, so the MFMAs leave
// S - LSE/scale and dP - D: P = exp2(scale*log2(e) * that) and dS = P (dP - D).
// MASK (a tile on the causal diagonal): S starts at -inf where the key
// follows the query, which makes P and dS zero there.
template <int D, bool MASK>
__device__ __forceinline__ void dkdv_scores(const BwdArgs& a, const bf16x8 (&kf)[KvCfg<D>::KS], const bf16x8 (&vf)[KvCfg<D>::KS],
                                            const __bf16* stg, __bf16* hand, int t, int kw, int lane) {
  using C = KvCfg<D>;
  const int lr = lane % 32, hf = lane / 32;
  const int key = kw + lr;
  const __bf16* Qs = stg;
  const __bf16* dOs = stg + C::TILE;
  const float* sts = reinterpret_cast<const float*>(stg + 2 * C::TILE);
  const int rsw = swz<C::CPR>(lr);
  // every LDS read of the tile is issued before the first MFMA, so their
  // latencies overlap instead of adding up
  bf16x8 qa[C::KS], da[C::KS];
  f32x16 s, dp;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const int off = lr * D + 8 * ((2 * ks + hf) ^ rsw);
    qa[ks] = ld16(Qs + off);
    da[ks] = ld16(dOs + off);
  }
  // accumulator register r = 4g + i: row 8g + 4hf + i of the tile
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 l4 = *reinterpret_cast<const f32x4*>(sts + 8 * g + 4 * hf);
    const f32x4 d4 = *reinterpret_cast<const f32x4*>(sts + 32 + 8 * g + 4 * hf);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[4 * g + i] = (MASK && key > 32 * t + 8 * g + 4 * hf + i) ? -INFINITY : l4[i];
      dp[4 * g + i] = d4[i];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // the score wave goes first on the SIMD's matrix unit; its partner's MFMAs
  // then run while it does the softmax
  __builtin_amdgcn_s_setprio(2);
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    s = mfma32(qa[ks], kf[ks], s);
    dp = mfma32(da[ks], vf[ks], dp);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  // accumulator register r: query 32t + 8(r/4) + 4hf + r%4, key `key`
  bf16x8 pb[2], db[2];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      const float p = fast_exp2(s[r] * a.scale_log2);
      pb[r / 8][r % 8] = to_bf16(p);
      db[r / 8][r % 8] = to_bf16(p * dp[r]);
    }
  }
  u32x4* h = reinterpret_cast<u32x4*>(hand) + lane;
  h[0] = __builtin_bit_cast(u32x4, pb[0]);
  h[64] = __builtin_bit_cast(u32x4, pb[1]);
  h[128] = __builtin_bit_cast(u32x4, db[0]);
  h[192] = __builtin_bit_cast(u32x4, db[1]);
}

// Gradient wave, one tile: dV^T += dO^T P, dK^T += Q^T dS for its column
// block cb of d and its CB key groups (KvCfg::kgroup).  The A operand (column
// d = 32cb + lane%32, k-slots = queries) comes from two transposing reads of
// the row-major tile, rows 16*s2 + 4hf + 0..3 and 16*s2 + 8 + 4hf + 0..3 (the
// query order of the P / dS k-slots), and serves every key group.
template <int D>
__device__ __forceinline__ void dkdv_grads(f32x16 (&dkt)[4], f32x16 (&dvt)[4], const __bf16* stg, const __bf16* hands,
                                           int gw, int lane) {
  using C = KvCfg<D>;
  const int hf = lane / 32, g16 = lane % 16, csub = (lane / 16) % 2;
  const int cb = gw % C::CB;
  const __bf16* Qs = stg;
  const __bf16* dOs = stg + C::TILE;
  // element (r, c) of a row-major swizzled tile
  auto at = [](int r, int c) { return r * D + 8 * ((c >> 3) ^ swz<C::CPR>(r)) + (c & 7); };
  bf16x8 ao[2], aq[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const int r0 = 16 * s2 + 4 * hf + g16 / 4;
    const int c0 = 32 * cb + 16 * csub + 4 * (g16 % 4);
    ao[s2] = join_tr(lds_read_tr(dOs + at(r0, c0)), lds_read_tr(dOs + at(r0 + 8, c0)));
    aq[s2] = join_tr(lds_read_tr(Qs + at(r0, c0)), lds_read_tr(Qs + at(r0 + 8, c0)));
  }
  u32x4 pb[C::CB][2], db[C::CB][2];
#pragma unroll
  for (int i = 0; i < C::CB; ++i) {
    const u32x4* h = reinterpret_cast<const u32x4*>(hands + C::kgroup(gw, i) * C::HAND_GRP) + lane;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      pb[i][s2] = h[64 * s2];
      db[i][s2] = h[128 + 64 * s2];
    }
  }
  // all reads in flight before the first MFMA
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < C::CB; ++i)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      dvt[i] = mfma32(ao[s2], __builtin_bit_cast(bf16x8, pb[i][s2]), dvt[i]);
      dkt[i] = mfma32(aq[s2], __builtin_bit_cast(bf16x8, db[i][s2]), dkt[i]);
    }
}

// Work list of the dK/dV launch.  The launch is persistent: kv_nwg
// workgroups (as many as are resident on the chip at once) each run a fixed
// list of items (head, key block) back to back as one stream of query tiles,
// each item walked from its last query tile down.  No workgroup waits on the
// dispatcher between items (with one workgroup per CU a finished workgroup's
// CU idled about 6 us, median, before the next one started), and the tile
// copies, key loads and gradient stores of consecutive items overlap.
//   causal mask: item pairs (key block k, key block nkb-1-k) of one head, whose
//     tile counts add up to the same total for every k when Tq = Tk, dealt
//     round-robin over the workgroups (pair wg + r*kv_nwg, round r).  One
//     XCD's workgroups (consecutive logical ids, xcd_remap) take consecutive
//     pairs, i.e. the blocks of one or two heads, which stream the same query
//     tiles and share them in L2; the longer block of a pair goes first.
//     (Alternating the order between neighbouring workgroups, so that they
//     stream different tiles, measured the same.)
//   no mask: every item has the same tiles; items in head-major order are
//     dealt round-robin (item wg + r*kv_nwg), so that one XCD's workgroups
//     again hold consecutive key blocks of one or two heads in each round.
struct KvItem {
  int bh, kb;
  int tb;  // first (lowest) query tile of the item; nqt: no query reaches its keys
};

template <bool CAUSAL>
__device__ __forceinline__ bool kv_item(const BwdArgs& a, int wg, int m, int nqt, KvItem& it) {
  const int nkb = a.kv_nkb;
  if (CAUSAL) {
    const int npair = (nkb + 1) >> 1;
    const int q = wg + (m >> 1) * a.kv_nwg;
    if (q >= a.BH * npair) return false;
    it.bh = q / npair;
    const int k = q - it.bh * npair;
    it.kb = (m & 1) ? nkb - 1 - k : k;
    // the middle block of an odd count pairs with itself: walked once
    it.tb = ((m & 1) && nkb - 1 - k == k) ? -1 : min(it.kb * (kKvBlock / 32), nqt);
  } else {
    const int i = wg + m * a.kv_nwg;
    if (i >= a.BH * nkb) return false;
    it.bh = i / nkb;
    it.kb = i - it.bh * nkb;
    it.tb = 0;
  }
  return true;
}

// Position in a workgroup's tile stream: item m - 1 of its list, tile t.
struct KvCursor {
  KvItem it;
  int m, t;
};

// Moves to the first tile of the next item that has one (items no query
// reaches are written by the zero pass instead); false at the end of the list.
template <bool CAUSAL>
__device__ __forceinline__ bool kv_seek(const BwdArgs& a, int wg, int nqt, KvCursor& c) {
  while (kv_item<CAUSAL>(a, wg, c.m, nqt, c.it)) {
    ++c.m;
    if (c.it.tb >= 0 && c.it.tb < nqt) {
      c.t = nqt - 1;
      return true;
    }
  }
  return false;
}
template <bool CAUSAL>
__device__ __forceinline__ bool kv_step(const BwdArgs& a, int wg, int nqt, KvCursor& c) {
  return --c.t >= c.it.tb || kv_seek<CAUSAL>(a, wg, nqt, c);
}

// dK = scale * (dK^T)^T and dV of one item's 128 keys, bf16.  Register r of
// accumulator i is column 32cb + 8(r/4) + 4hf + r%4 of key k0 + 32 kgroup(gw, i)
// + lane%32; lanes l and l+32 (the same key) trade halves with
// v_permlane32_swap so that each holds 8 consecutive columns and writes them
// as one 16-byte store.  Buffer stores with the record size set to the rows
// before Tk drop the rows past it while every store is still issued: the
// gradient waves count their vector-memory operations to wait for tile
// copies, so the number of stores per item must not depend on the data.
template <int D>
__device__ __forceinline__ void dkdv_store(const BwdArgs& a, const f32x16 (&dkt)[4], const f32x16 (&dvt)[4],
                                           const KvItem& it, int gw, int lane) {
  using C = KvCfg<D>;
  const int lr = lane % 32, hf = lane / 32;
  const int k0 = it.kb * C::BK;
  const int rows = min(C::BK, a.Tk - k0);
  const size_t base = ((size_t)it.bh * a.Tk + k0) * D;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(a.dk + base, 0, rows * D * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(a.dv + base, 0, rows * D * 2, kBufferWord3);
  const int cb = gw % C::CB;
#pragma unroll
  for (int i = 0; i < C::CB; ++i) {
    const int row = 32 * C::kgroup(gw, i) + lr;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int off = (row * D + 32 * cb + 16 * j + 8 * hf) * 2;
      // groups 2j (columns 16j + 4hf + 0..3) and 2j+1 (16j + 8 + 4hf + 0..3)
      auto half_swap = [&](const f32x16& acc, float f) {
        const unsigned x0 = pack_bf16x2(acc[8 * j] * f, acc[8 * j + 1] * f);
        const unsigned x1 = pack_bf16x2(acc[8 * j + 2] * f, acc[8 * j + 3] * f);
        const unsigned y0 = pack_bf16x2(acc[8 * j + 4] * f, acc[8 * j + 5] * f);
        const unsigned y1 = pack_bf16x2(acc[8 * j + 6] * f, acc[8 * j + 7] * f);
        const auto r0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
        return u32x4{(unsigned)r0[0], (unsigned)r1[0], (unsigned)r0[1], (unsigned)r1[1]};
      };
      __builtin_amdgcn_raw_buffer_store_b128(half_swap(dkt[i], a.scale), rk, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(half_swap(dvt[i], 1.f), rv, off, 0, 0);
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, D == 64 ? 4 : 1) void bwd_dkdv_kernel(BwdArgs a) {
  using C = KvCfg<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 stages[C::NSTAGE * C::STAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 hands[2 * C::HAND];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int lr = lane % 32, hf = lane / 32;
  const int wg = xcd_remap(blockIdx.x, a.kv_nwg);
  const int grp = wave & 3;
  const int nqt = (a.Tq + 31) / 32;
  auto stage = [&](int g) { return stages + (g % C::NSTAGE) * C::STAGE; };
  auto hand = [&](int g) { return hands + (g & 1) * C::HAND + grp * C::HAND_GRP; };

  // Step g (g = 0 .. S, S tiles in the workgroup's stream): tile g has landed
  // and is published by the barrier; the copy of tile g+AHEAD goes into the
  // stage of tile g-2; score waves work on tile g, gradient waves on tile
  // g-1.  Both roles pass S+1 barriers.
  static_assert(C::AHEAD == 2, "the gradient waves' waits assume copies two tiles ahead");
  if (wave < 4) {
    // K and V rows of this wave's 32 keys of an item's key block, as B
    // operands.  At d = 128 two register sets alternate between consecutive
    // items: the next item's rows are loaded while the current item runs
    // (loaded at the item boundary instead, they took about 8 us to arrive
    // behind the tile copies in flight).  At d = 64 one set, reloaded at the
    // boundary, keeps the kernel within 128 registers (two workgroups per CU).
    constexpr bool PREFETCH = D == 128;
    bf16x8 k0[C::KS], v0[C::KS], k1[C::KS], v1[C::KS];
    auto load_keys = [&](const KvItem& it, bf16x8(&kf)[C::KS], bf16x8(&vf)[C::KS]) {
      const __bf16* Kh = a.k + (size_t)it.bh * a.Tk * D;
      const __bf16* Vh = a.v + (size_t)it.bh * a.Tk * D;
      const int kr = min(it.kb * C::BK + 32 * grp + lr, a.Tk - 1);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        kf[ks] = ld16(Kh + (size_t)kr * D + 16 * ks + 8 * hf);
        vf[ks] = ld16(Vh + (size_t)kr * D + 16 * ks + 8 * hf);
      }
    };
    KvCursor c;
    c.m = 0;
    bool live = kv_seek<CAUSAL>(a, wg, nqt, c);
    if (live) load_keys(c.it, k0, v0);
    int g = 0;
    // The steps of the cursor's item with keys (kf, vf); the next item's keys
    // go into (kn, vn).  False when the list has no next item.
    auto run_item = [&](const bf16x8(&kf)[C::KS], const bf16x8(&vf)[C::KS], bf16x8(&kn)[C::KS],
                        bf16x8(&vn)[C::KS]) __attribute__((always_inline)) {
      KvCursor nx = c;
      nx.t = nx.it.tb;
      const bool more = kv_step<CAUSAL>(a, wg, nqt, nx);
      if (PREFETCH && more) load_keys(nx.it, kn, vn);
      const int kw = c.it.kb * C::BK + 32 * grp;
      for (int t = nqt - 1; t >= c.it.tb; --t, ++g) {
        barrier();
        // a tile is skipped when the group lies past the keys, or when every
        // query of it precedes every key of the group
        if (kw >= a.Tk || (CAUSAL && 32 * t + 31 < kw)) {
          u32x4* h = reinterpret_cast<u32x4*>(hand(g)) + lane;
          const u32x4 z = {0u, 0u, 0u, 0u};
          h[0] = z;
          h[64] = z;
          h[128] = z;
          h[192] = z;
        } else if (CAUSAL && 32 * t < kw + 31) {
          dkdv_scores<D, true>(a, kf, vf, stage(g), hand(g), t, kw, lane);
        } else {
          dkdv_scores<D, false>(a, kf, vf, stage(g), hand(g), t, kw, lane);
        }
      }
      if (!PREFETCH && more) load_keys(nx.it, kn, vn);
      c = nx;
      return more;
    };
    while (live) {
      if (!PREFETCH) {
        live = run_item(k0, v0, k0, v0);
        continue;
      }
      live = run_item(k0, v0, k1, v1);
      if (!live) break;
      live = run_item(k1, v1, k0, v0);
    }
    barrier();  // step S
  } else {
    f32x16 dkt[4], dvt[4];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
      dkt[cb] = f32x16{};
      dvt[cb] = f32x16{};
    }
    // items no query reaches (causal, keys past Tq) get zero gradients
    // before the stream starts
    if (CAUSAL && a.kv_zero_items) {
      KvItem it;
      for (int m = 0; kv_item<CAUSAL>(a, wg, m, nqt, it); ++m)
        if (it.tb == nqt) dkdv_store<D>(a, dkt, dvt, it, grp, lane);
    }
    KvCursor ci, cg;  // the next tile to copy, the tile the gradient step takes
    ci.m = 0;
    bool li = kv_seek<CAUSAL>(a, wg, nqt, ci);
    cg = ci;
    bool lg = li;
    int issued = 0;
    for (int j = 0; j < C::AHEAD && li; ++j) {
      dkdv_issue<D>(a, ci.it.bh, ci.t, stage(issued++), grp, lane);
      li = kv_step<CAUSAL>(a, wg, nqt, ci);
    }
    // Vector-memory operations after tile g's copies, in issue order: the
    // stores of step g-2, the copies of tile g+1, the stores of step g-1
    // (operations complete in issue order, so waiting until at most that many
    // are outstanding waits for tile g).
    constexpr int NST = 4 * C::CB;  // stores per item and wave
    bool st1 = false, st2 = false;  // stores issued in steps g-1, g-2
    for (int g = 0;; ++g) {
      if (g < issued) {
        const int k = (st1 ? 1 : 0) + (st2 ? 1 : 0);
        const bool later = g + 1 < issued;
        if (k == 0) later ? wait_vm<C::VM>() : wait_vm<0>();
        else if (k == 1) later ? wait_vm<NST + C::VM>() : wait_vm<NST>();
        else later ? wait_vm<2 * NST + C::VM>() : wait_vm<2 * NST>();
      }
      barrier();
      if (li) {
        dkdv_issue<D>(a, ci.it.bh, ci.t, stage(issued++), grp, lane);
        li = kv_step<CAUSAL>(a, wg, nqt, ci);
      }
      st2 = st1;
      st1 = false;
      if (g >= 1) {
        dkdv_grads<D>(dkt, dvt, stage(g - 1), hands + ((g - 1) & 1) * C::HAND, grp, lane);
        if (cg.t == cg.it.tb) {  // tile g-1 closed its item
          dkdv_store<D>(a, dkt, dvt, cg.it, grp, lane);
#pragma unroll
          for (int cb = 0; cb < C::CB; ++cb) {
            dkt[cb] = f32x16{};
            dvt[cb] = f32x16{};
          }
          st1 = true;
        }
        lg = kv_step<CAUSAL>(a, wg, nqt, cg);
      }
      if (!lg) break;
    }
  }
}

// ---------------------------------------------------------------------------------
// bwd_dq
template <int D>
struct DqCfg {
  static constexpr int KS = D / 16;
  static constexpr int CB = D / 32;
  static constexpr int CPR = D / 8;                    // 16-byte chunks per K / V row
  static constexpr int WAVES = 8;
  static constexpr int BM = 32 * WAVES;                // queries per workgroup
  static constexpr int TILE = 64 * D;                  // bf16 elements of one K or V tile
  static constexpr int DMA = TILE * 2 / 1024 / WAVES;  // wave copies per tensor and tile
  static constexpr int VM = 2 * DMA;
  static constexpr int STAGE = 2 * TILE;
  static_assert(DMA >= 1 && TILE * 2 == DMA * WAVES * 1024, "tile copy split");
};

// acc + the sum over 8 bf16 pairs, in fp32, as one chain of dot products in
// a fixed order (the running sum is each step's accumulator, so that the
// compiler has no additions of its own to contract differently from one
// build to the next)
__device__ __forceinline__ float dot8_bf16(const bf16x8& a, const bf16x8& b, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const u32x4 x = __builtin_bit_cast(u32x4, a), y = __builtin_bit_cast(u32x4, b);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // copy the element out first: a bit cast of a vector-element lvalue reads
    // element 0 with this compiler
    const unsigned xe = x[e], ye = y[e];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xe), __builtin_bit_cast(bf16x2, ye), acc, false);
  }
  return acc;
}

struct DqWave {
  bf16x8 qf[8], df[8];  // Q, dO rows of this lane's query as B operands
  f32x16 dqt[4];
  float lse2, ndsum;  // LSE * log2(e), -D of this lane's query
};

template <int D>
__device__ __forceinline__ void dq_issue(const BwdArgs& a, int bh, int j, __bf16* stg, int wave, int lane) {
  using C = DqCfg<D>;
  const __bf16* Kh = a.k + (size_t)bh * a.Tk * D;
  const __bf16* Vh = a.v + (size_t)bh * a.Tk * D;
#pragma unroll
  for (int n = 0; n < C::DMA; ++n) {
    const int i = wave * C::DMA + n;
    const int p = 64 * i + lane;
    const int row = p / C::CPR, c = (p % C::CPR) ^ swz<C::CPR>(row);
    const int kk = min(64 * j + row, a.Tk - 1);
    dma16(Kh + (size_t)kk * D + 8 * c, stg + 512 * i);
    dma16(Vh + (size_t)kk * D + 8 * c, stg + C::TILE + 512 * i);
  }
}

// dS^T of one 32-key unit as bf16 B operands: accumulator register r is key
// key0 + 8(r/4) + 4hf + r%4 for query my_q.  MASK: the unit holds a blocked
// (key, query) pair (causal diagonal or keys past Tk).
template <bool CAUSAL, bool MASK>
__device__ __forceinline__ void dq_softmax(const BwdArgs& a, const DqWave& w, const f32x16& st, const f32x16& dpt,
                                           int key0, int my_q, int hf, bf16x8 (&db)[2]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float p = fast_exp2(__builtin_fmaf(st[r], a.scale_log2, -w.lse2));
    if (MASK) {
      const int kk = key0 + 8 * (r / 4) + 4 * hf + (r % 4);
      p = ((CAUSAL && kk > my_q) || kk >= a.Tk) ? 0.f : p;
    }
    db[r / 8][r % 8] = to_bf16(p * dpt[r]);  // dP^T - D: the accumulator started at -D
  }
}

template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_compute(const BwdArgs& a, DqWave& w, const __bf16* stg, int j, int qw, int kend,
                                           int lane) {
  using C = DqCfg<D>;
  const int lr = lane % 32, hf = lane / 32;
  const int my_q = qw + lr;
  const __bf16* Ks = stg;
  const __bf16* Vs = stg + C::TILE;
  const int rsw = swz<C::CPR>(lr);
  // K^T fragments (A operand of dQ^T += K^T dS^T: column 32cb + lane%32 of K,
  // k-slots = the keys of dS's k-slots) by two transposing reads of the
  // row-major K tile: rows 32u + 16s2 + 4hf + 0..3 and the same + 8
  // (the swizzle of row r + 16k equals that of row r, so a fragment's address
  // is a per-lane offset for its column block plus a constant for u, s2)
  const int g16 = lane % 16, csub = (lane / 16) % 2;
  auto at = [](int r, int cc) { return r * D + 8 * ((cc >> 3) ^ swz<C::CPR>(r)) + (cc & 7); };
  int kofs[C::CB][2];
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) {
    const int c0 = 32 * cb + 16 * csub + 4 * (g16 % 4);
    kofs[cb][0] = at(4 * hf + g16 / 4, c0);
    kofs[cb][1] = at(8 + 4 * hf + g16 / 4, c0);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int key0 = 64 * j + 32 * u;
    if (key0 >= kend) break;
    // K and V fragments four k-steps ahead of their MFMAs (each read issued
    // after the MFMA that frees its registers); the S^T and dP^T chains
    // alternate
    constexpr int LA = C::KS < 4 ? C::KS : 4;
    bf16x8 kfr[C::KS], vfr[C::KS];
    auto rd = [&](int ks) {
      const int off = (32 * u + lr) * D + 8 * ((2 * ks + hf) ^ rsw);
      kfr[ks] = ld16(Ks + off);
      vfr[ks] = ld16(Vs + off);
    };
#pragma unroll
    for (int ks = 0; ks < LA; ++ks) rd(ks);
    f32x16 st = {}, dpt;
#pragma unroll
    for (int r = 0; r < 16; ++r) dpt[r] = w.ndsum;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      __builtin_amdgcn_sched_barrier(0);
      st = mfma32(kfr[ks], w.qf[ks], st);
      dpt = mfma32(vfr[ks], w.df[ks], dpt);
      if (ks + LA < C::KS) rd(ks + LA);
    }
    __builtin_amdgcn_sched_barrier(0);
    // K^T fragments read while the softmax runs
    bf16x8 ka[C::CB][2];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const __bf16* kb = Ks + (32 * u + 16 * s2) * D;
        ka[cb][s2] = join_tr(lds_read_tr(kb + kofs[cb][0]), lds_read_tr(kb + kofs[cb][1]));
      }
    bf16x8 db[2];
    if ((CAUSAL && key0 + 31 > qw) || key0 + 32 > a.Tk) dq_softmax<CAUSAL, true>(a, w, st, dpt, key0, my_q, hf, db);
    else dq_softmax<CAUSAL, false>(a, w, st, dpt, key0, my_q, hf, db);
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) w.dqt[cb] = mfma32(ka[cb][s2], db[s2], w.dqt[cb]);
  }
}

// SPLIT: the workgroup covers key tiles [split * dq_tiles_per_split, ...) of
// its query block and writes an fp32 partial dQ (scaled) that dq_reduce_kernel
// sums over the splits in a fixed order; every split writes its partial,
// zeros when its range holds no key of the block.
template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(BwdArgs a) {
  using C = DqCfg<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 stg0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 stg1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 stg2[C::STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int lr = lane % 32, hf = lane / 32;
  const int nqb = (a.Tq + C::BM - 1) / C::BM;
  const int ns = SPLIT ? a.dq_splits : 1;
  const WorkItem wi = work_item(xcd_remap(blockIdx.x, a.BH * nqb * ns), a.BH, nqb, ns, a.dq_head_group);
  const int split = wi.split;
  const int bh = wi.bh;
  const int qi = wi.blk;
  const int qb = CAUSAL ? nqb - 1 - qi : qi;  // most causal work first
  const int q0 = qb * C::BM;
  const int qw = q0 + 32 * wave;
  const int my_q = qw + lr;

  DqWave w;
  {
    const __bf16* Qh = a.q + (size_t)bh * a.Tq * D;
    const __bf16* dOh = a.dout + (size_t)bh * a.Tq * D;
    const int qr = min(my_q, a.Tq - 1);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      w.qf[ks] = ld16(Qh + (size_t)qr * D + 16 * ks + 8 * hf);
      w.df[ks] = ld16(dOh + (size_t)qr * D + 16 * ks + 8 * hf);
    }
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) w.dqt[cb] = f32x16{};
    // This row's statistics ("Gradient of S": D = ROW_SUM(dO o O), with the
    // forward's O): lanes l and l+32 hold the two halves of the row's dO and
    // load the same halves of O.  With an upstream gradient dLSE on the
    // log-sum-exp, dS gains dLSE_i P_ij, i.e. D becomes D - dLSE.  Split 0
    // of every query block also writes -LSE/scale and -D for the dK/dV
    // kernel, launched after this one (rows past Tq: -inf and 0, so that
    // their P is 0).
    const __bf16* Oh = a.o + (size_t)bh * a.Tq * D;
    bf16x8 of[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) of[ks] = ld16(Oh + (size_t)qr * D + 16 * ks + 8 * hf);
    const bool in = my_q < a.Tq;
    float l = -INFINITY, dl = 0.f;
    if (in) {
      l = a.lse[(size_t)bh * a.Tq + my_q];
      if (a.dlse) dl = a.dlse[(size_t)bh * a.Tq + my_q];
    }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      settle(w.qf[ks]);
      settle(w.df[ks]);
    }
    float dsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) dsum = dot8_bf16(w.df[ks], of[ks], dsum);
    dsum = pair_sum(dsum);
    w.lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
    w.ndsum = in ? dl - dsum : 0.f;
    if ((!SPLIT || split == 0) && hf == 0 && my_q < a.nqb32 * 32) {
      float* blk = a.stats + ((size_t)bh * a.nqb32 + my_q / 32) * kStatsPerBlock;
      blk[my_q % 32] = (l == -INFINITY) ? -INFINITY : -l / a.scale;
      blk[32 + my_q % 32] = w.ndsum;
    }
    settle(w.lse2);
    settle(w.ndsum);
  }

  const int nkt_all = (a.Tk + 63) / 64;
  const int last_q = min(q0 + C::BM - 1, a.Tq - 1);
  const int n_all = CAUSAL ? min(nkt_all, last_q / 64 + 1) : nkt_all;
  // this workgroup's key tiles: [jb, jb + n)
  const int jb = SPLIT ? min(n_all, split * a.dq_tiles_per_split) : 0;
  const int n = SPLIT ? min(n_all - jb, a.dq_tiles_per_split) : n_all;
  // keys this wave needs: [0, kend)
  const int kend = qw >= a.Tq ? 0 : (CAUSAL ? min(a.Tk, min(qw + 31, a.Tq - 1) + 1) : a.Tk);

  // local tiles 0, 1 in flight before the loop; local tile i+2 is issued at step i
  if (n > 0) dq_issue<D>(a, bh, jb, stg0, wave, lane);
  if (n > 1) dq_issue<D>(a, bh, jb + 1, stg1, wave, lane);

  auto step = [&](int i, const __bf16* cur, __bf16* ahead) {
    if (i + 1 < n) wait_vm<C::VM>();
    else wait_vm<0>();
    barrier();
    if (i + 2 < n) dq_issue<D>(a, bh, jb + i + 2, ahead, wave, lane);
    if (64 * (jb + i) < kend) dq_compute<D, CAUSAL>(a, w, cur, jb + i, qw, kend, lane);
  };
  for (int i = 0; i < n; i += 3) {
    step(i, stg0, stg2);
    if (i + 1 < n) step(i + 1, stg1, stg0);
    if (i + 2 < n) step(i + 2, stg2, stg1);
  }

  // dQ = scale * (dQ^T)^T: register r of block cb is column 32cb + 8(r/4) + 4hf + r%4
  if (SPLIT) {
    if (my_q < a.Tq) {
      float* pr = a.dq_part + (((size_t)split * a.BH + bh) * a.Tq + my_q) * D;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(pr + 32 * cb + 8 * g + 4 * hf) =
              f32x4{w.dqt[cb][4 * g] * a.scale, w.dqt[cb][4 * g + 1] * a.scale, w.dqt[cb][4 * g + 2] * a.scale,
                    w.dqt[cb][4 * g + 3] * a.scale};
    }
    return;
  }
  if (my_q < a.Tq) {
    __bf16* dqr = a.dq + ((size_t)bh * a.Tq + my_q) * D;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 wq = {pack_bf16x2(w.dqt[cb][4 * g] * a.scale, w.dqt[cb][4 * g + 1] * a.scale),
                          pack_bf16x2(w.dqt[cb][4 * g + 2] * a.scale, w.dqt[cb][4 * g + 3] * a.scale)};
        *reinterpret_cast<u32x2*>(dqr + 32 * cb + 8 * g + 4 * hf) = wq;
      }
  }
}

// dQ = sum over the key-range splits of the partials, in split order; four
// values per thread.
__global__ __launch_bounds__(256) void dq_reduce_kernel(const float* __restrict__ part, __bf16* __restrict__ dq,
                                                        size_t n4, int splits) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const f32x4* p = reinterpret_cast<const f32x4*>(part) + i;
  f32x4 acc = p[0];
  for (int s = 1; s < splits; ++s) acc += p[(size_t)s * n4];
  *reinterpret_cast<u32x2*>(dq + 4 * i) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
}

// ---------------------------------------------------------------------------------
// Key-range splits of the dQ kernel: only when the query blocks alone leave the
// CUs under-filled (fewer than two workgroups per CU), about 1024 workgroups
// then, each split at least 8 key tiles (512 keys) long.
struct DqSplit {
  int splits, tiles_per_split;
};

int dq_default_splits(int BH, int Tq, int Tk) {
  const int nqb = (Tq + 255) / 256;
  const int nkt = (Tk + 63) / 64;
  const long long items = (long long)BH * nqb;
  int s = 1;
  if (items < 512) {
    s = (int)((1024 + items - 1) / items);
    s = std::min(s, std::max(1, nkt / 8));
  }
  return s;
}

// s requested splits -> tiles per split, and the splits that are non-empty
DqSplit dq_split(int Tk, int s) {
  const int nkt = (Tk + 63) / 64;
  s = std::max(1, std::min(s, nkt));
  const int tps = (nkt + s - 1) / s;
  return {(nkt + tps - 1) / tps, tps};
}

struct BwdLayout {
  size_t stats, dq_part, total;
};

BwdLayout bwd_layout(int BH, int Tq, int Tk, int d, int dq_splits) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t nqb32 = (size_t)(Tq + 31) / 32;
  const DqSplit sp = dq_split(Tk, dq_splits);
  BwdLayout L;
  L.stats = 0;
  L.dq_part = up(L.stats + (size_t)BH * nqb32 * kStatsPerBlock * sizeof(float));
  L.total = L.dq_part + (sp.splits > 1 ? up((size_t)sp.splits * BH * Tq * d * sizeof(float)) : 0);
  return L;
}

template <int D>
hipError_t bwd_launch_d(BwdArgs& args, bool causal, hipStream_t stream) {
  // dQ first: it also writes the row statistics the dK/dV kernel reads
  const int nqb = (args.Tq + DqCfg<D>::BM - 1) / DqCfg<D>::BM;
  const int ns = args.dq_splits;
  prof_begin(4, stream);
  const dim3 grid((unsigned)(args.BH * nqb * ns));
  if (ns > 1) {
    if (causal)
      hipLaunchKernelGGL((bwd_dq_kernel<D, true, true>), grid, dim3(512), 0, stream, args);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, false, true>), grid, dim3(512), 0, stream, args);
    const size_t n4 = (size_t)args.BH * args.Tq * D / 4;
    hipLaunchKernelGGL(dq_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, args.dq_part,
                       args.dq, n4, ns);
  } else {
    if (causal)
      hipLaunchKernelGGL((bwd_dq_kernel<D, true, false>), grid, dim3(512), 0, stream, args);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, false, false>), grid, dim3(512), 0, stream, args);
  }
  prof_end(4, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int nkb = (args.Tk + KvCfg<D>::BK - 1) / KvCfg<D>::BK;
  const int nqt = (args.Tq + 31) / 32;
  const long long items = causal ? (long long)args.BH * ((nkb + 1) / 2) : (long long)args.BH * nkb;
  const int resident = causal ? resident_workgroups<bwd_dkdv_kernel<D, true>>(512)
                              : resident_workgroups<bwd_dkdv_kernel<D, false>>(512);
  if (resident <= 0) return hipErrorInvalidDevice;
  args.kv_nkb = nkb;
  args.kv_nwg = (int)std::min<long long>(items, resident);
  args.kv_zero_items = causal && (nkb - 1) * (KvCfg<D>::BK / 32) >= nqt;
  prof_begin(3, stream);
  if (causal)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3(args.kv_nwg), dim3(512), 0, stream, args);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3(args.kv_nwg), dim3(512), 0, stream, args);
  prof_end(3, stream);
  return hipGetLastError();
}

}  // namespace

int bwd_bf16_dq_splits(int BH, int Tq, int Tk, int d, size_t ws_cap) {
  // the default plan, or the most splits whose partials still fit ws_cap
  // (1: no partials); 0 when not even the row statistics fit.  Workspace
  // grows with the split count, so the first fit going down is the largest.
  int s = dq_default_splits(BH, Tq, Tk);
  for (;;) {
    const int eff = dq_split(Tk, s).splits;
    if (bwd_layout(BH, Tq, Tk, d, eff).total <= ws_cap) return eff;
    if (eff <= 1) return 0;
    s = eff - 1;
  }
}

size_t bwd_bf16_workspace_bytes(int BH, int Tq, int Tk, int d, int dq_splits) {
  return bwd_layout(BH, Tq, Tk, d, dq_splits).total;
}

hipError_t bwd_bf16_launch(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const float* dlse, const void* dout, void* dq, void* dk, void* dv, int BH, int Tq, int Tk,
                           int d, float scale, int causal, int dq_splits, void* workspace, hipStream_t stream) {
  const BwdLayout L = bwd_layout(BH, Tq, Tk, d, dq_splits);
  char* ws = static_cast<char*>(workspace);
  BwdArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.dout = static_cast<const __bf16*>(dout);
  a.o = static_cast<const __bf16*>(o);
  a.lse = lse;
  a.dlse = dlse;
  a.stats = reinterpret_cast<float*>(ws + L.stats);
  a.dq = static_cast<__bf16*>(dq);
  a.dk = static_cast<__bf16*>(dk);
  a.dv = static_cast<__bf16*>(dv);
  a.BH = BH;
  a.Tq = Tq;
  a.Tk = Tk;
  a.nqb32 = (Tq + 31) / 32;
  const DqSplit sp = dq_split(Tk, dq_splits);
  a.dq_splits = sp.splits;
  a.dq_head_group = head_group(BH, ((Tq + DqCfg<128>::BM - 1) / DqCfg<128>::BM) * sp.splits);
  a.dq_tiles_per_split = sp.tiles_per_split;
  a.dq_part = sp.splits > 1 ? reinterpret_cast<float*>(ws + L.dq_part) : nullptr;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  return d == 128 ? bwd_launch_d<128>(a, causal != 0, stream) : bwd_launch_d<64>(a, causal != 0, stream);
}

// ---- scratch memory of the entry point that allocates nothing -------------------
// A file-scope device array: every GPU the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as an
// address (on the host it is only a stand-in): the device address of each
// GPU's copy comes from hipGetSymbolAddress, taken once per device on that
// device's first call and kept.
namespace {
__device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
}  // namespace

hipError_t bwd_bf16_noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace attn
