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
// Kernels:
//   bwd_preprocess  D_i = sum_c dO_ic O_ic (fp32) and zero the fp32 dQ workspace
//   bwd_bf16_kernel one workgroup (4 waves) per 128 keys of one (batch, head);
//                   each wave keeps its 32 keys' K, V rows as MFMA operands and
//                   its dK^T, dV^T accumulators in registers, and walks the
//                   query tiles (64 rows) that can see those keys:
//                     S  = Q K^T, dP = dO V^T   (queries on the M side)
//                     P  = exp2(S*scale*log2e - LSE*log2e), dS = P o (dP - D)
//                     dV^T += dO^T P, dK^T += Q^T dS  (Q, dO read transposed
//                                                      from LDS)
//                     dS^T -> LDS; dQ_tile += dS K over the 128 keys, added to
//                     the fp32 workspace with device atomics
//   bwd_finalize    dQ = scale * workspace, rounded to bf16
#include "attn_common.hpp"
#include "attn_launch.hpp"

namespace attn {

namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = kBwdWaves * 64;
constexpr int kBK = 32 * kBwdWaves;  // keys per workgroup
constexpr int kBQ = 64;              // query rows per inner tile

template <int D>
struct BwdCfg {
  static constexpr int KS = D / 16;
  static constexpr int CB = D / 32;
  static constexpr int STR = D + 8;            // LDS row stride of Q, dO, K tiles
  static constexpr int STRS = kBQ + 8;         // LDS row stride of the dS^T tile
  static constexpr int QCHUNKS = kBQ * D / 8;  // 16-byte chunks of a Q or dO tile
  static constexpr int QPER = QCHUNKS / kBwdThreads;
  static constexpr int KCHUNKS = kBK * D / 8;
  static constexpr int KPER = KCHUNKS / kBwdThreads;
  // dQ output blocks (2 query blocks x CB column blocks) shared by the waves
  static constexpr int QBLK_PER_WAVE = (2 * CB) / kBwdWaves;
  static_assert(QCHUNKS % kBwdThreads == 0 && KCHUNKS % kBwdThreads == 0, "tile split");
  static_assert((2 * CB) % kBwdWaves == 0, "dQ block split");
};

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const float* lse;
  const float* dsum;  // D = rowsum(dO o O)   [BH][Tq]
  float* dq_acc;      // fp32 dQ / scale      [BH][Tq][D]
  __bf16* dk;
  __bf16* dv;
  int BH, Tq, Tk, num_kblocks;
  float scale, scale_log2;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_bf16_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 Qs[kBQ * C::STR];
  __shared__ __attribute__((aligned(16))) __bf16 dOs[kBQ * C::STR];
  __shared__ __attribute__((aligned(16))) __bf16 Ks[kBK * C::STR];
  __shared__ __attribute__((aligned(16))) __bf16 dSt[kBK * C::STRS];
  __shared__ float lse2s[kBQ];
  __shared__ float Dss[kBQ];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int lr = lane % 32, hf = lane / 32;
  const int g16 = lane % 16, csub = (lane / 16) % 2;
  const int n_items = a.BH * a.num_kblocks;
  const int item = xcd_remap(blockIdx.x, n_items);
  const int kb = item % a.num_kblocks;  // key block 0 (most causal work) first within a head
  const int bh = item / a.num_kblocks;
  const int k0 = kb * kBK;
  const int key = k0 + wave * 32 + lr;  // this lane's key (N index of S, dP)

  const __bf16* Qh = a.q + (size_t)bh * a.Tq * D;
  const __bf16* dOh = a.dout + (size_t)bh * a.Tq * D;
  const __bf16* Kh = a.k + (size_t)bh * a.Tk * D;
  const __bf16* Vh = a.v + (size_t)bh * a.Tk * D;
  const float* lseh = a.lse + (size_t)bh * a.Tq;
  const float* Dh = a.dsum + (size_t)bh * a.Tq;
  float* dQh = a.dq_acc + (size_t)bh * a.Tq * D;

  // K and V rows of this lane's key as B operands (lane holds row[16ks + 8hf + 0..7])
  bf16x8 kf[C::KS], vf[C::KS];
  {
    const bool ok = key < a.Tk;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      kf[ks] = __builtin_bit_cast(bf16x8, ok ? *reinterpret_cast<const u32x4*>(Kh + (size_t)key * D + 16 * ks + 8 * hf) : z);
      vf[ks] = __builtin_bit_cast(bf16x8, ok ? *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D + 16 * ks + 8 * hf) : z);
    }
  }
  // the workgroup's 128 K rows in LDS (B operand of dQ = dS K, read transposed)
  {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < C::KPER; ++i) {
      const int c = tid + i * kBwdThreads;
      const int r = c / CPR, col = (c % CPR) * 8;
      const int kk = k0 + r;
      u32x4 t = {0u, 0u, 0u, 0u};
      if (kk < a.Tk) t = *reinterpret_cast<const u32x4*>(Kh + (size_t)kk * D + col);
      *reinterpret_cast<u32x4*>(Ks + r * C::STR + col) = t;
    }
  }

  f32x16 dKt[C::CB], dVt[C::CB];
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) {
    dKt[cb] = f32x16{};
    dVt[cb] = f32x16{};
  }

  const int num_qt = (a.Tq + kBQ - 1) / kBQ;
  const int qt_begin = CAUSAL ? min(k0 / kBQ, num_qt) : 0;

  // stage one query tile (Q, dO rows and their LSE, D) into LDS
  auto load_qtile = [&](int q0, u32x4 (&qr)[C::QPER], u32x4 (&dr)[C::QPER], float& lv, float& dvv) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < C::QPER; ++i) {
      const int c = tid + i * kBwdThreads;
      const int r = c / CPR, col = (c % CPR) * 8;
      const int qq = q0 + r;
      u32x4 z = {0u, 0u, 0u, 0u};
      qr[i] = qq < a.Tq ? *reinterpret_cast<const u32x4*>(Qh + (size_t)qq * D + col) : z;
      dr[i] = qq < a.Tq ? *reinterpret_cast<const u32x4*>(dOh + (size_t)qq * D + col) : z;
    }
    if (tid < kBQ) {
      const int qq = q0 + tid;
      const float l = qq < a.Tq ? lseh[qq] : -INFINITY;
      // rows past Tq or with no allowed key get P = 0 through LSE = +inf
      lv = (l == -INFINITY) ? INFINITY : l * kLog2e;
      dvv = qq < a.Tq ? Dh[qq] : 0.f;
    }
  };
  auto store_qtile = [&](const u32x4 (&qr)[C::QPER], const u32x4 (&dr)[C::QPER], float lv, float dvv) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < C::QPER; ++i) {
      const int c = tid + i * kBwdThreads;
      const int r = c / CPR, col = (c % CPR) * 8;
      *reinterpret_cast<u32x4*>(Qs + r * C::STR + col) = qr[i];
      *reinterpret_cast<u32x4*>(dOs + r * C::STR + col) = dr[i];
    }
    if (tid < kBQ) {
      lse2s[tid] = lv;
      Dss[tid] = dvv;
    }
  };

  u32x4 qr[C::QPER], dr[C::QPER];
  float lv = 0.f, dvv = 0.f;
  if (qt_begin < num_qt) {
    load_qtile(qt_begin * kBQ, qr, dr, lv, dvv);
    store_qtile(qr, dr, lv, dvv);
  }
  __syncthreads();

  for (int qt = qt_begin; qt < num_qt; ++qt) {
    const int q0 = qt * kBQ;
    const bool more = qt + 1 < num_qt;
    if (more) load_qtile(q0 + kBQ, qr, dr, lv, dvv);

    // ---- S = Q K^T and dP = dO V^T (queries on M, this wave's keys on N) ----
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = f32x16{};
      dp[qb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qs + (32 * qb + lr) * C::STR + 16 * ks + 8 * hf);
        s[qb] = mfma32(qa, kf[ks], s[qb]);
      }
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 da = *reinterpret_cast<const bf16x8*>(dOs + (32 * qb + lr) * C::STR + 16 * ks + 8 * hf);
        dp[qb] = mfma32(da, vf[ks], dp[qb]);
      }
    }
    // ---- P = exp(S - LSE), dS = P o (dP - D) -------------------------------------
    const bool need_mask = (k0 + wave * 32 + 32 > a.Tk) || (CAUSAL && q0 < k0 + wave * 32 + 31);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qi = 32 * qb + 8 * g + 4 * hf;  // first of 4 consecutive local queries
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + qi);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(Dss + qi);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * g + j;
          float p = fast_exp2(__builtin_fmaf(s[qb][r], a.scale_log2, -l4[j]));
          if (need_mask) {
            const bool blocked = key >= a.Tk || (CAUSAL && key > q0 + qi + j);
            p = blocked ? 0.f : p;
          }
          s[qb][r] = p;
          dp[qb][r] = p * (dp[qb][r] - d4[j]);
        }
      }
    // k-slot 8*hf+e of (qb,u) <-> local query 32*qb + 16*u + (e<4 ? 4*hf+e : 8+4*hf+e-4)
    bf16x8 pb[2][2], sb[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[qb][u][e] = to_bf16(s[qb][8 * u + e]);
          sb[qb][u][e] = to_bf16(dp[qb][8 * u + e]);
        }
    // ---- dV^T += dO^T P and dK^T += Q^T dS --------------------------------------
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r0 = 32 * qb + 16 * u + 4 * hf + g16 / 4;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
          const int c0 = 32 * cb + 16 * csub + 4 * (g16 % 4);
          const i16x4 dlo = lds_read_tr(dOs + r0 * C::STR + c0);
          const i16x4 dhi = lds_read_tr(dOs + (r0 + 8) * C::STR + c0);
          dVt[cb] = mfma32(join_tr(dlo, dhi), pb[qb][u], dVt[cb]);
          const i16x4 qlo = lds_read_tr(Qs + r0 * C::STR + c0);
          const i16x4 qhi = lds_read_tr(Qs + (r0 + 8) * C::STR + c0);
          dKt[cb] = mfma32(join_tr(qlo, qhi), sb[qb][u], dKt[cb]);
        }
      }
    // ---- dS^T (bf16) to LDS: row = key, 4 consecutive queries per 8-byte write ---
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w = {pack_bf16x2(dp[qb][4 * g], dp[qb][4 * g + 1]), pack_bf16x2(dp[qb][4 * g + 2], dp[qb][4 * g + 3])};
        *reinterpret_cast<u32x2*>(dSt + (wave * 32 + lr) * C::STRS + 32 * qb + 8 * g + 4 * hf) = w;
      }
    __syncthreads();

    // ---- dQ_tile += dS K over the workgroup's 128 keys (fp32 atomics) -----------
#pragma unroll
    for (int ob = 0; ob < C::QBLK_PER_WAVE; ++ob) {
      const int blk = wave * C::QBLK_PER_WAVE + ob;
      const int qb = blk / C::CB, cb = blk % C::CB;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < kBK / 16; ++ks) {
        const int rr = 16 * ks + 8 * hf + g16 / 4;
        const i16x4 alo = lds_read_tr(dSt + rr * C::STRS + 32 * qb + 16 * csub + 4 * (g16 % 4));
        const i16x4 ahi = lds_read_tr(dSt + (rr + 4) * C::STRS + 32 * qb + 16 * csub + 4 * (g16 % 4));
        const i16x4 blo = lds_read_tr(Ks + rr * C::STR + 32 * cb + 16 * csub + 4 * (g16 % 4));
        const i16x4 bhi = lds_read_tr(Ks + (rr + 4) * C::STR + 32 * cb + 16 * csub + 4 * (g16 % 4));
        acc = mfma32(join_tr(alo, ahi), join_tr(blo, bhi), acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qq = q0 + 32 * qb + 8 * (r / 4) + 4 * hf + (r % 4);
        if (qq < a.Tq) unsafeAtomicAdd(dQh + (size_t)qq * D + 32 * cb + lr, acc[r]);
      }
    }

    if (more) store_qtile(qr, dr, lv, dvv);
    __syncthreads();
  }

  // ---- dK = scale * dK^T^T, dV: lane holds key row, 4 consecutive columns per group
  if (key < a.Tk) {
    __bf16* dkr = a.dk + ((size_t)bh * a.Tk + key) * D;
    __bf16* dvr = a.dv + ((size_t)bh * a.Tk + key) * D;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 32 * cb + 8 * g + 4 * hf;
        u32x2 wk = {pack_bf16x2(dKt[cb][4 * g] * a.scale, dKt[cb][4 * g + 1] * a.scale),
                    pack_bf16x2(dKt[cb][4 * g + 2] * a.scale, dKt[cb][4 * g + 3] * a.scale)};
        u32x2 wv = {pack_bf16x2(dVt[cb][4 * g], dVt[cb][4 * g + 1]),
                    pack_bf16x2(dVt[cb][4 * g + 2], dVt[cb][4 * g + 3])};
        *reinterpret_cast<u32x2*>(dkr + c) = wk;
        *reinterpret_cast<u32x2*>(dvr + c) = wv;
      }
  }
}

// D_i = sum_c dO_ic O_ic in fp32 and zero the fp32 dQ workspace row.
// 16 lanes per row, D/16 elements per lane.
template <int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const __bf16* __restrict__ o,
                                                             const __bf16* __restrict__ dout,
                                                             float* __restrict__ dsum, float* __restrict__ dq_acc,
                                                             int rows) {
  constexpr int PER = D / 16;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int row = t / 16, sub = t % 16;
  const bool ok = row < rows;
  float acc = 0.f;
  if (ok) {
    const uint16_t* op = reinterpret_cast<const uint16_t*>(o) + (size_t)row * D + sub * PER;
    const uint16_t* dp = reinterpret_cast<const uint16_t*>(dout) + (size_t)row * D + sub * PER;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc += bf16_to_f32(op[j]) * bf16_to_f32(dp[j]);
    float* z = dq_acc + (size_t)row * D + sub * PER;
#pragma unroll
    for (int j = 0; j < PER; j += 4) *reinterpret_cast<f32x4*>(z + j) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (ok && sub == 0) dsum[row] = acc;
}

// dQ = scale * dq_acc rounded to bf16, 8 elements per thread.
__global__ __launch_bounds__(256) void bwd_finalize_kernel(const float* __restrict__ dq_acc, __bf16* __restrict__ dq,
                                                           float scale, size_t n8) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const f32x4 x0 = *reinterpret_cast<const f32x4*>(dq_acc + i * 8);
  const f32x4 x1 = *reinterpret_cast<const f32x4*>(dq_acc + i * 8 + 4);
  u32x4 w = {pack_bf16x2(x0[0] * scale, x0[1] * scale), pack_bf16x2(x0[2] * scale, x0[3] * scale),
             pack_bf16x2(x1[0] * scale, x1[1] * scale), pack_bf16x2(x1[2] * scale, x1[3] * scale)};
  *reinterpret_cast<u32x4*>(dq + i * 8) = w;
}

template <int D>
hipError_t bwd_launch_d(const BwdArgs& args, const __bf16* o, __bf16* dq, bool causal, hipStream_t stream) {
  const int rows = args.BH * args.Tq;
  prof_begin(2, stream);
  hipLaunchKernelGGL(bwd_preprocess_kernel<D>, dim3((rows * 16 + 255) / 256), dim3(256), 0, stream, o, args.dout,
                     const_cast<float*>(args.dsum), args.dq_acc, rows);
  prof_end(2, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = args.BH * args.num_kblocks;
  prof_begin(3, stream);
  if (causal)
    hipLaunchKernelGGL((bwd_bf16_kernel<D, true>), dim3(n), dim3(kBwdThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((bwd_bf16_kernel<D, false>), dim3(n), dim3(kBwdThreads), 0, stream, args);
  prof_end(3, stream);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n8 = (size_t)rows * D / 8;
  prof_begin(4, stream);
  hipLaunchKernelGGL(bwd_finalize_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, args.dq_acc, dq,
                     args.scale, n8);
  prof_end(4, stream);
  return hipGetLastError();
}

}  // namespace

size_t bwd_bf16_workspace_bytes(int BH, int Tq, int d) {
  return (size_t)BH * Tq * d * sizeof(float) + (size_t)BH * Tq * sizeof(float);
}

hipError_t bwd_bf16_launch(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, int BH, int Tq, int Tk, int d,
                           float scale, int causal, void* workspace, hipStream_t stream) {
  BwdArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.dout = static_cast<const __bf16*>(dout);
  a.lse = lse;
  a.dq_acc = static_cast<float*>(workspace);
  a.dsum = a.dq_acc + (size_t)BH * Tq * d;
  a.dk = static_cast<__bf16*>(dk);
  a.dv = static_cast<__bf16*>(dv);
  a.BH = BH;
  a.Tq = Tq;
  a.Tk = Tk;
  a.num_kblocks = (Tk + kBK - 1) / kBK;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  const __bf16* ob = static_cast<const __bf16*>(o);
  __bf16* dqb = static_cast<__bf16*>(dq);
  return d == 128 ? bwd_launch_d<128>(a, ob, dqb, causal != 0, stream)
                  : bwd_launch_d<64>(a, ob, dqb, causal != 0, stream);
}

}  // namespace attn
