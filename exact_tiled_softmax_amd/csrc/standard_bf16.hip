// Standard (materialised) attention, bf16 in / bf16 out: the three steps of
// "The Hidden Recurrence in Softmax Attention", section "Standard Attention /
// Forward Pass", each a kernel of its own with the full score matrix in HBM:
//   S = scale * Q K^T  (fp32, [BH][Tq][Tk], blocked keys written as -inf)
//   P = softmax(S) by rows (bf16) and LSE = m + ln l per row
//   O = P V
// It exists to measure what the tiled method saves: S and P cost
// Tq*Tk*(4 + 4 + 2 + 2) bytes of HBM traffic per head (S written, S read
// twice by the two-pass row softmax, P written, P read), against reading
// Q, K, V and writing O once.  The arithmetic matches the forward kernel's
// (bf16 MFMA products, fp32 softmax, P rounded to bf16 before P V).
//
// Layouts: P is stored with the 16 columns of every 16-key group in the order
// of the transposed V copy (see group_row), so that the P V product reads
// both operands as 16-byte rows; P and V^T are zero past Tk (Tk padded to 64).
#include "attn_common.hpp"
#include "attn_launch.hpp"
#include "tile_stream.hpp"

namespace attn {
namespace {

// Row of a 16-row group that the transposed copies store at position p
// (0..15).  An MFMA accumulator gives lane half h the rows 4h..4h+3 and
// 8+4h..8+4h+3 of each 16-row group, and an operand read takes 8 consecutive
// positions, so position 8h+e holds row (e < 4 ? 4h+e : 8+4h+e-4).
__device__ __forceinline__ int group_row(int p) {
  const int h = (p >> 3) & 1, e = p & 7;
  return (e < 4) ? 4 * h + e : 8 + 4 * h + (e - 4);
}

// Transposed copy [d][Tpad] of a row-major [T][d] bf16 tensor (per head),
// rows of each 16-row group stored in group_row order, zero past T.
// One 64-row block of one head per workgroup.
// out[bh][c][tpos] = in[bh][t][c] with t = 16*(tpos/16) + group_row(tpos%16),
// zero for t >= T.
template <int D>
__global__ __launch_bounds__(256) void transpose_rows_kernel(const __bf16* __restrict__ in_all,
                                                            __bf16* __restrict__ out_all, int T, int Tpad) {
  constexpr int STR = D + 8;
  constexpr int CPR = D / 8;
  __shared__ __attribute__((aligned(16))) __bf16 tile[64 * STR];
  const int bh = blockIdx.y;
  const int t0 = blockIdx.x * 64;
  const __bf16* in = in_all + (size_t)bh * T * D;
  __bf16* out = out_all + (size_t)bh * D * Tpad;
  for (int c = threadIdx.x; c < 64 * CPR; c += 256) {
    const int r = c / CPR, col = (c % CPR) * 8;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (t0 + r < T) x = *reinterpret_cast<const u32x4*>(in + (size_t)(t0 + r) * D + col);
    *reinterpret_cast<u32x4*>(tile + r * STR + col) = x;
  }
  __syncthreads();
  const uint16_t* ts = reinterpret_cast<const uint16_t*>(tile);
  for (int it = threadIdx.x; it < D * 8; it += 256) {
    const int c = it / 8, m = it % 8;  // output row c, positions 8m..8m+7
    unsigned w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int p0 = 8 * m + e, p1 = p0 + 1;
      const int r0 = (p0 & ~15) + group_row(p0 & 15), r1 = (p1 & ~15) + group_row(p1 & 15);
      w[e / 2] = (unsigned)ts[r0 * STR + c] | ((unsigned)ts[r1 * STR + c] << 16);
    }
    const u32x4 v = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(out + (size_t)c * Tpad + t0 + 8 * m) = v;
  }
}


constexpr int kStdWaves = 4;                // one wave = 32 query rows
constexpr int kStdRows = 32 * kStdWaves;    // query rows per workgroup

// S = scale * Q K^T for 32 query rows per wave and all keys, 32 keys at a time
// (32x32x16 MFMA, query rows on the M side).  K rows come straight from
// memory (they are the B operand's natural layout).
template <int D>
__global__ __launch_bounds__(64 * kStdWaves) void std_scores_kernel(const __bf16* __restrict__ q,
                                                                    const __bf16* __restrict__ k,
                                                                    float* __restrict__ s, int Tq, int Tk,
                                                                    float scale, int causal) {
  constexpr int KS = D / 16;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int lr = lane % 32, hf = lane / 32;
  const int bh = blockIdx.y;
  const int q0 = blockIdx.x * kStdRows + wave * 32;
  if (q0 >= Tq) return;
  const __bf16* Qh = q + (size_t)bh * Tq * D;
  const __bf16* Kh = k + (size_t)bh * Tk * D;
  float* Sh = s + (size_t)bh * Tq * Tk;
  bf16x8 qf[KS];
  {
    const int qr = min(q0 + lr, Tq - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = ld16(Qh + (size_t)qr * D + 16 * ks + 8 * hf);
  }
  for (int key0 = 0; key0 < Tk; key0 += 32) {
    const int kr = min(key0 + lr, Tk - 1);
    bf16x8 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = ld16(Kh + (size_t)kr * D + 16 * ks + 8 * hf);
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mfma32(qf[ks], kf[ks], acc);
    const int key = key0 + lr;
    if (key < Tk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = q0 + 8 * (r / 4) + 4 * hf + (r % 4);
        if (row < Tq) Sh[(size_t)row * Tk + key] = (causal && key > row) ? -INFINITY : acc[r] * scale;
      }
    }
  }
}

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// Row softmax of S, one wave per row, two passes over the row: (max, sum)
// with a running max, then P = exp(s - m) / l written in the permuted column
// order, zero past Tk.  LSE = m + ln l (-inf for a row with no allowed key).
__global__ __launch_bounds__(256) void std_softmax_kernel(const float* __restrict__ s, __bf16* __restrict__ p,
                                                          float* __restrict__ lse, int rows, int Tk, int Tk_pad) {
  const size_t row = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / 64;
  const int lane = threadIdx.x % 64;
  if (row >= (size_t)rows) return;
  const float* Sr = s + row * Tk;
  float m = -INFINITY, l = 0.f;
  for (int j = lane; j < Tk; j += 64) {
    const float x = Sr[j];
    if (x > m) {
      l = l * __expf(m - x);  // m = -inf -> 0
      m = x;
    }
    if (x != -INFINITY) l += __expf(x - m);
  }
  const float M = wave_max64(m);
  l = (m == -INFINITY) ? 0.f : l * __expf(m - M);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off, 64);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float mu = (M == -INFINITY) ? 0.f : M;
  __bf16* Pr = p + row * Tk_pad;
  for (int pos = lane; pos < Tk_pad; pos += 64) {
    const int key = (pos & ~15) + group_row(pos & 15);
    const float x = key < Tk ? Sr[key] : -INFINITY;
    Pr[pos] = to_bf16(__expf(x - mu) * inv);
  }
  if (lane == 0) lse[row] = l > 0.f ? M + __logf(l) : -INFINITY;
}

// O = P V for 32 query rows per wave: P rows (A operand) and V^T rows (B
// operand) are read as 16-byte runs of 8 keys in the same permuted order.
template <int D>
__global__ __launch_bounds__(64 * kStdWaves) void std_pv_kernel(const __bf16* __restrict__ p,
                                                                const __bf16* __restrict__ vt, __bf16* __restrict__ o,
                                                                int Tq, int Tk_pad) {
  constexpr int CB = D / 32;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int lr = lane % 32, hf = lane / 32;
  const int bh = blockIdx.y;
  const int q0 = blockIdx.x * kStdRows + wave * 32;
  if (q0 >= Tq) return;
  const __bf16* Pr = p + ((size_t)bh * Tq + min(q0 + lr, Tq - 1)) * Tk_pad;
  const __bf16* VTh = vt + (size_t)bh * D * Tk_pad;
  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
  for (int k0 = 0; k0 < Tk_pad; k0 += 16) {
    const bf16x8 a = ld16(Pr + k0 + 8 * hf);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      acc[cb] = mfma32(a, ld16(VTh + (size_t)(32 * cb + lr) * Tk_pad + k0 + 8 * hf), acc[cb]);
  }
  // accumulator register r of block cb: row 8(r/4) + 4hf + r%4, column 32cb + lr
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = q0 + 8 * (r / 4) + 4 * hf + (r % 4);
      if (row < Tq) o[((size_t)bh * Tq + row) * D + 32 * cb + lr] = to_bf16(acc[cb][r]);
    }
}

struct StdLayout {
  size_t s, p, vt, total;
};

StdLayout std_layout(int BH, int Tq, int Tk, int d) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t tk_pad = (size_t)(Tk + 63) / 64 * 64;
  StdLayout L;
  L.s = 0;
  L.p = up((size_t)BH * Tq * Tk * sizeof(float));
  L.vt = L.p + up((size_t)BH * Tq * tk_pad * 2);
  L.total = L.vt + up((size_t)BH * d * tk_pad * 2);
  return L;
}

}  // namespace

size_t std_bf16_workspace_bytes(int BH, int Tq, int Tk, int d) { return std_layout(BH, Tq, Tk, d).total; }

hipError_t std_bf16_launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Tq, int Tk,
                           int d, float scale, int causal, void* workspace, hipStream_t stream) {
  const StdLayout L = std_layout(BH, Tq, Tk, d);
  char* ws = static_cast<char*>(workspace);
  float* S = reinterpret_cast<float*>(ws + L.s);
  __bf16* P = reinterpret_cast<__bf16*>(ws + L.p);
  __bf16* VT = reinterpret_cast<__bf16*>(ws + L.vt);
  const int tk_pad = (Tk + 63) / 64 * 64;
  const dim3 tiles((unsigned)((Tq + kStdRows - 1) / kStdRows), (unsigned)BH);
  prof_begin(6, stream);
  if (d == 128)
    hipLaunchKernelGGL(std_scores_kernel<128>, tiles, dim3(64 * kStdWaves), 0, stream,
                       static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), S, Tq, Tk, scale, causal);
  else
    hipLaunchKernelGGL(std_scores_kernel<64>, tiles, dim3(64 * kStdWaves), 0, stream,
                       static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), S, Tq, Tk, scale, causal);
  const size_t rows = (size_t)BH * Tq;
  hipLaunchKernelGGL(std_softmax_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, S, P, lse, (int)rows,
                     Tk, tk_pad);
  if (d == 128) {
    hipLaunchKernelGGL(transpose_rows_kernel<128>, dim3(tk_pad / 64, BH), dim3(256), 0, stream,
                       static_cast<const __bf16*>(v), VT, Tk, tk_pad);
    hipLaunchKernelGGL(std_pv_kernel<128>, tiles, dim3(64 * kStdWaves), 0, stream, P, VT, static_cast<__bf16*>(o), Tq,
                       tk_pad);
  } else {
    hipLaunchKernelGGL(transpose_rows_kernel<64>, dim3(tk_pad / 64, BH), dim3(256), 0, stream,
                       static_cast<const __bf16*>(v), VT, Tk, tk_pad);
    hipLaunchKernelGGL(std_pv_kernel<64>, tiles, dim3(64 * kStdWaves), 0, stream, P, VT, static_cast<__bf16*>(o), Tq,
                       tk_pad);
  }
  prof_end(6, stream);
  return hipGetLastError();
}

}  // namespace attn
