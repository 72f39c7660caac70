// fp32 attention kernels that follow the pages' block loop literally.  They
// serve the fp32 entry points (attn_fwd_f32 / attn_bwd_f32): small problems,
// any head dim up to 128, any key-block size, fp32 throughout.
//
// Forward: one wave per query row.  Keys are visited in blocks of `block_n`
// starting at 0, block_n, 2*block_n, ... with a shorter last block, and each
// block performs one online-softmax step on (m, l, a) ("Tiled attention with
// an online softmax", section "Task"):
//   m' = max(m, max_j s_j); mu = (m' == -inf) ? 0 : m'
//   c  = exp(m - mu); p_j = exp(s_j - mu)
//   l' = c l + sum_j p_j;  a' = c a + sum_j p_j v_j
// After the last block the row is a / l and its log-sum-exp m + log l.
//
// RESCALE == false is the chunk-wise mode of "The Hidden Recurrence in
// Softmax Attention" (section "Chunk-wise Mode") before its rescale: the same
// block loop with no max, l += sum_j exp(s_j), a += sum_j exp(s_j) v_j, and
// LSE = log l.  fp32 exp overflows once a score passes about 88.7, and the
// row then turns into inf / nan: a negative control for the rescale, not a
// path to use.
//
// Backward: D_i = sum_c dO_ic O_ic; P_ij = exp(s_ij - LSE_i);
// dS_ij = P_ij (dO_i . V_j - D_i)  ("attention backprop", "Gradient of S");
// dQ_i = scale sum_j dS_ij K_j (one wave per query row) and
// dK_j = scale sum_i dS_ij Q_i, dV_j = sum_i P_ij dO_i (one wave per key row)
// ("attention backprop", "Gradient of V and P", "Gradient of Q and K").
// No atomics: every output element is written by exactly one lane.
#include <math.h>

#include "attn_common.hpp"
#include "attn_launch.hpp"

namespace attn {

namespace {

constexpr int kMaxBlock = 1024;
constexpr int kMaxDim = 128;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// one wave (64 threads) per (bh, query row)
template <bool RESCALE>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                     const float* __restrict__ v, float* __restrict__ o,
                                                     float* __restrict__ lse, int Tq, int Tk, int d, int dv,
                                                     float scale, int causal, int block_n) {
  __shared__ float qrow[kMaxDim];
  __shared__ float pblk[kMaxBlock];
  const int lane = threadIdx.x;
  const int i = blockIdx.x % Tq;
  const size_t bh = blockIdx.x / Tq;
  const float* Q = q + (bh * Tq + i) * d;
  const float* K = k + bh * Tk * d;
  const float* V = v + bh * Tk * dv;
  for (int c = lane; c < d; c += 64) qrow[c] = Q[c];
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float acc0 = 0.f, acc1 = 0.f;  // columns lane and lane + 64
  for (int start = 0; start < Tk; start += block_n) {
    const int stop = min(Tk, start + block_n);
    // scores of the block (blocked keys: -inf)
    float bmax = -INFINITY;
    for (int j = start + lane; j < stop; j += 64) {
      float s = -INFINITY;
      if (!(causal && j > i)) {
        float dot = 0.f;
        for (int c = 0; c < d; ++c) dot = fmaf(qrow[c], K[(size_t)j * d + c], dot);
        s = dot * scale;
      }
      pblk[j - start] = s;
      bmax = fmaxf(bmax, s);
    }
    float m_new = 0.f, mu = 0.f, cfac = 1.f;
    if (RESCALE) {
      bmax = wave_max(bmax);
      m_new = fmaxf(m, bmax);
      mu = (m_new == -INFINITY) ? 0.f : m_new;
      cfac = expf(m - mu);
    }
    float psum = 0.f;
    for (int j = start + lane; j < stop; j += 64) {
      const float p = expf(pblk[j - start] - mu);
      pblk[j - start] = p;
      psum += p;
    }
    psum = wave_sum(psum);
    __syncthreads();
    float add0 = 0.f, add1 = 0.f;
    for (int j = start; j < stop; ++j) {
      const float p = pblk[j - start];
      if (lane < dv) add0 = fmaf(p, V[(size_t)j * dv + lane], add0);
      if (lane + 64 < dv) add1 = fmaf(p, V[(size_t)j * dv + lane + 64], add1);
    }
    acc0 = cfac * acc0 + add0;
    acc1 = cfac * acc1 + add1;
    l = cfac * l + psum;
    m = m_new;
    __syncthreads();
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* O = o + (bh * Tq + i) * dv;
  if (lane < dv) O[lane] = acc0 * inv;
  if (lane + 64 < dv) O[lane + 64] = acc1 * inv;
  if (RESCALE) {
    if (lane == 0) lse[bh * Tq + i] = l > 0.f ? m + logf(l) : -INFINITY;
  } else {
    if (lane == 0) lse[bh * Tq + i] = logf(l);  // log 0 = -inf; overflowed rows give inf or nan
  }
}

// dQ: one wave per (bh, query row i)
__global__ __launch_bounds__(64) void bwd_f32_dq_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                        const float* __restrict__ v, const float* __restrict__ o,
                                                        const float* __restrict__ lse, const float* __restrict__ dout,
                                                        float* __restrict__ dq, int Tq, int Tk, int d, int dv,
                                                        float scale, int causal) {
  __shared__ float qrow[kMaxDim];
  __shared__ float drow[kMaxDim];
  __shared__ float dsblk[64];
  const int lane = threadIdx.x;
  const int i = blockIdx.x % Tq;
  const size_t bh = blockIdx.x / Tq;
  const float* Q = q + (bh * Tq + i) * d;
  const float* K = k + bh * Tk * d;
  const float* V = v + bh * Tk * dv;
  const float* O = o + (bh * Tq + i) * dv;
  const float* dO = dout + (bh * Tq + i) * dv;
  for (int c = lane; c < d; c += 64) qrow[c] = Q[c];
  for (int c = lane; c < dv; c += 64) drow[c] = dO[c];
  float part = 0.f;
  for (int c = lane; c < dv; c += 64) part = fmaf(dO[c], O[c], part);
  const float Di = wave_sum(part);
  const float L = lse[bh * Tq + i];
  __syncthreads();
  float acc0 = 0.f, acc1 = 0.f;
  for (int j0 = 0; j0 < Tk; j0 += 64) {
    const int j = j0 + lane;
    float ds = 0.f;
    if (j < Tk && !(causal && j > i) && L != -INFINITY) {
      float s = 0.f, dp = 0.f;
      for (int c = 0; c < d; ++c) s = fmaf(qrow[c], K[(size_t)j * d + c], s);
      for (int c = 0; c < dv; ++c) dp = fmaf(drow[c], V[(size_t)j * dv + c], dp);
      const float p = expf(s * scale - L);
      ds = p * (dp - Di);
    }
    dsblk[lane] = ds;
    __syncthreads();
    const int jn = min(64, Tk - j0);
    for (int jj = 0; jj < jn; ++jj) {
      const float w = dsblk[jj];
      if (lane < d) acc0 = fmaf(w, K[(size_t)(j0 + jj) * d + lane], acc0);
      if (lane + 64 < d) acc1 = fmaf(w, K[(size_t)(j0 + jj) * d + lane + 64], acc1);
    }
    __syncthreads();
  }
  float* dQ = dq + (bh * Tq + i) * d;
  if (lane < d) dQ[lane] = scale * acc0;
  if (lane + 64 < d) dQ[lane + 64] = scale * acc1;
}

// dK, dV: one wave per (bh, key row j)
__global__ __launch_bounds__(64) void bwd_f32_dkdv_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                          const float* __restrict__ v, const float* __restrict__ o,
                                                          const float* __restrict__ lse,
                                                          const float* __restrict__ dout, float* __restrict__ dk,
                                                          float* __restrict__ dvg, int Tq, int Tk, int d, int dv,
                                                          float scale, int causal) {
  __shared__ float krow[kMaxDim];
  __shared__ float vrow[kMaxDim];
  __shared__ float pblk[64];
  __shared__ float dsblk[64];
  const int lane = threadIdx.x;
  const int j = blockIdx.x % Tk;
  const size_t bh = blockIdx.x / Tk;
  const float* Qh = q + bh * Tq * d;
  const float* Oh = o + bh * Tq * dv;
  const float* dOh = dout + bh * Tq * dv;
  for (int c = lane; c < d; c += 64) krow[c] = k[(bh * Tk + j) * d + c];
  for (int c = lane; c < dv; c += 64) vrow[c] = v[(bh * Tk + j) * dv + c];
  __syncthreads();
  float dk0 = 0.f, dk1 = 0.f, dv0 = 0.f, dv1 = 0.f;
  for (int i0 = 0; i0 < Tq; i0 += 64) {
    const int i = i0 + lane;
    float p = 0.f, ds = 0.f;
    if (i < Tq && !(causal && j > i)) {
      const float L = lse[bh * Tq + i];
      if (L != -INFINITY) {
        float s = 0.f, dp = 0.f, Di = 0.f;
        for (int c = 0; c < d; ++c) s = fmaf(Qh[(size_t)i * d + c], krow[c], s);
        for (int c = 0; c < dv; ++c) {
          const float g = dOh[(size_t)i * dv + c];
          dp = fmaf(g, vrow[c], dp);
          Di = fmaf(g, Oh[(size_t)i * dv + c], Di);
        }
        p = expf(s * scale - L);
        ds = p * (dp - Di);
      }
    }
    pblk[lane] = p;
    dsblk[lane] = ds;
    __syncthreads();
    const int in = min(64, Tq - i0);
    for (int ii = 0; ii < in; ++ii) {
      const float pw = pblk[ii], sw = dsblk[ii];
      const size_t r = (size_t)(i0 + ii);
      if (lane < dv) dv0 = fmaf(pw, dOh[r * dv + lane], dv0);
      if (lane + 64 < dv) dv1 = fmaf(pw, dOh[r * dv + lane + 64], dv1);
      if (lane < d) dk0 = fmaf(sw, Qh[r * d + lane], dk0);
      if (lane + 64 < d) dk1 = fmaf(sw, Qh[r * d + lane + 64], dk1);
    }
    __syncthreads();
  }
  float* dK = dk + (bh * Tk + j) * d;
  float* dV = dvg + (bh * Tk + j) * dv;
  if (lane < d) dK[lane] = scale * dk0;
  if (lane + 64 < d) dK[lane + 64] = scale * dk1;
  if (lane < dv) dV[lane] = dv0;
  if (lane + 64 < dv) dV[lane + 64] = dv1;
}

}  // namespace

hipError_t fwd_f32_launch(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int Tq,
                          int Tk, int d, int dv, float scale, int causal, int block_n, int rescale,
                          hipStream_t stream) {
  const dim3 grid((unsigned)((size_t)BH * Tq));
  if (rescale)
    hipLaunchKernelGGL(fwd_f32_kernel<true>, grid, dim3(64), 0, stream, q, k, v, o, lse, Tq, Tk, d, dv, scale, causal,
                       block_n);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<false>, grid, dim3(64), 0, stream, q, k, v, o, lse, Tq, Tk, d, dv, scale,
                       causal, block_n);
  return hipGetLastError();
}

hipError_t bwd_f32_launch(const float* q, const float* k, const float* v, const float* o, const float* lse,
                          const float* dout, float* dq, float* dk, float* dv_grad, int BH, int Tq, int Tk, int d,
                          int dv, float scale, int causal, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_f32_dq_kernel, dim3((unsigned)((size_t)BH * Tq)), dim3(64), 0, stream, q, k, v, o, lse,
                     dout, dq, Tq, Tk, d, dv, scale, causal);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_f32_dkdv_kernel, dim3((unsigned)((size_t)BH * Tk)), dim3(64), 0, stream, q, k, v, o, lse,
                     dout, dk, dv_grad, Tq, Tk, d, dv, scale, causal);
  return hipGetLastError();
}

}  // namespace attn
