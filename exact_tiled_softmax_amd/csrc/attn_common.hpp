// Internal helpers shared by the gfx950 attention kernels (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32x16 bf16 MFMA with fp32 accumulation.  Operand lane layout (checked on
// gfx950 against a host matmul): lane l holds A[l%32][8*(l/32) + e] and
// B[8*(l/32) + e][l%32] for e = 0..7; accumulator register r of lane l holds
// C[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing 8-byte LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, let lane t point at 4 consecutive 16-bit values M[t][0..3]; lane i
// receives M[4e + i/4][i%4] for e = 0..3.  Pointing lane t at row
// (r0 + t/4), column (c0 + 4*(t%4)) of a row-major 16-bit matrix therefore
// gives lane i the column c0 + i of rows r0..r0+3.
__device__ __forceinline__ i16x4 lds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}

__device__ __forceinline__ bf16x8 join_tr(const i16x4& lo, const i16x4& hi) {
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value held by lane (l ^ 32).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// max / sum of the values held by lanes l and l ^ 32.  v_permlane32_swap(v, v)
// returns, in its two results, the lower-half and upper-half value of every
// lane pair (lane order of the pair differs per half, which max and + ignore).
__device__ __forceinline__ float pair_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Word 3 of a raw buffer resource on gfx9 (data format 32, no swizzle, no
// index stride): a buffer access past the record size the resource gives is
// dropped (stores) or reads zero (loads) instead of touching memory.
constexpr int kBufferWord3 = 0x00020000;

// Byte permute: result byte i = byte sel[i] of the 8-byte value {hi:lo}.
__device__ __forceinline__ unsigned perm_b32(unsigned hi, unsigned lo, unsigned sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// {lo16(a), lo16(b)} and {hi16(a), hi16(b)} of two packed bf16 pairs.
__device__ __forceinline__ unsigned pack_lo16(unsigned a, unsigned b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ unsigned pack_hi16(unsigned a, unsigned b) { return perm_b32(b, a, 0x07060302u); }

// Map the hardware workgroup id to a logical work item so that logical items
// that are adjacent in number run on the same XCD (workgroups are dealt to
// the 8 XCDs round robin, and each XCD has its own L2).  Logical items
// [x*per + min(x, rem) ...) go to XCD x.
__device__ __forceinline__ int xcd_remap(int wg, int n) {
  const int per = n / 8, rem = n % 8;
  const int x = wg % 8, slot = wg / 8;
  return (x < rem) ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
}

// Work item of a launch over (head, block, split), block 0 the heaviest: the
// logical items of each group of G consecutive heads are ordered block-major
// (block, then head, then split), so that a group's heaviest blocks of all
// its heads are dispatched before any of their lighter ones.  G = 1 is
// head-major.  With xcd_remap, a group whose items fill one XCD's range
// keeps its heads on that XCD.
struct WorkItem {
  int bh, blk, split;
};
__device__ __forceinline__ WorkItem work_item(int item, int BH, int nblk, int nsplit, int G) {
  const int full = G * nblk * nsplit;
  const int g = item / full, r = item % full;
  const int gsize = min(G, BH - g * G);
  WorkItem w;
  w.blk = r / (gsize * nsplit);
  w.bh = g * G + (r / nsplit) % gsize;
  w.split = r % nsplit;
  return w;
}

}  // namespace attn
