// Internal helpers for streaming bf16 tiles through LDS on gfx950: the
// direct-to-LDS copy, its waits, a barrier and the LDS swizzle.  Not part of
// the ABI.
#pragma once

#include "attn_common.hpp"

namespace attn {
namespace {

typedef __attribute__((address_space(3))) const void lds_cvoid;

// One wave copies 16 bytes per lane from `src` (per lane) to LDS; lane l's
// bytes land at lds_base + 16*l (lds_base must be the same in every lane).
// Issued as inline assembly so that the compiler neither reorders LDS
// accesses across it nor adds waits of its own for it: every copy is waited
// for explicitly (wait_vm) before a barrier that publishes the tile.  The
// LDS base goes through M0, which the compiler reserves but keeps no value
// in for any instruction these kernels use (the generated code writes M0
// only here), so clobbering it is safe.
__device__ __forceinline__ void dma16(const __bf16* src, const __bf16* lds_base) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cvoid*)lds_base));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
#pragma clang diagnostic pop
}

// The same copy from a wave-uniform 64-bit base in SGPRs plus a 32-bit
// per-lane byte offset: no per-lane address arithmetic per copy.
__device__ __forceinline__ void dma16_sbase(const void* sbase, uint32_t voff, const __bf16* lds_base) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_cvoid*)lds_base));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier after this wave's LDS reads and writes have completed;
// it also keeps the compiler from moving memory accesses across it.  Tile
// copies into LDS are waited for separately (wait_vm) before it.
__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ bf16x8 ld16(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Make the compiler complete a register load here, before the tile copies
// that follow are issued: its own waits count only its own loads, so a wait
// for this value inside the tile loop would also drain the copies.
__device__ __forceinline__ void settle(const bf16x8& x) { asm volatile("" ::"v"(__builtin_bit_cast(u32x4, x))); }
__device__ __forceinline__ void settle(float x) { asm volatile("" ::"v"(x)); }

// Swizzle of a row-major LDS tile with CPR 16-byte chunks per row: logical
// chunk c of row r is stored at chunk r*CPR + (c ^ swz<CPR>(r)).  For every
// CPR, 16 consecutive rows read at one logical chunk hit 16 different
// 16-byte bank groups (a 16-byte read of 32 rows has no bank conflict), and
// for CPR 8 and 16 the 4 rows x 4 chunks that half a wave touches in a
// transposing read (rows 4a..4a+3, chunks 4m..4m+3) are 16 different bank
// groups as well.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  static_assert(CPR == 4 || CPR == 8 || CPR == 16, "chunks per row");
  if constexpr (CPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else if constexpr (CPR == 8) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return (r >> 2) & 3;
}

}  // namespace
}  // namespace attn
