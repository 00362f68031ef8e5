// Streaming K/V tiles through LDS rings: the wait, barrier and load primitives
// the LDS-sharing attention kernels are built from.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace wmtp {

// Wait until at most N vector-memory operations of this wave are outstanding.
// gfx9 encoding: vmcnt in bits [3:0] and [15:14]; expcnt (bits [6:4]) and
// lgkmcnt (bits [11:8]) left at their maxima (no wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int enc = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  __builtin_amdgcn_s_waitcnt(enc);
}

// Workgroup barrier that does not wait for outstanding global loads, so the
// next tiles' direct-to-LDS loads stay in flight across it.  Visibility of a
// tile is established before the barrier by each wave's own vmcnt wait (a
// direct-to-LDS load is counted until its data is in LDS); the memory clobber
// keeps the compiler from moving LDS accesses across the barrier, and every LDS
// read of a tile is consumed by that tile's MFMAs before the next barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_barrier" ::: "memory");
}

// N 1 KB global-to-LDS loads (global_load_lds_dwordx4, non-temporal) under one
// M0: load j takes lane i's 16 bytes at base + voff + STRIDE j (base
// wave-uniform, voff the lane's byte offset) to dst + STRIDE j + 16 i.  The
// instruction's immediate offset moves the global address and the LDS address
// alike, so one M0 value serves the run (M0 is saved and restored around it).
// Written as inline asm because the compiler treats the builtin as an LDS write
// that may alias every LDS read in flight and, with one anywhere in the kernel,
// drains all LDS reads at every LDS wait; the slots refilled here are never read
// while their loads are outstanding (a barrier separates the last read of a
// slot from its refill, and the explicit vmcnt waits plus a barrier its refill
// from the next read), so no such wait is needed.  The loads are counted in
// vmcnt like any other, which the callers' explicit waits account for.
template <int N, int STRIDE = 1024>
__device__ __forceinline__ void lds_load_run(const void* base, uint32_t voff, unsigned char* dst) {
  static_assert(N == 1 || N == 2 || N == 4, "runs of 1, 2 or 4 loads");
  static_assert(STRIDE % 1024 == 0 && (N - 1) * STRIDE < 4096, "immediate offsets below 4 KB");
  const unsigned m0 = (unsigned)(size_t)((__attribute__((address_space(3))) unsigned char*)dst);
  unsigned saved;
  if constexpr (N == 1) {
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %2 nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(voff), "s"(base), "s"(m0) : "memory");
  } else if constexpr (N == 2) {
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %2 nt\n\t"
                 "global_load_lds_dwordx4 %1, %2 offset:%4 nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(voff), "s"(base), "s"(m0), "i"(STRIDE) : "memory");
  } else {
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %2 nt\n\t"
                 "global_load_lds_dwordx4 %1, %2 offset:%4 nt\n\t"
                 "global_load_lds_dwordx4 %1, %2 offset:%5 nt\n\t"
                 "global_load_lds_dwordx4 %1, %2 offset:%6 nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(voff), "s"(base), "s"(m0), "i"(STRIDE), "i"(2 * STRIDE), "i"(3 * STRIDE)
                 : "memory");
  }
}

// Compiler-level fence for memory operations: LDS reads after it are not hoisted
// above it, which bounds how many operand registers are live at once.
__device__ __forceinline__ void operand_fence() { asm volatile("" ::: "memory"); }

// Scheduling anchors: an empty volatile asm that "redefines" a register.  The
// volatile statements keep their relative order, so a value produced before one
// anchor and consumed after the next cannot move across either; this is how the
// fast tiles keep their interleaved issue order.
template <typename T>
__device__ __forceinline__ void anchor(T& v) { asm volatile("" : "+v"(v)); }

}  // namespace wmtp
