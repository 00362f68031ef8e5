// Shared device types and helpers for the gfx950 kernels of libwmtp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wmtp {

constexpr int kPage = 64;        // positions per KV page
constexpr int kTile = 32;        // positions per tile (one MFMA contraction step over keys)
constexpr int kWave = 64;        // wavefront width on CDNA

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte global load as 8 bf16 lanes.
__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

// The same, as a non-temporal load: streamed K/V is read once per call, so it
// should not displace reusable lines (measured ~7.0 TB/s streaming vs ~6.1 TB/s
// for ordinary loads on MI355X).
__device__ __forceinline__ bf16x8 ld_bf16x8_stream(const uint16_t* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return __builtin_bit_cast(bf16x8, v);
}

// 8-byte load (8 fp8 values of a K/V tile read again later), and its
// non-temporal form for streamed tiles.
__device__ __forceinline__ u32x2 ld_u32x2(const uint8_t* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ u32x2 ld_u32x2_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// Zero the bf16 lanes whose bit in `keep` (bit i = lane i) is clear.
__device__ __forceinline__ bf16x8 mask_bf16x8(bf16x8 v, uint32_t keep) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t m = ((keep >> (2 * w)) & 1u ? 0x0000FFFFu : 0u) |
                 ((keep >> (2 * w + 1)) & 1u ? 0xFFFF0000u : 0u);
    u[w] &= m;
  }
  return __builtin_bit_cast(bf16x8, u);
}

// C[16x16] += A[16x32] * B[32x16], bf16 inputs, fp32 accumulate.
// Lane l supplies A row (l % 16) and B column (l % 16), 8 contraction
// elements each (the same 8 for A and B); it receives C column (l % 16),
// rows 4 * (l / 16) + 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// C[32x32] += A[32x16] * B[16x32], bf16 inputs, fp32 accumulate.
// Lane l supplies A row (l % 32) and B column (l % 32), 8 contraction elements
// each (the same 8 for A and B); it receives C column (l % 32), rows
// 8 * (i / 4) + 4 * (l / 32) + i % 4 in register i (i = 0..15).  On gfx950 this
// shape runs at the full bf16 matrix rate even with one wave per SIMD, where
// 16x16x32 reaches about a third of it.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Butterfly max / sum over the four lanes that share (lane % 16).
__device__ __forceinline__ float max_over_lane_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float sum_over_lane_groups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;   // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, h);
}

// Two floats rounded to bf16 (nearest even) and packed: a in bits 0..15, b in
// bits 16..31 (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

}  // namespace wmtp
