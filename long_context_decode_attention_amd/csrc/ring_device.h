// Device-side ring writer shared by the ring append kernels (append.hip) and
// the fused windowed draft step (attn.hip): the tiled-page store of one
// position's K/V and the write of the positions that survive an append.
//
// Tiled pages: tile t = (page * Hkv + g) * 2 + (pos % 64) / 32 holds 32 * D
// elements; with tok = pos % 32, K tile element (tok, d) at (d / 16) * 512 +
// tok * 16 + d % 16, V tile element (tok, d) at (tok / 16) * 16 * D + d * 16 +
// tok % 16.
#pragma once

#include "common.h"
#include "internal.h"

namespace wmtp {

// Store the 8 dims d0 .. d0+7 of one position (16 bytes of K and of V from the
// row-major source) into tile `tile`, position-in-tile `tok`.
__device__ __forceinline__ void store_kv8(uint16_t* kc, uint16_t* vc, size_t tile, int tok, int d0,
                                          int D, const uint16_t* ksrc, const uint16_t* vsrc) {
  const u32x4 kv = *reinterpret_cast<const u32x4*>(ksrc);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(vsrc);
  uint16_t* kt = kc + tile * (size_t)(32 * D);
  uint16_t* vt = vc + tile * (size_t)(32 * D);
  *reinterpret_cast<u32x4*>(kt + (d0 >> 4) * 512 + tok * 16 + (d0 & 15)) = kv;
  uint16_t* vp = vt + (tok >> 4) * (16 * D) + (tok & 15);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    vp[(d0 + 2 * w) * 16] = (uint16_t)(vv[w] & 0xFFFFu);
    vp[(d0 + 2 * w + 1) * 16] = (uint16_t)(vv[w] >> 16);
  }
}

// Of the appended positions [T0, T0 + n_new), a sink position keeps its slot for
// good, and a later position survives iff no later appended position shares its
// slot, i.e. iff p >= T1 - M.  Only survivors are written: items
// [first, total) with stride `step` of the survivors' 16-byte pieces.
__device__ __forceinline__ void ring_write(const RingAppendArgs& a, int b, int64_t T0, int first,
                                           int step) {
  const int64_t T1 = T0 + a.n_new;
  const int64_t M = a.C - a.n_sink;
  const int64_t s_lo = T0;
  const int64_t s_hi = T1 < a.n_sink ? T1 : (int64_t)a.n_sink;
  int64_t r_lo = T0 > a.n_sink ? T0 : (int64_t)a.n_sink;
  if (T1 - M > r_lo) r_lo = T1 - M;
  const int64_t r_hi = T1;
  const int n_s = s_hi > s_lo ? (int)(s_hi - s_lo) : 0;
  const int n_r = r_hi > r_lo ? (int)(r_hi - r_lo) : 0;
  const int chunks = a.Hkv * (a.D >> 3);      // 16-byte pieces per position
  const int total = (n_s + n_r) * chunks;
  for (int idx = first; idx < total; idx += step) {
    const int e = idx / chunks;
    const int c = idx - e * chunks;
    const int64_t p = e < n_s ? s_lo + e : r_lo + (e - n_s);
    const int64_t t_in = p - T0;
    const int slot = p < a.n_sink ? (int)p : a.n_sink + (int)((p - a.n_sink) % M);
    const int g = c / (a.D >> 3);
    const int d0 = (c - g * (a.D >> 3)) * 8;
    const size_t src = (((size_t)b * a.n_new + t_in) * a.Hkv + g) * a.D + d0;
    const int page = b * (a.C >> 6) + (slot >> 6);
    const int off = slot & 63;
    const size_t tile = ((size_t)page * a.Hkv + g) * 2 + (off >> 5);
    store_kv8(a.kc, a.vc, tile, off & 31, d0, a.D, a.k_new + src, a.v_new + src);
    if (c == 0) a.ring_pos[(size_t)b * a.C + slot] = (int32_t)p;
  }
}

// Append of a few positions to ring b by one workgroup of 256 threads: every
// thread reads the old count before thread 0 stores the new one.
__device__ __forceinline__ void ring_append_block(const RingAppendArgs& a, int b) {
  int64_t T0 = a.ring_T[b];
  if (T0 < 0) T0 = 0;
  __syncthreads();
  ring_write(a, b, T0, threadIdx.x, 256);
  __syncthreads();
  if (threadIdx.x == 0) a.ring_T[b] = T0 + a.n_new;
}

}  // namespace wmtp
