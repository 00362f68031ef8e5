// Device-side pieces shared by the split-KV attention kernels (attn.hip,
// attn_shared.hip): operand addressing in the tiled page layout, the
// online-softmax update, and the partial / final output write.
#pragma once

#include "common.h"
#include "internal.h"

#include <climits>
#include <cmath>

namespace wmtp {

constexpr float kLn2 = 0.693147180559945309f;

// Element offset, inside a 32-position K tile, of the 16 bytes lane (n, j)
// feeds as the MFMA A operand of key block bb, head-dim step ks.  A row n of
// key block bb is key 8*(n/4) + 4*bb + n%4 of the tile, so that the S^T
// accumulator rows a lane receives are keys 8*(lane/16) .. +7.
__device__ __forceinline__ int k_operand_offset(int bb, int ks, int n, int j) {
  const int tok = 8 * (n >> 2) + 4 * bb + (n & 3);
  return ks * 1024 + tok * 32 + j * 8;
}

// Element offset, inside a 32-position V tile, of lane (n, j)'s 16 bytes of
// the V^T operand of head-dim block db: dims 16*db + n, keys 8*j .. +7.
__device__ __forceinline__ int v_operand_offset(int db, int n, int j) {
  return (db * 16 + n) * 32 + j * 8;
}

template <int D, bool RING>
struct KTile {
  bf16x8 k[2][D / 32];   // K operands: key block bb, head-dim step ks
  int32_t pos[RING ? 8 : 1];   // ring mode: positions held by this lane's 8 slots
};

template <int D>
struct VTile {
  bf16x8 v[D / 16];      // V^T operands: head-dim block db
};

// Physical 32-key tile index of tile kb of (b, g), or ok = false when the
// page id is outside the cache (its keys then count as absent).
template <bool RING>
__device__ __forceinline__ size_t tile_index(const AttnArgs& a, int b, int g, int kb, bool& ok) {
  const int lpage = kb >> 1;
  int ppage;
  if constexpr (RING) {
    ppage = b * (a.C >> 6) + lpage;
  } else {
    ppage = a.block_table[(size_t)b * a.max_pages + lpage];
  }
  ok = (unsigned)ppage < (unsigned)a.num_pages;
  return ((size_t)ppage * a.Hkv + g) * 2 + (kb & 1);
}

template <int D, bool RING>
__device__ __forceinline__ void load_k(KTile<D, RING>& t, const AttnArgs& a, size_t tile, int b,
                                       int kb, int n, int j) {
  constexpr int KS = D / 32;
  const uint16_t* kt = a.kc + tile * (size_t)(32 * D);
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      t.k[bb][ks] = ld_bf16x8_stream(kt + k_operand_offset(bb, ks, n, j));
  }
  if constexpr (RING) {
    const int32_t* rp = a.ring_pos + (size_t)b * a.C + kb * 32 + j * 8;
    const int4 p0 = *reinterpret_cast<const int4*>(rp);
    const int4 p1 = *reinterpret_cast<const int4*>(rp + 4);
    t.pos[0] = p0.x; t.pos[1] = p0.y; t.pos[2] = p0.z; t.pos[3] = p0.w;
    t.pos[4] = p1.x; t.pos[5] = p1.y; t.pos[6] = p1.z; t.pos[7] = p1.w;
  }
}

template <int D>
__device__ __forceinline__ void load_v(VTile<D>& t, const AttnArgs& a, size_t tile, int n, int j) {
  constexpr int DB = D / 16;
  const uint16_t* vt = a.vc + tile * (size_t)(32 * D);
#pragma unroll
  for (int db = 0; db < DB; ++db) t.v[db] = ld_bf16x8_stream(vt + v_operand_offset(db, n, j));
}

template <int D, int NRB>
struct SoftmaxState {
  f32x4 acc[NRB][D / 16];   // O^T accumulators: lane (n, j) holds d = 16*db + 4*j + i, row n
  float m[NRB];             // running row max of the scaled logits (log2 units)
  float l[NRB];             // this lane's share of the running sum of weights
};

// Keys of this lane's 8 (kbase .. kbase+7) that exist for every row: inside the
// sequence length, or (ring) holding a position of the current window.
template <int D, bool RING>
__device__ __forceinline__ uint32_t present_keys(const KTile<D, RING>& t, const AttnArgs& a,
                                                 int kbase, int L, int T) {
  uint32_t keep;
  if constexpr (RING) {
    keep = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = t.pos[i];
      const bool ok = p >= 0 && p < T && (p < a.n_sink || p >= T - a.n_recent);
      keep |= (ok ? 1u : 0u) << i;
    }
  } else {
    const int rem = L - kbase;
    keep = rem >= 8 ? 0xFFu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
  }
  return keep;
}

// Online-softmax update of one row block from its S^T accumulators.  The weights
// this lane feeds to the PV product are returned as two bf16 parts, p = hi + lo
// (hi = bf16(p), lo = bf16(p - hi)), so that PV sees p to about 2^-16 relative
// instead of bf16's 2^-9; the running sum adds the fp32 weights.
//
// The running maximum m (log2 units, uniform over the four lanes of a row) is
// only raised when some score of the wave exceeds it by more than kLazyMax:
// weights are exp2(x - m) <= 2^kLazyMax either way, so nothing overflows, and
// the result (sum p v / sum p, lse = m + log2 sum p) does not depend on which m
// was used.  Most tiles then need neither the cross-lane max nor a rescale of
// the accumulators.
constexpr float kLazyMax = 8.0f;

template <int D, int NRB>
__device__ __forceinline__ void softmax_update(SoftmaxState<D, NRB>& st, int rb, f32x4 s0,
                                               f32x4 s1, uint32_t keep, int lr, float scale_log2,
                                               bf16x8& p_hi, bf16x8& p_lo) {
  constexpr int DB = D / 16;
  // s0[i] is key kbase + i, s1[i] is key kbase + 4 + i, for this lane's row.
  float x[8];
  if (keep == 0xFFu && lr >= 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (i < 4 ? s0[i] : s1[i - 4]) * scale_log2;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = (i < 4 ? s0[i] : s1[i - 4]) * scale_log2;
      const bool ok = ((keep >> i) & 1u) && (i < lr);
      x[i] = ok ? v : -INFINITY;
    }
  }
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
  // m = -inf: -inf <= -inf holds only when this lane saw no key either.
  const bool raise = !(mx <= st.m[rb] + kLazyMax);
  if (__any(raise)) {
    const float m_new = fmaxf(st.m[rb], max_over_lane_groups(mx));
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(st.m[rb] - m_use);
    st.m[rb] = m_new;
    st.l[rb] *= alpha;
    if (!__all(alpha == 1.0f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) st.acc[rb][db] *= alpha;
    }
  }
  const float m_use = (st.m[rb] == -INFINITY) ? 0.f : st.m[rb];

  u32x4 hw, lw;
  float psum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float p0 = fast_exp2(x[2 * w] - m_use);
    const float p1 = fast_exp2(x[2 * w + 1] - m_use);
    psum += p0 + p1;
    const uint32_t h0 = f32_to_bf16_bits(p0);
    const uint32_t h1 = f32_to_bf16_bits(p1);
    const uint32_t l0 = f32_to_bf16_bits(p0 - bf16_bits_to_f32(h0));
    const uint32_t l1 = f32_to_bf16_bits(p1 - bf16_bits_to_f32(h1));
    hw[w] = h0 | (h1 << 16);
    lw[w] = l0 | (l1 << 16);
  }
  st.l[rb] += psum;
  p_hi = __builtin_bit_cast(bf16x8, hw);
  p_lo = __builtin_bit_cast(bf16x8, lw);
}

}  // namespace wmtp
