// Device-side pieces shared by the split-KV attention kernels (attn.hip,
// attn_shared.hip): MFMA operand addressing in the tiled page layout, the
// online-softmax steps, and the output write.
//
// Products per 32-position tile and 32 query rows (MFMA 32x32x16, bf16 in, fp32
// accumulate):
//     S^T[key][row] = K[key][:] . Q[row][:]         D/16 steps
//     O^T[d][row]  += V^T[d][key] . P^T[key][row]   D/32 blocks x 2 steps (x2: P hi, lo)
// Keys sit on the M axis of S^T.  The K rows are fed in an order (bits 2 and 3 of
// the MFMA row index swapped) that makes S^T register i of lane (n, h), n = lane
// % 32, h = lane / 32, hold key 16*(i/8) + 8*h + i%8 of row n; registers 0..7 and
// 8..15 are then exactly the lane's contraction slices of P^T for the two PV
// steps (keys 8h..8h+7 and 16+8h..16+8h+7), and the matching V^T operand is 16
// contiguous bytes of the V tile.  No value crosses lanes between the products
// except the row maximum, over the two lanes n and n + 32.
#pragma once

#include "common.h"
#include "internal.h"

#include <climits>
#include <cmath>

namespace wmtp {

constexpr float kLn2 = 0.693147180559945309f;

// MFMA row m of the S^T product holds tile key m with bits 2 and 3 swapped.
__device__ __forceinline__ int s_row_key(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Element offset, inside a 32-position K tile ([D/16][32 pos][16 dims]), of the
// 16 bytes lane (m, h) feeds as A operand of head-dim step ks (dims 16*ks + 8*h
// ..).  The 64 lanes of one step read the step's whole 1 KB block.
__device__ __forceinline__ int k_operand_offset(int ks, int m, int h) {
  return ks * 512 + s_row_key(m) * 16 + h * 8;
}

// Element offset, inside a 32-position V tile ([2][D][16 pos]), of lane (m, h)'s
// 16 bytes of the V^T operand of head-dim block db, key step kk: dim 32*db + m,
// keys 16*kk + 8*h .. +7.  The 64 lanes read one contiguous 1 KB block.
template <int D>
__device__ __forceinline__ int v_operand_offset(int db, int kk, int m, int h) {
  return kk * (16 * D) + (db * 32 + m) * 16 + h * 8;
}

// Tile-relative key held by S^T register i of lane group h.
__host__ __device__ constexpr int s_key(int i, int h) { return 16 * (i >> 3) + 8 * h + (i & 7); }

template <int D, int NB>
struct SoftmaxState {
  f32x16 acc[NB][D / 32];   // O^T: lane (n, h) register i holds d = 32*db + 8*(i/4) + 4*h + i%4
  float m[NB];              // running row max of the scaled logits (log2 units)
  float l[NB];              // this lane's share of the running sum of weights
  float l_drop[NB];         // the part of l that PV did not see: the low bf16 parts of
                            // the weights of tiles whose PV took the high parts only
};

// 16 bits: which of this lane's keys are below `count` (tile-relative): keys
// 8h..8h+7 are bits 0..7, keys 16+8h..16+8h+7 bits 8..15.
__device__ __forceinline__ uint32_t keys_below(int count, int h) {
  const int r0 = count - 8 * h;
  const int r1 = r0 - 16;
  const uint32_t b0 = r0 >= 8 ? 0xFFu : (r0 <= 0 ? 0u : ((1u << r0) - 1u));
  const uint32_t b1 = r1 >= 8 ? 0xFFu : (r1 <= 0 ? 0u : ((1u << r1) - 1u));
  return b0 | (b1 << 8);
}

// Max / sum over the two lanes of a row (n and n + 32).  v_permlane32_swap of v
// with itself leaves lanes n and n + 32 holding (v[n], v[n]) in the first result
// and (v[n + 32], v[n + 32]) in the second, so one swap and one VALU operation
// combine the pair in every lane, with no LDS round trip.
__device__ __forceinline__ float max_over_row(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_over_row(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Eight fp8 e4m3 values (bytes 0..7 of r, element j = byte j) as the bf16 MFMA
// operand of the same element order.  Every e4m3 value is a bf16 value, so the
// conversion is exact: gfx950 widens two fp8 bytes to two packed bf16 in one
// instruction (scale 1, so nothing is rounded).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 r) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, 1.0f, false);
  const bf16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, 1.0f, true);
  const bf16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, 1.0f, false);
  const bf16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, 1.0f, true);
  return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                                          __builtin_bit_cast(uint32_t, h2), __builtin_bit_cast(uint32_t, h3)});
}
__device__ __forceinline__ bf16x8 as_operand(bf16x8 v) { return v; }
__device__ __forceinline__ bf16x8 as_operand(u32x2 r) { return fp8x8_to_bf16(r); }

// Verify under a tree of proposals: of this lane's 16 keys, which are appended
// positions that `mask` marks (bit a: the appended position a, 0 <= a < 64).
// rel0 is the appended index of the tile's key 0 (negative when the tile starts
// before the appended positions).
__device__ __forceinline__ uint32_t tree_keys(uint64_t mask, int rel0, int h) {
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int a = rel0 + (i < 8 ? 8 * h + i : 16 + 8 * h + (i - 8));
    const bool on = a >= 0 && a < 64 && ((mask >> (a & 63)) & 1u);
    bits |= (on ? 1u : 0u) << i;
  }
  return bits;
}

// Online softmax in log2 units: scores x = s * c with c = scale * log2(e) > 0,
// weights p = exp2(x - m).  The running maximum m of a row (the same on its two
// lanes) is raised lazily, only when a score exceeds it by more than kLazyMax.
// Weights then stay below 2^kLazyMax and row sums below 2^(kLazyMax + 32), far
// inside the fp32 and bf16 range, and the result (sum p v / sum p, lse = m +
// log2 sum p) does not depend on which m was used.  With so wide a margin a
// raise after a row's first visible key is rare, so the kernels run a fast loop
// that never rescales the accumulators and fall back to a general loop only
// when a rescale is due; a row whose m is still -inf takes its first maximum in
// the fast loop, since its accumulators and sum are still zero.  The weights
// reach PV as two bf16 parts, p = hi + lo (hi = bf16(p), lo = bf16(p - hi)), so
// PV sees p to about 2^-16 relative instead of bf16's 2^-9; the running sum adds
// the fp32 weights.
constexpr float kLazyMax = 64.0f;

// This lane's keys visible to a row whose keys below `lr` (tile-relative) are in
// its causal range, among the present ones.
__device__ __forceinline__ uint32_t visible_keys(uint32_t keep, int lr, int h) {
  return keep & keys_below(lr, h);
}

__device__ __forceinline__ float lane_max16(const float (&x)[16]) {
  float a = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  float b = fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]));
  float c = fmaxf(fmaxf(x[8], x[9]), fmaxf(x[10], x[11]));
  float d = fmaxf(fmaxf(x[12], x[13]), fmaxf(x[14], x[15]));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Raw scores of one row block, -inf where the key is not visible, and the lane
// maximum in log2 units.  all_vis (wave-uniform): every key is visible to every
// row, the common case, which skips the masking.
__device__ __forceinline__ float masked_scores(float (&x)[16], const f32x16& s, uint32_t vis,
                                               bool all_vis, float c) {
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = s[i];
  if (!all_vis) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = ((vis >> i) & 1u) ? x[i] : -INFINITY;
  }
  return lane_max16(x) * c;
}

// Does this lane's row need its maximum raised?  (m = -inf: -inf <= -inf holds
// only when this lane saw no key either.)
__device__ __forceinline__ bool needs_raise(float lane_mx, float m) {
  return !(lane_mx <= m + kLazyMax);
}

// Ties an accumulator block to the accumulation registers at this point, so that
// the compiler keeps the O^T blocks there for the whole loop.
__device__ __forceinline__ void pin_acc(f32x16& v) { asm volatile("" : "+a"(v)); }

// Fast-loop maximum update: rows without a maximum take their first one.
// Returns true (wave-uniform) when some row that has a maximum needs it raised:
// the caller then hands the tile to the general loop.
template <int D, int NB>
__device__ __forceinline__ bool first_max_or_rescale(SoftmaxState<D, NB>& st,
                                                     const float (&mx)[NB]) {
  bool raise = false, rescale = false;
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const bool r = needs_raise(mx[rb], st.m[rb]);
    raise |= r;
    rescale |= r && st.m[rb] != -INFINITY;
  }
  if (__any(rescale)) return true;
  if (__any(raise)) {
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      const float row_mx = max_over_row(mx[rb]);
      if (st.m[rb] == -INFINITY) st.m[rb] = row_mx;
    }
  }
  return false;
}

// General-loop maximum update: raise where needed and rescale the row's
// accumulators and sum by exp2(m_old - m_new); also(rb, alpha) rescales whatever
// else the caller keeps in the same units.
template <int D, int NB, typename Also>
__device__ __forceinline__ void raise_and_rescale(SoftmaxState<D, NB>& st, const float (&mx)[NB],
                                                  Also&& also) {
  constexpr int DB = D / 32;
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    if (!__any(needs_raise(mx[rb], st.m[rb]))) continue;
    const float m_new = fmaxf(st.m[rb], max_over_row(mx[rb]));
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(st.m[rb] - m_use);
    st.m[rb] = m_new;
    st.l[rb] *= alpha;
    st.l_drop[rb] *= alpha;
    if (!__all(alpha == 1.0f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        st.acc[rb][db] *= alpha;
        pin_acc(st.acc[rb][db]);
      }
      also(rb, alpha);
    }
  }
}
template <int D, int NB>
__device__ __forceinline__ void raise_and_rescale(SoftmaxState<D, NB>& st, const float (&mx)[NB]) {
  raise_and_rescale(st, mx, [](int, float) {});
}

// Weights of one row block as the P^T operands of the two PV steps.
template <int D, int NB>
__device__ __forceinline__ void weights(SoftmaxState<D, NB>& st, int rb, const float (&x)[16],
                                        float c, bf16x8 (&p_hi)[2], bf16x8 (&p_lo)[2]) {
  const float neg_m = (st.m[rb] == -INFINITY) ? 0.f : -st.m[rb];
  float psum = 0.f;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    u32x4 hw, lw;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float p0 = fast_exp2(fmaf(x[8 * kk + 2 * w], c, neg_m));
      const float p1 = fast_exp2(fmaf(x[8 * kk + 2 * w + 1], c, neg_m));
      psum += p0 + p1;
      const uint32_t hp = pack_bf16x2(p0, p1);
      const uint32_t lp = pack_bf16x2(p0 - __builtin_bit_cast(float, hp << 16),
                                      p1 - __builtin_bit_cast(float, hp & 0xFFFF0000u));
      hw[w] = hp;
      lw[w] = lp;
    }
    p_hi[kk] = __builtin_bit_cast(bf16x8, hw);
    p_lo[kk] = __builtin_bit_cast(bf16x8, lw);
  }
  st.l[rb] += psum;
}

// Zero the bf16 lanes of an 8-key operand whose keep bits (bit j = key j of the
// operand) are clear, so that absent keys (any bits, even NaN) add 0 in PV.
__device__ __forceinline__ bf16x8 mask8(bf16x8 v, uint32_t bits8) { return mask_bf16x8(v, bits8); }

// PV of one tile for NB row blocks: V^T operands v[db][kk]; the hi products of
// every accumulator first, then the lo products, so that no MFMA waits on the
// one just before it.
template <int D, int NB>
__device__ __forceinline__ void pv(SoftmaxState<D, NB>& st, const bf16x8 (&v)[D / 32][2],
                                   const bf16x8 (&p_hi)[NB][2], const bf16x8 (&p_lo)[NB][2]) {
  constexpr int DB = D / 32;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int rb = 0; rb < NB; ++rb)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        st.acc[rb][db] = mfma32x32x16(v[db][kk], p_hi[rb][kk], st.acc[rb][db]);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int rb = 0; rb < NB; ++rb)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        st.acc[rb][db] = mfma32x32x16(v[db][kk], p_lo[rb][kk], st.acc[rb][db]);
}

// Normalised output of one row block of this lane: o[d] for the lane's 16 dims.
template <int D, int NB>
__device__ __forceinline__ void write_row(float* op, const SoftmaxState<D, NB>& st, int rb,
                                          float inv, int h) {
  constexpr int DB = D / 32;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 v = {st.acc[rb][db][4 * c] * inv, st.acc[rb][db][4 * c + 1] * inv,
                       st.acc[rb][db][4 * c + 2] * inv, st.acc[rb][db][4 * c + 3] * inv};
      *reinterpret_cast<f32x4*>(op + db * 32 + 8 * c + 4 * h) = v;
    }
}

}  // namespace wmtp
