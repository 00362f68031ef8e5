// Device-side log-sum-exp merge of per-split attention results, the core of the
// merge kernels (combine.hip):
//     lse = ln sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) * o_s.
#pragma once

#include "common.h"

namespace wmtp {

constexpr int kMergeUnroll = 8;   // (o_s, lse_s) pairs a lane loads at a time

// One split lane's share of a merge, in a single pass over its splits
// p0 + sl, p0 + sl + SL, ... < p1: kMergeUnroll pairs are loaded at a time, all
// independent of one another, and folded into a running maximum m (log2 units;
// -inf while the lane has seen no key) and sums acc = sum_s 2^(l_s - m) * o_s,
// wsum = sum_s 2^(l_s - m), rescaled when m rises.  The lanes' states are then
// brought to their common maximum by the caller.  base points at column col of
// row `row` of partial 0; partial q's row is base + q * stride, its lse
// lse[q * R + row].
struct LaneMerge {
  f32x4 acc;
  float wsum;
  float m;
};

__device__ __forceinline__ LaneMerge merge_lane(const float* base, const float* lse, size_t stride,
                                                int R, int row, int p0, int p1, int sl, int SL) {
  constexpr float kLog2eM = 1.4426950408889634f;
  LaneMerge s = {f32x4{0.f, 0.f, 0.f, 0.f}, 0.f, -INFINITY};
  for (int p = p0 + sl; p < p1; p += SL * kMergeUnroll) {
    f32x4 v[kMergeUnroll];
    float l[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int q = p + u * SL;
      if (q < p1) {
        v[u] = *reinterpret_cast<const f32x4*>(base + (size_t)q * stride);
        l[u] = lse[(size_t)q * R + row] * kLog2eM;
      } else {
        v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        l[u] = -INFINITY;
      }
    }
    float bm = l[0];
#pragma unroll
    for (int u = 1; u < kMergeUnroll; ++u) bm = fmaxf(bm, l[u]);
    if (bm == -INFINITY) continue;   // no keys in this batch
    if (bm > s.m) {
      const float f = s.m == -INFINITY ? 0.f : fast_exp2(s.m - bm);
      s.acc *= f;
      s.wsum *= f;
      s.m = bm;
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const float w = l[u] == -INFINITY ? 0.f : fast_exp2(l[u] - s.m);
      s.acc += v[u] * w;
      s.wsum += w;
    }
  }
  return s;
}

}  // namespace wmtp
