// Log-sum-exp merge of per-split attention results:
//     lse = ln sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) * o_s
// One workgroup per (group, query row); thread t owns output column d = t.
// Partials are read in split order, so the result does not depend on timing.
#include "common.h"
#include "internal.h"

#include <cmath>

namespace wmtp {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kChunk = 1024;   // split weights staged in LDS per pass

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs c) {
  const int t = threadIdx.x;
  const int row = blockIdx.x % c.R;
  const int grp = blockIdx.x / c.R;
  int p0, p1;
  if (c.indptr) {
    p0 = min(max(c.indptr[grp], 0), c.n_parts);
    p1 = min(max(c.indptr[grp + 1], p0), c.n_parts);
  } else {
    p0 = grp * c.splits_per_group;
    p1 = p0 + c.splits_per_group;
  }

  __shared__ float red[4];
  __shared__ float w_sm[kChunk];

  // pass 1: the largest split lse of this row
  float mx = -INFINITY;
  for (int p = p0 + t; p < p1; p += 256) mx = fmaxf(mx, c.part_lse[(size_t)p * c.R + row]);
  mx = fmaxf(mx, __shfl_xor(mx, 1));
  mx = fmaxf(mx, __shfl_xor(mx, 2));
  mx = fmaxf(mx, __shfl_xor(mx, 4));
  mx = fmaxf(mx, __shfl_xor(mx, 8));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float Mu = (M == -INFINITY) ? 0.f : M;

  // pass 2: weights exp(lse_s - M), their sum, and the weighted column sum
  float acc = 0.f;
  float wsum = 0.f;
  for (int base = p0; base < p1; base += kChunk) {
    const int cnt = min(kChunk, p1 - base);
    __syncthreads();
    for (int q = t; q < cnt; q += 256) {
      const float l = c.part_lse[(size_t)(base + q) * c.R + row];
      w_sm[q] = (l == -INFINITY) ? 0.f : fast_exp2((l - Mu) * kLog2e);
    }
    __syncthreads();
    for (int q = 0; q < cnt; ++q) wsum += w_sm[q];
    if (t < c.D) {
      const float* src = c.part_o + ((size_t)base * c.R + row) * c.D + t;
      const size_t stride = (size_t)c.R * c.D;
      for (int q = 0; q < cnt; ++q) acc += w_sm[q] * src[(size_t)q * stride];
    }
  }

  const int qi = row / c.G;
  const int hl = row - qi * c.G;
  const int b = grp / c.Hkv;
  const int g = grp - b * c.Hkv;
  const size_t oidx = (size_t)(b * c.n_q + qi) * (c.Hkv * c.G) + g * c.G + hl;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (t < c.D) c.o[oidx * c.D + t] = acc * inv;
  if (t == 0 && c.lse) c.lse[oidx] = wsum > 0.f ? M + fast_log2(wsum) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& c, hipStream_t stream) {
  CombineArgs arg = c;
  void* args[] = {&arg};
  const int grid = c.B * c.Hkv * c.R;
  return hipLaunchKernel(reinterpret_cast<const void*>(&combine_kernel), dim3(grid), dim3(256),
                         args, 0, stream);
}

}  // namespace wmtp
