// Log-sum-exp merge of per-split attention results:
//     lse = ln sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) * o_s
//
// One workgroup per (group, query row, column chunk): 256 threads = SL split
// lanes x CL column lanes (a float4 each), SL * CL = 256.  The host picks CL
// per shape: wide chunks (contiguous 1 KB reads of a partial row) when there are
// many rows, narrow ones when there are few, so that the grid fills the chip.
// Split lane sl visits splits sl, sl + SL, ... with eight independent 16-byte
// loads in flight; the split lanes are then summed through LDS in a fixed
// order, so the result does not depend on timing.
#include "common.h"
#include "internal.h"

#include <cmath>

namespace wmtp {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs c, int CL) {
  const int SL = 256 / CL;
  const int t = threadIdx.x;
  const int cl = t % CL;
  const int sl = t / CL;
  const int nchunk = c.D / (4 * CL);
  const int chunk = blockIdx.x % nchunk;
  const int rest = blockIdx.x / nchunk;
  const int row = rest % c.R;
  const int grp = rest / c.R;
  int p0, p1;
  if (c.indptr) {
    p0 = min(max(c.indptr[grp], 0), c.n_parts);
    p1 = min(max(c.indptr[grp + 1], p0), c.n_parts);
  } else {
    p0 = grp * c.splits_per_group;
    p1 = p0 + c.splits_per_group;
  }
  const int col = chunk * 4 * CL + cl * 4;

  __shared__ float red[4];
  __shared__ f32x4 sm_acc[256];
  __shared__ float sm_w[256];

  // pass 1: the largest split lse of this row
  float mx = -INFINITY;
  for (int p = p0 + t; p < p1; p += 256) mx = fmaxf(mx, c.part_lse[(size_t)p * c.R + row]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float Mu = (M == -INFINITY) ? 0.f : M;

  // pass 2: this lane's share of sum_s w_s * o_s and sum_s w_s
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  const size_t stride = (size_t)c.R * c.D;
  const float* base = c.part_o + (size_t)row * c.D + col;
  for (int p = p0 + sl; p < p1; p += SL * kUnroll) {
    f32x4 v[kUnroll];
    float w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int q = p + u * SL;
      if (q < p1) {
        v[u] = *reinterpret_cast<const f32x4*>(base + (size_t)q * stride);
        const float l = c.part_lse[(size_t)q * c.R + row];
        w[u] = (l == -INFINITY) ? 0.f : fast_exp2((l - Mu) * kLog2e);
      } else {
        v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        w[u] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      acc += v[u] * w[u];
      wsum += w[u];
    }
  }
  sm_acc[t] = acc;
  sm_w[t] = wsum;
  __syncthreads();
  if (sl == 0) {
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
    float wt = 0.f;
    for (int i = 0; i < SL; ++i) {
      tot += sm_acc[i * CL + cl];
      wt += sm_w[i * CL + cl];
    }
    const int qi = row / c.G;
    const int hl = row - qi * c.G;
    const int b = grp / c.Hkv;
    const int g = grp - b * c.Hkv;
    const size_t oidx = (size_t)(b * c.n_q + qi) * (c.Hkv * c.G) + g * c.G + hl;
    const float inv = wt > 0.f ? 1.f / wt : 0.f;
    *reinterpret_cast<f32x4*>(c.o + oidx * c.D + col) = tot * inv;
    if (chunk == 0 && cl == 0 && c.lse)
      c.lse[oidx] = wt > 0.f ? M + fast_log2(wt) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& c, hipStream_t stream) {
  CombineArgs arg = c;
  // Widest column chunk that still gives about 512 workgroups; at least 16 columns.
  const long pairs = (long)c.B * c.Hkv * c.R;
  // CL: a power of two (so that 256 / CL split lanes is whole) dividing D / 4.
  int CL = 4;
  while (CL < 64 && (c.D / 4) % (2 * CL) == 0) CL *= 2;
  while (CL > 4 && pairs * (c.D / (4 * CL)) < 512) CL /= 2;
  int cl_arg = CL;
  void* args[] = {&arg, &cl_arg};
  const long grid = pairs * (c.D / (4 * CL));
  return hipLaunchKernel(reinterpret_cast<const void*>(&combine_kernel), dim3((unsigned)grid),
                         dim3(256), args, 0, stream);
}

}  // namespace wmtp
