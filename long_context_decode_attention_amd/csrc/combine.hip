// Log-sum-exp merge of per-split attention results:
//     lse = ln sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) * o_s
//
// Two mappings of a workgroup's 256 threads onto (split lanes) x (column chunks
// of a float4 each), chosen per shape by the host:
//  * few rows (R < 64): SL split lanes of a chunk adjacent in one wave, summed by
//    a butterfly of lane shuffles; SL is the smallest power of two covering the
//    split count (at most 64), so small merges leave no lane idle.
//  * many rows: CL column lanes adjacent (a contiguous 16 * CL-byte piece of a
//    partial row per load) and the split lanes in different waves, summed
//    through LDS; CL is the widest that still gives about 512 workgroups.  The
//    partials of a many-row verify are tens of MB: coalescing decides there.
// Either way split lane sl visits splits sl, sl + SL, ... in one pass, with
// eight independent (o_s, lse_s) loads in flight and a running maximum (one
// memory round trip when a lane has at most eight splits), and the sums run in
// a fixed order, so the result does not depend on timing.
#include "common.h"
#include "internal.h"
#include "merge_device.h"
#include "ring_device.h"

#include <cmath>

namespace wmtp {

namespace {

constexpr float kLn2 = 0.693147180559945309f;

template <int SL>
__device__ __forceinline__ float max_over_split_lanes(float v) {
#pragma unroll
  for (int o = 1; o < SL; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <int SL>
__device__ __forceinline__ float sum_over_split_lanes(float v) {
#pragma unroll
  for (int o = 1; o < SL; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// Many rows: CL column lanes adjacent, SL = 256 / CL split lanes in LDS.
__global__ __launch_bounds__(256) void combine_wide_kernel(CombineArgs c, int CL) {
  const int SL = 256 / CL;
  const int t = threadIdx.x;
  const int cl = t % CL;
  const int sl = t / CL;
  const int nchunk = c.D / (4 * CL);
  if (c.append) {
    // fused draft step: the workgroups after the combine's append to the rings
    const int merge_blocks = c.B * c.Hkv * c.R * nchunk;
    if ((int)blockIdx.x >= merge_blocks) {
      ring_append_block(c.app, blockIdx.x - merge_blocks);
      return;
    }
  }
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

  LaneMerge st = merge_lane(c.part_o + (size_t)row * c.D + col, c.part_lse, (size_t)c.R * c.D,
                            c.R, row, p0, p1, sl, SL);
  // the row's maximum M over all the threads, then each thread's state brought to it
  float mx = st.m;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float f = st.m == -INFINITY ? 0.f : fast_exp2(st.m - M);
  const f32x4 acc = st.acc * f;
  const float wsum = st.wsum * f;
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
    if (chunk == 0 && cl == 0 && c.lse) c.lse[oidx] = wt > 0.f ? (M + fast_log2(wt)) * kLn2 : -INFINITY;
  }
}

// Few rows: SL split lanes adjacent in a wave.
template <int SL>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs c) {
  constexpr int CL = 256 / SL;
  const int t = threadIdx.x;
  const int sl = t % SL;
  const int cl = t / SL;
  const int nblk = c.D / (4 * CL);            // column-chunk blocks per row
  if (c.append) {
    // fused draft step: the workgroups after the combine's append to the rings
    const int merge_blocks = c.B * c.Hkv * c.R * nblk;
    if ((int)blockIdx.x >= merge_blocks) {
      ring_append_block(c.app, blockIdx.x - merge_blocks);
      return;
    }
  }
  const int blk = blockIdx.x % nblk;
  const int rest = blockIdx.x / nblk;
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
  const int col = (blk * CL + cl) * 4;

  LaneMerge st = merge_lane(c.part_o + (size_t)row * c.D + col, c.part_lse, (size_t)c.R * c.D,
                            c.R, row, p0, p1, sl, SL);
  // bring the lanes to the row's maximum M, then sum them
  const float M = max_over_split_lanes<SL>(st.m);
  const float f = st.m == -INFINITY ? 0.f : fast_exp2(st.m - M);
  f32x4 acc = st.acc * f;
  float wsum = st.wsum * f;
  acc.x = sum_over_split_lanes<SL>(acc.x);
  acc.y = sum_over_split_lanes<SL>(acc.y);
  acc.z = sum_over_split_lanes<SL>(acc.z);
  acc.w = sum_over_split_lanes<SL>(acc.w);
  wsum = sum_over_split_lanes<SL>(wsum);
  if (sl == 0) {
    const int qi = row / c.G;
    const int hl = row - qi * c.G;
    const int b = grp / c.Hkv;
    const int g = grp - b * c.Hkv;
    const size_t oidx = (size_t)(b * c.n_q + qi) * (c.Hkv * c.G) + g * c.G + hl;
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    *reinterpret_cast<f32x4*>(c.o + oidx * c.D + col) = acc * inv;
    if (col == 0 && c.lse) c.lse[oidx] = wsum > 0.f ? (M + fast_log2(wsum)) * kLn2 : -INFINITY;
  }
}

template <int SL>
hipError_t launch_sl(const CombineArgs& c, hipStream_t stream) {
  constexpr int CL = 256 / SL;
  CombineArgs arg = c;
  void* args[] = {&arg};
  const long grid = (long)c.B * c.Hkv * c.R * (c.D / (4 * CL)) + (c.append ? c.app.B : 0);
  return hipLaunchKernel(reinterpret_cast<const void*>(&combine_kernel<SL>), dim3((unsigned)grid),
                         dim3(256), args, 0, stream);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& c, hipStream_t stream) {
  if (c.R >= 64) {
    // CL: a power of two dividing D / 4, the widest that gives about 512 workgroups
    // and enough split lanes (256 / CL) that each lane loads its splits in one
    // batch of kMergeUnroll (one memory round trip instead of several).
    const long pairs = (long)c.B * c.Hkv * c.R;
    const int splits = c.indptr ? 64 : c.splits_per_group;
    int CL = 4;
    while (CL < 64 && (c.D / 4) % (2 * CL) == 0) CL *= 2;
    while (CL > 4 && pairs * (c.D / (4 * CL)) < 512) CL /= 2;
    while (CL > 4 && (256 / CL) * kMergeUnroll < splits) CL /= 2;
    CombineArgs arg = c;
    int cl_arg = CL;
    void* args[] = {&arg, &cl_arg};
    const long grid = pairs * (c.D / (4 * CL)) + (c.append ? c.app.B : 0);
    return hipLaunchKernel(reinterpret_cast<const void*>(&combine_wide_kernel), dim3((unsigned)grid),
                           dim3(256), args, 0, stream);
  }
  // Split lanes: the smallest power of two covering the splits of a group (all 64
  // with a CSR split list, whose counts the host does not see), and no fewer
  // than make the column lanes 256 / sl a divisor of D / 4, so that a row's column
  // blocks cover it exactly (D is a multiple of 16: sl = 64 gives 4 column lanes,
  // which always divide D / 4).
  int splits = c.indptr ? 64 : c.splits_per_group;
  int sl = 1;
  while (sl < splits && sl < 64) sl *= 2;
  while (sl < 64 && (256 / sl > c.D / 4 || (c.D / 4) % (256 / sl) != 0)) sl *= 2;
  switch (sl) {
    case 1: return launch_sl<1>(c, stream);
    case 2: return launch_sl<2>(c, stream);
    case 4: return launch_sl<4>(c, stream);
    case 8: return launch_sl<8>(c, stream);
    case 16: return launch_sl<16>(c, stream);
    case 32: return launch_sl<32>(c, stream);
    default: return launch_sl<64>(c, stream);
  }
}

}  // namespace wmtp
