// Writers of the tiled page layout: the draft ring append and the paged append.
//
// Tiled pages: tile t = (page * Hkv + g) * 2 + (pos % 64) / 32 holds 32 * D
// elements; with tok = pos % 32, K tile element (tok, d) at (d / 16) * 512 +
// tok * 16 + d % 16, V tile element (tok, d) at (tok / 16) * 16 * D + d * 16 +
// tok % 16 (the 1 KB MFMA operand blocks the attention kernels read).
#include "common.h"
#include "internal.h"
#include "ring_device.h"

namespace wmtp {

namespace {

// fp8 e4m3 form of 8 bf16 values: code(clamp(x * inv, +-448)), round to nearest
// even (the conversion instruction's rounding); byte j holds element j.
__device__ __forceinline__ u32x2 bf16x8_to_fp8(const uint16_t* src, float inv) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(src);
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16) * inv;
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u) * inv;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = fminf(fmaxf(f[i], -448.f), 448.f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
  return u32x2{(uint32_t)lo, (uint32_t)hi};
}

// The same store as store_kv8 into fp8 tiles (one byte per element, the bf16
// tiles' element order).
__device__ __forceinline__ void store_kv8_fp8(uint8_t* kc, uint8_t* vc, size_t tile, int tok,
                                              int d0, int D, const uint16_t* ksrc,
                                              const uint16_t* vsrc, float k_inv, float v_inv) {
  const u32x2 kq = bf16x8_to_fp8(ksrc, k_inv);
  const u32x2 vq = bf16x8_to_fp8(vsrc, v_inv);
  uint8_t* kt = kc + tile * (size_t)(32 * D);
  uint8_t* vt = vc + tile * (size_t)(32 * D);
  *reinterpret_cast<u32x2*>(kt + (d0 >> 4) * 512 + tok * 16 + (d0 & 15)) = kq;
  uint8_t* vp = vt + (tok >> 4) * (16 * D) + (tok & 15);
#pragma unroll
  for (int i = 0; i < 8; ++i) vp[(d0 + i) * 16] = (uint8_t)(vq[i >> 2] >> (8 * (i & 3)));
}

// Appends of a few positions (the decode steps): one workgroup per request;
// every thread reads the old count before thread 0 stores the new one.
__global__ __launch_bounds__(256) void ring_append_kernel(RingAppendArgs a) {
  ring_append_block(a, blockIdx.x);
}

// Bulk fills (a prefill or a resume): the survivors' pieces spread over
// gridDim.x workgroups per request; the count is advanced afterwards by
// ring_count_kernel, launched next on the same stream, so that no workgroup
// can read a count another has already advanced.
__global__ __launch_bounds__(256) void ring_fill_kernel(RingAppendArgs a) {
  const int b = blockIdx.y;
  int64_t T0 = a.ring_T[b];
  if (T0 < 0) T0 = 0;
  ring_write(a, b, T0, blockIdx.x * 256 + threadIdx.x, gridDim.x * 256);
}

__global__ __launch_bounds__(256) void ring_count_kernel(int64_t* ring_T, int B, int n_new) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  int64_t T0 = ring_T[b];
  if (T0 < 0) T0 = 0;
  ring_T[b] = T0 + n_new;
}

__global__ __launch_bounds__(256) void paged_append_kernel(PagedAppendArgs a) {
  const int b = blockIdx.y;
  const int chunks = a.Hkv * (a.D >> 3);
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)a.n_new * chunks) return;
  const int t_in = (int)(idx / chunks);
  const int c = (int)(idx - (long)t_in * chunks);
  const long pos = (long)a.start_pos[b] + t_in;
  if (pos < 0) return;
  const long lpage = pos >> 6;
  if (lpage >= a.max_pages) return;
  const int ppage = a.block_table[(size_t)b * a.max_pages + lpage];
  if ((unsigned)ppage >= (unsigned)a.num_pages) return;
  const int g = c / (a.D >> 3);
  const int d0 = (c - g * (a.D >> 3)) * 8;
  const size_t src = (((size_t)b * a.n_new + t_in) * a.Hkv + g) * a.D + d0;
  const int off = (int)(pos & 63);
  const size_t tile = ((size_t)ppage * a.Hkv + g) * 2 + (off >> 5);
  if (a.kv8)
    store_kv8_fp8(reinterpret_cast<uint8_t*>(a.kc), reinterpret_cast<uint8_t*>(a.vc), tile,
                  off & 31, d0, a.D, a.k_new + src, a.v_new + src, a.k_inv, a.v_inv);
  else
    store_kv8(a.kc, a.vc, tile, off & 31, d0, a.D, a.k_new + src, a.v_new + src);
}

// Appends longer than this take the multi-workgroup fill.
constexpr int kRingBulkFrom = 64;

}  // namespace

hipError_t launch_ring_append(const RingAppendArgs& a, hipStream_t stream) {
  RingAppendArgs arg = a;
  void* args[] = {&arg};
  if (a.n_new <= kRingBulkFrom) {
    return hipLaunchKernel(reinterpret_cast<const void*>(&ring_append_kernel), dim3(a.B),
                           dim3(256), args, 0, stream);
  }
  // at most C survivors per request, 8 pieces per thread
  const long pieces = (long)(a.n_new < a.C ? a.n_new : a.C) * a.Hkv * (a.D >> 3);
  long gx = (pieces + 2047) / 2048;
  if (gx > 1024) gx = 1024;
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&ring_fill_kernel),
                                 dim3((unsigned)gx, a.B), dim3(256), args, 0, stream);
  if (e != hipSuccess) return e;
  int64_t* ring_T = a.ring_T;
  int B = a.B, n_new = a.n_new;
  void* cargs[] = {&ring_T, &B, &n_new};
  return hipLaunchKernel(reinterpret_cast<const void*>(&ring_count_kernel), dim3((B + 255) / 256),
                         dim3(256), cargs, 0, stream);
}

hipError_t launch_paged_append(const PagedAppendArgs& a, hipStream_t stream) {
  PagedAppendArgs arg = a;
  void* args[] = {&arg};
  const long work = (long)a.n_new * a.Hkv * (a.D >> 3);
  const unsigned gx = (unsigned)((work + 255) / 256);
  return hipLaunchKernel(reinterpret_cast<const void*>(&paged_append_kernel), dim3(gx, a.B),
                         dim3(256), args, 0, stream);
}

}  // namespace wmtp
