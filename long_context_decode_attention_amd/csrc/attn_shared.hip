// Split-KV attention for many query rows per kv head (the verify of n_q
// proposed positions: n_q * G rows), with every K/V tile shared by all rows.
//
// One workgroup (NW = 8 waves, two per SIMD so that one wave's LDS latency
// hides under the other's MFMAs) owns one key split of one (sequence, kv head)
// pair and up to 16 * RBW * NW query rows; wave w owns rows
// [16*RBW*NW*rg + 16*RBW*w, +16*RBW).
// The 32-key tiles of the split stream through a ring of LDS stages, filled
// by direct global-to-LDS loads (global_load_lds_dwordx4): each of the tile's
// 2*D/32 K operands and D/16 V^T operands is one 1 KB wave load that lands in
// LDS in exactly the lane order the MFMA reads it back, so the LDS reads are
// contiguous 16-byte-per-lane accesses.  Tiles t+1 .. t+kStages-1 are in
// flight while tile t is computed; one barrier per tile both publishes tile t
// and frees the stage the loads of tile t+kStages-1 overwrite.
//
// The per-wave math is the one of attn.hip (S^T and PV on MFMA 16x16x32, online
// softmax with P as bf16 hi + lo parts); a wave's rows never meet another
// wave's, so each wave writes its own rows' (o, lse).
#include "attn_device.h"

namespace wmtp {

namespace {

#ifndef WMTP_SHARED_STAGES
#define WMTP_SHARED_STAGES 4
#endif
constexpr int kStages = WMTP_SHARED_STAGES;   // LDS tile stages: kStages - 1 tiles in flight
static_assert(kStages >= 2 && kStages <= 4, "the vmcnt waits cover up to 3 tiles in flight");
constexpr int kPageRegs = 4;   // page ids preloaded per split: 64 per register

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

template <int D, int RBW, int NW>
__global__ __launch_bounds__(64 * NW, 1) void attn_shared_kernel(AttnArgs a) {
  constexpr int KS = D / 32;
  constexpr int DB = D / 16;
  constexpr int NOPS = 2 * KS + DB;      // 1 KB operands per tile
  constexpr int NL = NOPS / NW;          // wave loads per tile per wave
  constexpr int STAGE = NOPS * 1024;     // bytes per stage
  static_assert(NOPS % NW == 0, "operands split evenly over the waves");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int j = lane >> 4;

  int item, rg;
  if (a.nrg == 1) {
    item = blockIdx.x;
    rg = 0;
  } else {   // row groups of one item on one XCD, as in attn.hip
    const int w = blockIdx.x;
    const int k = w >> 3;
    rg = k % a.nrg;
    item = (k / a.nrg) * 8 + (w & 7);
  }
  if (item >= a.items) return;
  const int s = item % a.nsplit;
  const int bg = item / a.nsplit;
  const int g = bg % a.Hkv;
  const int b = bg / a.Hkv;
  const int row0 = (rg * NW + wave) * 16 * RBW;

  const int l_in = a.seq_lens[b];
  const int L = l_in < 0 ? 0 : (l_in > a.max_keys ? a.max_keys : l_in);
  const int nkb = (L + 31) >> 5;
  const int kb0 = s * a.kb_per_split;
  const int kb1 = min(kb0 + a.kb_per_split, nkb);
  const int ntile = kb1 > kb0 ? kb1 - kb0 : 0;

  // Q^T operands of this wave's rows.
  bf16x8 qop[RBW][KS];
  int lim[RBW];
  bool any_row = false;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int row = row0 + rb * 16 + n;
    if (row < a.R) {
      const int qi = row / a.G;
      const int hl = row - qi * a.G;
      const uint16_t* qp = a.q + ((size_t)(b * a.n_q + qi) * a.Hq + g * a.G + hl) * D + j * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[rb][ks] = ld_bf16x8(qp + ks * 32);
      lim[rb] = L - a.n_q + qi + 1;
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[rb][ks] = zero_bf16x8();
      lim[rb] = L;
    }
  }
  any_row = row0 < a.R;   // wave-uniform: does this wave own a real row?

  SoftmaxState<D, RBW> st;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    st.m[rb] = -INFINITY;
    st.l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) st.acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Page ids of this split (at most 256 pages): lane i of register r holds
  // logical page kb0/2 + 64*r + i, read once here so that no load other than
  // the tiles' is outstanding inside the pipeline.
  const int page0 = kb0 >> 1;
  const int last_page = ntile > 0 ? (kb1 - 1) >> 1 : -1;
  int my_page[kPageRegs];
#pragma unroll
  for (int r = 0; r < kPageRegs; ++r) {
    const int pg = page0 + 64 * r + lane;
    my_page[r] = pg <= last_page ? a.block_table[(size_t)b * a.max_pages + pg] : -1;
  }
  wait_vmcnt<0>();

  // Issue the NL wave loads of tile kb into stage `stage`.  A page id outside
  // the cache still issues its loads (from page 0) so that every tile costs the
  // same number of outstanding loads; the tile is then skipped.
  auto issue = [&](int kb, int stage) -> bool {
    const int idx = (kb >> 1) - page0;   // 0 .. 64*kPageRegs - 1, wave-uniform
    int ppage = -1;
#pragma unroll
    for (int r = 0; r < kPageRegs; ++r)
      if ((idx >> 6) == r) ppage = __builtin_amdgcn_readlane(my_page[r], idx & 63);
    const bool ok = (unsigned)ppage < (unsigned)a.num_pages;
    if (!ok) ppage = 0;
    const size_t tile = ((size_t)ppage * a.Hkv + g) * 2 + (kb & 1);
    const uint16_t* kt = a.kc + tile * (size_t)(32 * D);
    const uint16_t* vt = a.vc + tile * (size_t)(32 * D);
    unsigned char* base = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int op = wave + NW * i;
      const uint16_t* src;
      if (op < 2 * KS) {
        src = kt + k_operand_offset(op / KS, op % KS, n, j);
      } else {
        src = vt + v_operand_offset(op - 2 * KS, n, j);
      }
      // cache policy 2 = non-temporal (the tile is read from HBM once)
      __builtin_amdgcn_global_load_lds(
          (void*)src, (__attribute__((address_space(3))) void*)(base + op * 1024), 16, 0, 2);
    }
    return ok;
  };

  constexpr int AHEAD = kStages - 1;   // tiles in flight while one is computed
  bool ok_stage[kStages];
#pragma unroll
  for (int i = 0; i < kStages; ++i) ok_stage[i] = false;
#pragma unroll
  for (int i = 0; i < AHEAD; ++i)
    if (i < ntile) ok_stage[i] = issue(kb0 + i, i);

  for (int t = 0; t < ntile; ++t) {
    // Tile t has landed once at most (tiles issued after it) * NL loads remain.
    const int later = min(ntile - 1 - t, AHEAD - 1);
    if (later >= 3) {
      wait_vmcnt<3 * NL>();
    } else if (later == 2) {
      wait_vmcnt<2 * NL>();
    } else if (later == 1) {
      wait_vmcnt<NL>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    const int stage = t % kStages;
    if (t + AHEAD < ntile) ok_stage[(t + AHEAD) % kStages] = issue(kb0 + t + AHEAD, (t + AHEAD) % kStages);
    if (!ok_stage[stage] || !any_row) continue;

    const int kb = kb0 + t;
    const int kbase = kb * 32 + 8 * j;
    const int rem = L - kbase;
    const uint32_t keep = rem >= 8 ? 0xFFu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
    const unsigned char* base = smem + stage * STAGE + lane * 16;

    f32x4 sacc[RBW][2];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      sacc[rb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      sacc[rb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bf16x8 kop[2][KS];     // all K operands first: one LDS latency, then the MFMAs
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kop[0][ks] = *reinterpret_cast<const bf16x8*>(base + (0 * KS + ks) * 1024);
      kop[1][ks] = *reinterpret_cast<const bf16x8*>(base + (1 * KS + ks) * 1024);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        sacc[rb][0] = mfma16x16x32(kop[0][ks], qop[rb][ks], sacc[rb][0]);
        sacc[rb][1] = mfma16x16x32(kop[1][ks], qop[rb][ks], sacc[rb][1]);
      }
    }
    bf16x8 p_hi[RBW], p_lo[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
      softmax_update<D, RBW>(st, rb, sacc[rb][0], sacc[rb][1], keep, lim[rb] - kbase,
                             a.scale_log2, p_hi[rb], p_lo[rb]);
    const bool all_keep = __all(keep == 0xFFu);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(base + (2 * KS + db) * 1024);
      if (!all_keep) v = mask_bf16x8(v, keep);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) {
        st.acc[rb][db] = mfma16x16x32(v, p_hi[rb], st.acc[rb][db]);
        st.acc[rb][db] = mfma16x16x32(v, p_lo[rb], st.acc[rb][db]);
      }
    }
  }

  // Each wave writes its own rows.
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int row = row0 + rb * 16 + n;
    const float Ltot = sum_over_lane_groups(st.l[rb]);
    if (row >= a.R) continue;
    const float inv = Ltot > 0.f ? 1.f / Ltot : 0.f;
    float* op;
    float* lp;
    if (a.direct) {
      const int qi = row / a.G;
      const int hl = row - qi * a.G;
      const size_t oidx = (size_t)(b * a.n_q + qi) * a.Hq + g * a.G + hl;
      op = a.out_o + oidx * D;
      lp = a.out_lse ? a.out_lse + oidx : nullptr;
    } else {
      op = a.out_o + ((size_t)item * a.R + row) * D;
      lp = a.out_lse + (size_t)item * a.R + row;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<f32x4*>(op + db * 16 + 4 * j) = st.acc[rb][db] * inv;
    if (j == 0 && lp) *lp = Ltot > 0.f ? (st.m[rb] + fast_log2(Ltot)) * kLn2 : -INFINITY;
  }
}

constexpr int kWaves = 8;

template <int D, int RBW>
hipError_t launch_shared_one(const AttnArgs& a, int grid, hipStream_t stream) {
  AttnArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_shared_kernel<D, RBW, kWaves>),
                         dim3(grid), dim3(64 * kWaves), args, 0, stream);
}

}  // namespace

int shared_kernel_waves() { return kWaves; }
int shared_kernel_max_tiles() { return 2 * 64 * kPageRegs; }

hipError_t launch_attention_shared(const AttnArgs& a, const AttnPlan& p, hipStream_t stream) {
  switch (a.D) {
    case 64:
      return p.nrb == 1 ? launch_shared_one<64, 1>(a, p.grid, stream)
                        : launch_shared_one<64, 2>(a, p.grid, stream);
    case 128:
      return p.nrb == 1 ? launch_shared_one<128, 1>(a, p.grid, stream)
                        : launch_shared_one<128, 2>(a, p.grid, stream);
    case 256:
      return p.nrb == 1 ? launch_shared_one<256, 1>(a, p.grid, stream) : hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace wmtp
