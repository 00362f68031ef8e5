// Split-KV attention for many query rows per kv head (the verify of n_q
// proposed positions: n_q * G rows), with every K/V tile shared by all rows.
//
// One workgroup (NW = 4 waves, one per SIMD, each with the whole register file)
// owns one key split of one (sequence, kv head) pair and up to 32 * RBW * NW
// query rows; wave w owns rows [32*RBW*NW*rg + 32*RBW*w, +32*RBW), so every K/V
// operand read from LDS feeds RBW row blocks.
//
// The 32-key tiles of the split stream through a ring of 4 LDS stages, filled by
// direct global-to-LDS loads (global_load_lds_dwordx4, non-temporal): each of the
// tile's D/16 K operands and D/16 V^T operands is one 1 KB wave load that lands
// in LDS in exactly the lane order the MFMA reads it back.
//
// The loop is software-pipelined across tiles.  Iteration t issues the S^T
// products of tile t+1 first; they run on the matrix cores while the VALU does
// the softmax of tile t, whose PV products follow.  Tiles t and t+1 are resident
// in LDS while tiles t+2 and t+3 are in flight; one barrier per iteration both
// publishes tile t+1 and frees the stage of tile t-1, which the loads of tile
// t+3 overwrite.
//
// The per-tile math is the one of attn.hip (MFMA 32x32x16, online softmax with
// P as bf16 hi + lo parts); a wave's rows never meet another wave's, so each
// wave writes its own rows' (o, lse).
#include "attn_device.h"

namespace wmtp {

namespace {

constexpr int kStages = 4;      // LDS tile stages: tiles t, t+1 resident, t+2, t+3 in flight
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

// Compiler-level fence for memory operations: LDS reads after it are not hoisted
// above it, which bounds how many operand registers are live at once.
__device__ __forceinline__ void operand_fence() { asm volatile("" ::: "memory"); }

// S^T of one tile for this wave's RBW row blocks: K operands read from the LDS
// stage at `base` (offset by lane * 16) in two halves.  The MFMAs are only
// issued here; their results are used one iteration later.
template <int D, int RBW>
__device__ __forceinline__ void s_tile(f32x16 (&sacc)[RBW], const bf16x8 (&qop)[RBW][D / 16],
                                       const unsigned char* base) {
  constexpr int KS = D / 16;
  constexpr int KH = KS / 2;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) sacc[rb] = f32x16{};
#pragma unroll
  for (int k0 = 0; k0 < KS; k0 += KH) {
    bf16x8 kop[KH];
#pragma unroll
    for (int ks = 0; ks < KH; ++ks)
      kop[ks] = *reinterpret_cast<const bf16x8*>(base + (k0 + ks) * 1024);
#pragma unroll
    for (int ks = 0; ks < KH; ++ks)
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) sacc[rb] = mfma32x32x16(kop[ks], qop[rb][k0 + ks], sacc[rb]);
    operand_fence();
  }
}

// Weights and PV of one tile from its masked scores x; V^T operands from the LDS
// stage at `base`, in two halves.  mask_v (wave-uniform): some key of the tile
// is past the sequence length, and its values, which may hold any bits (even
// NaN), are zeroed so that 0-weight * value stays 0 in the PV product.
template <int D, int RBW>
__device__ __forceinline__ void pv_tile(SoftmaxState<D, RBW>& st, const float (&x)[RBW][16],
                                        float c, const unsigned char* base, uint32_t keep,
                                        bool mask_v) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int DH = DB > 1 ? DB / 2 : 1;
  bf16x8 p_hi[RBW][2], p_lo[RBW][2];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) weights<D, RBW>(st, rb, x[rb], c, p_hi[rb], p_lo[rb]);
#pragma unroll
  for (int d0 = 0; d0 < DB; d0 += DH) {
    bf16x8 vop[DH][2];
#pragma unroll
    for (int db = 0; db < DH; ++db)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        vop[db][kk] = *reinterpret_cast<const bf16x8*>(base + (KS + 2 * (d0 + db) + kk) * 1024);
    if (mask_v) {
#pragma unroll
      for (int db = 0; db < DH; ++db)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) vop[db][kk] = mask8(vop[db][kk], (keep >> (8 * kk)) & 0xFFu);
    }
    // the hi products of the half's accumulators, then the lo products, so that no
    // MFMA waits on the one just before it
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int db = 0; db < DH; ++db)
          st.acc[rb][d0 + db] = mfma32x32x16(vop[db][kk], p_hi[rb][kk], st.acc[rb][d0 + db]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int db = 0; db < DH; ++db)
          st.acc[rb][d0 + db] = mfma32x32x16(vop[db][kk], p_lo[rb][kk], st.acc[rb][d0 + db]);
    operand_fence();
  }
}

template <int D, int RBW, int NW>
__global__ __launch_bounds__(64 * NW, 1) void attn_shared_kernel(AttnArgs a) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NOPS = 2 * KS;           // 1 KB operands per tile: D/16 of K, D/16 of V^T
  constexpr int NL = NOPS / NW;          // wave loads per tile per wave
  constexpr int STAGE = NOPS * 1024;     // bytes per stage
  static_assert(NOPS % NW == 0, "operands split evenly over the waves");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 31;
  const int h = lane >> 5;

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
  const int row0 = (rg * NW + wave) * 32 * RBW;

  const int l_in = a.seq_lens[b];
  const int L = l_in < 0 ? 0 : (l_in > a.max_keys ? a.max_keys : l_in);
  const int nkb = (L + 31) >> 5;
  const int kb0 = s * a.kb_per_split;
  const int kb1 = min(kb0 + a.kb_per_split, nkb);
  const int ntile = kb1 > kb0 ? kb1 - kb0 : 0;

  // Q^T operands of this wave's rows: lane (m, h) holds row row0 + 32*rb + m,
  // dims 16*ks + 8*h .. +7.
  bf16x8 qop[RBW][KS];
  int lim[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int row = row0 + rb * 32 + m;
    if (row < a.R) {
      const int qi = row / a.G;
      const int hl = row - qi * a.G;
      const uint16_t* qp = a.q + ((size_t)(b * a.n_q + qi) * a.Hq + g * a.G + hl) * D + h * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[rb][ks] = ld_bf16x8(qp + ks * 16);
      lim[rb] = L - a.n_q + qi + 1;
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[rb][ks] = zero_bf16x8();
      lim[rb] = L;
    }
  }
  const bool any_row = row0 < a.R;   // wave-uniform: does this wave own a real row?
  // Q^T is only an MFMA operand: park it in the accumulation registers.
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(qop[rb][ks]));

  SoftmaxState<D, RBW> st;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    st.m[rb] = -INFINITY;
    st.l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) st.acc[rb][db] = f32x16{};
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
      if (op < KS) {
        src = kt + k_operand_offset(op, m, h);
      } else {
        const int vo = op - KS;
        src = vt + v_operand_offset<D>(vo >> 1, vo & 1, m, h);
      }
      // cache policy 2 = non-temporal (the tile is read from HBM once)
      __builtin_amdgcn_global_load_lds(
          (void*)src, (__attribute__((address_space(3))) void*)(base + op * 1024), 16, 0, 2);
    }
    return ok;
  };

  // Pipeline: issue tiles 0..2, publish tile 0, issue S(0); step t then publishes
  // tile t+1, issues tile t+3, issues S(t+1) and finishes tile t.
  uint32_t ok_stage = 0;               // bit s: the tile in stage s has a valid page
#pragma unroll
  for (int i = 0; i < 3; ++i)
    if (i < ntile && issue(kb0 + i, i)) ok_stage |= 1u << i;
  f32x16 s_cur[RBW], s_next[RBW];
  if (ntile > 0) {
    if (ntile >= 3) {
      wait_vmcnt<2 * NL>();
    } else if (ntile == 2) {
      wait_vmcnt<NL>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    if (any_row) s_tile<D, RBW>(s_cur, qop, smem + lane * 16);
  }

  // Publish tile t+1, refill the stage of tile t-1 with tile t+3, issue S(t+1).
  auto advance = [&](int t) {
    // Tile t+1 has landed once only the loads of tile t+2 (if issued) remain.
    if (t + 2 < ntile) {
      wait_vmcnt<NL>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    if (t + 3 < ntile) {
      const int st3 = (t + 3) % kStages;
      ok_stage = (ok_stage & ~(1u << st3)) | ((issue(kb0 + t + 3, st3) ? 1u : 0u) << st3);
    }
    if (any_row && t + 1 < ntile)
      s_tile<D, RBW>(s_next, qop, smem + ((t + 1) % kStages) * STAGE + lane * 16);
  };

  // Masked scores of tile t (from s_cur) and the facts its PV needs.
  float x[RBW][16], mx[RBW];
  uint32_t keep = 0;
  bool mask_v = false;
  auto scores_of = [&](int t) {
    const int kb = kb0 + t;
    // every key of the tile is present and visible to every row (the smallest
    // causal limit of any row is L - n_q + 1)
    const bool all_vis = (kb + 1) * 32 <= L - a.n_q + 1;
    keep = keys_below(L - kb * 32, h);
    mask_v = (kb + 1) * 32 > L;
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
      mx[rb] = masked_scores(x[rb], s_cur[rb], keys_below(lim[rb] - kb * 32, h), all_vis,
                             a.scale_log2);
  };
  auto tile_ok = [&](int t) { return any_row && ((ok_stage >> (t % kStages)) & 1u); };
  auto stage_base = [&](int t) { return smem + (t % kStages) * STAGE + lane * 16; };

  // Fast loop: no accumulator rescale.  Leaves with t < ntile when tile t needs
  // one; its scores are then already in x / mx.
  int t = 0;
  for (; t < ntile; ++t) {
    advance(t);
    if (tile_ok(t)) {
      scores_of(t);
      if (first_max_or_rescale<D, RBW>(st, mx)) break;
      pv_tile<D, RBW>(st, x, a.scale_log2, stage_base(t), keep, mask_v);
    }
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) s_cur[rb] = s_next[rb];
  }
  // General loop, from the tile the fast loop left on.
  if (t < ntile) {
    raise_and_rescale<D, RBW>(st, mx);
    pv_tile<D, RBW>(st, x, a.scale_log2, stage_base(t), keep, mask_v);
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) s_cur[rb] = s_next[rb];
    for (++t; t < ntile; ++t) {
      advance(t);
      if (tile_ok(t)) {
        scores_of(t);
        raise_and_rescale<D, RBW>(st, mx);
        pv_tile<D, RBW>(st, x, a.scale_log2, stage_base(t), keep, mask_v);
      }
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) s_cur[rb] = s_next[rb];
    }
  }

  // Each wave writes its own rows.
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int row = row0 + rb * 32 + m;
    const float Ltot = sum_over_row(st.l[rb]);
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
    write_row<D, RBW>(op, st, rb, inv, h);
    if (h == 0 && lp) *lp = Ltot > 0.f ? (st.m[rb] + fast_log2(Ltot)) * kLn2 : -INFINITY;
  }
}

constexpr int kWaves = 4;

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
