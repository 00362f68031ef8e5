// Split-KV decode attention for gfx950: the native draft (every cached key),
// the windowed draft (the valid slots of a sink-plus-recent ring) and the
// causal verify of n_q proposed positions share this kernel.
//
// Work decomposition.  One workgroup (4 waves) owns one key split of one
// (sequence b, kv head g) pair and a group of up to 16 * NRB query rows of that
// kv head (the G query heads of the group, times n_q verify queries).  The
// split is a run of 32-key tiles; wave w of the workgroup takes tiles
// w, w + 4, w + 8, ... so the four waves stream neighbouring memory.  Each wave
// keeps its own online-softmax state; the four are merged through LDS at the
// end and the workgroup writes one partial (o, lse) per row, or the final
// result when the sequence has a single split.
//
// Per 32-key tile a wave computes, with bf16 MFMA 16x16x32 and fp32 accumulation,
//     S^T[key][row] = K[key][:] . Q[row][:]          (2 key blocks x D/32 steps)
//     O^T[d][row]  += V^T[d][key] . P^T[key][row]    (D/16 blocks, 2 steps:
//                                                     P as bf16 hi + lo parts)
// Keys sit on the MFMA M axis of S^T, so the S^T accumulator a lane receives
// (column = its query row, rows 4*(lane/16)+i) holds exactly the 8 keys that
// the same lane must feed as the contraction slice of P^T for the PV product;
// the key order inside the first product is chosen so that these are keys
// 8*(lane/16) .. +7.  No value crosses lanes between the two products except
// the row maximum, reduced over the four lane groups.
//
// Operand loads are 16 bytes per lane straight from the tiled page layout:
// a K operand fetches 16 rows of 64 contiguous bytes (a 2 KB dim-tile per key
// block pair), a V operand 1 KB contiguous.  Each wave double-buffers its tiles
// in registers: the loads of tile t+4 are in flight while tile t is computed.
#include "attn_device.h"

// Workgroups the split planner aims at: two per CU for the split-keys kernel
// (one resident at a time), one per CU for the shared kernel.
#ifndef WMTP_TARGET_WG_SPLIT
#define WMTP_TARGET_WG_SPLIT 512
#endif
#ifndef WMTP_TARGET_WG_SHARED
#define WMTP_TARGET_WG_SHARED 256
#endif

namespace wmtp {

namespace {

template <int D, int NRB, bool RING>
__global__ __launch_bounds__(256, 1) void attn_split_kernel(AttnArgs a) {
  constexpr int KS = D / 32;
  constexpr int DB = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int j = lane >> 4;

  // Workgroup -> (item, row group).  With several row groups, the workgroups of
  // one item are spaced 8 apart in launch order so that they land on the same
  // XCD (workgroups are dealt to the 8 XCDs round-robin) at about the same time
  // and re-read the item's keys from that XCD's L2.
  int item, rg;
  if (a.nrg == 1) {
    item = blockIdx.x;
    rg = 0;
  } else {
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
  const int row0 = rg * 16 * NRB;

  int L, T = 0;
  if (RING) {
    L = a.C;
    const int64_t t64 = a.ring_T[b];
    T = t64 < 0 ? 0 : (t64 > (int64_t)INT_MAX ? INT_MAX : (int)t64);
  } else {
    const int l = a.seq_lens[b];
    L = l < 0 ? 0 : (l > a.max_keys ? a.max_keys : l);
  }
  const int nkb = (L + 31) >> 5;
  const int kb0 = s * a.kb_per_split;
  const int kb1 = min(kb0 + a.kb_per_split, nkb);

  // Q^T operands: lane (n, j) holds row row0 + 16*rb + n, dims 32*ks + 8*j .. +7.
  bf16x8 qop[NRB][KS];
  int lim[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int row = row0 + rb * 16 + n;
    if (row < a.R) {
      const int qi = row / a.G;
      const int hl = row - qi * a.G;
      const uint16_t* qp =
          a.q + ((size_t)(b * a.n_q + qi) * a.Hq + g * a.G + hl) * D + j * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[rb][ks] = ld_bf16x8(qp + ks * 32);
      lim[rb] = RING ? L : L - a.n_q + qi + 1;
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[rb][ks] = zero_bf16x8();
      lim[rb] = L;
    }
  }

  SoftmaxState<D, NRB> st;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    st.m[rb] = -INFINITY;
    st.l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) st.acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Main loop over this wave's tiles.  K registers are refilled with the next
  // tile as soon as the S^T products have consumed them, V registers as soon as
  // the PV products have: one tile of each is always in flight.
  KTile<D, RING> kt;
  VTile<D> vt;
  int kb = kb0 + wave;
  bool ok = false;
  if (kb < kb1) {
    const size_t tile = tile_index<RING>(a, b, g, kb, ok);
    if (ok) {
      load_k<D, RING>(kt, a, tile, b, kb, n, j);
      load_v<D>(vt, a, tile, n, j);
    }
  }
  while (kb < kb1) {
    const int kbn = kb + 4;
    bool ok_n = false;
    size_t tile_n = 0;
    if (kbn < kb1) tile_n = tile_index<RING>(a, b, g, kbn, ok_n);
    const int kbase = kb * 32 + 8 * j;   // this lane's 8 keys: kbase .. kbase + 7
    if (ok) {
      const uint32_t keep = present_keys<D, RING>(kt, a, kbase, L, T);
      f32x4 s[NRB][2];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        s[rb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        s[rb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s[rb][0] = mfma16x16x32(kt.k[0][ks], qop[rb][ks], s[rb][0]);
          s[rb][1] = mfma16x16x32(kt.k[1][ks], qop[rb][ks], s[rb][1]);
        }
      }
      if (ok_n) load_k<D, RING>(kt, a, tile_n, b, kbn, n, j);
      bf16x8 p_hi[NRB], p_lo[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        softmax_update<D, NRB>(st, rb, s[rb][0], s[rb][1], keep, lim[rb] - kbase, a.scale_log2,
                               p_hi[rb], p_lo[rb]);
      // Absent keys may hold any bits (even NaN): zero their values so that
      // 0-weight * value stays 0 in the PV product.
      if (!__all(keep == 0xFFu)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) vt.v[db] = mask_bf16x8(vt.v[db], keep);
      }
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          st.acc[rb][db] = mfma16x16x32(vt.v[db], p_hi[rb], st.acc[rb][db]);
          st.acc[rb][db] = mfma16x16x32(vt.v[db], p_lo[rb], st.acc[rb][db]);
        }
      }
      if (ok_n) load_v<D>(vt, a, tile_n, n, j);
    } else if (ok_n) {
      load_k<D, RING>(kt, a, tile_n, b, kbn, n, j);
      load_v<D>(vt, a, tile_n, n, j);
    }
    ok = ok_n;
    kb = kbn;
  }

  // ---- merge the four waves' states through LDS, one row block at a time ----
  __shared__ float sm_m[4][16];
  __shared__ float sm_l[4][16];
  __shared__ f32x4 sm_acc[3][DB][64];

#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float lsum = sum_over_lane_groups(st.l[rb]);
    __syncthreads();   // previous round's readers are done with the buffers
    if (j == 0) {
      sm_m[wave][n] = st.m[rb];
      sm_l[wave][n] = lsum;
    }
    __syncthreads();
    float M = sm_m[0][n];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm_m[w][n]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Ltot = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) Ltot += sm_l[w][n] * fast_exp2(sm_m[w][n] - Mu);
    const float f = fast_exp2(st.m[rb] - Mu);
    if (wave > 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db) sm_acc[wave - 1][db][lane] = st.acc[rb][db] * f;
    }
    __syncthreads();
    if (wave == 0) {
      const int row = row0 + rb * 16 + n;
      if (row < a.R) {
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
        for (int db = 0; db < DB; ++db) {
          f32x4 v = st.acc[rb][db] * f;
          v += sm_acc[0][db][lane];
          v += sm_acc[1][db][lane];
          v += sm_acc[2][db][lane];
          *reinterpret_cast<f32x4*>(op + db * 16 + 4 * j) = v * inv;
        }
        if (j == 0 && lp) *lp = Ltot > 0.f ? (M + fast_log2(Ltot)) * kLn2 : -INFINITY;
      }
    }
  }
}

template <int D, int NRB, bool RING>
hipError_t launch_one(const AttnArgs& a, int grid, hipStream_t stream) {
  AttnArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_split_kernel<D, NRB, RING>),
                         dim3(grid), dim3(256), args, 0, stream);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& p, bool ring, hipStream_t stream) {
  if constexpr (D == 256) {   // one row block per wave only (two would spill)
    if (p.nrb != 1) return hipErrorInvalidValue;
    return ring ? launch_one<D, 1, true>(a, p.grid, stream)
                : launch_one<D, 1, false>(a, p.grid, stream);
  } else {
    if (ring) {
      return p.nrb == 1 ? launch_one<D, 1, true>(a, p.grid, stream)
                        : launch_one<D, 2, true>(a, p.grid, stream);
    }
    return p.nrb == 1 ? launch_one<D, 1, false>(a, p.grid, stream)
                      : launch_one<D, 2, false>(a, p.grid, stream);
  }
}

}  // namespace

bool plan_attention(int B, int Hq, int Hkv, int D, int n_q, int max_keys, int num_splits,
                    int partials_only, bool ring, AttnPlan* p) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || n_q < 1 || max_keys < 0 || num_splits < 0)
    return false;
  if (D != 64 && D != 128 && D != 256) return false;
  p->G = Hq / Hkv;
  p->R = n_q * p->G;
  if (p->R > 256) return false;
  p->nkb = (max_keys + 31) / 32;
  const long groups = (long)B * Hkv;
  long target;    // workgroups to aim at
  int cap;        // most 32-key tiles per split
  // Few rows: each wave holds every row and the four waves split the keys.
  // Two row blocks per wave need too many registers at D = 256 (they spill).
  if (ring || p->R <= 16 || (p->R <= 32 && D != 256)) {
    p->shared = 0;
    p->nrb = (p->R <= 16 || D == 256) ? 1 : 2;
    p->nrg = (p->R + 16 * p->nrb - 1) / (16 * p->nrb);
    target = WMTP_TARGET_WG_SPLIT;
    cap = INT_MAX;
  } else {
    // Many rows: the waves split the rows and share each K/V tile through LDS.
    // A workgroup holds 16 * rbw rows per wave; two row blocks per wave are too
    // many registers at D = 256 for two waves per SIMD.
    p->shared = 1;
    const int nw = shared_kernel_waves();
    const int rbw = (p->R > 16 * nw && D != 256) ? 2 : 1;
    p->nrb = rbw;
    p->nrg = (p->R + 16 * nw * rbw - 1) / (16 * nw * rbw);
    target = WMTP_TARGET_WG_SHARED;
    cap = shared_kernel_max_tiles();
  }
  int kbps;
  if (num_splits > 0) {
    kbps = (p->nkb + num_splits - 1) / num_splits;
  } else {
    // Rounded down (to a multiple of 4: one share per wave) so that a length just
    // past a round number adds a small last split instead of stretching all.
    const long tiles = (long)p->nkb * groups * p->nrg;
    long per = tiles / target;
    per = (per / 4) * 4;
    kbps = (int)(per < 4 ? 4 : (per > INT_MAX ? INT_MAX : per));
  }
  if (p->shared) kbps = (kbps + 1) & ~1;   // even: a split then spans at most cap/2 whole pages
  if (kbps > cap) kbps = cap;
  if (kbps < 1) kbps = 1;
  p->kb_per_split = kbps;
  p->nsplit = p->nkb == 0 ? 1 : (p->nkb + kbps - 1) / kbps;
  p->direct = (p->nsplit == 1 && !partials_only) ? 1 : 0;
  const long items = groups * p->nsplit;
  if (items * p->nrg > INT_MAX / 16) return false;
  p->items = (int)items;
  p->grid = p->nrg == 1 ? p->items : ((p->items + 7) / 8) * 8 * p->nrg;
  if (p->direct) {
    p->part_o_bytes = 0;
    p->lse_offset = 0;
    p->ws_bytes = 0;
  } else {
    p->part_o_bytes = (size_t)items * p->R * D * sizeof(float);
    p->lse_offset = ((p->part_o_bytes + 255) / 256) * 256;
    p->ws_bytes = p->lse_offset + (size_t)items * p->R * sizeof(float);
  }
  return true;
}

hipError_t launch_attention(const AttnArgs& a, const AttnPlan& p, bool ring, hipStream_t stream) {
  if (p.shared) return ring ? hipErrorInvalidValue : launch_attention_shared(a, p, stream);
  switch (a.D) {
    case 64: return launch_d<64>(a, p, ring, stream);
    case 128: return launch_d<128>(a, p, ring, stream);
    case 256: return launch_d<256>(a, p, ring, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wmtp
