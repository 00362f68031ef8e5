// Split-KV attention for many query rows per kv head (the verify of n_q
// proposed positions: n_q * G rows), with every K/V tile shared by all rows.
//
// One workgroup (NW = 4 waves, one per SIMD, each with the whole register file;
// or NW = 8, two per SIMD, at head dim 128 with more than 128 rows) owns one key
// split of one (sequence, kv head) pair and up to 32 * RBW * NW query rows; wave
// w owns rows [32*RBW*NW*rg + 32*RBW*w, +32*RBW), so every K/V operand read from
// LDS feeds RBW row blocks.
//
// The K and V halves of the split's 32-key tiles stream through two rings of
// kSlots LDS slots, filled by direct global-to-LDS loads (global_load_lds_dwordx4,
// non-temporal): each of a half's D/16 operands is one 1 KB block in the lane
// order the MFMA reads it back, the blocks in the order the tile holds them in
// memory, so that a wave loads its share of a half as one run of loads.
//
// The loop is software-pipelined across tiles.  Iteration t issues the S^T
// products of tile t+1 first; they run on the matrix cores while the VALU does
// the softmax of tile t, whose PV products follow.  K(t+1) and V(t) are resident
// while the next kSlots - 1 halves of each ring are in flight; one barrier per
// iteration both publishes K(t+1), V(t) and frees the slots of K(t) and V(t-1),
// which the refill (K(t+kSlots), V(t+kSlots-1)) overwrites.
//
// The per-tile math is the one of attn.hip (MFMA 32x32x16, online softmax with
// P as bf16 hi + lo parts); a wave's rows never meet another wave's, so each
// wave writes its own rows' (o, lse).
//
// fp8 caches (KV8): a tile keeps the bf16 tile's element order at one byte per
// element, so its K half and its V half are each copied into LDS as they lie in
// memory (1 KB direct loads of contiguous bytes, half as many as for bf16); an
// operand is then 8 bytes per lane, read at the element offset the bf16 layout
// gives and turned into the bf16 MFMA operand right before its product (every
// e4m3 value is a bf16 value: exact).
#include "attn_device.h"
#include "lds_stream.h"

#include <type_traits>

namespace wmtp {

namespace {

constexpr int kSlots = 5;       // LDS slots per ring (K, V): one resident, four in flight
constexpr int kPageRegs = 4;   // page ids preloaded per split: 64 per register
// A tile in which some weight exceeds this fraction of its row's running sum is
// heavy: PV takes the hi and lo parts of its weights (see the kernel).
constexpr float kHeavyWeight = 1.0f / 32.0f;

// An MFMA operand as it sits in LDS: 16 bytes of bf16, or 8 bytes of fp8 codes.
template <bool KV8>
using LdsOp = std::conditional_t<KV8, u32x2, bf16x8>;

template <bool KV8>
__device__ __forceinline__ LdsOp<KV8> lds_op(const unsigned char* p) {
  return *reinterpret_cast<const LdsOp<KV8>*>(p);
}

// LDS byte offsets, inside a stage, of K operand ks and of V^T operand (db, kk),
// without the lane's own offset (k_lane / v_lane).  bf16: each operand is a
// 1 KB block in MFMA lane order, the blocks in the order the tile holds them
// in memory (K by ks, V^T by kk and then db).  fp8: the stage holds the tile's
// bytes as in memory, so the offsets are the tile's element offsets.
template <int D, bool KV8>
__device__ __forceinline__ int k_lds(int ks) { return KV8 ? ks * 512 : ks * 1024; }
template <int D, bool KV8>
__device__ __forceinline__ int v_lds(int db, int kk) {
  return KV8 ? kk * (16 * D) + db * 512 : (kk * (D / 32) + db) * 1024;
}
template <bool KV8>
__device__ __forceinline__ int k_lane(int lane) {
  const int m = lane & 31, h = lane >> 5;
  return KV8 ? s_row_key(m) * 16 + 8 * h : lane * 16;
}
template <bool KV8>
__device__ __forceinline__ int v_lane(int lane) {
  const int m = lane & 31, h = lane >> 5;
  return KV8 ? m * 16 + 8 * h : lane * 16;
}

// S^T of one tile for this wave's RBW row blocks: K operands read from the LDS
// stage at `base` (offset by lane * 16) in two halves.  The MFMAs are only
// issued here; their results are used one iteration later.
template <int D, int RBW, bool KV8>
__device__ __forceinline__ void s_tile(f32x16 (&sacc)[RBW], const bf16x8 (&qop)[RBW][D / 16],
                                       const unsigned char* base) {
  constexpr int KS = D / 16;
  constexpr int KH = KS / 2;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) sacc[rb] = f32x16{};
#pragma unroll
  for (int k0 = 0; k0 < KS; k0 += KH) {
    LdsOp<KV8> kop[KH];
#pragma unroll
    for (int ks = 0; ks < KH; ++ks) kop[ks] = lds_op<KV8>(base + k_lds<D, KV8>(k0 + ks));
#pragma unroll
    for (int ks = 0; ks < KH; ++ks) {
      const bf16x8 k = as_operand(kop[ks]);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) sacc[rb] = mfma32x32x16(k, qop[rb][k0 + ks], sacc[rb]);
    }
    operand_fence();
  }
}

// Weights and PV of one tile from its masked scores x; V^T operands from the LDS
// stage at `base`, in two halves.  mask_v (wave-uniform): some key of the tile
// is past the sequence length, and its values, which may hold any bits (even
// NaN), are zeroed so that 0-weight * value stays 0 in the PV product.
template <int D, int RBW, bool KV8>
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
        vop[db][kk] = as_operand(lds_op<KV8>(base + v_lds<D, KV8>(d0 + db, kk)));
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

// One tile of the fast loop, as one block (branch-free up to a heavy tile's lo
// products at its end): S(t+1) into s_acc from the LDS stage at kbase, the
// weights of tile t from its scores x, and PV(t) from the stage at vbase.  Every
// key of tile t is present and visible to every row, and
// no rescale is due.  Step ks issues the S^T MFMA(s) of head-dim step ks and
// then the softmax work of 256/D of tile t's scores per row block, which the
// VALU executes while the matrix core runs the MFMA; anchors at every step keep
// that order.  K operand reads run four steps ahead of their MFMAs and the V
// operand reads are spread over the same steps, so PV(t) finds them in
// registers.  dma(0) and dma(1) issue the wave's global-to-LDS loads of the K
// and the V half of the refill for later tiles, right after the S^T MFMAs of
// steps 0 and KS / 2.  PV(t) takes the hi bf16 parts of the weights only (the
// precision argument is at the fast loop in the kernel), unless keep_lo (a
// heavy tile) adds the lo parts' products after them.  What hi alone leaves out
// goes to the output's normaliser in one of three ways (DROP).  kDropMfma:
// l_drop sums the fast tiles' exact weights, and two more products with a V^T
// of ones sum their hi parts into hs (every register of lane (n, h) holds row
// n's sum), two issue slots.  kDropDot: l_drop as there, and a bf16 dot
// product with (1, 1) adds each pair of hi parts to hsd (this lane's share):
// one VALU instruction per pair and no registers.  kDropLo: l_drop sums the
// dropped lo parts on the VALU (six instructions per pair).  The tile ends with
// the check of tile t+1 (copy_and_check), VALU work beside the PV products.
constexpr int kDropLo = 0, kDropMfma = 1, kDropDot = 2;

// Copies a tile's scores out of s_acc into x and checks this lane's rows:
// raise, a score above the running maximum by more than the lazy margin (or
// no maximum yet), which bars the tile from the fast path; heavy, a weight
// above kHeavyWeight of the row's running sum (the row's keys are split over
// lanes n and n + 32), which makes the fast tile keep the weights' lo parts.
template <int D, int RBW>
__device__ __forceinline__ void copy_and_check(const SoftmaxState<D, RBW>& st,
                                               const f32x16 (&s_acc)[RBW], float (&x)[RBW][16],
                                               float c, bool& raise, bool& heavy) {
  raise = false;
  heavy = false;
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      x[rb][i] = s_acc[rb][i];
      asm volatile("" : "+v"(x[rb][i]));   // a vector register copy, carried as such
    }
    const float mxf = lane_max16(x[rb]) * c;
    raise |= needs_raise(mxf, st.m[rb]);
    heavy |= fast_exp2(mxf - st.m[rb]) > sum_over_row(st.l[rb]) * kHeavyWeight;
  }
  // the flags are computed here, beside the caller's products, not sunk past
  // the branch that follows (the compiler moves them to their first use)
  int r = raise, hv = heavy;
  asm volatile("" : "+v"(r), "+v"(hv));
  raise = r != 0;
  heavy = hv != 0;
}

template <int D, int RBW, bool KV8, int DROP, typename Dma>
__device__ __forceinline__ void fast_tile(SoftmaxState<D, RBW>& st, f32x16 (&s_acc)[RBW],
                                          f32x16 (&hs)[RBW], float (&hsd)[RBW],
                                          const bf16x8 (&qop)[RBW][D / 16],
                                          float (&x)[RBW][16], bool keep_lo, bool& raise_next,
                                          bool& heavy_next, float c,
                                          const unsigned char* kbase, const unsigned char* vbase,
                                          Dma&& dma) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int kAhead = KS < 4 ? KS : 4;
  constexpr int E = 256 / D;                   // scores per row block handled per step
  static_assert(E * KS == 16, "scores per step");

  float neg_m[RBW], p[RBW][16], psum[RBW], pdrop[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    neg_m[rb] = -st.m[rb];                     // finite: every row has seen a full tile
    psum[rb] = 0.f;
    pdrop[rb] = 0.f;
  }
  uint32_t hw[RBW][8];                         // packed P^T words: key pair w of row block
  LdsOp<KV8> kop[KS];
  LdsOp<KV8> vop[KS];                          // V operand (db, kk) at index 2 * db + kk
#pragma unroll
  for (int ks = 0; ks < kAhead; ++ks) kop[ks] = lds_op<KV8>(kbase + k_lds<D, KV8>(ks));
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) s_acc[rb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    // step boundary: the previous step's results and this step's inputs (the K
    // operand and the V operand read with it in one statement, so that one LDS
    // wait covers both)
    if (ks >= kAhead) {
      asm volatile("" : "+v"(kop[ks]), "+v"(vop[ks - kAhead]));
    } else {
      anchor(kop[ks]);
    }
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      anchor(psum[rb]);
      anchor(pdrop[rb]);
#pragma unroll
      for (int j = 0; j < E; ++j) anchor(x[rb][ks * E + j]);
      if (ks > 0 && (E > 1 || (ks & 1) == 0)) {
        // pairs completed by the previous step
#pragma unroll
        for (int j = 0; j < (E + 1) / 2; ++j) {
          const int w = ((ks - 1) * E) / 2 + j;
          anchor(hw[rb][w]);
        }
      }
    }
    if (ks + kAhead < KS) kop[ks + kAhead] = lds_op<KV8>(kbase + k_lds<D, KV8>(ks + kAhead));
    vop[ks] = lds_op<KV8>(vbase + v_lds<D, KV8>(ks >> 1, ks & 1));
    {
      const bf16x8 k = as_operand(kop[ks]);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) s_acc[rb] = mfma32x32x16(k, qop[rb][ks], s_acc[rb]);
    }
    if (ks == 0) dma(0);
    if (ks == KS / 2) dma(1);
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const int i = ks * E + j;
        p[rb][i] = fast_exp2(fmaf(x[rb][i], c, neg_m[rb]));
        psum[rb] += p[rb][i];
        if (i & 1) {
          const uint32_t hp = pack_bf16x2(p[rb][i - 1], p[rb][i]);
          hw[rb][i >> 1] = hp;
          if constexpr (DROP == kDropLo) {
            const float d0 = p[rb][i - 1] - __builtin_bit_cast(float, hp << 16);
            const float d1 = p[rb][i] - __builtin_bit_cast(float, hp & 0xFFFF0000u);
            pdrop[rb] += d0 + d1;
          } else if constexpr (DROP == kDropDot) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
            hsd[rb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, hp), ones, hsd[rb],
                                                       false);
          }
        }
      }
    }
  }
#pragma unroll
  for (int ks = KS - kAhead; ks < KS; ++ks) anchor(vop[ks]);
  bf16x8 p_hi[RBW][2];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    st.l[rb] += psum[rb];
    st.l_drop[rb] += DROP == kDropLo ? pdrop[rb] : psum[rb];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      p_hi[rb][kk] = __builtin_bit_cast(bf16x8, u32x4{hw[rb][4 * kk], hw[rb][4 * kk + 1],
                                                      hw[rb][4 * kk + 2], hw[rb][4 * kk + 3]});
  }
  // PV(t) with the hi parts of the weights; l_drop (and hs) hold what they
  // leave out, so that the output is normalised by exactly the weights PV saw.
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 v = as_operand(vop[2 * db + kk]);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) st.acc[rb][db] = mfma32x32x16(v, p_hi[rb][kk], st.acc[rb][db]);
    }
  if constexpr (DROP == kDropMfma) {
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) hs[rb] = mfma32x32x16(ones, p_hi[rb][kk], hs[rb]);
  }
  // tile t+1's check, on its finished scores and tile t's running sums: VALU
  // work beside the PV products instead of ahead of the next tile's
  copy_and_check<D, RBW>(st, s_acc, x, c, raise_next, heavy_next);
  if (keep_lo) {
    // a heavy tile (wave-uniform): the lo parts of its weights as well, so that
    // PV sees hi + lo as on the general path, and the normaliser term of the
    // dropped parts counts them as seen (ones products or dot products of the
    // lo parts, or l_drop less this tile's dropped parts)
    bf16x8 p_lo[RBW][2];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 lw;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int w = 4 * kk + j;
          const uint32_t hp = hw[rb][w];
          // a scalar, not the vector element: bit-casting lw[j] itself made the
          // compiler read element 0 for every j
          const uint32_t lp = pack_bf16x2(p[rb][2 * w] - __builtin_bit_cast(float, hp << 16),
                                          p[rb][2 * w + 1] - __builtin_bit_cast(float, hp & 0xFFFF0000u));
          lw[j] = lp;
          if constexpr (DROP == kDropDot) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
            hsd[rb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lp), ones, hsd[rb],
                                                       false);
          }
        }
        p_lo[rb][kk] = __builtin_bit_cast(bf16x8, lw);
      }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 v = as_operand(vop[2 * db + kk]);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) st.acc[rb][db] = mfma32x32x16(v, p_lo[rb][kk], st.acc[rb][db]);
      }
    if constexpr (DROP == kDropMfma) {
      const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) hs[rb] = mfma32x32x16(ones, p_lo[rb][kk], hs[rb]);
    }
    if constexpr (DROP == kDropLo) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) st.l_drop[rb] -= pdrop[rb];
    }
  }
}

// TREE: the appended positions form a tree (a.tree_mask), else a causal chain.
// KV8: the caches hold fp8 e4m3 codes (K's scale folded into scale_log2, V's
// applied to the output).
template <int D, int RBW, int NW, bool TREE, bool KV8>
__global__ __launch_bounds__(64 * NW, 1) void attn_shared_kernel(AttnArgs a) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  // bytes of a K (or V) half of a tile in LDS: KS operands of 1 KB (bf16) or 512 B (fp8)
  constexpr int HALF = KS * (KV8 ? 512 : 1024);
  constexpr int NCH = HALF / 1024;               // 1 KB wave loads per half tile
  constexpr int NH = (NCH + NW - 1) / NW;        // loads per half of each wave that loads
  // every wave issues NH loads per half, or (fewer chunks than waves) none: the
  // vmcnt waits below count NH per half
  static_assert(NCH % NW == 0 || NCH < NW, "chunks split evenly over the loading waves");

  // How the fast tiles' hi weight parts are summed (see fast_tile): on the
  // matrix cores where a wave has the registers for the sums, else by bf16 dot
  // products on the VALU.
#ifndef WMTP_SHARED_DROP
  constexpr int DROP = (NW <= 4 && !(D == 128 && RBW == 2)) ? kDropMfma : kDropDot;
#else
  constexpr int DROP = WMTP_SHARED_DROP;
#endif

  // K ring then V ring, kSlots half tiles each (160 KB at D = 256).
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kSlots * HALF];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 31;
  const int h = lane >> 5;
  const int klane = k_lane<KV8>(lane);   // the lane's byte offset in a K / V stage operand
  const int vlane = v_lane<KV8>(lane);

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
  const int nkb = (int)(((unsigned)L + 31u) >> 5);   // L >= 0
  const int kb0 = s * a.kb_per_split;
  const int kb1 = min(kb0 + a.kb_per_split, nkb);
  const int ntile = kb1 > kb0 ? kb1 - kb0 : 0;
  // keys below vis_end are visible to every row: the causal limit of the first
  // query, or (tree) the start of the appended positions
  const int vis_end = L - a.n_q + (TREE ? 0 : 1);

  // Q^T operands of this wave's rows: lane (m, h) holds row row0 + 32*rb + m,
  // dims 16*ks + 8*h .. +7.
  bf16x8 qop[RBW][KS];
  int lim[RBW];
  uint64_t tmask[TREE ? RBW : 1];   // tree: the row's ancestor mask over the appended positions
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
      if constexpr (TREE) tmask[rb] = a.tree_mask[(size_t)b * a.n_q + qi];
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[rb][ks] = zero_bf16x8();
      lim[rb] = L;
      if constexpr (TREE) tmask[rb] = 0;
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
    st.l_drop[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) st.acc[rb][db] = f32x16{};
  }
  // hi parts of the fast tiles' weights: summed per row (kDropMfma: any
  // register) or this lane's share (kDropDot)
  f32x16 hs[RBW];
  float hsd[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    hs[rb] = f32x16{};
    hsd[rb] = 0.f;
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
  // Every page of the split inside the cache (the same for every wave): only
  // then do tiles take the fast path, which then tracks no page validity.
  bool pages_in = true;
#pragma unroll
  for (int r = 0; r < kPageRegs; ++r)
    pages_in = pages_in && (page0 + 64 * r + lane > last_page || (unsigned)my_page[r] < (unsigned)a.num_pages);
  const bool pages_ok = __all(pages_in);

  // Half tiles stream through two rings of LDS slots, K and V, filled by
  // direct global-to-LDS loads: the K half of tile u goes to K slot u % kSlots,
  // its V half to V slot u % kSlots.  Step t reads K(t+1) (for S(t+1)) and V(t)
  // (for PV(t)), so each ring has one resident half and kSlots - 1 in flight:
  // after the barrier of step t, K(t+kSlots) refills the slot K(t) left and
  // V(t+kSlots-1) the slot V(t-1) left.  A page id outside the cache still issues its loads (from page
  // 0) so that every half costs the same number of loads; the tile is skipped.
  uint32_t ok_tile = 0;                 // bit u % 32: tile u has a valid page
  // tile index of tile u, whose page the split's preloaded ids hold (ok: the page
  // is inside the cache; else page 0 stands in)
  auto page_of = [&](int u, bool& ok) -> size_t {
    const int kb = kb0 + u;
    const int idx = (kb >> 1) - page0;   // 0 .. 64*kPageRegs - 1, wave-uniform
    // every register's lane idx % 64, then a select: no branch per register
    int cand[kPageRegs];
#pragma unroll
    for (int r = 0; r < kPageRegs; ++r) cand[r] = __builtin_amdgcn_readlane(my_page[r], idx & 63);
    int ppage = -1;
#pragma unroll
    for (int r = 0; r < kPageRegs; ++r) ppage = (idx >> 6) == r ? cand[r] : ppage;
    ok = (unsigned)ppage < (unsigned)a.num_pages;
    if (!ok) ppage = 0;
    return ((size_t)ppage * a.Hkv + g) * 2 + (kb & 1);
  };
  auto k_slot = [&](int u) { return smem + (u % kSlots) * HALF; };
  auto v_slot = [&](int u) { return smem + (kSlots + u % kSlots) * HALF; };
  // Bytes of tile `tile` in a cache, and the byte offset, inside it, of this
  // lane's 16 bytes of the wave's 1 KB load number c of the K (kv = 0) or V half
  // (bf16: operand c in MFMA lane order; fp8: the half's bytes c KB on, as stored).
  auto tile_bytes = [&](const uint16_t* cache, size_t tile) {
    return reinterpret_cast<const unsigned char*>(cache) + tile * (size_t)(32 * D) * (KV8 ? 1 : 2);
  };
  // Chunk c of a half sits at c KB in the tile's half and in the stage alike;
  // the lane's 16 bytes sit at c KB + k_goff / v_goff in the tile (bf16: MFMA
  // lane order; fp8: as stored) and at c KB + 16 * lane in the stage.  Wave w
  // loads chunks NH*w .. NH*w + NH - 1 (or, with fewer chunks than waves, chunk w).
  const uint32_t k_goff = KV8 ? (uint32_t)(lane * 16) : 2u * k_operand_offset(0, m, h);
  const uint32_t v_goff = KV8 ? (uint32_t)(lane * 16) : 2u * v_operand_offset<D>(0, 0, m, h);
  const bool loads = !(NCH < NW && wave >= NCH);   // wave-uniform
  const int c0 = wave * NH;                         // the wave's first chunk
  auto issue_k = [&](int u) {
    bool ok;
    const unsigned char* kt = tile_bytes(a.kc, page_of(u, ok));
    ok_tile = (ok_tile & ~(1u << (u & 31))) | ((ok ? 1u : 0u) << (u & 31));
    if (loads) lds_load_run<NH>(kt + c0 * 1024, k_goff, k_slot(u) + c0 * 1024);
  };
  auto issue_v = [&](int u) {
    bool ok;
    const unsigned char* vt = tile_bytes(a.vc, page_of(u, ok));
    if (loads) lds_load_run<NH>(vt + c0 * 1024, v_goff, v_slot(u) + c0 * 1024);
  };

  // Prologue: K(0..kSlots-1) and V(0..kSlots-2) in the order the steps would have issued them,
  // publish K(0), issue S(0).
#pragma unroll
  for (int u = 0; u < kSlots; ++u) {
    if (u < ntile) issue_k(u);
    if (u >= 1 && u - 1 < ntile) issue_v(u - 1);
  }
  f32x16 s_acc[RBW];
  if (ntile > 0) {
    if (ntile >= kSlots) {
      wait_vmcnt<(kSlots - 1) * 2 * NH>();   // K(1..), V(0..) may still be in flight
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    if (any_row) s_tile<D, RBW, KV8>(s_acc, qop, k_slot(0) + klane);
  }

  // Publish K(t+1) and V(t); then refill the freed slots (issue_for).
  auto publish = [&](int t) {
    // Issued after K(t+1), V(t): K(t+2..t+kSlots-1) and V(t+1..t+kSlots-2),
    // all present unless the split ends within the next few tiles.
    if (t + kSlots - 1 < ntile) {
      wait_vmcnt<(kSlots - 2) * 2 * NH>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
  };
  auto issue_for = [&](int t) {
    if (t + kSlots < ntile) issue_k(t + kSlots);
    if (t + kSlots - 1 < ntile) issue_v(t + kSlots - 1);
  };
  auto sync_stage = [&](int t) {
    publish(t);
    issue_for(t);
  };
  auto next_scores = [&](int t) {
    if (any_row && t + 1 < ntile) s_tile<D, RBW, KV8>(s_acc, qop, k_slot(t + 1) + klane);
  };

  // Masked scores of tile t (from s_acc, which then is free) and the facts its
  // PV needs.
  float x[RBW][16], mx[RBW];
  uint32_t keep = 0;
  bool mask_v = false;
  auto scores_of = [&](int t) {
    const int kb = kb0 + t;
    // every key of the tile is present and visible to every row (the smallest
    // causal limit of any row is L - n_q + 1)
    const bool all_vis = (kb + 1) * 32 <= vis_end;
    keep = keys_below(L - kb * 32, h);
    mask_v = (kb + 1) * 32 > L;
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      uint32_t vis;
      if constexpr (TREE)
        vis = keys_below(L - a.n_q - kb * 32, h) | tree_keys(tmask[rb], kb * 32 - (L - a.n_q), h);
      else
        vis = keys_below(lim[rb] - kb * 32, h);
      mx[rb] = masked_scores(x[rb], s_acc[rb], vis, all_vis,
                             a.scale_log2);
#pragma unroll
      for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(x[rb][i]));
    }
  };
  auto tile_ok = [&](int t) { return any_row && (pages_ok || ((ok_tile >> (t & 31)) & 1u)); };

  // Tiles run through a fast path or a general one.  The fast path takes a tile
  // that is full (every key present and visible to every row), whose rows all
  // have a running maximum that no score of the tile exceeds by more than the
  // lazy margin, and whose refill, K(t+kSlots) and V(t+kSlots-1), exists: one branch-free
  // block, no cross-lane work.  Any other tile (a split's first and last
  // tiles, the causal boundary, bad pages, a rescale) takes the general path,
  // and the fast path resumes after it.  Waves that own no row take only part
  // in the stage pipeline.  s_acc holds S(t) when tile t starts either way.
  //
  // Precision of the fast path.  The general path feeds PV each weight as two
  // bf16 parts (hi + lo, relative error ~2^-17); the fast path feeds the hi
  // parts alone and takes the dropped lo parts out of the output's normaliser
  // (l_drop), so o stays an exact weighted mean with each of those weights
  // perturbed by at most 2^-9 relative: |error| <= 2^-9 * sum_i w_i |v_i - o|
  // over the fast tiles' keys.  A heavy tile, where some weight exceeds
  // kHeavyWeight of its row's running sum (a needle, a few dominant keys, the
  // start of a split), stays on the fast path but feeds PV the hi and lo parts,
  // as the general path does, so no key that is a large share of the mass is
  // rounded (with scores ~N(0, 1), ~15 of a wave's 256 tiles in a split, most
  // of them near its start).  lse uses the exact sum.
  int t = 0;
  while (t < ntile) {
    bool synced = false;   // tile t is published, its refill not yet issued
    if (any_row && pages_ok && t + kSlots < ntile) {
      // Kept across the fast tiles: t % kSlots, and the tile index of the next V
      // refill, which is the tile the previous K refill took.
      int sj = t % kSlots;
      bool ok_v;
      size_t v_tix = page_of(t + kSlots - 1, ok_v);
      // the fast path's own copy of tile t's scores (the general path takes
      // them from s_acc again) and its check; each fast tile leaves both for the
      // tile after it
      float xf[RBW][16];
      bool raise_t, heavy_t;
      copy_and_check<D, RBW>(st, s_acc, xf, a.scale_log2, raise_t, heavy_t);
      for (; t + kSlots < ntile; ++t) {
        publish(t);
        const int kb = kb0 + t;
        const bool slow = raise_t || (kb + 1) * 32 > vis_end;
        if (__any(slow)) {
          synced = true;
          break;
        }
        // K(t+kSlots): an odd 32-key tile shares its page with the tile before
        // it, V(t+kSlots-1), one tile on in the cache
        size_t k_tix;
        if ((kb + kSlots) & 1) {
          k_tix = v_tix + 1;
        } else {
          bool ok_k;
          k_tix = page_of(t + kSlots, ok_k);
        }
        const unsigned char* kt = tile_bytes(a.kc, k_tix);
        const unsigned char* vt = tile_bytes(a.vc, v_tix);
        v_tix = k_tix;
        // slots: K(t+kSlots) refills K(t)'s, V(t+kSlots-1) V(t-1)'s; reads K(t+1), V(t)
        const int sj1 = sj == kSlots - 1 ? 0 : sj + 1;
        const int sjm = sj == 0 ? kSlots - 1 : sj - 1;
        unsigned char* kdst = smem + sj * HALF;
        unsigned char* vdst = smem + (kSlots + sjm) * HALF;
        auto dma = [&](int i) {
          if (!loads) return;
          if (i == 0) lds_load_run<NH>(kt + c0 * 1024, k_goff, kdst + c0 * 1024);
          else lds_load_run<NH>(vt + c0 * 1024, v_goff, vdst + c0 * 1024);
        };
        const bool keep_lo = __any(heavy_t);
        fast_tile<D, RBW, KV8, DROP>(st, s_acc, hs, hsd, qop, xf, keep_lo, raise_t, heavy_t, a.scale_log2,
                                     smem + sj1 * HALF + klane, smem + (kSlots + sj) * HALF + vlane,
                                     dma);
        sj = sj1;
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
#pragma unroll
          for (int db = 0; db < DB; ++db) pin_acc(st.acc[rb][db]);
          if (DROP == kDropMfma) pin_acc(hs[rb]);
        }
      }
    }
    if (t >= ntile) break;
    // general path for tile t
    if (synced) {
      issue_for(t);
    } else {
      sync_stage(t);
    }
    const bool ok_t = tile_ok(t);
    if (ok_t) scores_of(t);
    next_scores(t);
    if (ok_t) {
      raise_and_rescale<D, RBW>(st, mx, [&](int rb, float alpha) {
        if constexpr (DROP == kDropMfma) {
          hs[rb] *= alpha;
          pin_acc(hs[rb]);
        }
        if constexpr (DROP == kDropDot) hsd[rb] *= alpha;
      });
      pv_tile<D, RBW, KV8>(st, x, a.scale_log2, v_slot(t) + vlane, keep, mask_v);
    }
    ++t;
  }

  // Each wave writes its own rows.
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int row = row0 + rb * 32 + m;
    const float Ltot = sum_over_row(st.l[rb]);
    // the weights PV saw: all of them, less the fast tiles' dropped lo parts
    float Lpv;
    if constexpr (DROP == kDropMfma) {
      Lpv = Ltot - (sum_over_row(st.l_drop[rb]) - hs[rb][0]);
    } else if constexpr (DROP == kDropDot) {
      Lpv = Ltot - (sum_over_row(st.l_drop[rb]) - sum_over_row(hsd[rb]));
    } else {
      Lpv = Ltot - sum_over_row(st.l_drop[rb]);
    }
    if (row >= a.R) continue;
    const float inv = (Lpv > 0.f ? 1.f / Lpv : 0.f) * (KV8 ? a.v_scale : 1.f);
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

template <int D, int RBW, int NW = kWaves>
hipError_t launch_shared_one(const AttnArgs& a, int grid, hipStream_t stream) {
  AttnArgs arg = a;
  void* args[] = {&arg};
  const void* k;
  if (a.kv8) {   // fp8 caches: causal verify only
    if (a.tree_mask) return hipErrorInvalidValue;
    k = reinterpret_cast<const void*>(&attn_shared_kernel<D, RBW, NW, false, true>);
  } else {
    k = a.tree_mask ? reinterpret_cast<const void*>(&attn_shared_kernel<D, RBW, NW, true, false>)
                    : reinterpret_cast<const void*>(&attn_shared_kernel<D, RBW, NW, false, false>);
  }
  return hipLaunchKernel(k, dim3(grid), dim3(64 * NW), args, 0, stream);
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
      if (p.nw == 8) return p.nrb == 1 ? launch_shared_one<128, 1, 8>(a, p.grid, stream)
                                       : hipErrorInvalidValue;
      return p.nrb == 1 ? launch_shared_one<128, 1>(a, p.grid, stream)
                        : launch_shared_one<128, 2>(a, p.grid, stream);
    case 256:
      return p.nrb == 1 ? launch_shared_one<256, 1>(a, p.grid, stream) : hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace wmtp
