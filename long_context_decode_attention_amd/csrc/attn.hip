// Split-KV decode attention for gfx950: the native draft (every cached key),
// the windowed draft (the valid slots of a sink-plus-recent ring) and a verify
// with at most 32 query rows per kv head share this kernel.
//
// Work decomposition.  One workgroup (NW = 4 waves) owns one key split of one
// (sequence b, kv head g) pair and a group of up to 32 * NB query rows of that
// kv head (the G query heads of the group, times n_q verify queries).  The
// split is a run of 32-key tiles; wave w of the workgroup takes tiles w,
// w + NW, ..., so the four waves stream neighbouring memory.  Each wave keeps
// its own online-softmax state; the four are merged through LDS at the end and
// the workgroup writes one partial (o, lse) per row, or the final result when
// the sequence has a single split.
//
// Per tile a wave runs the products of attn_device.h on MFMA 32x32x16.  K and V
// operands are 16-byte non-temporal loads straight from the tiled page layout
// into registers; the next tile's K loads are issued as soon as the S^T
// products have consumed the current ones, V likewise after PV, so one tile of
// each is always in flight.
#include "attn_device.h"
#include "ring_device.h"

#include <type_traits>

// Workgroups the split planner aims at: one per CU for both kernels, so that a
// long sequence runs in a single round (measured at 1M keys: 256 workgroups
// stream at 6.85 TB/s against 6.55 TB/s for 512, whose second round adds a
// workgroup prologue, a merge and a tail).
#ifndef WMTP_TARGET_WG_SPLIT
#define WMTP_TARGET_WG_SPLIT 256
#endif
#ifndef WMTP_TARGET_WG_SHARED
#define WMTP_TARGET_WG_SHARED 256
#endif

namespace wmtp {

namespace {


// KV8: the operands stay as loaded (8 fp8 bytes) until their MFMA.
template <int D, bool RING, bool KV8>
struct KTile {
  std::conditional_t<KV8, u32x2, bf16x8> k[D / 16];   // K operands, head-dim step ks
  int32_t pos[RING ? 16 : 1];   // ring mode: positions held by this lane's 16 slots
};

template <int D, bool KV8>
struct VTile {
  std::conditional_t<KV8, u32x2, bf16x8> v[D / 32][2];   // V^T operands (db, kk)
};

// Physical 32-key tile index of tile kb of (b, g); ok = false when the page id
// is outside the cache: the index is then that of page 0, and the tile's keys
// count as absent.
template <bool RING>
__device__ __forceinline__ size_t tile_index(const AttnArgs& a, int b, int g, int kb, bool& ok) {
  const int lpage = kb >> 1;
  int ppage;
  if constexpr (RING) {
    ppage = b * (a.C >> 6) + lpage;
  } else {
    ppage = a.block_table[(size_t)b * a.max_pages + lpage];
  }
  ok = (unsigned)ppage < (unsigned)a.num_pages;
  if (!ok) ppage = 0;   // still loaded (so that every load is unconditional), then ignored
  return ((size_t)ppage * a.Hkv + g) * 2 + (kb & 1);
}

// Tile index of tile kb of kv head g on physical page `ppage` (paged caches), with
// the same bad-page rule as tile_index.
__device__ __forceinline__ size_t tile_of_page(const AttnArgs& a, int ppage, int g, int kb,
                                               bool& ok) {
  ok = (unsigned)ppage < (unsigned)a.num_pages;
  if (!ok) ppage = 0;
  return ((size_t)ppage * a.Hkv + g) * 2 + (kb & 1);
}

// The fp8 tiles keep the bf16 tiles' element order at one byte per element, so
// the operand offsets are the same numbers in bytes.
// KEEP: the tiles are read again at the next draft step (a ring, or a window
// through the truncated paged index): ordinary loads.  The window still misses
// L2 at every step, by the fetch counters, but the step is faster without the
// streaming hint, which keeps the window out of the memory-side cache.  A full
// pass streams bytes it reads once.
template <int D, bool RING, bool KV8, bool KEEP>
__device__ __forceinline__ void load_k(KTile<D, RING, KV8>& t, const AttnArgs& a, size_t tile,
                                       int b, int kb, int m, int h) {
  if constexpr (KV8) {
    const uint8_t* kt = reinterpret_cast<const uint8_t*>(a.kc) + tile * (size_t)(32 * D);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      t.k[ks] = KEEP ? ld_u32x2(kt + k_operand_offset(ks, m, h)) : ld_u32x2_stream(kt + k_operand_offset(ks, m, h));
  } else {
    const uint16_t* kt = a.kc + tile * (size_t)(32 * D);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      t.k[ks] = KEEP ? ld_bf16x8(kt + k_operand_offset(ks, m, h)) : ld_bf16x8_stream(kt + k_operand_offset(ks, m, h));
  }
  if constexpr (RING) {
    // slots 8h..8h+7 and 16+8h..16+8h+7 of the tile
    const int32_t* rp = a.ring_pos + (size_t)b * a.C + kb * 32 + 8 * h;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int4 p0 = *reinterpret_cast<const int4*>(rp + 16 * r);
      const int4 p1 = *reinterpret_cast<const int4*>(rp + 16 * r + 4);
      t.pos[8 * r + 0] = p0.x; t.pos[8 * r + 1] = p0.y; t.pos[8 * r + 2] = p0.z;
      t.pos[8 * r + 3] = p0.w; t.pos[8 * r + 4] = p1.x; t.pos[8 * r + 5] = p1.y;
      t.pos[8 * r + 6] = p1.z; t.pos[8 * r + 7] = p1.w;
    }
  }
}

template <int D, bool KV8, bool KEEP>
__device__ __forceinline__ void load_v(VTile<D, KV8>& t, const AttnArgs& a, size_t tile, int m,
                                       int h) {
  if constexpr (KV8) {
    const uint8_t* vt = reinterpret_cast<const uint8_t*>(a.vc) + tile * (size_t)(32 * D);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        t.v[db][kk] = KEEP ? ld_u32x2(vt + v_operand_offset<D>(db, kk, m, h))
                           : ld_u32x2_stream(vt + v_operand_offset<D>(db, kk, m, h));
  } else {
    const uint16_t* vt = a.vc + tile * (size_t)(32 * D);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        t.v[db][kk] = KEEP ? ld_bf16x8(vt + v_operand_offset<D>(db, kk, m, h))
                           : ld_bf16x8_stream(vt + v_operand_offset<D>(db, kk, m, h));
  }
}

// Fused draft step: K operands of the tile of new positions (key j = position
// T0 + j of app.k_new, j < n_new; the other keys load key 0 and are marked
// absent).  The loads do not depend on T0; new_positions() sets the positions
// the window test reads once T0 is known.
template <int D>
__device__ __forceinline__ void load_k_new(KTile<D, true, false>& t, const AttnArgs& a, int b, int g,
                                           int m, int h) {
  const int key = s_row_key(m);
  const int kk = key < a.app.n_new ? key : 0;
  const uint16_t* src = a.app.k_new + (((size_t)b * a.app.n_new + kk) * a.Hkv + g) * D + 8 * h;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) t.k[ks] = ld_bf16x8(src + 16 * ks);
}

template <int D>
__device__ __forceinline__ void new_positions(KTile<D, true, false>& t, const AttnArgs& a, int T0,
                                              int h) {
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 16 * r + 8 * h + i;
      t.pos[8 * r + i] = j < a.app.n_new ? T0 + j : -1;
    }
}

// V^T of the new positions, staged in LDS as [D][kVtRow] bf16, keys 0..31 of a
// row first (keys >= n_new left as they are: the window test marks them absent
// and PV zeroes them).  Rows are padded from 32 to 40 keys (80 bytes): the 16
// lanes of a 16-byte read then start 20 banks apart and hit distinct banks,
// where 64-byte rows would put eight lanes on the same ones.
constexpr int kVtRow = 40;
template <int D, int NT>
__device__ __forceinline__ void stage_v_new(uint16_t* sm_vt, const AttnArgs& a, int b, int g) {
  const int pieces = a.app.n_new * (D / 8);
  for (int idx = threadIdx.x; idx < pieces; idx += NT) {
    const int j = idx / (D / 8);
    const int d0 = (idx - j * (D / 8)) * 8;
    const u32x4 w = *reinterpret_cast<const u32x4*>(
        a.app.v_new + (((size_t)b * a.app.n_new + j) * a.Hkv + g) * D + d0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sm_vt[(d0 + 2 * e) * kVtRow + j] = (uint16_t)(w[e] & 0xFFFFu);
      sm_vt[(d0 + 2 * e + 1) * kVtRow + j] = (uint16_t)(w[e] >> 16);
    }
  }
}

template <int D>
__device__ __forceinline__ void load_v_new(VTile<D, false>& t, const uint16_t* sm_vt, int m, int h) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      t.v[db][kk] =
          *reinterpret_cast<const bf16x8*>(sm_vt + (32 * db + m) * kVtRow + 16 * kk + 8 * h);
}

// Which of this lane's 16 keys exist for every row: inside the sequence length
// (and, for a truncated paged index, below sink_end or from r0 on), or (ring)
// holding a position of the current window.  Ring mode reads positions below
// p_end only: T for a window over the ring; the count before the append for the
// ring splits of a fused step, whose slots may still hold positions at or past
// that count from before a rollback (the new positions come from k_new alone).
template <int D, bool RING, bool KV8>
__device__ __forceinline__ uint32_t present_keys(const KTile<D, RING, KV8>& t, const AttnArgs& a,
                                                 int kb, int L, int T, int p_end, int h,
                                                 int sink_end, int r0) {
  if constexpr (RING) {
    uint32_t keep = 0;
    // in the window of some query: the last n_q positions T - n_q .. T - 1 each
    // see the sink and their own last n_recent positions (bitwise tests: no
    // branches; p_end >= 0, so the unsigned compare is 0 <= p < p_end)
    const int lo = T - (a.n_q - 1) - a.n_recent;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int p = t.pos[i];
      const bool ok = ((unsigned)p < (unsigned)p_end) & ((p < a.n_sink) | (p >= lo));
      keep |= (ok ? 1u : 0u) << i;
    }
    return keep;
  } else {
    uint32_t keep = keys_below(L - kb * 32, h);
    if (a.win) keep &= keys_below(sink_end - kb * 32, h) | (~keys_below(r0 - kb * 32, h) & 0xFFFFu);
    return keep;
  }
}

// WIN: the call reads a window through the truncated paged index (a.win), whose
// tiles the next draft step reads again (ordinary loads).
template <int D, int NB, bool RING, bool KV8, bool STEP = false, bool WIN = false>
__global__ __launch_bounds__(256, 1) void attn_split_kernel(AttnArgs a) {
  static_assert(!STEP || (RING && !KV8 && NB == 1), "the fused step reads a bf16 ring");
  constexpr int NW = 4;         // waves
  constexpr int NT = 64 * NW;   // threads
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 31;   // MFMA row / column of this lane
  const int h = lane >> 5;   // lane group

  // The arguments the prologue reads are fetched in one round trip: held in
  // registers here, they no longer wait one after another behind the branches
  // that use them.
  asm volatile("" ::"s"(a.nrg), "s"(a.items), "s"(a.nsplit), "s"(a.Hkv), "s"(a.kb_per_split),
               "s"(a.q), "s"(a.kc), "s"(a.vc), "s"(a.Hq), "s"(a.G), "s"(a.n_q), "s"(a.R),
               "s"(a.num_pages));
  if constexpr (RING) {
    asm volatile("" ::"s"(a.ring_pos), "s"(a.ring_T), "s"(a.C));
  } else {
    asm volatile("" ::"s"(a.block_table), "s"(a.seq_lens), "s"(a.max_pages), "s"(a.max_keys),
                 "s"(a.win));
  }

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
  // fused step: each group has a.nsplit ring splits and then one workgroup that
  // reads the new positions (split index a.nsplit)
  const int nparts = STEP ? a.nsplit + 1 : a.nsplit;
  const int s = item % nparts;
  const int bg = item / nparts;
  const bool newk = STEP && s == a.nsplit;
  const int g = bg % a.Hkv;
  const int b = bg / a.Hkv;
  const int row0 = rg * 32 * NB;


  // Q^T operands, staged once in LDS in MFMA lane order (sm_q[rb][ks][lane]:
  // row row0 + 32*rb + m, dims 16*ks + 8*h .. +7) and read back per tile; in
  // registers they would push the tile buffers into scratch at D = 256.  The Q
  // loads go out first, then the wave's first tile, and only then are the Q
  // values stored and published, so that the two memory latencies overlap.
  __shared__ bf16x8 sm_q[NB][KS][64];
  // the four waves' O^T chunks for the final merge (fused step: first the V^T
  // staging of the new positions, which is consumed before the merge starts)
  constexpr int U = DB * 4;
  __shared__ f32x4 sm_acc[NW][U][64];
  static_assert(sizeof(sm_acc) >= D * kVtRow * sizeof(uint16_t), "V^T staging fits the merge buffer");
  constexpr int kQPer = NB * KS * 64 / NT;   // Q operands per thread
  static_assert(kQPer * NT == NB * KS * 64, "Q operands split evenly over the threads");
  // The sequence length and the wave's first page id are read first: the tile
  // loads depend on them.  The tiles of a ring do not depend on its position
  // count, which is read after they are issued (except by the workgroup of a
  // fused step's new positions, whose positions are counted from it).
  const int len_raw = RING ? 0 : a.seq_lens[b];
  const int64_t t_raw = RING ? a.ring_T[b] : 0;   // issued here, waited for below
  const int kb_first = s * a.kb_per_split + wave;
  const int page_first =
      RING ? 0 : a.block_table[(size_t)b * a.max_pages + min(kb_first >> 1, a.max_pages - 1)];
  bf16x8 qv[kQPer];
#pragma unroll
  for (int r = 0; r < kQPer; ++r) {
    const int idx = threadIdx.x + NT * r;
    const int ln = idx & 63;
    const int ks = (idx >> 6) % KS;
    const int rb = idx / (64 * KS);
    const int row = row0 + rb * 32 + (ln & 31);
    // rows past R repeat row 0: their results are never written
    const int rr = row < a.R ? row : 0;
    const int qi = rr / a.G;
    const int hl = rr - qi * a.G;
    qv[r] = ld_bf16x8(a.q + ((size_t)(b * a.n_q + qi) * a.Hq + g * a.G + hl) * D + ks * 16 +
                      (ln >> 5) * 8);
  }
  // ring: the position count, clamped (step: room for the new positions).  The
  // empty asm is its first use: the wait for the load goes there, after the
  // tile loads issued before it, and not before them.
  auto ring_count = [&]() {
    int64_t t64 = t_raw;
    asm volatile("" : "+v"(t64));
    const int64_t t_max = STEP ? INT_MAX - 64 : INT_MAX;
    return t64 < 0 ? 0 : (t64 > t_max ? (int)t_max : (int)t64);
  };
  const int L = RING ? a.C : (len_raw < 0 ? 0 : (len_raw > a.max_keys ? a.max_keys : len_raw));
  const int nkb = (int)(((unsigned)L + 31u) >> 5);   // L >= 0
  // Truncated paged index (win): the key set [0, sink_end) u [r0, L) as virtual
  // tiles, the sink tiles [0, st_end) then the recent tiles from kr on; phys()
  // maps a virtual tile to its 32-key tile of the sequence.
  int sink_end = L, r0 = 0, st_end = 0, kr = 0, nvt = nkb;
  if (!RING && a.win) {
    sink_end = min(a.n_sink, L);
    r0 = max(a.n_sink, L - a.n_recent);
    st_end = (int)(((unsigned)sink_end + 31u) >> 5);
    kr = max(r0 >> 5, st_end);
    nvt = st_end + max(nkb - kr, 0);
  }
  auto phys = [&](int u) { return (!RING && a.win && u >= st_end) ? kr + (u - st_end) : u; };
  const int kb0 = newk ? 0 : s * a.kb_per_split;
  const int kb1 = newk ? 1 : min(kb0 + a.kb_per_split, nvt);   // new positions: one tile
  asm volatile("" ::: "memory");
  // Loop over this wave's tiles.  K registers are refilled with the next tile as
  // soon as the S^T products have consumed them, V registers as soon as the PV
  // products have: one tile of each is always in flight.  Loads are
  // unconditional (a tile with a bad page id is loaded from page 0 and then
  // masked), so the loop carries the tile registers without copies.
  KTile<D, RING, KV8> kt;
  VTile<D, KV8> vt;
  int kb = kb0 + wave;
  bool ok = false;
  int T0 = 0;
  // Store the loaded Q operands and publish them: the barrier waits for this
  // wave's LDS stores only, so the tile loads stay in flight across it.  Each
  // path below stages Q itself, after its own tile loads: with one shared copy
  // after the paths join, the wait for the Q loads would be counted as if
  // either path's loads might be the newer ones, and the ring splits would
  // wait for their whole first tile before staging Q.
  auto stage_q = [&]() {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int r = 0; r < kQPer; ++r) {
      const int idx = threadIdx.x + NT * r;
      sm_q[idx / (64 * KS)][(idx >> 6) % KS][idx & 63] = qv[r];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  {
    // unconditional (a wave without tiles loads a valid tile it never uses), so
    // that the Q stores wait only for the Q loads
    const int kbl = kb < kb1 ? kb : 0;
    size_t tile;
    if (newk) {
      tile = 0;
    } else if (RING) {
      tile = tile_index<RING>(a, b, g, kbl, ok);
    } else if (a.win) {   // the page of the first tile depends on L here
      tile = tile_index<RING>(a, b, g, phys(kbl), ok);
    } else {
      tile = tile_of_page(a, kb < kb1 ? page_first : 0, g, kbl, ok);
    }
    if (STEP && newk) {
      if constexpr (STEP) {
        load_k_new<D>(kt, a, b, g, m, h);
        ok = true;
        stage_v_new<D, NT>(reinterpret_cast<uint16_t*>(&sm_acc[0][0][0]), a, b, g);
        stage_q();
        load_v_new<D>(vt, reinterpret_cast<const uint16_t*>(&sm_acc[0][0][0]), m, h);
        T0 = ring_count();
        new_positions<D>(kt, a, T0, h);
      }
    } else {
      load_k<D, RING, KV8, RING || WIN>(kt, a, tile, b, kbl, m, h);
      load_v<D, KV8, RING || WIN>(vt, a, tile, m, h);
      asm volatile("" ::: "memory");
      if (RING) T0 = ring_count();
      stage_q();
    }
  }
  // Ring: the window ends at T.  Fused step: T counts the new positions too; the
  // slots they will overwrite hold positions outside the window, so the window
  // test skips them, and p_end stops the ring splits at the count before the
  // append (slots holding positions >= T0, left by a rollback, are skipped; the
  // new positions' workgroup reads T0 .. T - 1).
  const int T = RING ? (STEP ? T0 + a.app.n_new : T0) : 0;
  const int p_end = (STEP && !newk) ? T0 : T;
  int lim[NB];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int row = row0 + rb * 32 + m;
    // paged: keys visible to the row (causal limit); ring: the row's query position
    if (RING)
      lim[rb] = T - a.n_q + (row < a.R ? row / a.G : a.n_q - 1);
    else
      lim[rb] = row < a.R ? L - a.n_q + row / a.G + 1 : L;
  }
  // tree verify: each row's ancestor mask over the appended positions
  uint64_t tmask[NB];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const int row = row0 + rb * 32 + m;
    tmask[rb] = (!RING && a.tree_mask && row < a.R) ? a.tree_mask[(size_t)b * a.n_q + row / a.G] : 0;
  }

  // The accumulators are set to zero right before a wave's first PV (or at
  // the end, for a wave without tiles), so that the products start from the
  // constant instead of a zeroed register block.
  SoftmaxState<D, NB> st;
  auto zero_acc = [&]() {
#pragma unroll
    for (int rb = 0; rb < NB; ++rb)
#pragma unroll
      for (int db = 0; db < DB; ++db) st.acc[rb][db] = f32x16{};
  };
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    st.m[rb] = -INFINITY;
    st.l[rb] = 0.f;
    st.l_drop[rb] = 0.f;
  }

  int kbn = kb;
  bool ok_n = false;
  size_t tile_n = 0;
  float x[NB][16], mx[NB];
  uint32_t keep = 0;
  bool mask_v = false;
  auto next_tile = [&]() {
    kbn = kb + NW;
    tile_n = tile_index<RING>(a, b, g, phys(kbn), ok_n);
  };
  auto advance = [&]() {
    ok = ok_n;
    kb = kbn;
  };
  // S^T of tile kb, refill K (when there is a next tile), masked scores.
  auto scores_of = [&](auto has_next) {
    const int pk = phys(kb);   // the tile's place in the sequence
    keep = ok ? present_keys<D, RING, KV8>(kt, a, pk, L, T, p_end, h, sink_end, r0) : 0u;
    bool all_vis;
    uint32_t rvis[NB];   // ring, several queries: the keys in each row's own window
    if (RING) {
      mask_v = !__all(keep == 0xFFFFu);
      bool rows_all = true;
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) {
        rvis[rb] = keep;
        if (a.n_q > 1) {
          const int pq = lim[rb];
          uint32_t v = 0;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int p = kt.pos[i];
            v |= ((p <= pq) & ((p < a.n_sink) | (p > pq - a.n_recent)) ? 1u : 0u) << i;
          }
          rvis[rb] &= v;
        }
        rows_all = rows_all && rvis[rb] == 0xFFFFu;
      }
      all_vis = __all(rows_all);
    } else {
      // every key present and visible to every row (smallest causal limit L - n_q + 1)
      const bool in_set = !a.win || pk * 32 >= r0 || (pk + 1) * 32 <= sink_end;
      // (a tree's first appended position need not be visible to every row)
      all_vis = ok && in_set && (pk + 1) * 32 <= L - a.n_q + (a.tree_mask ? 0 : 1);
      mask_v = !ok || !in_set || (pk + 1) * 32 > L;
    }
    f32x16 sacc[NB];
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      sacc[rb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sacc[rb] = mfma32x32x16(as_operand(kt.k[ks]), sm_q[rb][ks][lane], sacc[rb]);
      // A wave's last tile, bf16 K: keep four Q reads from LDS in flight ahead
      // of the products (left to itself, the scheduler serialises them at
      // D = 256, where the registers are short: one LDS round trip per
      // product).  That tile's products are on the wave's critical path; the
      // others overlap the next tile's loads, and there the constraint costs
      // more than it saves (native draft at 1M keys: 84 % of peak HBM
      // bandwidth without it, 82 % with it).  fp8 K converts each operand
      // first, which spaces the reads out already, and at D = 128 the extra
      // registers would cost it its second workgroup per CU.
      if constexpr (!KV8 && !decltype(has_next)::value) {
        constexpr int QD = KS < 4 ? KS : 4;
        __builtin_amdgcn_sched_group_barrier(0x100, QD, 0);   // LDS reads
#pragma unroll
        for (int ks = 0; ks < KS - QD; ++ks) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, QD, 0);
      }
    }
    if constexpr (decltype(has_next)::value) load_k<D, RING, KV8, RING || WIN>(kt, a, tile_n, b, kbn, m, h);
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      uint32_t vis;
      if (RING)
        vis = rvis[rb];
      else if (a.tree_mask)
        vis = keep & (keys_below(L - a.n_q - pk * 32, h) |
                      tree_keys(tmask[rb], pk * 32 - (L - a.n_q), h));
      else
        vis = keep & keys_below(lim[rb] - pk * 32, h);
      mx[rb] = masked_scores(x[rb], sacc[rb], vis, all_vis, a.scale_log2);
    }
  };
  // Weights, PV, refill V (when there is a next tile).
  auto finish = [&](auto has_next) {
    bf16x8 p_hi[NB][2], p_lo[NB][2];
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) weights<D, NB>(st, rb, x[rb], a.scale_log2, p_hi[rb], p_lo[rb]);
    if constexpr (KV8) {
      bf16x8 vv[DB][2];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          vv[db][kk] = fp8x8_to_bf16(vt.v[db][kk]);
          // absent keys may hold any bits (an fp8 NaN too): zero them
          if (mask_v) vv[db][kk] = mask8(vv[db][kk], (keep >> (8 * kk)) & 0xFFu);
        }
      // the raw V bytes are converted: refill them now, so that the next tile's V
      // loads run under this tile's PV products
      if constexpr (decltype(has_next)::value) load_v<D, KV8, RING || WIN>(vt, a, tile_n, m, h);
      pv<D, NB>(st, vv, p_hi, p_lo);
    } else {
      if (mask_v) {
        // Absent keys may hold any bits (even NaN): zero their values so that
        // 0-weight * value stays 0 in the PV product.
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) vt.v[db][kk] = mask8(vt.v[db][kk], (keep >> (8 * kk)) & 0xFFu);
      }
      pv<D, NB>(st, vt.v, p_hi, p_lo);
    }
    if constexpr (!KV8 && decltype(has_next)::value) load_v<D, KV8, RING || WIN>(vt, a, tile_n, m, h);
  };
  const std::true_type more;
  const std::false_type last;

  // Ring windows (a tile or two per wave): a wave's first tile takes the rows'
  // first maxima (no row has one yet, so nothing is rescaled) and its PV starts
  // the accumulators, which are then never zeroed in registers.  The long
  // paged passes zero them up front and keep one copy of the loop body: there
  // the saving is one tile's worth in dozens.  (The two structures are written
  // out in full: at D = 256 the register allocation of either is fragile.)
  if constexpr (RING) {
    if (kb >= kb1) {
      zero_acc();   // no tiles
    } else if (kb + NW >= kb1) {
      scores_of(last);   // the only tile
      first_max_or_rescale<D, NB>(st, mx);
      zero_acc();
      finish(last);
    } else {
      next_tile();
      scores_of(more);
      first_max_or_rescale<D, NB>(st, mx);
      zero_acc();
      finish(more);
      advance();
      // Fast loop over the tiles that have a successor: no accumulator rescale.
      // It leaves early when tile kb needs one; its scores are then already in
      // x / mx.
      bool general = false;
      while (kb + NW < kb1) {
        next_tile();
        scores_of(more);
        if (first_max_or_rescale<D, NB>(st, mx)) {
          general = true;
          break;
        }
        finish(more);
        advance();
      }
      // General loop, from the tile the fast loop left on.
      if (general) {
        raise_and_rescale<D, NB>(st, mx);
        finish(more);
        advance();
        while (kb + NW < kb1) {
          next_tile();
          scores_of(more);
          raise_and_rescale<D, NB>(st, mx);
          finish(more);
          advance();
        }
      }
      // The wave's last tile.
      scores_of(last);
      if (general || first_max_or_rescale<D, NB>(st, mx)) raise_and_rescale<D, NB>(st, mx);
      finish(last);
    }
  } else {
    zero_acc();
    // Fast loop over the tiles that have a successor: no accumulator rescale.
    // It leaves early when tile kb needs one; its scores are then already in
    // x / mx.
    bool general = false;
    while (kb + NW < kb1) {
      next_tile();
      scores_of(more);
      if (first_max_or_rescale<D, NB>(st, mx)) {
        general = true;
        break;
      }
      finish(more);
      advance();
    }
    // General loop, from the tile the fast loop left on.
    if (general) {
      raise_and_rescale<D, NB>(st, mx);
      finish(more);
      advance();
      while (kb + NW < kb1) {
        next_tile();
        scores_of(more);
        raise_and_rescale<D, NB>(st, mx);
        finish(more);
        advance();
      }
    }
    // The wave's last tile.
    if (kb < kb1) {
      scores_of(last);
      if (general || first_max_or_rescale<D, NB>(st, mx)) raise_and_rescale<D, NB>(st, mx);
      finish(last);
    }
  }

  // ---- merge the four waves' states through LDS, one row block at a time ----
  // Every wave stores its rescaled O^T chunks (chunk u = 4*db + c: dims
  // 32*db + 8*c + 4*h .. +3 of row m), then wave w sums and writes chunks
  // [w*U/4, (w+1)*U/4) of all four waves.  When the row group holds at most 16
  // query rows, lanes m >= 16 carry no results: a swap of 16-lane rows then
  // packs two chunks into one register (lanes 16..31 and 48..63 take the next
  // chunk of rows m - 16), which halves the LDS traffic and the stores.
  __shared__ float sm_m[NW][32];
  __shared__ float sm_l[NW][32];
  const bool pack = NB == 1 && a.R - row0 <= 16;   // uniform
  // the query row this lane writes, and which chunk of a packed pair it carries
  const int orow = pack ? (lane & 15) : m;
  const int half = pack ? (lane >> 4) & 1 : 0;

#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const float lsum = sum_over_row(st.l[rb]);
    __syncthreads();   // previous round's readers are done with the buffers
    if (h == 0) {
      sm_m[wave][m] = st.m[rb];
      sm_l[wave][m] = lsum;
    }
    __syncthreads();
    // this lane's own row m: the factor that brings its state to the row maximum
    float Mo = sm_m[0][m];
#pragma unroll
    for (int w = 1; w < NW; ++w) Mo = fmaxf(Mo, sm_m[w][m]);
    const float f = fast_exp2(st.m[rb] - ((Mo == -INFINITY) ? 0.f : Mo));
    // the row it writes: maximum and total weight
    float M = sm_m[0][orow];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][orow]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Ltot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) Ltot += sm_l[w][orow] * fast_exp2(sm_m[w][orow] - Mu);
    auto chunk = [&](int u) {
      const int db = u >> 2, c = u & 3;
      const f32x4 v = {st.acc[rb][db][4 * c], st.acc[rb][db][4 * c + 1],
                       st.acc[rb][db][4 * c + 2], st.acc[rb][db][4 * c + 3]};
      return v * f;
    };
    if (pack) {
#pragma unroll
      for (int v = 0; v < U / 2; ++v) {
        f32x4 x = chunk(2 * v);
        const f32x4 y = chunk(2 * v + 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // 16-lane rows 1 and 3 of x (lanes 16..31, 48..63) take rows 0 and 2 of y
          const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[e]),
                                                          __float_as_uint(y[e]), false, false);
          x[e] = __uint_as_float(r[0]);
        }
        sm_acc[wave][v][lane] = x;
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) sm_acc[wave][u][lane] = chunk(u);
    }
    __syncthreads();
    const int row = row0 + rb * 32 + orow;
    if (row < a.R) {
      const float inv = (Ltot > 0.f ? 1.f / Ltot : 0.f) * (KV8 ? a.v_scale : 1.f);
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
      // this wave's share of the stored entries: n from j0 on; entry j holds
      // chunk 2 j + half (packed) or chunk j
      auto write = [&](int j0, int n) {
#pragma unroll
        for (int j = 0; j < n; ++j) {
          const int jj = j0 + j;
          f32x4 v = sm_acc[0][jj][lane];
#pragma unroll
          for (int w = 1; w < NW; ++w) v += sm_acc[w][jj][lane];
          const int u = pack ? 2 * jj + half : jj;
          *reinterpret_cast<f32x4*>(op + (u >> 2) * 32 + 8 * (u & 3) + 4 * h) = v * inv;
        }
      };
      if (pack)
        write(wave * (U / 2 / NW), U / 2 / NW);
      else
        write(wave * (U / NW), U / NW);
      if (wave == 0 && lane < (pack ? 16 : 32) && lp)
        *lp = Ltot > 0.f ? (M + fast_log2(Ltot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int NB, bool RING, bool KV8, bool WIN = false>
hipError_t launch_one(const AttnArgs& a, int grid, hipStream_t stream) {
  AttnArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_split_kernel<D, NB, RING, KV8, false, WIN>),
                         dim3(grid), dim3(256), args, 0, stream);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& p, bool ring, hipStream_t stream) {
  if (p.nrb != 1) return hipErrorInvalidValue;
  if (ring) return launch_one<D, 1, true, false>(a, p.grid, stream);
  if (a.win)
    return a.kv8 ? launch_one<D, 1, false, true, true>(a, p.grid, stream)
                 : launch_one<D, 1, false, false, true>(a, p.grid, stream);
  return a.kv8 ? launch_one<D, 1, false, true>(a, p.grid, stream)
               : launch_one<D, 1, false, false>(a, p.grid, stream);
}

template <int D>
hipError_t launch_step_d(const AttnArgs& a, int grid, hipStream_t stream) {
  AttnArgs arg = a;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_split_kernel<D, 1, true, false, true>),
                         dim3(grid), dim3(256), args, 0, stream);
}

}  // namespace

bool plan_window_step(int B, int Hq, int Hkv, int D, int n_q, int C, int num_splits,
                      AttnPlan* p) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || n_q < 1 || num_splits < 0 || C < 64 ||
      C % 64 != 0)
    return false;
  if (D != 64 && D != 128 && D != 256) return false;
  p->G = Hq / Hkv;
  if ((long)n_q * p->G > 256) return false;
  p->R = n_q * p->G;
  p->shared = 0;
  p->nrb = 1;
  p->nrg = (p->R + 31) / 32;
  p->nkb = C / 32;
  // default: the windowed draft's plan (one workgroup per CU, at least four
  // tiles, one per wave, per split).  Measured at 2 x 128 tiles, D = 256: four
  // waves of one tile each in 64 workgroups take 12.7 us a step against 13.8 us
  // for 256 one-wave workgroups, whose four times as many partials the merge
  // launch then reads.
  int kbps;
  if (num_splits > 0) {
    kbps = (int)(((long)p->nkb + num_splits - 1) / num_splits);
  } else {
    const long units = (long)B * Hkv * p->nrg;
    const long per_unit = units < WMTP_TARGET_WG_SPLIT ? WMTP_TARGET_WG_SPLIT / units : 1;
    const long per = ((long)p->nkb + per_unit - 1) / per_unit;
    kbps = (int)(per < 4 ? 4 : per);
  }
  p->kb_per_split = kbps;
  p->nsplit = (p->nkb + kbps - 1) / kbps;
  p->direct = 0;
  const long items = (long)B * Hkv * (p->nsplit + 1);
  if (items * p->nrg > INT_MAX / 16) return false;
  p->items = (int)items;
  p->grid = p->nrg == 1 ? p->items : ((p->items + 7) / 8) * 8 * p->nrg;
  p->part_o_bytes = (size_t)items * p->R * D * sizeof(float);
  p->lse_offset = ((p->part_o_bytes + 255) / 256) * 256;
  p->ws_bytes = p->lse_offset + (size_t)items * p->R * sizeof(float);
  return true;
}

hipError_t launch_window_step(const AttnArgs& a, const AttnPlan& p, hipStream_t stream) {
  switch (a.D) {
    case 64: return launch_step_d<64>(a, p.grid, stream);
    case 128: return launch_step_d<128>(a, p.grid, stream);
    case 256: return launch_step_d<256>(a, p.grid, stream);
    default: return hipErrorInvalidValue;
  }
}

bool plan_attention(int B, int Hq, int Hkv, int D, int n_q, int max_keys, int num_splits,
                    int partials_only, bool ring, AttnPlan* p, bool kv8) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || n_q < 1 || max_keys < 0 || num_splits < 0)
    return false;
  if (D != 64 && D != 128 && D != 256) return false;
  p->G = Hq / Hkv;
  if ((long)n_q * p->G > 256) return false;
  p->R = n_q * p->G;
  p->nkb = (int)(((long)max_keys + 31) / 32);
  const long groups = (long)B * Hkv;
  long target;    // workgroups to aim at
  int cap;        // most 32-key tiles per split
  // Few rows: each wave holds every row and the four waves split the keys.
  // Two row blocks per wave need too many registers at D = 256 (they spill).
  p->nw = 0;
  if (ring || p->R <= 32) {
    p->shared = 0;
    p->nrb = 1;                             // one 32-row block per wave
    p->nrg = (p->R + 31) / 32;
    target = WMTP_TARGET_WG_SPLIT;
    cap = INT_MAX;
  } else {
    // Many rows: the waves split the rows and share each K/V tile through LDS.
    // A wave holds 32 * rbw rows: the fewest that cover R, at most one block at
    // D = 256 and two below (register file); beyond that the rows go to row groups.
    p->shared = 1;
    int nw = shared_kernel_waves();
    const int rbw_max = D == 256 ? 1 : 2;
    int rbw = 1;
    if (D == 128 && p->R > 32 * nw) {
      // more rows than four waves of 32 hold at D = 128: eight waves of 32 rows, two
      // per SIMD, so that one wave's refill and softmax stalls overlap the other's
      // MFMAs (instead of four waves of 64 rows, one per SIMD)
      nw = 8;
    } else {
      while (rbw < rbw_max && 32 * nw * rbw < p->R) rbw *= 2;
    }
    p->nw = nw;
    p->nrb = rbw;
    p->nrg = (p->R + 32 * nw * rbw - 1) / (32 * nw * rbw);
    target = WMTP_TARGET_WG_SHARED;
    cap = shared_kernel_max_tiles();
  }
  // Several long sequences: their lengths are on the device, so the plan cannot
  // balance them.  It aims at four workgroups per CU instead of one and lets the
  // dispatcher, which gives a CU its next workgroup when one ends, even out the
  // unequal lengths (measured on 8 sequences of 256K..1M keys: the native draft
  // pass at 81 % of peak HBM bandwidth against 72 % with one round, the verify
  // at 79 % against 72 %).  One sequence keeps one round (its second round
  // would add a prologue, a merge and a tail), and short key ranges (windows) too.
  if (!ring && B > 1 && p->nkb >= 2048) target *= 4;
  // fp8 caches at D = 128: the split kernel fits two workgroups per CU (246
  // registers per wave, 73 KB of LDS), and with 8 KB per tile it needs the second
  // one's loads in flight: twice the workgroups for long key ranges (measured at
  // 128K keys, 32/4 heads: 33 us against 44 us; the bf16 kernel, at 283
  // registers, stays at one per CU)
  if (kv8 && D == 128 && !ring && !p->shared && p->nkb >= 2048) target *= 2;
  int kbps;
  if (num_splits > 0) {
    kbps = (int)(((long)p->nkb + num_splits - 1) / num_splits);
  } else {
    // As many splits per (group, row group) as keep the workgroups within the
    // target, the tiles spread evenly over them: at one workgroup per CU, a
    // workgroup past the target would run as a second round on its own (a
    // length just past a round number would otherwise add a one-tile split).
    const long units = groups * p->nrg;
    const long per_unit = units < target ? target / units : 1;
    const long per = ((long)p->nkb + per_unit - 1) / per_unit;
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
