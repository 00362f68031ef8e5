// Host-side launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wmtp {

struct RingAppendArgs {
  uint16_t* kc;
  uint16_t* vc;
  int32_t* ring_pos;
  int64_t* ring_T;
  const uint16_t* k_new;
  const uint16_t* v_new;
  int B, n_new, Hkv, D, C, n_sink;
};

// Arguments of the split-KV attention kernel (draft full, draft window, verify).
struct AttnArgs {
  const uint16_t* q;            // bf16 [B][n_q][Hq][D]
  const uint16_t* kc;           // K tiled pages
  const uint16_t* vc;           // V tiled pages
  const int32_t* block_table;   // paged mode: [B][max_pages]
  const int32_t* seq_lens;      // paged mode: [B]
  const int32_t* ring_pos;      // ring mode: [B][C]
  const int64_t* ring_T;        // ring mode: [B]
  const uint64_t* tree_mask;    // paged verify: [B][n_q] ancestor masks, or null (causal)
  float* out_o;                 // partials (split mode) or final o (direct mode)
  float* out_lse;               // partials or final lse (may be null in direct mode)
  int B, Hq, Hkv, G, n_q, R, D;
  int num_pages;                // pages addressable through kc/vc
  int max_pages;                // block-table row stride (paged mode)
  int max_keys;                 // keys considered per sequence: min(max_seq_len, max_pages*64) or C
  int nsplit;                   // key splits per (b, g)
  int kb_per_split;             // 32-key tiles per split
  int items;                    // B * Hkv * nsplit
  int nrg;                      // row groups (16 * NRB rows each)
  int direct;                   // 1: write final o/lse, 0: write partials
  int C, n_sink, n_recent;      // ring mode; paged mode with win: the key set
  int win;                      // paged mode: 1 = keys [0, n_sink) and the last n_recent only
  int kv8;                      // paged mode: kc/vc hold fp8 e4m3 tiles (1 byte per element)
  float v_scale;                // kv8: value of a V code = code value * v_scale (K's scale is
                                // folded into scale_log2)
  float scale_log2;             // softmax_scale * log2(e)
  // Fused windowed draft step (ring mode): the n_new positions ring_T ..
  // ring_T + n_new - 1 come from app.k_new / app.v_new, read by one more
  // workgroup per group (split index nsplit); the ring itself is read as it
  // stands and written afterwards by the combine launch.
  RingAppendArgs app;
};

struct AttnPlan {
  int shared;   // 0: attn_split_kernel (one wave holds all rows, waves split keys)
                // 1: attn_shared_kernel (waves split rows, K/V tiles shared in LDS)
  int G, R, nrb, nrg, nkb, kb_per_split, nsplit, items, grid;
  int nw;       // attn_shared_kernel: waves per workgroup (4, or 8 at D = 128 with many rows)
  int direct;
  size_t part_o_bytes, lse_offset, ws_bytes;
};

// kv8: the call reads fp8 caches (the plan may then aim at more workgroups)
bool plan_attention(int B, int Hq, int Hkv, int D, int n_q, int max_keys, int num_splits,
                    int partials_only, bool ring, AttnPlan* p, bool kv8 = false);

hipError_t launch_attention(const AttnArgs& a, const AttnPlan& p, bool ring, hipStream_t stream);

// Fused windowed draft step (n_q queries): ring splits as the windowed draft plans
// them, plus one workgroup per group (and row group) for the new positions; items =
// B * Hkv * (nsplit + 1) partials of R = n_q * Hq / Hkv <= 256 rows.
bool plan_window_step(int B, int Hq, int Hkv, int D, int n_q, int C, int num_splits,
                      AttnPlan* p);
hipError_t launch_window_step(const AttnArgs& a, const AttnPlan& p, hipStream_t stream);
hipError_t launch_attention_shared(const AttnArgs& a, const AttnPlan& p, hipStream_t stream);
int shared_kernel_waves();
int shared_kernel_max_tiles();   // most 32-key tiles one split of the shared kernel covers

struct CombineArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* indptr;   // may be null
  int n_parts;             // partials addressable; indptr entries are clamped to it
  int splits_per_group;
  int B, Hkv, G, n_q, D, R;
  float* o;
  float* lse;              // may be null
  // Fused windowed draft step: after the combine's workgroups, app.B more append
  // app.n_new positions to the rings (one workgroup per request, as
  // wmtp_ring_append does).  Only with R < 64.
  int append;
  RingAppendArgs app;
};

hipError_t launch_combine(const CombineArgs& c, hipStream_t stream);

hipError_t launch_ring_append(const RingAppendArgs& a, hipStream_t stream);

struct PagedAppendArgs {
  uint16_t* kc;
  uint16_t* vc;
  const int32_t* block_table;
  const int32_t* start_pos;
  const uint16_t* k_new;
  const uint16_t* v_new;
  int B, n_new, Hkv, D, num_pages, max_pages;
  int kv8;                      // kc/vc hold fp8 e4m3 tiles: store code(x * k_inv) etc.
  float k_inv, v_inv;
};

hipError_t launch_paged_append(const PagedAppendArgs& a, hipStream_t stream);

}  // namespace wmtp
