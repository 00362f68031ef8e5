// C ABI of libwmtp (declared in include/wmtp.h): host-side argument checks,
// split planning and kernel launches.  No call allocates device memory; the one
// library-owned buffer is the static scratch below, part of the code object.
#include "wmtp.h"

#include "internal.h"

#include <climits>
#include <cmath>
#include <mutex>

using namespace wmtp;

namespace {

// Library-owned scratch for wmtp_draft_step_window_static: the split partials of
// one fused windowed draft step, for callers that cannot allocate a workspace.
// One copy per GPU, alive until the process ends.  In host code `scratch` names
// a host-side stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, once per device (static_scratch below).
__device__ __align__(256) unsigned char scratch[WMTP_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch (the current device, which must be the
// stream's): looked up on the first call on a device and kept.
wmtp_status static_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WMTP_ERR_HIP;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return WMTP_ERR_HIP;
    if (sdev != dev) return WMTP_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WMTP_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return WMTP_OK;
}

constexpr float kLog2e = 1.4426950408889634f;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
bool head_dim_ok(int D) { return D == 64 || D == 128 || D == 256; }

wmtp_status from_hip(hipError_t e) { return e == hipSuccess ? WMTP_OK : WMTP_ERR_HIP; }

// Keys to plan a truncated paged index for (window n_sink + n_recent = w): its
// virtual tiles number at most ceil(w / 32) + 2 (the sink part and the recent part
// may each start or end inside a tile).
int window_plan_keys(long w, int max_keys) {
  const long k = 32 * ((w + 31) / 32 + 2);
  return k < max_keys ? (int)k : max_keys;
}

// Common tail of the attention calls: plan (for plan_keys keys per sequence),
// check the workspace, launch the split pass and, when there is more than one
// split, the combine.
wmtp_status run_attention(AttnArgs a, bool ring, int max_keys, int plan_keys, float* o,
                          float* lse, void* workspace, size_t workspace_bytes, int num_splits,
                          unsigned flags, hipStream_t stream) {
  const int partials_only = (flags & WMTP_FLAG_PARTIALS_ONLY) ? 1 : 0;
  AttnPlan p;
  if (!plan_attention(a.B, a.Hq, a.Hkv, a.D, a.n_q, plan_keys, num_splits, partials_only, ring,
                      &p, a.kv8 != 0))
    return ((long)a.n_q * (a.Hq / a.Hkv) > 256) ? WMTP_ERR_UNSUPPORTED : WMTP_ERR_INVALID_ARG;
  if (a.win && p.shared) return WMTP_ERR_UNSUPPORTED;   // truncated index: split kernel only
  if (p.ws_bytes > 0) {
    if (!workspace || !aligned16(workspace)) return WMTP_ERR_WORKSPACE;
    if (workspace_bytes < p.ws_bytes) return WMTP_ERR_WORKSPACE;
  }
  a.G = p.G;
  a.R = p.R;
  a.nsplit = p.nsplit;
  a.kb_per_split = p.kb_per_split;
  a.items = p.items;
  a.nrg = p.nrg;
  a.direct = p.direct;
  a.max_keys = max_keys;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = p.ws_bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                          p.lse_offset)
                               : nullptr;
  if (p.direct) {
    a.out_o = o;
    a.out_lse = lse;
  } else {
    a.out_o = part_o;
    a.out_lse = part_lse;
  }
  hipError_t e = launch_attention(a, p, ring, stream);
  if (e != hipSuccess) return WMTP_ERR_HIP;
  if (p.direct || partials_only) return WMTP_OK;
  CombineArgs c = {};
  c.part_o = part_o;
  c.part_lse = part_lse;
  c.indptr = nullptr;
  c.n_parts = p.items;
  c.splits_per_group = p.nsplit;
  c.B = a.B;
  c.Hkv = a.Hkv;
  c.G = p.G;
  c.n_q = a.n_q;
  c.D = a.D;
  c.R = p.R;
  c.o = o;
  c.lse = lse;
  return from_hip(launch_combine(c, stream));
}

bool attn_dims_ok(int B, int Hq, int Hkv, int D) {
  return B >= 1 && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0;
}

}  // namespace

extern "C" {

const char* wmtp_status_string(int status) {
  switch (status) {
    case WMTP_OK: return "ok";
    case WMTP_ERR_INVALID_ARG: return "invalid argument";
    case WMTP_ERR_UNSUPPORTED: return "unsupported configuration";
    case WMTP_ERR_WORKSPACE: return "workspace missing or too small";
    case WMTP_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

int wmtp_plan_splits(int call, int B, int Hq, int Hkv, int D, int n_q, int max_keys,
                     int num_splits) {
  AttnPlan p;
  if (call == WMTP_CALL_RING_STEP) {
    if (!plan_window_step(B, Hq, Hkv, D, n_q, max_keys, num_splits, &p)) return -1;
    return p.nsplit;
  }
  if (call != WMTP_CALL_PAGED && call != WMTP_CALL_RING && call != WMTP_CALL_PAGED_WINDOW &&
      call != WMTP_CALL_PAGED_FP8)
    return -1;
  if (call == WMTP_CALL_PAGED_WINDOW) {
    if (max_keys < 0) return -1;
    max_keys = window_plan_keys(max_keys, INT_MAX);
  }
  if (!plan_attention(B, Hq, Hkv, D, n_q, max_keys, num_splits, 0, call == WMTP_CALL_RING, &p,
                      call == WMTP_CALL_PAGED_FP8))
    return -1;
  return p.nsplit;
}

size_t wmtp_workspace_bytes(int call, int B, int Hq, int Hkv, int D, int n_q, int max_keys,
                            int num_splits, int partials_only) {
  AttnPlan p;
  if (call == WMTP_CALL_RING_STEP) {
    if (!plan_window_step(B, Hq, Hkv, D, n_q, max_keys, num_splits, &p)) return 0;
    return p.ws_bytes;
  }
  if (call != WMTP_CALL_PAGED && call != WMTP_CALL_RING && call != WMTP_CALL_PAGED_WINDOW &&
      call != WMTP_CALL_PAGED_FP8)
    return 0;
  if (call == WMTP_CALL_PAGED_WINDOW) {
    if (max_keys < 0) return 0;
    max_keys = window_plan_keys(max_keys, INT_MAX);
  }
  if (!plan_attention(B, Hq, Hkv, D, n_q, max_keys, num_splits, partials_only,
                      call == WMTP_CALL_RING, &p, call == WMTP_CALL_PAGED_FP8))
    return 0;
  return p.ws_bytes;
}

// win: keys [0, n_sink) and the last n_recent of each sequence only.
static wmtp_status paged_attention(const uint16_t* q, const uint16_t* k_cache,
                                   const uint16_t* v_cache, const int32_t* block_table,
                                   const int32_t* seq_lens, int B, int n_q, int Hq, int Hkv,
                                   int D, int num_pages, int max_pages, int max_seq_len,
                                   float softmax_scale, float* o, float* lse, void* workspace,
                                   size_t workspace_bytes, int num_splits, unsigned flags,
                                   void* stream, bool win = false, int n_sink = 0,
                                   int n_recent = 0, const uint64_t* tree_mask = nullptr,
                                   bool kv8 = false, float k_scale = 1.f, float v_scale = 1.f) {
  if (!attn_dims_ok(B, Hq, Hkv, D) || n_q < 1) return WMTP_ERR_INVALID_ARG;
  if (!head_dim_ok(D)) return WMTP_ERR_UNSUPPORTED;
  if ((long)n_q * (Hq / Hkv) > 256) return WMTP_ERR_UNSUPPORTED;
  if (num_pages < 1 || max_pages < 1 || max_seq_len < 0 || num_splits < 0)
    return WMTP_ERR_INVALID_ARG;
  if ((flags & ~WMTP_FLAG_PARTIALS_ONLY) != 0) return WMTP_ERR_INVALID_ARG;
  // the kernels take row maxima of raw scores before scaling: the scale must be positive
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return WMTP_ERR_INVALID_ARG;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens) return WMTP_ERR_INVALID_ARG;
  if (!(flags & WMTP_FLAG_PARTIALS_ONLY) && !o) return WMTP_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || (o && !aligned16(o)) ||
      !aligned4(block_table) || !aligned4(seq_lens) || (lse && !aligned4(lse)))
    return WMTP_ERR_INVALID_ARG;
  if ((long)max_pages * 64 > (long)INT_MAX) return WMTP_ERR_INVALID_ARG;
  const int max_keys = max_seq_len < max_pages * 64 ? max_seq_len : max_pages * 64;
  AttnArgs a = {};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_q = n_q;
  a.D = D;
  a.num_pages = num_pages;
  a.max_pages = max_pages;
  a.scale_log2 = softmax_scale * kLog2e;
  a.tree_mask = tree_mask;
  if (kv8) {
    if (!std::isfinite(k_scale) || !(k_scale > 0.f) || !std::isfinite(v_scale) ||
        !(v_scale > 0.f))
      return WMTP_ERR_INVALID_ARG;
    // fp8 caches: a draft (one query) reads them through the split kernel only,
    // up to 32 query rows per kv head; a verify also through the shared kernel
    if (n_q == 1 && Hq / Hkv > 32) return WMTP_ERR_UNSUPPORTED;
    if (tree_mask) return WMTP_ERR_UNSUPPORTED;   // no fp8 tree verify
    a.kv8 = 1;
    a.scale_log2 = softmax_scale * k_scale * kLog2e;   // logits of the K codes
    a.v_scale = v_scale;
  }
  int plan_keys = max_keys;
  if (win) {
    if (n_sink < 0 || n_recent < 1) return WMTP_ERR_INVALID_ARG;
    a.win = 1;
    a.n_sink = n_sink;
    a.n_recent = n_recent;
    plan_keys = window_plan_keys((long)n_sink + n_recent, max_keys);
  }
  return run_attention(a, false, max_keys, plan_keys, o, lse, workspace, workspace_bytes,
                       num_splits, flags, static_cast<hipStream_t>(stream));
}

wmtp_status wmtp_draft_attn_full(const uint16_t* q, const uint16_t* k_cache,
                                 const uint16_t* v_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                                 int num_pages, int max_pages, int max_seq_len,
                                 float softmax_scale, float* o, float* lse, void* workspace,
                                 size_t workspace_bytes, int num_splits, unsigned flags,
                                 void* stream) {
  return paged_attention(q, k_cache, v_cache, block_table, seq_lens, B, 1, Hq, Hkv, D, num_pages,
                         max_pages, max_seq_len, softmax_scale, o, lse, workspace,
                         workspace_bytes, num_splits, flags, stream);
}

wmtp_status wmtp_draft_attn_window_paged(const uint16_t* q, const uint16_t* k_cache,
                                         const uint16_t* v_cache, const int32_t* block_table,
                                         const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                                         int num_pages, int max_pages, int max_seq_len,
                                         int n_sink, int n_recent, float softmax_scale, float* o,
                                         float* lse, void* workspace, size_t workspace_bytes,
                                         int num_splits, unsigned flags, void* stream) {
  return paged_attention(q, k_cache, v_cache, block_table, seq_lens, B, 1, Hq, Hkv, D, num_pages,
                         max_pages, max_seq_len, softmax_scale, o, lse, workspace,
                         workspace_bytes, num_splits, flags, stream, true, n_sink, n_recent);
}

wmtp_status wmtp_verify_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, int B, int n_q,
                             int Hq, int Hkv, int D, int num_pages, int max_pages,
                             int max_seq_len, float softmax_scale, float* o, float* lse,
                             void* workspace, size_t workspace_bytes, int num_splits,
                             unsigned flags, void* stream) {
  return paged_attention(q, k_cache, v_cache, block_table, seq_lens, B, n_q, Hq, Hkv, D,
                         num_pages, max_pages, max_seq_len, softmax_scale, o, lse, workspace,
                         workspace_bytes, num_splits, flags, stream);
}

// The ring calls: n_q = 1 (a draft step) or the n_q positions of a draft
// context pass, query i at position ring_T - n_q + i.
static wmtp_status ring_attention(const uint16_t* q, const uint16_t* ring_k,
                                  const uint16_t* ring_v, const int32_t* ring_pos,
                                  const int64_t* ring_T, int B, int n_q, int Hq, int Hkv, int D,
                                  int C, int n_sink, int n_recent, float softmax_scale, float* o,
                                  float* lse, void* workspace, size_t workspace_bytes,
                                  int num_splits, unsigned flags, void* stream) {
  if (!attn_dims_ok(B, Hq, Hkv, D) || n_q < 1) return WMTP_ERR_INVALID_ARG;
  if (!head_dim_ok(D)) return WMTP_ERR_UNSUPPORTED;
  if ((long)n_q * (Hq / Hkv) > 256) return WMTP_ERR_UNSUPPORTED;
  if (C < 64 || C % 64 != 0 || n_sink < 0 || n_sink >= C || n_recent < 1 ||
      n_recent > C - n_sink || num_splits < 0)
    return WMTP_ERR_INVALID_ARG;
  // the earliest query's window must still be in the ring: slack >= n_q - 1
  if (n_q - 1 > C - n_sink - n_recent) return WMTP_ERR_INVALID_ARG;
  if ((long)B * C > (long)INT_MAX) return WMTP_ERR_INVALID_ARG;
  if ((flags & ~WMTP_FLAG_PARTIALS_ONLY) != 0) return WMTP_ERR_INVALID_ARG;
  // the kernels take row maxima of raw scores before scaling: the scale must be positive
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return WMTP_ERR_INVALID_ARG;
  if (!q || !ring_k || !ring_v || !ring_pos || !ring_T) return WMTP_ERR_INVALID_ARG;
  if (!(flags & WMTP_FLAG_PARTIALS_ONLY) && !o) return WMTP_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(ring_k) || !aligned16(ring_v) || !aligned16(ring_pos) ||
      !aligned8(ring_T) || (o && !aligned16(o)) || (lse && !aligned4(lse)))
    return WMTP_ERR_INVALID_ARG;
  AttnArgs a = {};
  a.q = q;
  a.kc = ring_k;
  a.vc = ring_v;
  a.ring_pos = ring_pos;
  a.ring_T = ring_T;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_q = n_q;
  a.D = D;
  a.num_pages = B * (C / 64);
  a.max_pages = C / 64;
  a.C = C;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  a.scale_log2 = softmax_scale * kLog2e;
  return run_attention(a, true, C, C, o, lse, workspace, workspace_bytes, num_splits, flags,
                       static_cast<hipStream_t>(stream));
}

wmtp_status wmtp_draft_attn_full_fp8(const uint16_t* q, const uint8_t* k_cache,
                                     const uint8_t* v_cache, const int32_t* block_table,
                                     const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                                     int num_pages, int max_pages, int max_seq_len, float k_scale,
                                     float v_scale, float softmax_scale, float* o, float* lse,
                                     void* workspace, size_t workspace_bytes, int num_splits,
                                     unsigned flags, void* stream) {
  return paged_attention(q, reinterpret_cast<const uint16_t*>(k_cache),
                         reinterpret_cast<const uint16_t*>(v_cache), block_table, seq_lens, B, 1,
                         Hq, Hkv, D, num_pages, max_pages, max_seq_len, softmax_scale, o, lse,
                         workspace, workspace_bytes, num_splits, flags, stream, false, 0, 0,
                         nullptr, true, k_scale, v_scale);
}

wmtp_status wmtp_draft_attn_window_paged_fp8(
    const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache, const int32_t* block_table,
    const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int num_pages, int max_pages,
    int max_seq_len, int n_sink, int n_recent, float k_scale, float v_scale, float softmax_scale,
    float* o, float* lse, void* workspace, size_t workspace_bytes, int num_splits, unsigned flags,
    void* stream) {
  return paged_attention(q, reinterpret_cast<const uint16_t*>(k_cache),
                         reinterpret_cast<const uint16_t*>(v_cache), block_table, seq_lens, B, 1,
                         Hq, Hkv, D, num_pages, max_pages, max_seq_len, softmax_scale, o, lse,
                         workspace, workspace_bytes, num_splits, flags, stream, true, n_sink,
                         n_recent, nullptr, true, k_scale, v_scale);
}

wmtp_status wmtp_verify_attn_fp8(const uint16_t* q, const uint8_t* k_cache,
                                 const uint8_t* v_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, int B, int n_q, int Hq, int Hkv, int D,
                                 int num_pages, int max_pages, int max_seq_len, float k_scale,
                                 float v_scale, float softmax_scale, float* o, float* lse,
                                 void* workspace, size_t workspace_bytes, int num_splits,
                                 unsigned flags, void* stream) {
  return paged_attention(q, reinterpret_cast<const uint16_t*>(k_cache),
                         reinterpret_cast<const uint16_t*>(v_cache), block_table, seq_lens, B, n_q,
                         Hq, Hkv, D, num_pages, max_pages, max_seq_len, softmax_scale, o, lse,
                         workspace, workspace_bytes, num_splits, flags, stream, false, 0, 0,
                         nullptr, true, k_scale, v_scale);
}

wmtp_status wmtp_verify_attn_tree(const uint16_t* q, const uint16_t* k_cache,
                                  const uint16_t* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, const uint64_t* tree_mask, int B,
                                  int n_q, int Hq, int Hkv, int D, int num_pages, int max_pages,
                                  int max_seq_len, float softmax_scale, float* o, float* lse,
                                  void* workspace, size_t workspace_bytes, int num_splits,
                                  unsigned flags, void* stream) {
  if (!tree_mask || !aligned8(tree_mask) || n_q < 1 || n_q > 64) return WMTP_ERR_INVALID_ARG;
  return paged_attention(q, k_cache, v_cache, block_table, seq_lens, B, n_q, Hq, Hkv, D,
                         num_pages, max_pages, max_seq_len, softmax_scale, o, lse, workspace,
                         workspace_bytes, num_splits, flags, stream, false, 0, 0, tree_mask);
}

wmtp_status wmtp_draft_attn_window(const uint16_t* q, const uint16_t* ring_k,
                                   const uint16_t* ring_v, const int32_t* ring_pos,
                                   const int64_t* ring_T, int B, int Hq, int Hkv, int D, int C,
                                   int n_sink, int n_recent, float softmax_scale, float* o,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   int num_splits, unsigned flags, void* stream) {
  return ring_attention(q, ring_k, ring_v, ring_pos, ring_T, B, 1, Hq, Hkv, D, C, n_sink,
                        n_recent, softmax_scale, o, lse, workspace, workspace_bytes, num_splits,
                        flags, stream);
}

wmtp_status wmtp_draft_context_window(const uint16_t* q, const uint16_t* ring_k,
                                      const uint16_t* ring_v, const int32_t* ring_pos,
                                      const int64_t* ring_T, int B, int n_q, int Hq, int Hkv,
                                      int D, int C, int n_sink, int n_recent,
                                      float softmax_scale, float* o, float* lse, void* workspace,
                                      size_t workspace_bytes, int num_splits, unsigned flags,
                                      void* stream) {
  return ring_attention(q, ring_k, ring_v, ring_pos, ring_T, B, n_q, Hq, Hkv, D, C, n_sink,
                        n_recent, softmax_scale, o, lse, workspace, workspace_bytes, num_splits,
                        flags, stream);
}

// Fused ring step for the last n_q of the positions the ring holds once the n_new
// new ones are appended.
static wmtp_status ring_step(const uint16_t* q, uint16_t* ring_k, uint16_t* ring_v,
                             int32_t* ring_pos, int64_t* ring_T, const uint16_t* k_new,
                             const uint16_t* v_new, int B, int n_new, int n_q, int Hq, int Hkv,
                             int D, int C, int n_sink, int n_recent, float softmax_scale,
                             float* o, float* lse, void* workspace, size_t workspace_bytes,
                             int num_splits, void* stream, bool use_static = false) {
  if (!attn_dims_ok(B, Hq, Hkv, D) || n_q < 1) return WMTP_ERR_INVALID_ARG;
  if (!head_dim_ok(D)) return WMTP_ERR_UNSUPPORTED;
  if ((long)n_q * (Hq / Hkv) > 256) return WMTP_ERR_UNSUPPORTED;
  if (n_new < 1 || n_new > 32 || num_splits < 0) return WMTP_ERR_INVALID_ARG;
  if (C < 64 || C % 64 != 0 || n_sink < 0 || n_sink >= C || n_recent < 1 ||
      n_recent > C - n_sink)
    return WMTP_ERR_INVALID_ARG;
  // slack >= n_q - 1: the earliest query's window is still in the ring after the
  // append, and every slot the append overwrites holds a position before it
  if (n_q - 1 > C - n_sink - n_recent) return WMTP_ERR_INVALID_ARG;
  if ((long)B * C > (long)INT_MAX) return WMTP_ERR_INVALID_ARG;
  // the kernels take row maxima of raw scores before scaling: the scale must be positive
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return WMTP_ERR_INVALID_ARG;
  if (!q || !ring_k || !ring_v || !ring_pos || !ring_T || !k_new || !v_new || !o)
    return WMTP_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(ring_k) || !aligned16(ring_v) || !aligned16(ring_pos) ||
      !aligned8(ring_T) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(o) ||
      (lse && !aligned4(lse)))
    return WMTP_ERR_INVALID_ARG;
  AttnPlan p;
  if (!plan_window_step(B, Hq, Hkv, D, n_q, C, num_splits, &p)) return WMTP_ERR_INVALID_ARG;
  if (use_static) {
    // the partials go to this GPU's static scratch; sizes beyond it are refused
    if (p.ws_bytes > (size_t)WMTP_STATIC_SCRATCH_BYTES) return WMTP_ERR_WORKSPACE;
    const wmtp_status s = static_scratch(static_cast<hipStream_t>(stream), &workspace);
    if (s != WMTP_OK) return s;
    workspace_bytes = WMTP_STATIC_SCRATCH_BYTES;
  }
  if (!workspace || !aligned16(workspace) || workspace_bytes < p.ws_bytes)
    return WMTP_ERR_WORKSPACE;
  RingAppendArgs app;
  app.kc = ring_k;
  app.vc = ring_v;
  app.ring_pos = ring_pos;
  app.ring_T = ring_T;
  app.k_new = k_new;
  app.v_new = v_new;
  app.B = B;
  app.n_new = n_new;
  app.Hkv = Hkv;
  app.D = D;
  app.C = C;
  app.n_sink = n_sink;
  // launch 1: the window over the ring as it stands, ending after the new
  // positions, plus one workgroup per group over the new positions themselves
  AttnArgs a = {};
  a.q = q;
  a.kc = ring_k;
  a.vc = ring_v;
  a.ring_pos = ring_pos;
  a.ring_T = ring_T;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_q = n_q;
  a.D = D;
  a.G = p.G;
  a.R = p.R;
  a.num_pages = B * (C / 64);
  a.max_pages = C / 64;
  a.max_keys = C;
  a.C = C;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  a.scale_log2 = softmax_scale * kLog2e;
  a.nsplit = p.nsplit;
  a.kb_per_split = p.kb_per_split;
  a.items = p.items;
  a.nrg = p.nrg;
  a.direct = 0;
  a.out_o = static_cast<float*>(workspace);
  a.out_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.lse_offset);
  a.app = app;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (launch_window_step(a, p, st) != hipSuccess) return WMTP_ERR_HIP;
  // launch 2: merge the nsplit + 1 partials of each group, and append the new
  // positions to the rings (every read of the rings has finished by then)
  CombineArgs c = {};
  c.part_o = a.out_o;
  c.part_lse = a.out_lse;
  c.indptr = nullptr;
  c.n_parts = p.items;
  c.splits_per_group = p.nsplit + 1;
  c.B = B;
  c.Hkv = Hkv;
  c.G = p.G;
  c.n_q = n_q;
  c.D = D;
  c.R = p.R;
  c.o = o;
  c.lse = lse;
  c.append = 1;
  c.app = app;
  return from_hip(launch_combine(c, st));
}

wmtp_status wmtp_draft_step_window(const uint16_t* q, uint16_t* ring_k, uint16_t* ring_v,
                                   int32_t* ring_pos, int64_t* ring_T, const uint16_t* k_new,
                                   const uint16_t* v_new, int B, int n_new, int Hq, int Hkv, int D,
                                   int C, int n_sink, int n_recent, float softmax_scale, float* o,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   int num_splits, void* stream) {
  return ring_step(q, ring_k, ring_v, ring_pos, ring_T, k_new, v_new, B, n_new, 1, Hq, Hkv, D, C,
                   n_sink, n_recent, softmax_scale, o, lse, workspace, workspace_bytes,
                   num_splits, stream);
}

wmtp_status wmtp_draft_step_window_static(const uint16_t* q, uint16_t* ring_k, uint16_t* ring_v,
                                          int32_t* ring_pos, int64_t* ring_T,
                                          const uint16_t* k_new, const uint16_t* v_new, int B,
                                          int n_new, int Hq, int Hkv, int D, int C, int n_sink,
                                          int n_recent, float softmax_scale, float* o, float* lse,
                                          int num_splits, void* stream) {
  return ring_step(q, ring_k, ring_v, ring_pos, ring_T, k_new, v_new, B, n_new, 1, Hq, Hkv, D, C,
                   n_sink, n_recent, softmax_scale, o, lse, nullptr, 0, num_splits, stream, true);
}

wmtp_status wmtp_draft_context_step_window(const uint16_t* q, uint16_t* ring_k, uint16_t* ring_v,
                                           int32_t* ring_pos, int64_t* ring_T,
                                           const uint16_t* k_new, const uint16_t* v_new, int B,
                                           int n_new, int n_q, int Hq, int Hkv, int D, int C,
                                           int n_sink, int n_recent, float softmax_scale,
                                           float* o, float* lse, void* workspace,
                                           size_t workspace_bytes, int num_splits, void* stream) {
  return ring_step(q, ring_k, ring_v, ring_pos, ring_T, k_new, v_new, B, n_new, n_q, Hq, Hkv, D,
                   C, n_sink, n_recent, softmax_scale, o, lse, workspace, workspace_bytes,
                   num_splits, stream);
}

wmtp_status wmtp_ring_append(uint16_t* ring_k, uint16_t* ring_v, int32_t* ring_pos,
                             int64_t* ring_T, const uint16_t* k_new, const uint16_t* v_new,
                             int B, int n_new, int Hkv, int D, int C, int n_sink, void* stream) {
  if (B < 1 || Hkv < 1 || n_new < 0) return WMTP_ERR_INVALID_ARG;
  if (!head_dim_ok(D)) return WMTP_ERR_UNSUPPORTED;
  if (C < 64 || C % 64 != 0 || n_sink < 0 || n_sink >= C) return WMTP_ERR_INVALID_ARG;
  if ((long)B * C > (long)INT_MAX) return WMTP_ERR_INVALID_ARG;
  if (!ring_k || !ring_v || !ring_pos || !ring_T) return WMTP_ERR_INVALID_ARG;
  if (n_new > 0 && (!k_new || !v_new)) return WMTP_ERR_INVALID_ARG;
  if (!aligned16(ring_k) || !aligned16(ring_v) || !aligned4(ring_pos) || !aligned8(ring_T) ||
      (k_new && !aligned16(k_new)) || (v_new && !aligned16(v_new)))
    return WMTP_ERR_INVALID_ARG;
  if (n_new == 0) return WMTP_OK;
  RingAppendArgs a;
  a.kc = ring_k;
  a.vc = ring_v;
  a.ring_pos = ring_pos;
  a.ring_T = ring_T;
  a.k_new = k_new;
  a.v_new = v_new;
  a.B = B;
  a.n_new = n_new;
  a.Hkv = Hkv;
  a.D = D;
  a.C = C;
  a.n_sink = n_sink;
  return from_hip(launch_ring_append(a, static_cast<hipStream_t>(stream)));
}

// kv8: quantize to fp8 e4m3 with the scales (k_scale, v_scale > 0, finite).
static wmtp_status paged_append(void* k_cache, void* v_cache, const int32_t* block_table,
                                const int32_t* start_pos, const uint16_t* k_new,
                                const uint16_t* v_new, int B, int n_new, int Hkv, int D,
                                int num_pages, int max_pages, void* stream, bool kv8,
                                float k_scale, float v_scale) {
  if (B < 1 || B > 65535 || Hkv < 1 || n_new < 0 || num_pages < 1 || max_pages < 1)
    return WMTP_ERR_INVALID_ARG;
  if (!head_dim_ok(D)) return WMTP_ERR_UNSUPPORTED;
  if (!k_cache || !v_cache || !block_table || !start_pos) return WMTP_ERR_INVALID_ARG;
  if (n_new > 0 && (!k_new || !v_new)) return WMTP_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned4(block_table) ||
      !aligned4(start_pos) || (k_new && !aligned16(k_new)) || (v_new && !aligned16(v_new)))
    return WMTP_ERR_INVALID_ARG;
  if (kv8 && (!std::isfinite(k_scale) || !(k_scale > 0.f) || !std::isfinite(v_scale) ||
              !(v_scale > 0.f)))
    return WMTP_ERR_INVALID_ARG;
  if ((long)n_new * Hkv * (D / 8) / 256 + 1 > (long)INT_MAX) return WMTP_ERR_INVALID_ARG;
  if (n_new == 0) return WMTP_OK;
  PagedAppendArgs a = {};
  a.kc = static_cast<uint16_t*>(k_cache);
  a.vc = static_cast<uint16_t*>(v_cache);
  a.block_table = block_table;
  a.start_pos = start_pos;
  a.k_new = k_new;
  a.v_new = v_new;
  a.B = B;
  a.n_new = n_new;
  a.Hkv = Hkv;
  a.D = D;
  a.num_pages = num_pages;
  a.max_pages = max_pages;
  a.kv8 = kv8 ? 1 : 0;
  a.k_inv = kv8 ? 1.0f / k_scale : 1.0f;
  a.v_inv = kv8 ? 1.0f / v_scale : 1.0f;
  return from_hip(launch_paged_append(a, static_cast<hipStream_t>(stream)));
}

wmtp_status wmtp_paged_append(uint16_t* k_cache, uint16_t* v_cache, const int32_t* block_table,
                              const int32_t* start_pos, const uint16_t* k_new,
                              const uint16_t* v_new, int B, int n_new, int Hkv, int D,
                              int num_pages, int max_pages, void* stream) {
  return paged_append(k_cache, v_cache, block_table, start_pos, k_new, v_new, B, n_new, Hkv, D,
                      num_pages, max_pages, stream, false, 1.f, 1.f);
}

wmtp_status wmtp_paged_append_fp8(uint8_t* k_cache, uint8_t* v_cache, const int32_t* block_table,
                                  const int32_t* start_pos, const uint16_t* k_new,
                                  const uint16_t* v_new, int B, int n_new, int Hkv, int D,
                                  int num_pages, int max_pages, float k_scale, float v_scale,
                                  void* stream) {
  return paged_append(k_cache, v_cache, block_table, start_pos, k_new, v_new, B, n_new, Hkv, D,
                      num_pages, max_pages, stream, true, k_scale, v_scale);
}

wmtp_status wmtp_split_combine(const float* part_o, const float* part_lse, int n_parts,
                               const int32_t* split_indptr, int splits_per_group, int B, int Hkv,
                               int G, int n_q, int D, float* o, float* lse, void* stream) {
  if (B < 1 || Hkv < 1 || G < 1 || n_q < 1 || D < 16 || D > 256 || D % 16 != 0 || n_parts < 0)
    return WMTP_ERR_INVALID_ARG;
  if (!split_indptr && (splits_per_group < 0 || (long)B * Hkv * splits_per_group > n_parts))
    return WMTP_ERR_INVALID_ARG;
  if ((long)B * Hkv * n_q * G * (D / 16) > (long)INT_MAX) return WMTP_ERR_INVALID_ARG;
  if (!part_o || !part_lse || !o) return WMTP_ERR_INVALID_ARG;
  if (!aligned16(part_o) || !aligned4(part_lse) || !aligned16(o) || (lse && !aligned4(lse)) ||
      (split_indptr && !aligned4(split_indptr)))
    return WMTP_ERR_INVALID_ARG;
  CombineArgs c = {};
  c.part_o = part_o;
  c.part_lse = part_lse;
  c.indptr = split_indptr;
  c.n_parts = n_parts;
  c.splits_per_group = splits_per_group;
  c.B = B;
  c.Hkv = Hkv;
  c.G = G;
  c.n_q = n_q;
  c.D = D;
  c.R = n_q * G;
  c.o = o;
  c.lse = lse;
  return from_hip(launch_combine(c, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
