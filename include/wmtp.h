/*
 * wmtp.h - C ABI of the Windowed-MTP draft/verify attention library for
 * MI355X (gfx950).  Library file: libwmtp.so.
 *
 * What the calls compute (sources are the three pages on arXiv 2607.21535,
 * cited by title and part):
 *   - native draft: the draft head's single query per head attends over the
 *     whole draft KV at every draft step ("Windowed-MTP: Removing the
 *     Full-Context Draft-KV Tax at Million-Token Context", English abstract);
 *   - windowed draft: the same attention over the first n_sink positions plus
 *     the most recent n_recent positions only, held in a compact per-request
 *     ring (pith.science verdict page: key machinery; referee minor comment on
 *     the App. A pseudocode, slot = ring_base(r) + logical_pos);
 *   - verify: the target's full-context causal attention of the gamma+1
 *     proposed positions, the same in both arms (English abstract; verdict
 *     page, key machinery: the verify term is untouched);
 *   - split combine: log-sum-exp merge of attention over disjoint key subsets
 *     (not on the pages; how split-KV decoding is put back together).
 *
 * Conventions for every call
 *   - Pointers are device pointers unless marked (host).  The caller allocates
 *     and owns every buffer, including the workspace; the library never
 *     allocates or frees device memory and keeps no state between calls (the
 *     one exception, wmtp_draft_step_window_static, uses a static scratch
 *     buffer the library holds on each GPU instead of a workspace).
 *   - bf16 tensors are passed as uint16_t bit patterns.  Every bf16/float
 *     pointer must be 16-byte aligned.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and return after the launches are queued.
 *   - Arguments are checked on the host before anything is launched; a
 *     failed check returns an error code and launches nothing.  A fault
 *     inside a kernel shows up at the caller's next synchronisation.  The
 *     library never exits or aborts.
 *   - Values the host cannot check (lengths, page ids, ring state) are
 *     clamped on the device so that no access leaves the buffers described
 *     by the size arguments: a length above max_seq_len or above
 *     max_pages*64 is cut to the smaller bound; a key on a page id outside
 *     [0, num_pages) is treated as absent.
 *
 * KV layout ("tiled pages").  KV is stored in pages of WMTP_PAGE_TOKENS = 64
 * positions.  Page p, kv head g holds two tiles of 32 positions; tile
 * t = (p * Hkv + g) * 2 + (pos % 64) / 32 occupies 32 * D bf16 elements at
 * element offset t * 32 * D of its cache, laid out as
 *     K tile: [D/16][32 positions][16 dims]: (pos, d) at
 *             (d / 16) * 512 + (pos % 32) * 16 + d % 16
 *     V tile: [2][D][16 positions]:          (pos, d) at
 *             ((pos % 32) / 16) * 16 * D + d * 16 + pos % 16
 * so a cache of num_pages pages holds num_pages * Hkv * 64 * D elements.
 * A draft ring of capacity C (a multiple of 64) for request r is the same
 * layout: C / 64 pages, ring page i of request r is page r * (C / 64) + i,
 * and ring slot s is position s of that request's pages.
 *
 * Query rows.  With G = Hq / Hkv, query head h reads kv head h / G.
 */
#ifndef WMTP_H
#define WMTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WMTP_PAGE_TOKENS 64

typedef enum wmtp_status {
  WMTP_OK = 0,
  WMTP_ERR_INVALID_ARG = 1,  /* null or misaligned pointer, bad size, inconsistent sizes */
  WMTP_ERR_UNSUPPORTED = 2,  /* valid but not built: D not in {64,128,256}, too many query rows */
  WMTP_ERR_WORKSPACE = 3,    /* workspace missing or smaller than wmtp_workspace_bytes() */
  WMTP_ERR_HIP = 4           /* the HIP runtime refused a launch */
} wmtp_status;

/* flags for the attention calls */
#define WMTP_FLAG_PARTIALS_ONLY 1u /* stop after the split pass: leave per-split (o, lse)
                                      in the workspace (layout below) and do not write
                                      o/lse; merge them later with wmtp_split_combine(),
                                      e.g. after gathering partials of a sequence that is
                                      split across devices */

/* Human-readable name of a status code (static string, never NULL).  Takes a
 * plain int, so that any value a caller holds is valid input: codes outside
 * wmtp_status give "unknown status". */
const char* wmtp_status_string(int status);

/* `call` argument of the two planning queries below */
#define WMTP_CALL_PAGED 0        /* wmtp_draft_attn_full, wmtp_verify_attn */
#define WMTP_CALL_RING 1         /* wmtp_draft_attn_window */
#define WMTP_CALL_PAGED_WINDOW 2 /* wmtp_draft_attn_window_paged */
#define WMTP_CALL_RING_STEP 3    /* wmtp_draft_step_window (n_q = 1) and
                                    wmtp_draft_context_step_window; max_keys = C */
#define WMTP_CALL_PAGED_FP8 4    /* wmtp_draft_attn_full_fp8, wmtp_verify_attn_fp8 */

/*
 * Split plan of the attention calls.  n_q = 1 for the draft calls;
 * max_keys = min(max_seq_len, max_pages * 64) for the paged calls, C for
 * the ring calls and n_sink + n_recent for the truncated paged index (its
 * plan then covers any max_seq_len); num_splits = 0 lets the library choose.  Returns the number
 * of key splits per (sequence, kv head) that a call with these arguments
 * will use, or -1 if the sizes are invalid.  For WMTP_CALL_RING_STEP it is the
 * number of ring splits; each (sequence, kv head) then has one more partial,
 * the new positions'.  With num_splits = 0, paged calls over several sequences
 * of 64K keys or more plan about four workgroups per compute unit (the lengths
 * are on the device, and the extra rounds even out unequal ones), other calls
 * about one; WMTP_CALL_PAGED_FP8 at D = 128 over 64K keys or more aims at twice
 * the workgroups of WMTP_CALL_PAGED (two fit on a compute unit; whole tiles per
 * split, so the count is about twice).
 */
int wmtp_plan_splits(int call, int B, int Hq, int Hkv, int D, int n_q, int max_keys,
                     int num_splits);

/*
 * Workspace bytes the same call needs (0 when one split suffices and the
 * result is written directly, unless partials_only is non-zero; never 0 for
 * WMTP_CALL_RING_STEP).  Layout: with P = B * Hkv * splits partials
 * (splits + 1 for WMTP_CALL_RING_STEP) of R = n_q * Hq / Hkv rows each,
 *   part_o   fp32 [P][R][D] at byte 0 (partial p = (b * Hkv + g) * splits + s;
 *            row r = i * G + (h - g * G) for query i, head h),
 *   part_lse fp32 [P][R]    at byte ((P * R * D * 4 + 255) / 256) * 256;
 * each partial is a normalised output and its natural-log log-sum-exp
 * (-inf and zeros for a split with no key).
 */
size_t wmtp_workspace_bytes(int call, int B, int Hq, int Hkv, int D, int n_q, int max_keys,
                            int num_splits, int partials_only);

/*
 * Native (full-context) draft attention, one decode query per head.
 * (Field-notes entry, English abstract: the native MTP draft attends over the whole KV cache at
 * every draft step.)
 *   q            bf16 [B][Hq][D]
 *   k_cache      bf16 tiled pages, num_pages pages (layout above)
 *   v_cache      bf16 tiled pages, num_pages pages
 *   block_table  int32 [B][max_pages]: logical page i of sequence b is
 *                physical page block_table[b * max_pages + i]
 *   seq_lens     int32 [B]: keys of sequence b, this step's appended
 *                position included; sequence b reads positions [0, L_b)
 *   B, Hq, Hkv, D, num_pages, max_pages, max_seq_len   (host) sizes;
 *                max_seq_len bounds every seq_lens entry
 *   softmax_scale (host) logits are softmax_scale * (q . k); finite and
 *                > 0 (1/sqrt(D) in the usual case), else WMTP_ERR_INVALID_ARG
 *   o            fp32 [B][Hq][D] out
 *   lse          fp32 [B][Hq] out, natural log; may be NULL
 *   workspace, workspace_bytes   scratch of wmtp_workspace_bytes() bytes
 *   num_splits   (host) 0 = automatic, else a requested split count
 *   flags        WMTP_FLAG_PARTIALS_ONLY or 0
 * A sequence with no key gets o = 0 and lse = -inf.
 */
wmtp_status wmtp_draft_attn_full(const uint16_t* q, const uint16_t* k_cache,
                                 const uint16_t* v_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                                 int num_pages, int max_pages, int max_seq_len,
                                 float softmax_scale, float* o, float* lse, void* workspace,
                                 size_t workspace_bytes, int num_splits, unsigned flags,
                                 void* stream);

/*
 * fp8 draft KV.  (Verdict page, forward implications: the window composes with
 * KV quantization to fp8.)  The format is OCP fp8 E4M3 (1 sign, 4 exponent
 * bits of bias 7, 3 mantissa bits; no infinity, largest magnitude 448).  An fp8
 * cache has the tile layout of the bf16 caches with one byte per element: a
 * page of 64 positions is Hkv * 2 tiles of 32 * D bytes for K and the same
 * for V.  A bf16 value x is stored as the code nearest to x / scale (the
 * product with the float32 inverse of the scale, clamped to +-448, rounded to
 * nearest with ties to the even code); its value is code value * scale.  One
 * scale per cache (k_scale, v_scale: finite, > 0).
 *
 * wmtp_paged_append_fp8: as wmtp_paged_append, quantizing into fp8 caches.
 * wmtp_draft_attn_full_fp8 / wmtp_draft_attn_window_paged_fp8: as the bf16
 * calls, reading fp8 caches: the attention over the dequantized keys and
 * values (every e4m3 value is a bf16 value, so the MFMA operands are exact);
 * k_scale folds into the logit scale, v_scale into the output.  At most 32
 * query rows per kv head (Hq / Hkv), else WMTP_ERR_UNSUPPORTED.  Workspace and
 * plan: wmtp_draft_attn_full_fp8 as WMTP_CALL_PAGED_FP8 (below),
 * wmtp_draft_attn_window_paged_fp8 as the bf16 truncated index.
 */
wmtp_status wmtp_paged_append_fp8(uint8_t* k_cache, uint8_t* v_cache, const int32_t* block_table,
                                  const int32_t* start_pos, const uint16_t* k_new,
                                  const uint16_t* v_new, int B, int n_new, int Hkv, int D,
                                  int num_pages, int max_pages, float k_scale, float v_scale,
                                  void* stream);

wmtp_status wmtp_draft_attn_full_fp8(const uint16_t* q, const uint8_t* k_cache,
                                     const uint8_t* v_cache, const int32_t* block_table,
                                     const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                                     int num_pages, int max_pages, int max_seq_len, float k_scale,
                                     float v_scale, float softmax_scale, float* o, float* lse,
                                     void* workspace, size_t workspace_bytes, int num_splits,
                                     unsigned flags, void* stream);

wmtp_status wmtp_draft_attn_window_paged_fp8(
    const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache, const int32_t* block_table,
    const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int num_pages, int max_pages,
    int max_seq_len, int n_sink, int n_recent, float k_scale, float v_scale, float softmax_scale,
    float* o, float* lse, void* workspace, size_t workspace_bytes, int num_splits, unsigned flags,
    void* stream);

/*
 * The causal verify over fp8 caches: as wmtp_verify_attn (n_q queries, the
 * attention over the dequantized keys and values of the caches described above
 * for wmtp_draft_attn_full_fp8; k_scale folds into the logit scale, v_scale into
 * the output).  (Verdict page, forward implications: the window composes with
 * fp8 KV quantization; the verify reads the target KV, which fp8 halves.)  Up to
 * 256 query rows per kv head (n_q * Hq / Hkv) as for bf16: more than 32 go
 * through the kernel that shares each tile among its waves in LDS, which copies
 * the fp8 bytes there and widens each operand to bf16 right before its product.
 *   k_cache, v_cache   uint8 fp8 caches (16-byte aligned)
 *   k_scale, v_scale   finite, > 0 (else WMTP_ERR_INVALID_ARG)
 *   other arguments as wmtp_verify_attn; workspace and plan as
 *   WMTP_CALL_PAGED_FP8 with this n_q
 */
wmtp_status wmtp_verify_attn_fp8(const uint16_t* q, const uint8_t* k_cache,
                                 const uint8_t* v_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, int B, int n_q, int Hq, int Hkv, int D,
                                 int num_pages, int max_pages, int max_seq_len, float k_scale,
                                 float v_scale, float softmax_scale, float* o, float* lse,
                                 void* workspace, size_t workspace_bytes, int num_splits,
                                 unsigned flags, void* stream);

/*
 * Verify of a tree of proposals: as wmtp_verify_attn, but the n_q appended
 * positions form a tree instead of a chain.  (Verdict page, forward
 * implications: the window composes with tree-shaped speculation.)  Query i
 * sees every key before the appended positions and the appended position
 * L_b - n_q + a exactly when bit a of tree_mask[b * n_q + i] is set (its
 * ancestors and itself; the causal verify is mask_i = 2^(i+1) - 1).
 *   tree_mask  uint64 [B][n_q] (device, 8-byte aligned); bits >= n_q ignored
 *   n_q        1 .. 64
 *   other arguments and the workspace as wmtp_verify_attn
 * A query that sees no key gets o = 0 and lse = -inf.
 */
wmtp_status wmtp_verify_attn_tree(const uint16_t* q, const uint16_t* k_cache,
                                  const uint16_t* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, const uint64_t* tree_mask, int B,
                                  int n_q, int Hq, int Hkv, int D, int num_pages, int max_pages,
                                  int max_seq_len, float softmax_scale, float* o, float* lse,
                                  void* workspace, size_t workspace_bytes, int num_splits,
                                  unsigned flags, void* stream);

/*
 * Windowed draft attention over the paged draft KV by index truncation: the
 * same key set as wmtp_draft_attn_window, read straight from the paged cache
 * instead of from a compact ring.  (Verdict page, key machinery: the draft
 * reads a per-request KV index cut down to the attention sink plus the recent
 * window; nothing is reclaimed, the full draft KV stays resident.)
 * Sequence b attends over keys [0, min(n_sink, L_b)) u [max(n_sink, L_b -
 * n_recent), L_b) of its pages, each key once.
 *   arguments as wmtp_draft_attn_full, plus
 *   n_sink, n_recent (host) the window: n_sink >= 0, n_recent >= 1
 * Workspace: wmtp_workspace_bytes(WMTP_CALL_PAGED_WINDOW, ..., max_keys =
 * n_sink + n_recent, ...).  More than 32 query rows per kv head (Hq / Hkv)
 * give WMTP_ERR_UNSUPPORTED.
 */
wmtp_status wmtp_draft_attn_window_paged(const uint16_t* q, const uint16_t* k_cache,
                                         const uint16_t* v_cache, const int32_t* block_table,
                                         const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                                         int num_pages, int max_pages, int max_seq_len,
                                         int n_sink, int n_recent, float softmax_scale, float* o,
                                         float* lse, void* workspace, size_t workspace_bytes,
                                         int num_splits, unsigned flags, void* stream);

/*
 * Windowed draft attention over a per-request ring of C slots.
 * (Verdict page, key machinery: the draft reads the first n_sink positions
 * plus the most recent ones; referee minor comment on App. A: the draft KV
 * lives in a ring addressed as ring_base(r) + logical_pos.)
 *   q          bf16 [B][Hq][D]
 *   ring_k     bf16 tiled pages, B * C / 64 pages
 *   ring_v     bf16 tiled pages, B * C / 64 pages
 *   ring_pos   int32 [B][C]: position held by each slot, -1 if empty
 *   ring_T     int64 [B]: positions appended so far (the context length L)
 *   B, Hq, Hkv, D, C, n_sink, n_recent   (host); C % 64 == 0,
 *              0 <= n_sink < C, 1 <= n_recent <= C - n_sink
 *   softmax_scale, o, lse, workspace, workspace_bytes, num_splits, flags,
 *   stream     as in wmtp_draft_attn_full
 * Slot s of request b is read iff its position p = ring_pos[b][s] satisfies
 * 0 <= p < L and (p < n_sink or p >= L - n_recent); slot order does not
 * matter because cached keys carry their positions already.
 */
wmtp_status wmtp_draft_attn_window(const uint16_t* q, const uint16_t* ring_k,
                                   const uint16_t* ring_v, const int32_t* ring_pos,
                                   const int64_t* ring_T, int B, int Hq, int Hkv, int D, int C,
                                   int n_sink, int n_recent, float softmax_scale, float* o,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   int num_splits, unsigned flags, void* stream);

/*
 * Draft context pass over the ring: the n_q positions the draft head
 * processes after a verify (the accepted ones), each attending causally over
 * its own window.  (Referee major comment on App. B / Eq. 1: the per-step cost
 * has a draft context term besides the draft forwards; its native form reads
 * the whole draft KV, which is wmtp_verify_attn over the paged draft cache.)
 * Query i is position ring_T[b] - n_q + i and sees the positions p <= its own
 * with p < n_sink or p > its own - n_recent.  The ring's slack must hold the
 * earlier queries' windows: n_q - 1 <= C - n_sink - n_recent, else
 * WMTP_ERR_INVALID_ARG.
 *   q     bf16 [B][n_q][Hq][D]; o fp32 [B][n_q][Hq][D]; lse fp32 [B][n_q][Hq]
 *   other arguments as wmtp_draft_attn_window; n_q * Hq / Hkv <= 256
 * Workspace: wmtp_workspace_bytes(WMTP_CALL_RING, B, Hq, Hkv, D, n_q, C, ...).
 */
wmtp_status wmtp_draft_context_window(const uint16_t* q, const uint16_t* ring_k,
                                      const uint16_t* ring_v, const int32_t* ring_pos,
                                      const int64_t* ring_T, int B, int n_q, int Hq, int Hkv,
                                      int D, int C, int n_sink, int n_recent,
                                      float softmax_scale, float* o, float* lse, void* workspace,
                                      size_t workspace_bytes, int num_splits, unsigned flags,
                                      void* stream);

/*
 * One windowed draft step: append n_new positions to each request's ring and
 * attend over the window that ends with them, in two launches instead of the
 * three of wmtp_ring_append + wmtp_draft_attn_window.  (Verdict page, key
 * machinery: per draft step the draft appends its new K/V and reads only the
 * sink plus the recent window; referee minor comment on App. A: the draft KV
 * lives in the ring.)  The result and the ring afterwards are those of
 * wmtp_ring_append(k_new, v_new) followed by wmtp_draft_attn_window with the
 * same arguments: the query attends over positions p < L = ring_T[b] + n_new
 * with p < n_sink or p >= L - n_recent, the new positions included.
 * How: the first launch reads the ring as it stands with the window ending at
 * L (the slots the new positions will take hold positions outside that
 * window) and, in one more workgroup per (request, kv head), the new positions
 * straight from k_new / v_new; the second merges the partial results and
 * appends the new positions to the rings.
 *   q                bf16 [B][Hq][D]; Hq / Hkv <= 256 (else WMTP_ERR_UNSUPPORTED)
 *   ring_k, ring_v   bf16 tiled pages (in/out), B * C / 64 pages
 *   ring_pos         int32 [B][C] (in/out)
 *   ring_T           int64 [B] (in/out); negative values count as 0, values
 *                    must stay below 2^31 - 64
 *   k_new, v_new     bf16 [B][n_new][Hkv][D], row-major; 1 <= n_new <= 32
 *   B, n_new, Hq, Hkv, D, C, n_sink, n_recent   (host) as wmtp_draft_attn_window
 *   softmax_scale, o, lse, stream   as in wmtp_draft_attn_full (o is required)
 *   workspace, workspace_bytes      wmtp_workspace_bytes(WMTP_CALL_RING_STEP, B,
 *                    Hq, Hkv, D, 1, C, num_splits, 0) bytes: the partials of
 *                    B * Hkv * (splits + 1) workgroups, in the layout described
 *                    there with splits + 1 partials per group (the last one
 *                    holds the new positions)
 *   num_splits       ring splits per (request, kv head); 0 = as the windowed
 *                    draft plans them
 * Errors as wmtp_draft_attn_window; the workspace is checked as there.
 */
wmtp_status wmtp_draft_step_window(const uint16_t* q, uint16_t* ring_k, uint16_t* ring_v,
                                   int32_t* ring_pos, int64_t* ring_T, const uint16_t* k_new,
                                   const uint16_t* v_new, int B, int n_new, int Hq, int Hkv, int D,
                                   int C, int n_sink, int n_recent, float softmax_scale, float* o,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   int num_splits, void* stream);

/*
 * wmtp_draft_step_window with no workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation.  The split partials go to a static scratch
 * buffer of WMTP_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends (its address is looked up once per device, on the
 * first call there).  Arguments, result and ring update as wmtp_draft_step_window;
 * the stream must belong to the current device (else WMTP_ERR_INVALID_ARG).
 * Sizes whose partials need more than the scratch
 * (wmtp_workspace_bytes(WMTP_CALL_RING_STEP, B, Hq, Hkv, D, 1, C, num_splits, 0)
 * > WMTP_STATIC_SCRATCH_BYTES) return WMTP_ERR_WORKSPACE and launch nothing.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time on
 * one GPU (on different streams, or from several threads without ordering) race
 * and give undefined results; calls ordered on one stream do not.  Nothing in the
 * scratch needs to start at zero.
 */
#define WMTP_STATIC_SCRATCH_BYTES (16u << 20)

wmtp_status wmtp_draft_step_window_static(const uint16_t* q, uint16_t* ring_k, uint16_t* ring_v,
                                          int32_t* ring_pos, int64_t* ring_T,
                                          const uint16_t* k_new, const uint16_t* v_new, int B,
                                          int n_new, int Hq, int Hkv, int D, int C, int n_sink,
                                          int n_recent, float softmax_scale, float* o, float* lse,
                                          int num_splits, void* stream);

/*
 * The draft context pass fused the same way: append n_new positions to each
 * request's ring, then the last n_q positions (the accepted ones the draft head
 * processes after a verify) attend causally over their own windows, in two
 * launches instead of the three of wmtp_ring_append + wmtp_draft_context_window.
 * (Referee major comment on App. B / Eq. 1: the draft context term of the
 * per-step cost; verdict page, key machinery: the draft reads only the sink and
 * the recent window.)  The result and the ring afterwards are those of
 * wmtp_ring_append(k_new, v_new) followed by wmtp_draft_context_window with the
 * same arguments: with L = ring_T[b] + n_new, query i is position L - n_q + i.
 * The slots the append overwrites hold positions before every query's window
 * because the slack condition n_q - 1 <= C - n_sink - n_recent holds (else
 * WMTP_ERR_INVALID_ARG); n_q may exceed n_new (the earlier queries' positions
 * are in the ring already).
 *   q     bf16 [B][n_q][Hq][D]; o fp32 [B][n_q][Hq][D]; lse fp32 [B][n_q][Hq];
 *         n_q * Hq / Hkv <= 256 (else WMTP_ERR_UNSUPPORTED)
 *   other arguments as wmtp_draft_step_window; the workspace is
 *   wmtp_workspace_bytes(WMTP_CALL_RING_STEP, B, Hq, Hkv, D, n_q, C, num_splits, 0)
 *   bytes (partials of n_q * Hq / Hkv rows)
 * With n_q = 1 this is wmtp_draft_step_window.
 */
wmtp_status wmtp_draft_context_step_window(const uint16_t* q, uint16_t* ring_k, uint16_t* ring_v,
                                           int32_t* ring_pos, int64_t* ring_T,
                                           const uint16_t* k_new, const uint16_t* v_new, int B,
                                           int n_new, int n_q, int Hq, int Hkv, int D, int C,
                                           int n_sink, int n_recent, float softmax_scale,
                                           float* o, float* lse, void* workspace,
                                           size_t workspace_bytes, int num_splits, void* stream);

/*
 * Append n_new consecutive positions to each request's draft ring.
 * (Referee minor comment on App. A: slot = ring_base(r) + logical_pos, with
 * slack beyond the window.)  Position p of request b goes to slot
 *     p                                    if p < n_sink
 *     n_sink + (p - n_sink) % (C - n_sink) otherwise
 * of ring b; the appended positions are ring_T[b] .. ring_T[b] + n_new - 1,
 * and ring_T[b] grows by n_new on the device.  Positions that a later
 * position of the same call overwrites are skipped, so n_new may exceed C
 * (bulk fill after prefill, or a rebuild on resume).  Capacity beyond
 * n_sink + n_recent is slack: the window call reads only the last n_recent,
 * so up to (C - n_sink - n_recent) rolled-back positions never evict a
 * position still in the window.  Rolling back is writing a smaller ring_T.
 * Up to 64 positions run as one launch (one workgroup per request); longer
 * appends run as a fill spread over many workgroups followed by a one-thread-
 * per-request launch that advances ring_T, both on `stream`.
 *   ring_k, ring_v   bf16 tiled pages (in/out), B * C / 64 pages
 *   ring_pos         int32 [B][C] (in/out)
 *   ring_T           int64 [B] (in/out); negative values count as 0
 *   k_new, v_new     bf16 [B][n_new][Hkv][D], row-major
 *   B, n_new, Hkv, D, C, n_sink   (host)
 */
wmtp_status wmtp_ring_append(uint16_t* ring_k, uint16_t* ring_v, int32_t* ring_pos,
                             int64_t* ring_T, const uint16_t* k_new, const uint16_t* v_new,
                             int B, int n_new, int Hkv, int D, int C, int n_sink, void* stream);

/*
 * Write n_new consecutive positions into paged caches: position
 * start_pos[b] + t of sequence b takes k_new/v_new[b][t].  Lengths are the
 * caller's: this call does not change seq_lens.  Positions on a logical page
 * >= max_pages or on a page id outside [0, num_pages) are skipped.
 *   k_cache, v_cache bf16 tiled pages (in/out), num_pages pages
 *   block_table      int32 [B][max_pages]
 *   start_pos        int32 [B]
 *   k_new, v_new     bf16 [B][n_new][Hkv][D], row-major
 *   B, n_new, Hkv, D, num_pages, max_pages  (host)
 */
wmtp_status wmtp_paged_append(uint16_t* k_cache, uint16_t* v_cache, const int32_t* block_table,
                              const int32_t* start_pos, const uint16_t* k_new,
                              const uint16_t* v_new, int B, int n_new, int Hkv, int D,
                              int num_pages, int max_pages, void* stream);

/*
 * Full-context causal verify of n_q proposed positions per sequence.
 * (English abstract: verification keeps full attention; verdict page, key
 * machinery: the verify term is the same in both arms.)
 *   q          bf16 [B][n_q][Hq][D]
 *   k_cache, v_cache, block_table, seq_lens, num_pages, max_pages,
 *   max_seq_len  as in wmtp_draft_attn_full; seq_lens counts the n_q
 *              appended positions, and query i sees the first
 *              seq_lens[b] - n_q + i + 1 positions
 *   o          fp32 [B][n_q][Hq][D] out
 *   lse        fp32 [B][n_q][Hq] out, may be NULL
 *   n_q * Hq / Hkv must not exceed 256.
 */
wmtp_status wmtp_verify_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, int B, int n_q,
                             int Hq, int Hkv, int D, int num_pages, int max_pages,
                             int max_seq_len, float softmax_scale, float* o, float* lse,
                             void* workspace, size_t workspace_bytes, int num_splits,
                             unsigned flags, void* stream);

/*
 * Merge per-split attention results (log-sum-exp combine):
 *     lse = ln sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) * o_s
 * over the splits of each (sequence b, kv head g) group.
 *   part_o        fp32 [n_parts][R][D], R = n_q * G, layout as in the workspace
 *   part_lse      fp32 [n_parts][R]; -inf marks an empty split
 *   n_parts       (host) partials in part_o / part_lse; split_indptr entries
 *                 are clamped to [0, n_parts] on the device
 *   split_indptr  int32 [B * Hkv + 1]: group (b * Hkv + g) owns partials
 *                 split_indptr[grp] .. split_indptr[grp + 1] - 1; or NULL,
 *                 then group grp owns grp * splits_per_group ..
 *                 (grp + 1) * splits_per_group - 1
 *   splits_per_group (host) used when split_indptr is NULL
 *   B, Hkv, G, n_q, D (host); D a multiple of 16, at most 256
 *   o             fp32 [B][n_q][Hkv * G][D] out
 *   lse           fp32 [B][n_q][Hkv * G] out, may be NULL
 * A group with no key gets o = 0 and lse = -inf.
 */
wmtp_status wmtp_split_combine(const float* part_o, const float* part_lse, int n_parts,
                               const int32_t* split_indptr, int splits_per_group, int B, int Hkv,
                               int G, int n_q, int D, float* o, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WMTP_H */
