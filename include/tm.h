/*
 * tm.h -- C ABI of the tile-routed mixed-precision causal attention library
 * (libtm.so, HIP for gfx950 / MI355X).
 *
 * What it computes.  Causal prefill attention in which every query-key score
 * tile is routed to SKIP, INT4, INT8 or FP16 computation by a compact per-head
 * policy, with every executed tile updating one shared online-softmax state;
 * and the decode step that reuses the quantized K/V produced for prefill as a
 * compressed cache.  Sources (the method pages):
 *   [TriAttention] "TriAttention: Unified Sparse Mixed-Precision Attention for
 *     Long-Context LLM Inference", abstract: skip / 4-bit / 8-bit tile routing,
 *     two diagonal-distance boundaries per head, precision-grouped traversals,
 *     one fused kernel that skips omitted tiles and merges both QK precisions
 *     into one normalized output, prefill codes reused as the decode KV cache.
 *   [TileMix] "TileMix: Tile-Centric Mixed-Precision Attention for LLM
 *     Inference Acceleration", abstract: hardware-aligned score tiles, routing
 *     decisions packed in compact bitmasks with one bit per group of adjacent
 *     key tiles, FP16 or INT8 score paths sharing one online-softmax state,
 *     all legal groups routed, GQA, variable-length batches, INT8 K/V caches.
 *   [HyQuant] "HyQuant Uses Hybrid Precision to Compress LLM Attention",
 *     sections "The observation behind the method" and "How HyQuant works":
 *     selected (vertical-line) tokens and a recent window kept FP16, the rest
 *     quantized, in prefill and in the decode cache, with dequantization
 *     fused into decode attention.
 * Policies: per-head boundaries, packed group bitmasks, the four-way
 * combination of the two, and the token-granular hybrid policy (with a
 * selection pass, tm_select_vertical).  Generation: tm_cache_append keeps a
 * growing cache quantized as if built from scratch.
 *
 * Conventions common to every entry point.
 *  - Pointers named *_dev or documented as "device" are device memory owned by
 *    the caller (e.g. PyTorch tensors).  Pointers documented as "host" are host
 *    memory read during the call only.  The library allocates no device
 *    memory (beyond one fixed array in its code object, for
 *    tm_decode_noalloc), frees nothing and keeps no pointer after a call returns (calls
 *    that stage small host tables copy them into caller buffers and
 *    synchronize the stream before returning).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    is asynchronous: buffers must stay valid until the stream has finished.
 *    Calls on different streams are independent (the library has no mutable
 *    global state apart from the lazily loaded code object and the scratch
 *    array of tm_decode_noalloc, which that entry point alone uses).
 *  - Every argument is validated on the host before anything is enqueued; on
 *    a nonzero status nothing has been enqueued and outputs are untouched.
 *    Launch failures return TM_E_HIP.  Faults inside kernels surface at the
 *    caller's next synchronization of the stream.  Nothing throws across the
 *    ABI.
 *  - Token-major 16-bit inputs are [T][heads][d] row-major, T = total tokens
 *    of all sequences; sequence s owns tokens cu_seqlens[s] .. cu_seqlens[s+1]-1.
 *  - Quantization blocks are 64 tokens and restart at each sequence start;
 *    nblk = sum over s of ceil(len_s / 64).  Key tiles are one block (bk = 64).
 */
#ifndef TM_H
#define TM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tm_status {
  TM_OK = 0,
  TM_E_ARG = 1,          /* NULL or out-of-range argument                      */
  TM_E_SHAPE = 2,        /* inconsistent sizes / unsupported head dim / tiles   */
  TM_E_POLICY = 3,       /* policy invalid (b8 > b4, a row with no key, ...)    */
  TM_E_SPACE = 4,        /* caller buffer (traversal, workspace) too small      */
  TM_E_UNSUPPORTED = 5,  /* valid request this build does not implement         */
  TM_E_HIP = 6           /* a HIP launch or copy failed                         */
} tm_status;

typedef enum tm_dtype { TM_F16 = 0, TM_BF16 = 1, TM_F32 = 2 } tm_dtype;

/* Per-tile precision.  INT4 tiles use 4-bit Q and K codes, INT8 tiles 8-bit
 * codes ([TriAttention] abstract); FP16 tiles use the 16-bit Q and K
 * ([TileMix] abstract; bf16 inputs run the bf16 MFMA on this path). */
typedef enum tm_prec { TM_SKIP = 0, TM_INT4 = 1, TM_INT8 = 2, TM_FP16 = 3 } tm_prec;

typedef enum tm_layout {
  TM_ROWS = 0,  /* codes [nblk][heads][64][d] and [nblk][heads][64][d/2]        */
  TM_COLS = 1   /* codes transposed per block: [nblk][heads][d][64], [d][32]   */
} tm_layout;

typedef enum tm_policy_kind {
  TM_POLICY_BOUNDARIES = 0,
  TM_POLICY_BITMASK = 1,
  TM_POLICY_FOURWAY = 2,
  TM_POLICY_HYBRID = 3
} tm_policy_kind;

/* Problem shape.  cu_seqlens (host) and cu_seqlens_dev (device) hold the same
 * nseq+1 non-decreasing int32 prefix sums starting at 0.
 * Supported: d in {64, 128}; bk == 64; bq in {64, 128}; hq % hkv == 0;
 * dtype TM_F16 or TM_BF16.  softmax_scale <= 0 selects 1/sqrt(d). */
typedef struct tm_shape {
  int32_t nseq;
  const int32_t* cu_seqlens;
  const int32_t* cu_seqlens_dev;
  int32_t hq, hkv, d;
  int32_t bq, bk;
  int32_t dtype;
  float softmax_scale;
} tm_shape;

/* Quantized tensor (device buffers, caller-allocated).  One symmetric scale
 * per (64-token block, head) over all d channels of the block's valid rows:
 * s8 = amax / 127, s4 = amax / 7 (IEEE binary32 divisions);
 * code = clamp(round_half_even(x / s), -qmax, qmax), binary32 division;
 * amax == 0 gives scale 0 and zero codes; rows past a sequence's end are zero.
 * INT4 codes are two's-complement nibbles packed along the last axis, element
 * 2t in the low nibble of byte t and 2t+1 in the high nibble.
 * ([TriAttention] abstract: keys and values quantized during prefill; the pages
 * give no formula, this symmetric block reading is the library's definition.)
 * Block-major: all heads of one 64-token block are adjacent, so the blocks a
 * decode step reads are dense in memory, and one block of every head is a
 * contiguous slice (entries [j*heads, (j+1)*heads)).
 *   TM_ROWS: c8 [nblk][heads][64][d]   c4 [nblk][heads][64][d/2]
 *   TM_COLS: c8 [nblk][heads][d][64]   c4 [nblk][heads][d][32]
 *            t16 (optional, TM_COLS only): the block's values as fp16,
 *            transposed, [nblk][heads][d][64] (bf16 input rounded to nearest
 *            even fp16, magnitudes beyond 65504 saturated to +-65504, NaN kept;
 *            zeros past the sequence end).
 *   s8, s4 [nblk][heads] float.
 *   c4x (optional, TM_ROWS only): the INT4 codes once more, one per byte
 *            (int8, -7..7), [nblk][heads][64][d] like c8.  tm_prefill
 *            requires it for K under boundary policies (the
 *            prefill kernel feeds these bytes to the int8 matrix cores as
 *            they are, without unpacking nibbles on every tile).
 * nblk must equal sum over sequences of ceil(len / 64) (tm_num_blocks). */
typedef struct tm_qtensor {
  int8_t* c8;
  uint8_t* c4;
  float* s8;
  float* s4;
  uint16_t* t16;
  int32_t heads;
  int32_t layout;
  int64_t nblk;
  int8_t* c4x;
} tm_qtensor;

/* Tile policy ([TriAttention] abstract: two diagonal-distance boundaries per
 * head; [TileMix] abstract: packed group bitmask; the four-way kind combines
 * the two; [HyQuant] "How HyQuant works": token-granular FP16 retention).  b8/b4 are host arrays (at most 256 query heads); bits is device
 * memory read by the expansion kernel.
 *  Boundaries: b8[hq], b4[hq] in key-tile units, 0 <= b8 <= b4.  For query
 *   tile i and key tile j, delta = max(0, floor((i*bq - j*bk) / bk));
 *   delta < b8 -> INT8, delta < b4 -> INT4, else SKIP; sink = 1 keeps key
 *   tile 0 INT8 for every query tile.  b4 == 0 without a sink leaves rows with
 *   no key and is rejected (TM_E_POLICY).
 *  Bitmask: bits[n_words] uint32 (device).  Bit = 1 -> FP16, 0 -> INT8;
 *   bit g of a row governs key tiles [g*group, (g+1)*group); each (sequence, query head,
 *   query tile) row holds ceil(ceil(nk_s / group) / 32) words, LSB first, rows
 *   ordered sequence, then head, then query tile.  Nothing is skipped.
 *  Four-way: b8, b4 and sink as for boundaries (same checks), plus bits with
 *   a 2-bit code per group: group g of a row is bits 2(g%16) .. 2(g%16)+1 of
 *   the row's word g/16; rows of ceil(ceil(nk_s / group) / 16) words in the
 *   bitmask's row order.  Code 0 leaves the group's tiles to the boundary
 *   rule (the only source of SKIP), codes 1, 2, 3 make them INT4, INT8, FP16.
 *   All-zero codes give the boundary policy; codes 2/3 only give the bitmask
 *   policy.
 *  Hybrid: precision per (row, key) instead of per tile: key c of row r
 *   (c <= r) is FP16 if c is in the selected list of the row's (sequence,
 *   query head) or r - c < window, else INT8; nothing is skipped.  The
 *   traversal holds, per work item, the tiles wholly inside the window
 *   (FP16), those wholly outside (INT8), the tiles the window edge crosses
 *   (run twice: FP16 on the pairs inside, INT8 on the rest), and the
 *   item's visible selected keys gathered into compact FP16 tiles of 64;
 *   selected keys are masked out of the regular tiles.  Lists are copied
 *   into the traversal buffer and its tables built by one kernel;
 *   tm_gather_selected fills the gathered tiles before tm_prefill.
 *  A tile is legal iff j*bk <= min((i+1)*bq, len) - 1; inside a legal tile key
 *  c is visible from row r iff c <= r. */
typedef struct tm_policy {
  int32_t kind;
  const int32_t* b8;
  const int32_t* b4;
  int32_t sink;
  const uint32_t* bits;
  int64_t n_words;
  int32_t group;
  /* TM_POLICY_HYBRID only (host arrays, read during tm_build_traversal and
   * tm_gather_selected): */
  const int32_t* sel_off;   /* [nseq*hq + 1]: list of row s*hq + h is sel_idx[sel_off[r], sel_off[r+1]) */
  const int32_t* sel_idx;   /* selected key positions within the sequence, strictly increasing per list */
  int32_t window;           /* sliding-window length in tokens, >= 0 */
  /* Hybrid lists in device memory instead (sel_idx == NULL): sel_idx_dev holds
   * the positions and sel_off_dev a device copy of sel_off (which is still
   * given on the host: it sizes the traversal).  The tables are then built by
   * a kernel, with no host copy and no wait, e.g. straight from the output of
   * tm_select_vertical.  The positions are not checked: lists must be
   * strictly increasing positions within their sequence (as
   * tm_select_vertical writes them); other lists give unspecified outputs,
   * but no access outside the buffers. */
  const int32_t* sel_off_dev;
  const int32_t* sel_idx_dev;
} tm_policy;

/* Tile counts of a traversal (host). */
typedef struct tm_census {
  int64_t legal, n_int8, n_int4, n_fp16, n_skip;
  int64_t n_items, max_runs;
} tm_census;

/* Decode cache policy (host arrays; at most 64 KV heads and 256 query heads),
 * in 64-token blocks.
 * For a cache of L tokens (the new token included) and block j:
 *  blocks overlapping the last tail_tokens tokens are FP16 (read from the
 *  16-bit keys and the t16 copy of V); otherwise delta = floor((L-1)/64) - j,
 *  INT8 if delta < b8 (or j == 0 with sink), INT4 if delta < b4, else SKIP.
 * per_q_head = 0: b8, b4 hold one map per KV head (hkv entries), shared by
 *  the KV head's query heads.  per_q_head = 1: one map per query head (hq
 *  entries).  Consecutive query heads of a KV head with equal maps are
 *  decoded together and share each cache block read; a group whose maps
 *  differ reads its blocks once per distinct run of maps.
 * ([HyQuant] "How HyQuant works": recent window FP16, rest quantized;
 * [TriAttention] abstract: prefill codes reused in the decode cache, two
 * boundaries per head.) */
typedef struct tm_dpolicy {
  const int32_t* b8;
  const int32_t* b4;
  int32_t sink;
  int32_t tail_tokens;
  const int32_t* lengths;   /* host [nseq] or NULL: current lengths, 1 <= lengths[s] <= the
                               cache shape's length of s (its capacity); NULL: the capacity */
  int32_t per_q_head;       /* 0: b8/b4 per KV head; 1: per query head */
  /* Selected tokens kept in FP16, or sel_off == NULL for none.  List of row
   * s*hkv + g (sequence s, KV head g) is sel_idx[sel_off[r], sel_off[r+1]):
   * positions below the sequence's current length, strictly increasing.  A
   * selected key is read in FP16 whatever its block's tag (SKIP included);
   * the other keys follow their block's tag.  sel_buf: device buffer that
   * tm_decode_select filled for these lists (host arrays read during the
   * calls).  tm_decode reads only the list lengths and trusts the positions
   * that tm_decode_select checked: after the lists or the lengths change,
   * call tm_decode_select again.  ([HyQuant] "How HyQuant works": selected
   * tokens and the recent window stay FP16 in the decode cache.) */
  const int32_t* sel_off;
  const int32_t* sel_idx;
  const void* sel_buf;
  /* Selected lists in device memory instead (sel_idx == NULL, read by
   * tm_decode_select only): positions sel_idx_dev and a device copy
   * sel_off_dev of sel_off (still given on the host).  tm_decode_select then
   * builds the tables with a kernel, with no host copy and no wait; the
   * positions are not checked (lists must be strictly increasing positions
   * below the current length; other lists give unspecified outputs but no
   * access outside the buffers). */
  const int32_t* sel_off_dev;
  const int32_t* sel_idx_dev;
} tm_dpolicy;

/* Traversal buffer layout (device, written by tm_build_traversal, read by
 * tm_prefill; documented so tests can decode it).  All fields little-endian.
 *  [0, 256)        header: uint32 magic 0x564D5454 ('TTMV'), version, kind,
 *                  n_items, max_runs, nseq, hq, hkv, bq, bk, d, nblk,
 *                  seq_off, item_off, run_off, bits_off (bytes);
 *                  at byte 128: int64 legal, int8, int4, fp16, skip.
 *  seq_off:        nseq x uint32[4] {tok_start, len, blk_start, nq}.
 *  item_off:       n_items x uint32[8] {seq, head, qtile, nruns,
 *                  n_int8, n_int4, n_fp16, n_skip}, heavy-first: query tiles
 *                  in descending index, then sequence, then head.
 *  run_off:        n_items x max_runs x uint32[2] {first key tile,
 *                  count | prec << 24}; an item's runs are grouped by
 *                  precision (boundaries: INT8 band, sink, INT4 band;
 *                  bitmask: FP16 runs, then INT8 runs; four-way: FP16,
 *                  then INT8, then INT4 runs, each in ascending key
 *                  order, adjacent equal tiles merged); SKIP tiles are never
 *                  listed ([TriAttention] abstract: precision-grouped
 *                  traversals; omitted tiles are skipped).
 *  bits_off:       0 (the bitmask stays in the caller's buffer).
 *  Hybrid traversals also hold (header words 16..23: window, n_gtiles and
 *  the byte offsets of the tables below):
 *   sel table      nseq*hq x uint32[4] {list start, list length, first
 *                  gathered tile, first column-mask word};
 *   sel off        nseq*hq + 1 int32: the list offsets, staged from host
 *                  lists (unused with device lists);
 *   sel idx        the selected positions (int32);
 *   column masks   u64 per (sequence, query head, key tile): bit k set when
 *                  key 64j + k is selected (masked out of regular tiles);
 *   gathered tiles per tile: a uint32[4] {tok_start, blk_start, kv head,
 *                  keys} entry, int32[64] key positions (INT32_MAX past the
 *                  list), K rows [64][d] 16-bit and V^T [d][64] fp16.
 *  Hybrid runs: prec 3 (FP16, whole tile in the window), 7 (FP16, window
 *  part of an edge tile), 2 (INT8, whole tile outside), 6 (INT8, outside part
 *  of an edge tile), 11 (gathered FP16 tiles: first = global gathered tile
 *  index); the census counts tile passes (edge tiles twice, gathered tiles
 *  as FP16) and no skips. */
#define TM_TRAV_MAGIC 0x564D5454u
#define TM_TRAV_VERSION 1u
#define TM_TRAV_HEADER_BYTES 256

/* ---------------------------------------------------------------- helpers */

/* Human-readable name of a status code (static string). */
const char* tm_status_string(int32_t status);

/* Library version, (major << 16) | minor. */
int32_t tm_version(void);

/* nblk for a shape (host only, no GPU work); -1 if the shape is invalid. */
int64_t tm_num_blocks(const tm_shape* shape);

/* ------------------------------------------------------------ entry points */

/* Quantize and pack x [T][heads][d] (shape->dtype, device) into `out`
 * (device buffers sized for out->heads, out->layout, out->nblk).
 * out->t16 may be NULL; it is written only for TM_COLS.
 * Errors: TM_E_ARG (NULL pointers, heads <= 0, bad layout), TM_E_SHAPE (d,
 * dtype, cu_seqlens, nblk mismatch).  ([TriAttention] abstract: quantized keys
 * and values prepared during prefill.) */
tm_status tm_quantize_pack(const tm_shape* shape, const void* x, int32_t heads,
                           tm_qtensor* out, void* stream);

/* Expand a policy into the precision-grouped traversal read by tm_prefill.
 * trav == NULL: write the required size to *trav_bytes and return TM_OK
 * without touching the GPU.  Otherwise *trav_bytes is the capacity of `trav`
 * (device); TM_E_SPACE if too small.  census (host, may be NULL): when given,
 * the counts are also summed on the GPU (into the traversal's header) and the
 * call synchronizes `stream` and fills it; without it the header's counts are
 * left as they were.
 * Errors: TM_E_ARG (unknown kind, NULL arrays), TM_E_SHAPE, TM_E_POLICY
 * (b8 > b4, negative boundaries, b4 == 0 without sink, group < 1, n_words too
 * small; hybrid: window < 0, offsets not starting at 0 or decreasing, a list
 * not strictly increasing or outside its sequence), TM_E_SPACE, TM_E_HIP.
 * Hybrid policies with host lists synchronize `stream` (the lists are staged
 * from the host); with device lists (sel_idx_dev) the call does not wait.
 * ([TriAttention] abstract: boundaries generate precision-grouped traversals;
 * [TileMix] abstract: compact bitmasks, one bit per group of key tiles.) */
tm_status tm_build_traversal(const tm_shape* shape, const tm_policy* policy,
                             void* trav, size_t* trav_bytes, tm_census* census,
                             void* stream);

/* Hybrid policies only: copy each selected key's 16-bit K row (from k
 * [T][hkv][d], device) and V row (from v [T][hkv][d], the same 16-bit V that
 * tm_prefill's fp16 copy is made from: converted to fp16 the same way, bf16
 * saturated to +-65504, and transposed) into the gathered tiles of a
 * traversal built from `policy` for this shape.  Call after
 * tm_build_traversal and before tm_prefill; K and V must not change in
 * between.  ([HyQuant] "How HyQuant works": selected tokens kept in FP16.)
 * Errors: TM_E_ARG (NULL pointers, policy not hybrid), TM_E_SHAPE, TM_E_POLICY
 * (invalid lists), TM_E_HIP. */
tm_status tm_gather_selected(const tm_shape* shape, const tm_policy* policy, void* trav,
                             const void* k, const void* v, void* stream);

/* tm_build_traversal followed by tm_gather_selected, for hybrid policies, in
 * one launch: one workgroup per list builds the tables as tm_build_traversal
 * does, one workgroup per gathered tile fills it as tm_gather_selected does
 * (both find the tile's keys from the same lists), so the traversal holds the
 * same bytes as after the two calls.  Arguments as for the two calls; trav ==
 * NULL is the size query of tm_build_traversal.  Waits as tm_build_traversal
 * does (host lists and census: yes; device lists: no).
 * Errors: those of the two calls; TM_E_ARG for a policy that is not hybrid or
 * NULL k or v.  ([HyQuant] "How HyQuant works": selected tokens kept in
 * FP16.) */
tm_status tm_build_traversal_gather(const tm_shape* shape, const tm_policy* policy, void* trav,
                                    size_t* trav_bytes, tm_census* census, const void* k,
                                    const void* v, void* stream);

/* Vertical-line token selection for the hybrid policies ([HyQuant] "The
 * observation behind the method" and "How HyQuant works": a few key positions
 * are attended by many queries; tokens to keep in FP16 are picked from
 * attention-pattern signals).  For every (sequence s, query head h) the
 * attention mass each key receives from the last min(n_obs, len_s) query rows
 * (softmax over each row's keys of scale * q . k on the 16-bit values, fp32):
 *   mass[h][t] (device float [hq][T], written; head-major, so that a list's
 *   keys are contiguous).
 * sel_idx (device int32, may be NULL): the counts[s] keys of largest mass of
 * each list, ascending (ties to the lower position); lists are per query head
 * (per_kv_head = 0: mass of the head) or per KV head (per_kv_head = 1: mass
 * summed over the KV head's query heads), ordered sequence, then head, each of
 * counts[s] entries -- the layout of the hybrid policy lists (sel_off follows
 * from counts).  q [T][hq][d], k [T][hkv][d] 16-bit (device); counts host
 * [nseq], 0 <= counts[s] <= len_s; 1 <= n_obs <= 64.
 * ws: workspace; ws == NULL writes the size to *ws_bytes and returns TM_OK.
 * Up to 64 sequences the per-sequence table travels in the kernel arguments
 * and the call does not wait; with more it is staged from the host into ws
 * and the call synchronizes `stream`.
 * Errors: TM_E_ARG, TM_E_SHAPE, TM_E_POLICY (counts, n_obs), TM_E_SPACE,
 * TM_E_HIP. */
tm_status tm_select_vertical(const tm_shape* shape, const void* q, const void* k, int32_t n_obs,
                             const int32_t* counts, int32_t per_kv_head, float* mass, int32_t* sel_idx,
                             void* ws, size_t* ws_bytes, void* stream);

/* Fused tile-routed causal prefill.
 *  trav: built by tm_build_traversal for this shape; policy_kind: the kind
 *    of the policy it was built from (selects the kernel specialization; a
 *    traversal of another kind leaves o untouched).
 *  q [T][hq][d], k [T][hkv][d]: 16-bit inputs (device; read on FP16 tiles).
 *  qq (TM_ROWS, hq heads), kq (TM_ROWS, hkv heads): quantized Q and K.
 *  vq (TM_COLS, hkv heads) with t16 set: V in fp16, transposed per block (the
 *    PV product always uses these unquantized values).
 *  o [T][hq][d] of o_dtype (TM_F32, TM_F16 or TM_BF16, device).
 *  lse [hq][T] float (device, may be NULL): natural-log sum of exponentials.
 *  dbg_qk / dbg_tiles / n_dbg (device, may be NULL / 0): for each listed
 *    integer tile {seq, head, qtile, ktile} the raw integer QK products of
 *    the whole tile are written to dbg_qk[n][bq][bk] (int32, INT4 tiles in
 *    code units) by the same kernel; listed tiles that are FP16 or skipped
 *    are left untouched.
 * Per row, the output is the softmax over the row's executed keys of the
 * tile scores (INT tiles: a * sq * sk * scale with a the exact integer dot
 * product of codes; FP16 tiles: scale * q . k), applied to V, with P rounded
 * to fp16 for the PV product ([TriAttention] abstract: one normalized output
 * from both QK precisions; [TileMix] abstract: shared online-softmax state).
 * Errors: TM_E_ARG, TM_E_SHAPE (tensors not matching the shape),
 * TM_E_ARG also when kq has no c4x under a boundary policy;
 * TM_E_UNSUPPORTED (a sequence whose 16-bit keys, or whose fp16 V copy, span
 * 2 GiB or more: len * hkv * d * 2 >= 2^31, or ceil(len / 64) * 64 * hkv * d
 * * 2 >= 2^31), TM_E_HIP. */
tm_status tm_prefill(const tm_shape* shape, const void* trav, int32_t policy_kind,
                     const void* q, const void* k,
                     const tm_qtensor* qq, const tm_qtensor* kq, const tm_qtensor* vq,
                     void* o, int32_t o_dtype, float* lse,
                     int32_t* dbg_qk, const int32_t* dbg_tiles, int32_t n_dbg,
                     void* stream);

/* Decode: one new query per sequence over the compressed cache.
 *  cache: shape of the cached sequences (nseq = batch, len = cache length L
 *    including the new token, or the capacity of a growing cache whose
 *    current lengths policy->lengths gives); dtype TM_F16 or TM_BF16 (type of q and k16;
 *    bf16 values are narrowed to fp16 for the MFMA, exact for magnitudes in
 *    [2^-14, 65504] and saturated to +-65504 beyond it); hq/hkv <= 16.
 *  q [nseq][hq][d] 16-bit (device).
 *  kq (TM_ROWS, hkv heads), vq (TM_COLS, hkv heads, t16 set): the cache, as
 *    produced by tm_quantize_pack over the cached tokens.
 *  k16 [T][hkv][d] 16-bit (device): keys read for FP16 blocks.
 *  policy: block tags per KV head or per query head (tm_dpolicy); with
 *    lengths set, the tags and the keys follow each sequence's current length.
 *    The workspace size depends on the maps only through their runs of equal
 *    maps (query the size with the policy that will be used).
 *  o [nseq][hq][d] of o_dtype (TM_F32 or TM_F16, device).
 *  ws (device): workspace; ws == NULL writes the required size to *ws_bytes
 *    and returns TM_OK without GPU work; otherwise *ws_bytes is its capacity.
 *    The size depends on the cache shape (capacities), not on lengths.
 * INT blocks: score = scale * sk * (q . ck), value = sv * cv; FP16 blocks:
 * score = scale * (q . k), value = v ([HyQuant] "How HyQuant works":
 * dequantization fused with attention).
 * Errors: TM_E_ARG, TM_E_SHAPE, TM_E_POLICY (bad boundaries, sink, tail or
 * per_q_head), TM_E_SPACE, TM_E_UNSUPPORTED
 * (hq/hkv > 16, more than 64 KV heads or 256 query heads, or a sequence whose 16-bit keys or
 * fp16 V copy span 2 GiB or more: ceil(len / 64) * 64 * hkv * d * 2 >= 2^31),
 * TM_E_HIP. */
/* Build the selected-token buffer of `policy` (its sel_off / sel_idx lists)
 * for a cache: column masks of every cache block and the selected keys'
 * 16-bit K rows (from k16 [T][hkv][d]) and fp16 V columns (from vq->t16)
 * gathered into tiles of 64.  sel_buf == NULL: write the required size to
 * *sel_bytes and return TM_OK without GPU work; otherwise *sel_bytes is its
 * capacity (TM_E_SPACE if too small).  Call again after the listed tokens'
 * K or V change.  With host lists it synchronizes `stream` (the tables are
 * staged from the host); with device lists (sel_idx_dev) the tables are built
 * by a kernel and the call does not wait.  Errors: TM_E_ARG, TM_E_SHAPE,
 * TM_E_POLICY (lists), TM_E_SPACE, TM_E_HIP. */
tm_status tm_decode_select(const tm_shape* cache, const tm_dpolicy* policy, const void* k16,
                           const tm_qtensor* vq, void* sel_buf, size_t* sel_bytes, void* stream);

tm_status tm_decode(const tm_shape* cache, const void* q,
                    const tm_qtensor* kq, const tm_qtensor* vq, const void* k16,
                    const tm_dpolicy* policy, void* o, int32_t o_dtype,
                    void* ws, size_t* ws_bytes, void* stream);

/* tm_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and errors as tm_decode;
 * the split-K partials live in a library-owned 8 MiB device array
 * (tm_decode_noalloc_max_workspace()), one per GPU, held until the process
 * ends.  The call allocates and frees nothing.  A request whose workspace
 * (the size tm_decode reports for the same arguments) exceeds 8 MiB returns
 * TM_E_SPACE before any GPU work; as a guide, 32 query heads of d = 128 fit
 * up to about 480 sequences.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (on different streams, or from
 * different host threads without ordering) race and give wrong outputs.
 * Consecutive calls on one stream are safe (nothing in the array needs to
 * start at zero; each call writes the partials it reads).  The first call on
 * a device looks the array's device address up (hipGetSymbolAddress) with
 * that device current.  Errors: those of tm_decode, TM_E_SPACE as above,
 * TM_E_HIP if the address lookup fails. */
tm_status tm_decode_noalloc(const tm_shape* cache, const void* q,
                            const tm_qtensor* kq, const tm_qtensor* vq, const void* k16,
                            const tm_dpolicy* policy, void* o, int32_t o_dtype, void* stream);

/* Size in bytes of tm_decode_noalloc's device array (host only). */
size_t tm_decode_noalloc_max_workspace(void);

/* Cache append during generation ([TriAttention] abstract: the codes made
 * during prefill are reused as the decode cache; [HyQuant] "How HyQuant
 * works": the recent tokens stay FP16 and older ones are quantized).
 *  cache: the cache shape with each sequence's capacity as its length (the
 *    layout of the quantized tensors and of x's rows).
 *  lengths (host [nseq]): current lengths after the append, 1 <= lengths[s]
 *    <= capacity; the caller has written the new tokens' rows of x.
 *  x [T][heads][d] 16-bit (device): K (out TM_ROWS) or V (out TM_COLS with
 *    t16) in the capacity layout.
 *  out: the cache tensor to update.
 * For every sequence, the 64-token block holding its newest token is
 * quantized again over the sequence's current length (the codes and scales
 * tm_quantize_pack would give for that length; V's fp16 copy too), so after
 * appending tokens one at a time the cache equals the one built from
 * scratch at the new lengths.  One launch per 128 sequences.
 * Errors: TM_E_ARG, TM_E_SHAPE (tensors not matching the shape, a length out
 * of range), TM_E_HIP. */
tm_status tm_cache_append(const tm_shape* cache, const int32_t* lengths, const void* x, int32_t heads,
                          tm_qtensor* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TM_H */
