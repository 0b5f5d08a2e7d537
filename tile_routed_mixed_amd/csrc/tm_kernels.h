// Kernel argument blocks and launchers shared by the HIP sources and the C ABI.
#pragma once

#include "tm_common.h"

namespace tmx {

constexpr int kMaxHeadsArg = 256;   // boundary tables passed by value
constexpr int kMaxKvArg = 64;
constexpr int kMaxClsArg = 64;     // decode head classes per launch (tables passed by value)
constexpr int kMaxSeqArg = 128;    // sequences per decode launch (tables passed by value)
constexpr int kMaxHeadArg = 64;    // query heads whose decode maps travel in the kernel arguments

struct QuantArgs {
  const uint16_t* x;
  const int32_t* cu;
  int nseq;
  int heads;
  int64_t nblk;
  int8_t* c8;
  uint8_t* c4;
  float* s8;
  float* s4;
  uint16_t* t16;
  int8_t* c4x;     // rows layout only, may be null: INT4 codes one per byte
};

struct AppendArgs {
  QuantArgs q;                  // x, heads, nblk and the outputs (cu and nseq unused)
  int n;                        // sequences of this launch
  int32_t blk[kMaxSeqArg];      // global block holding each sequence's newest token
  int32_t tok[kMaxSeqArg];      // its first token row in x
  int32_t nvalid[kMaxSeqArg];   // its valid rows
};

struct TravArgs {
  uint8_t* trav;
  const int32_t* cu;
  const uint32_t* bits;     // device bitmask (bitmask policies)
  int nseq, hq, hkv, d, bq, bk;
  int kind, sink, group;
  uint32_t n_items, max_runs, nblk;
  uint32_t seq_off, item_off, run_off, bits_off;
  int32_t b8[kMaxHeadsArg];
  int32_t b4[kMaxHeadsArg];
};

struct GatherArgs {
  uint8_t* trav;
  const uint16_t* k;        // [T][hkv][D] 16-bit
  const uint16_t* vt16;     // [nblk][hkv][D][64] fp16 (decode selection buffers)
  const uint16_t* v;        // [T][hkv][D] 16-bit (hybrid traversals), or null
  int hkv, bf16;
  uint32_t n_gtiles, gh_off, gk_off, gv_off;
};

// Hybrid traversal, built in one launch from the selected lists: one
// workgroup per (sequence, query head) list writes its list entry, positions,
// column masks, gathered-tile headers and the work items and runs of every
// query tile of that head (the TravArgs fields of the other kinds, plus the
// list tables).  off / idx: list offsets and positions in device memory, or
// the traversal's own staged copies (copy_idx = 0).
struct HybArgs {
  uint8_t* trav;
  const int32_t* cu;
  const int32_t* off;
  const int32_t* idx;
  int nseq, hq, hkv, d, bq, bk;
  uint32_t n_items, max_runs, nblk;
  uint32_t seq_off, item_off, run_off;
  uint32_t window, n_sel, n_gt, sel_tab_off, sel_idx_off, cm_off, gh_off, gk_off, gv_off;
  int copy_idx;
  // gather sources (16-bit K and V rows), or null: with them the same launch
  // also fills the gathered tiles, one workgroup per tile after the lists'
  const uint16_t* gk_src;
  const uint16_t* gv_src;
  int bf16;
};

// Decode selection tables built on the GPU from device-resident lists (one
// list per (sequence, KV head)).  n_sel and n_gt are the list entries and
// gathered tiles the host sized the buffer for: every write and every list
// read stays below them whatever the device offsets hold.
struct SelTabArgs {
  uint8_t* buf;
  const int32_t* cu;        // device cu_seqlens
  const int32_t* off;       // device list offsets [nseq * hkv + 1]
  const int32_t* idx;       // device positions
  int hkv;
  uint32_t n_sel, n_gt;
  uint32_t tab_off, cm_off, gh_off;
};

struct PrefillArgs {
  const uint8_t* trav;
  const uint16_t* q;
  const uint16_t* k;
  const int8_t* q8;
  const uint8_t* q4;
  const float* qs8;
  const float* qs4;
  const int8_t* k8;
  const uint8_t* k4;
  const int8_t* k4x;       // K's INT4 codes one per byte (boundary policies)
  const float* ks8;
  const float* ks4;
  const uint16_t* vt16;
  void* o;
  float* lse;
  int32_t* dbg_qk;
  const int32_t* dbg_tiles;
  int n_dbg;
  int o_dtype;
  int hq, hkv, T;
  int64_t nblk;
  uint32_t n_items;   // grid size; the traversal header holds the rest
  float tau_log2e;
};

struct DecodeArgs {
  const uint16_t* q;       // [B][hq][D] 16-bit
  const int8_t* k8;        // rows  [nblk][hkv][64][D]
  const uint8_t* k4;       // rows  [nblk][hkv][64][D/2]
  const float* ks8;
  const float* ks4;
  const int8_t* v8;        // cols  [nblk][hkv][D][64]
  const uint8_t* v4;       // cols  [nblk][hkv][D][32]
  const float* vs8;
  const float* vs4;
  const uint16_t* vt16;    // cols  [nblk][hkv][D][64] fp16
  const uint16_t* k16;     // [T][hkv][D] 16-bit
  float* ws;               // [B][hq][nsplit][D + 2]
  void* o;
  int o_dtype;
  int nseq, hq, hkv, nsplit, sink, tail;
  int64_t nblk;
  float tau_log2e;
  // head classes: class c (grid y) is `n` consecutive query heads from h0,
  // all of KV head kv, with one cache map (b8[c], b4[c]);
  // cls[c] = kv | h0 << 10 | n << 20 | uni << 30.  uni: the class holds the
  // whole group of a KV head whose query heads have different maps (hb8,
  // hb4 per query head); b8[c], b4[c] are then the group's largest and
  // b8min[c] its smallest b8
  int32_t cls[kMaxClsArg];
  int32_t b8[kMaxClsArg];
  int32_t b4[kMaxClsArg];
  int32_t b8min[kMaxClsArg];
  int32_t hb8[kMaxHeadArg];
  int32_t hb4[kMaxHeadArg];
  // selected tokens (kept in FP16): buffer written by tm_decode_select, or
  // null; list entries {first gathered tile, keys} per (sequence, KV head),
  // column masks [nblk][hkv] u64, gathered K rows and V^T (byte offsets)
  const uint8_t* sel;
  uint32_t sel_tab, sel_cm, sel_gk, sel_gv;
  int seq0;                     // first sequence of this launch
  int32_t cu[kMaxSeqArg + 1];   // token offsets of this launch's sequences (absolute)
  int32_t len[kMaxSeqArg];      // their current lengths (at most cu[i + 1] - cu[i])
  int32_t blk[kMaxSeqArg];      // their first cache block (absolute)
};

constexpr int kSelInline = 64;   // most sequences whose table travels in the kernel arguments
struct SelectArgs {
  const uint16_t* q;        // [T][hq][D] 16-bit
  const uint16_t* k;        // [T][hkv][D] 16-bit
  const int32_t* cu;        // device prefix sums
  int nseq, hq, hkv, n_obs, bf16, per_kv;
  float tau_log2e;
  float* part;              // [tiles][hq][64][2] partial (max, sum) per probe row
  float* rows;              // [nseq][hq][64][2] each probe row's (max, log2 sum)
  float* mass;              // [hq][T] attention mass of each key
  int64_t T;                // total tokens
  int tw;                   // key tiles per workgroup of passes 1 and 3 (set at launch)
  // per sequence: first tile, keys to select per list, first output entry of
  // its lists; as tab[3][nseq] in the workspace, or (nseq <= kSelInline,
  // tab == null) in itab, carried by the kernel arguments
  const int32_t* tab;
  int32_t* sel;             // output positions, or null (mass only)
  int32_t itab[3 * kSelInline];
};

__device__ __forceinline__ int sel_tab(const SelectArgs& a, int which, int b) {
  return a.tab != nullptr ? a.tab[which * a.nseq + b] : a.itab[which * a.nseq + b];
}

hipError_t launch_quantize(const QuantArgs& a, int d, bool bf16, bool cols, hipStream_t st);
hipError_t launch_append(const AppendArgs& p, int d, bool bf16, bool cols, hipStream_t st);
hipError_t launch_traversal(const TravArgs& a, bool census, hipStream_t st);   // census: also sum the counts into the header
hipError_t launch_gather(const GatherArgs& a, int d, hipStream_t st);        // V from the fp16 V^T copy
hipError_t launch_gather_rows(const GatherArgs& a, int d, hipStream_t st);   // V from 16-bit rows
hipError_t launch_sel_tables(const SelTabArgs& a, int n_lists, hipStream_t st);
hipError_t launch_hybrid_build(const HybArgs& a, bool census, hipStream_t st);
hipError_t launch_select(const SelectArgs& a, int d, int maxnt, int64_t tiles, hipStream_t st);
hipError_t launch_prefill(const PrefillArgs& a, int d, int bq, int kind, bool bf16, hipStream_t st);
// boundary policies: the software-pipelined kernel (k_prefill_pipe.hip)
hipError_t launch_prefill_pipe(const PrefillArgs& a, int d, int bq, hipStream_t st);
hipError_t launch_decode_split(const DecodeArgs& a, int ncls, bool small, int d, bool bf16, hipStream_t st);
// (a.sel selects the variant that reads selected tokens)
hipError_t launch_decode_combine(const DecodeArgs& a, int d, hipStream_t st);

}  // namespace tmx
