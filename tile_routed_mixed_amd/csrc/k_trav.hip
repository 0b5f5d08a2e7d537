// Policy expansion: per-head boundaries or a packed group bitmask become the
// precision-grouped traversal that the prefill kernel walks.
//
// [TriAttention] "TriAttention: Unified Sparse Mixed-Precision Attention for
// Long-Context LLM Inference", abstract: two diagonal-distance boundaries per
// head, storage independent of context length; the boundaries generate
// precision-grouped traversals and omitted tiles are skipped.
// [TileMix] "TileMix: Tile-Centric Mixed-Precision Attention for LLM Inference
// Acceleration", abstract: routing decisions packed into compact bitmasks; one
// bit governs a group of adjacent key tiles; FP16 or INT8 per group; all legal
// groups routed; variable-length batches.
// The four-way kind puts the two together: a 2-bit code per group either
// leaves its tiles to the boundary rule (code 0) or sets INT4, INT8 or FP16.
//
// One thread per work item (sequence, query head, query tile).  Items are
// ordered heavy-first: query tiles in descending index (more legal key tiles),
// then sequence, then head, so the 4 heads sharing a KV head are adjacent.
#include "tm_kernels.h"

namespace tmx {


__device__ __forceinline__ int seq_nq(const int32_t* cu, int s, int bq) {
  return (cu[s + 1] - cu[s] + bq - 1) / bq;
}

// Number of items in levels >= i (levels are query-tile indices).
__device__ __forceinline__ int64_t items_at_or_above(const TravArgs& a, int i) {
  int64_t n = 0;
  for (int s = 0; s < a.nseq; ++s) {
    const int nq = seq_nq(a.cu, s, a.bq);
    if (nq > i) n += nq - i;
  }
  return n * a.hq;
}

__device__ __forceinline__ void put_run(RunEntry* runs, uint32_t& n, uint32_t first, uint32_t count,
                                        uint32_t prec, uint32_t max_runs) {
  // max_runs bounds every item's runs by construction; the check keeps a
  // wrong bound from writing into the next item's slots
  if (count == 0 || n >= max_runs) return;
  runs[n].ktile = first;
  runs[n].count_prec = count | (prec << 24);
  ++n;
}

__global__ __launch_bounds__(256) void trav_items_kernel(TravArgs a) {
  const uint32_t k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k == 0) {
    TravHeader* h = reinterpret_cast<TravHeader*>(a.trav);
    h->magic = TM_TRAV_MAGIC;
    h->version = TM_TRAV_VERSION;
    h->kind = a.kind;
    h->n_items = a.n_items;
    h->max_runs = a.max_runs;
    h->nseq = a.nseq;
    h->hq = a.hq;
    h->hkv = a.hkv;
    h->bq = a.bq;
    h->bk = a.bk;
    h->d = a.d;
    h->nblk = a.nblk;
    h->seq_off = a.seq_off;
    h->item_off = a.item_off;
    h->run_off = a.run_off;
    h->bits_off = a.bits_off;
    h->window = h->n_gtiles = 0u;   // (hybrid traversals come from hyb_build_kernel)
    h->sel_tab_off = h->sel_idx_off = h->cm_off = h->gh_off = h->gk_off = h->gv_off = 0u;
  }
  if (k < static_cast<uint32_t>(a.nseq)) {
    SeqEntry* st = reinterpret_cast<SeqEntry*>(a.trav + a.seq_off);
    int blk = 0;
    for (int s = 0; s < static_cast<int>(k); ++s) blk += (a.cu[s + 1] - a.cu[s] + kBlock - 1) / kBlock;
    st[k].tok_start = a.cu[k];
    st[k].len = a.cu[k + 1] - a.cu[k];
    st[k].blk_start = blk;
    st[k].nq = seq_nq(a.cu, k, a.bq);
  }
  if (k >= a.n_items) return;

  // level (query tile index) of item k: largest i with items_at_or_above(i) > k
  int maxnq = 0;
  for (int s = 0; s < a.nseq; ++s) maxnq = max(maxnq, seq_nq(a.cu, s, a.bq));
  int lo = 0, hi = maxnq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (items_at_or_above(a, mid) > static_cast<int64_t>(k)) lo = mid; else hi = mid - 1;
  }
  const int qt = lo;
  const int64_t idx = static_cast<int64_t>(k) - items_at_or_above(a, qt + 1);
  const int rank = static_cast<int>(idx / a.hq);
  const int head = static_cast<int>(idx % a.hq);
  int seq = -1, cnt = 0;
  for (int s = 0; s < a.nseq; ++s) {
    if (seq_nq(a.cu, s, a.bq) > qt) {
      if (cnt == rank) { seq = s; break; }
      ++cnt;
    }
  }
  const int len = a.cu[seq + 1] - a.cu[seq];
  const int jmax = (min((qt + 1) * a.bq, len) - 1) / a.bk;
  const int legal = jmax + 1;
  RunEntry* runs = reinterpret_cast<RunEntry*>(a.trav + a.run_off) + static_cast<size_t>(k) * a.max_runs;
  uint32_t nr = 0, n8 = 0, n4 = 0, n16 = 0;

  if (a.kind == TM_POLICY_BOUNDARIES) {
    const int b8 = a.b8[head], b4 = a.b4[head];
    const int ri = qt * (a.bq / a.bk);
    // INT8 band [lo8, jmax]; INT4 band [lo4, hi4]; SKIP [0, lo4)
    const int lo8 = (b8 > 0) ? max(0, ri - b8 + 1) : legal;
    int lo4 = (b4 > 0) ? max(0, ri - b4 + 1) : legal;
    int hi4 = (b8 > 0) ? lo8 - 1 : jmax;
    if (b4 == 0) hi4 = -1;
    lo4 = min(lo4, legal);
    hi4 = min(hi4, jmax);
    const bool sink_extra = a.sink && lo8 > 0;
    if (sink_extra && lo4 == 0) lo4 = 1;   // tile 0 leaves the INT4 band for the sink run
    const uint32_t c8 = lo8 <= jmax ? static_cast<uint32_t>(jmax - lo8 + 1) : 0u;
    const uint32_t c4 = hi4 >= lo4 ? static_cast<uint32_t>(hi4 - lo4 + 1) : 0u;
    put_run(runs, nr, lo8, c8, TM_INT8, a.max_runs);
    if (sink_extra) put_run(runs, nr, 0, 1, TM_INT8, a.max_runs);
    put_run(runs, nr, lo4, c4, TM_INT4, a.max_runs);
    n8 = c8 + (sink_extra ? 1u : 0u);
    n4 = c4;
  } else {
    const int G = a.group;
    const bool four = a.kind == TM_POLICY_FOURWAY;
    const int per_word = four ? 16 : 32;
    int base = 0;
    for (int s = 0; s < seq; ++s) {
      const int ln = a.cu[s + 1] - a.cu[s];
      const int nk = (ln + a.bk - 1) / a.bk;
      const int wpr = ((nk + G - 1) / G + per_word - 1) / per_word;
      base += a.hq * seq_nq(a.cu, s, a.bq) * wpr;
    }
    const int nk = (len + a.bk - 1) / a.bk;
    const int wpr = ((nk + G - 1) / G + per_word - 1) / per_word;
    const int nq = seq_nq(a.cu, seq, a.bq);
    const uint32_t* row = a.bits + base + static_cast<size_t>(head * nq + qt) * wpr;
    const int ng = jmax / G + 1;
    if (!four) {
      for (int pass = 0; pass < 2; ++pass) {        // FP16 runs first, then INT8
        const uint32_t want = pass == 0 ? 1u : 0u;
        int g = 0;
        while (g < ng) {
          const uint32_t bit = (row[g >> 5] >> (g & 31)) & 1u;
          if (bit != want) { ++g; continue; }
          int g1 = g;
          while (g1 + 1 < ng && ((row[(g1 + 1) >> 5] >> ((g1 + 1) & 31)) & 1u) == want) ++g1;
          const int first = g * G;
          const int last = min((g1 + 1) * G - 1, jmax);
          const uint32_t c = static_cast<uint32_t>(last - first + 1);
          put_run(runs, nr, first, c, want ? TM_FP16 : TM_INT8, a.max_runs);
          if (want) n16 += c; else n8 += c;
          g = g1 + 1;
        }
      }
    } else {
      // boundary rule of this head: key tile j is INT8 from lo8, INT4 from lo4
      // (by diagonal distance ri - j), the sink tile 0 INT8, the rest SKIP
      const int b8 = a.b8[head], b4 = a.b4[head];
      const int ri = qt * (a.bq / a.bk);
      const int lo8 = b8 > 0 ? max(0, ri - b8 + 1) : (1 << 30);
      const int lo4 = b4 > 0 ? max(0, ri - b4 + 1) : (1 << 30);
      auto rule = [&](int j) -> uint32_t {
        if (a.sink && j == 0) return TM_INT8;
        return j >= lo8 ? TM_INT8 : (j >= lo4 ? TM_INT4 : TM_SKIP);
      };
      // one pass per precision (FP16, INT8, INT4) over constant pieces: a
      // piece ends at a group edge or where the boundary rule may change.  A
      // sink tile outside the INT8 band runs after the other INT8 tiles, the
      // order of the boundary traversal, so all-zero codes reproduce it.
      const bool late_sink = a.sink && lo8 > 0 && (row[0] & 3u) == 0u;
      const uint32_t order[3] = {TM_FP16, TM_INT8, TM_INT4};
      for (int pass = 0; pass < 3; ++pass) {
        const uint32_t want = order[pass];
        int rfirst = 0, rcount = 0;
        for (int g = 0; g < ng; ++g) {
          const uint32_t code = (row[g >> 4] >> (2 * (g & 15))) & 3u;
          const int gend = min(g * G + G - 1, jmax);
          int j = (late_sink && g == 0) ? 1 : g * G;
          while (j <= gend) {
            uint32_t p;
            int pend = gend;
            if (code != 0) {
              p = code == 1 ? TM_INT4 : (code == 2 ? TM_INT8 : TM_FP16);
            } else {
              p = rule(j);
              if (j == 0) pend = 0;                       // the sink tile stands alone
              if (lo4 > j && lo4 <= pend) pend = lo4 - 1;
              if (lo8 > j && lo8 <= pend) pend = lo8 - 1;
            }
            if (p == want) {
              if (rcount > 0 && rfirst + rcount == j) {
                rcount += pend - j + 1;
              } else {
                put_run(runs, nr, rfirst, static_cast<uint32_t>(rcount), want, a.max_runs);
                rfirst = j;
                rcount = pend - j + 1;
              }
            }
            j = pend + 1;
          }
        }
        put_run(runs, nr, rfirst, static_cast<uint32_t>(rcount), want, a.max_runs);
        if (want == TM_INT8 && late_sink) put_run(runs, nr, 0, 1, TM_INT8, a.max_runs);
        // counts of this pass
        uint32_t cnt = 0;
        for (uint32_t r = 0; r < nr; ++r)
          if ((runs[r].count_prec >> 24) == want) cnt += runs[r].count_prec & 0xFFFFFFu;
        if (want == TM_FP16) n16 = cnt; else if (want == TM_INT8) n8 = cnt; else n4 = cnt;
      }
    }
  }
  ItemEntry* it = reinterpret_cast<ItemEntry*>(a.trav + a.item_off) + k;
  it->seq = seq;
  it->head = head;
  it->qtile = qt;
  it->nruns = nr;
  it->n8 = n8;
  it->n4 = n4;
  it->n16 = n16;
  it->nskip = static_cast<uint32_t>(legal) - n8 - n4 - n16;
}

// Deterministic census: one workgroup sums the per-item counts.
__global__ __launch_bounds__(256) void trav_census_kernel(uint8_t* trav, uint32_t item_off, uint32_t n_items) {
  const ItemEntry* it = reinterpret_cast<const ItemEntry*>(trav + item_off);
  int64_t c[4] = {0, 0, 0, 0};
  for (uint32_t k = threadIdx.x; k < n_items; k += blockDim.x) {
    c[0] += it[k].n8;
    c[1] += it[k].n4;
    c[2] += it[k].n16;
    c[3] += it[k].nskip;
  }
  __shared__ int64_t red[4][256];
  for (int i = 0; i < 4; ++i) red[i][threadIdx.x] = c[i];
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (static_cast<int>(threadIdx.x) < s)
      for (int i = 0; i < 4; ++i) red[i][threadIdx.x] += red[i][threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    TravHeader* h = reinterpret_cast<TravHeader*>(trav);
    h->census[0] = red[0][0] + red[1][0] + red[2][0] + red[3][0];
    h->census[1] = red[0][0];
    h->census[2] = red[1][0];
    h->census[3] = red[2][0];
    h->census[4] = red[3][0];
  }
}

// Position of entry e of a list, or INT32_MAX (an empty slot: never
// gathered, and past every causal row) when it lies outside [0, len).
__device__ __forceinline__ int32_t clean_pos(int32_t c, int len) { return (c >= 0 && c < len) ? c : INT32_MAX; }

// A list's entries [lo, lo + n) of the positions, clamped to the n_sel
// entries the buffers were sized for.
__device__ __forceinline__ int2 list_span(const int32_t* off, int r, uint32_t n_sel) {
  const int32_t lo = min(max(off[r], 0), static_cast<int32_t>(n_sel));
  const int32_t hi = min(max(off[r + 1], lo), static_cast<int32_t>(n_sel));
  return make_int2(lo, hi - lo);
}

__device__ __forceinline__ int block_sum256(int v, int* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Exclusive prefix of v over the 256 threads of a workgroup; *total = sum.
__device__ __forceinline__ int block_scan256(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) red[w] = x;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) base += u < w ? red[u] : 0;
  *total = red[0] + red[1] + red[2] + red[3];
  return base + x - v;
}

// Decode selection tables from lists in device memory: one workgroup per list
// (sequence s, KV head g).  It writes the list's entry {first gathered tile,
// keys}, the column masks of its sequence's cache blocks (bit k of block j set
// when key 64 j + k is listed) and the headers and positions of its gathered
// tiles.  The list's first gathered tile and its sequence's first block are
// sums over the lists and sequences before it, reduced by the workgroup.  The
// lists are meant to be strictly increasing positions inside their sequence;
// they are not checked, but a position outside the sequence becomes an empty
// slot and no read or write leaves the buffers.
__global__ __launch_bounds__(256) void sel_tables_kernel(SelTabArgs a) {
  __shared__ int red[4];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int s = r / a.hkv, h = r % a.hkv;
  int blk = 0, gb = 0;
  for (int u = tid; u < s; u += 256) blk += (a.cu[u + 1] - a.cu[u] + kBlock - 1) / kBlock;
  for (int u = tid; u < r; u += 256) gb += (list_span(a.off, u, a.n_sel).y + kBlock - 1) / kBlock;
  blk = block_sum256(blk, red);
  gb = min(block_sum256(gb, red), static_cast<int>(a.n_gt));
  const int tok0 = a.cu[s], len = a.cu[s + 1] - tok0, nk = (len + kBlock - 1) / kBlock;
  const int2 sp = list_span(a.off, r, a.n_sel);
  const int cnt = min(sp.y, (static_cast<int>(a.n_gt) - gb) * kBlock);
  const int32_t* li = a.idx + sp.x;
  if (tid == 0) {
    uint32_t* te = reinterpret_cast<uint32_t*>(a.buf + a.tab_off);
    te[2 * r] = static_cast<uint32_t>(gb);
    te[2 * r + 1] = static_cast<uint32_t>(cnt);
  }
  // column masks: the entries of block j are contiguous in a sorted list
  uint64_t* cm = reinterpret_cast<uint64_t*>(a.buf + a.cm_off);
  for (int j = tid; j < nk; j += 256) {
    const int k0 = j * kBlock;
    int lo = 0, hi = cnt;   // first entry >= k0
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (li[mid] < k0) lo = mid + 1; else hi = mid;
    }
    uint64_t m = 0;
    for (int e = lo; e < cnt; ++e) {
      const int c = li[e];
      if (c < k0 || c >= k0 + kBlock) break;
      if (c < len) m |= uint64_t(1) << (c - k0);
    }
    cm[static_cast<size_t>(blk + j) * a.hkv + h] = m;
  }
  // gathered tiles: header {first token, first block, KV head, keys} and 64 positions
  const int ng = (cnt + kBlock - 1) / kBlock;
  for (int u = tid; u < ng * kBlock; u += 256) {
    const int t = u / kBlock, k = u % kBlock;
    uint8_t* gh = a.buf + a.gh_off + static_cast<size_t>(gb + t) * kGatherHdr;
    const int keys = min(kBlock, cnt - kBlock * t);
    if (k == 0)
      *reinterpret_cast<GatherEntry*>(gh) = GatherEntry{static_cast<uint32_t>(tok0), static_cast<uint32_t>(blk),
                                                        static_cast<uint32_t>(h), static_cast<uint32_t>(keys)};
    reinterpret_cast<int32_t*>(gh + 16)[k] = k < keys ? clean_pos(li[kBlock * t + k], len) : INT32_MAX;
  }
}

hipError_t launch_sel_tables(const SelTabArgs& a, int n_lists, hipStream_t st) {
  if (n_lists <= 0) return hipSuccess;
  hipLaunchKernelGGL(sel_tables_kernel, dim3(n_lists), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Hybrid traversal in one launch: one workgroup per (sequence s, query head
// h) list.  It writes the list entry {start, keys, first gathered tile, first
// column-mask word}, the positions (copied in from device lists), the column
// masks of the list's key tiles, the gathered-tile headers, and the work item
// and runs of every query tile of (s, h) (sequence and traversal headers from
// the first workgroups).  The column masks are built in LDS, kHybChunk key
// tiles at a time, with a popcount prefix over them, so each query tile's
// count of selected keys it can see (positions up to its last row) is read
// off the prefix: no search over the list.  Item k of (s, h, query tile i)
// keeps the heavy-first order of the other kinds (descending i, then
// sequence, then head).  The window classes of a query tile (key tiles wholly
// inside the window, crossed by its edge, wholly outside) are contiguous in
// the key-tile index.  Lists are meant to be strictly increasing positions
// inside their sequence (host lists are checked before the launch, device
// lists are not); a position outside the sequence becomes an empty slot and
// every write stays inside the sizes the host computed.
// Fill gathered tile t with the 16-bit K rows ([64][D]) and the fp16 V
// columns (V^T [D][64]) of the keys pos(0 .. keys - 1) of the sequence whose
// tokens start at tok0, KV head kv; both come from the token-major 16-bit
// inputs (each key's row is contiguous; V is converted to fp16, bf16
// saturated to the fp16 range, and transposed through LDS).  Slots past the
// keys and empty slots (position INT32_MAX) are zero.
template <int D, bool BF16, class Pos>
__device__ __forceinline__ void gather_rows_tile(uint8_t* trav, uint32_t gk_off, uint32_t gv_off, uint32_t t,
                                                 const uint16_t* k, const uint16_t* v, int hkv, uint32_t tok0,
                                                 uint32_t kv, int keys, Pos pos, _Float16* vl) {
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int VP = D + 8;     // LDS row pitch (fp16): rows start on different banks
  uint16_t* gk = reinterpret_cast<uint16_t*>(trav + gk_off) + static_cast<size_t>(t) * kBlock * D;
  uint16_t* gv = reinterpret_cast<uint16_t*>(trav + gv_off) + static_cast<size_t>(t) * D * kBlock;
  for (int u = threadIdx.x; u < kBlock * CPR; u += 256) {
    const int row = u / CPR, ch = u % CPR;
    u32x4 kx = u32x4{0u, 0u, 0u, 0u}, vx = u32x4{0u, 0u, 0u, 0u};
    const int32_t p = row < keys ? pos(row) : INT32_MAX;
    if (p != INT32_MAX) {
      const size_t off = ((static_cast<size_t>(tok0) + p) * hkv + kv) * D + ch * 8;
      kx = *reinterpret_cast<const u32x4*>(k + off);
      vx = *reinterpret_cast<const u32x4*>(v + off);
    }
    *reinterpret_cast<u32x4*>(gk + row * D + ch * 8) = kx;
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (BF16) {
        h[2 * e] = to_f16_sat(__uint_as_float(vx[e] << 16));
        h[2 * e + 1] = to_f16_sat(__uint_as_float(vx[e] & 0xFFFF0000u));
      } else {
        h[2 * e] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(vx[e] & 0xFFFFu));
        h[2 * e + 1] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(vx[e] >> 16));
      }
    }
    *reinterpret_cast<f16x8*>(vl + row * VP + ch * 8) = h;
  }
  __syncthreads();
  // V^T: channel rows of 64 slots, two slots per thread step
  for (int u = threadIdx.x; u < D * (kBlock / 2); u += 256) {
    const int c = u / (kBlock / 2), sl = 2 * (u % (kBlock / 2));
    f16x2 pr;
    pr[0] = vl[sl * VP + c];
    pr[1] = vl[(sl + 1) * VP + c];
    *reinterpret_cast<f16x2*>(gv + c * kBlock + sl) = pr;
  }
}

constexpr int kHybChunk = 1024;

// Workgroup g past the lists (when the gather sources are given) fills
// gathered tile g, as gather_rows_kernel does, from the list's positions:
// the lists' gathered tiles are numbered in list order, ceil(keys / 64) each,
// so the workgroup finds its list by a prefix over the list lengths (the
// numbering hyb_build_kernel gives the headers).
__device__ void hyb_gather(const HybArgs& a, int g, int* red) {
  __shared__ int hit[2];
  __shared__ _Float16 vl[kBlock * (128 + 8)];
  const int nl = a.nseq * a.hq, tid = threadIdx.x;
  if (tid == 0) hit[0] = -1;
  int carry = 0;
  for (int u0 = 0; u0 < nl; u0 += 256) {
    const int u = u0 + tid;
    const int nt = u < nl ? (list_span(a.off, u, a.n_sel).y + kBlock - 1) / kBlock : 0;
    int tot;
    const int ex = carry + block_scan256(nt, red, &tot);   // (synchronizes before writing red)
    if (nt > 0 && ex <= g && g < ex + nt) {
      hit[0] = u;
      hit[1] = ex;
    }
    carry += tot;
    __syncthreads();
    if (hit[0] >= 0 || carry > g) break;
  }
  const int r = hit[0];
  if (r < 0) return;   // (no list holds tile g: the host sized n_gt from the same lists)
  const int gb = hit[1], s = r / a.hq, h = r % a.hq;
  const uint32_t kv = static_cast<uint32_t>(h / (a.hq / a.hkv));
  const int tok0 = a.cu[s], len = a.cu[s + 1] - tok0;
  const int2 sp = list_span(a.off, r, a.n_sel);
  const int cnt = min(sp.y, (static_cast<int>(a.n_gt) - gb) * kBlock);
  const int tl = g - gb;
  const int keys = min(kBlock, cnt - kBlock * tl);
  const int32_t* li = a.idx + sp.x + kBlock * tl;
  auto pos = [&](int row) { return clean_pos(li[row], len); };
  const uint32_t tok = static_cast<uint32_t>(tok0);
  if (a.d == 128) {
    if (a.bf16) gather_rows_tile<128, true>(a.trav, a.gk_off, a.gv_off, g, a.gk_src, a.gv_src, a.hkv, tok, kv, keys, pos, vl);
    else gather_rows_tile<128, false>(a.trav, a.gk_off, a.gv_off, g, a.gk_src, a.gv_src, a.hkv, tok, kv, keys, pos, vl);
  } else {
    if (a.bf16) gather_rows_tile<64, true>(a.trav, a.gk_off, a.gv_off, g, a.gk_src, a.gv_src, a.hkv, tok, kv, keys, pos, vl);
    else gather_rows_tile<64, false>(a.trav, a.gk_off, a.gv_off, g, a.gk_src, a.gv_src, a.hkv, tok, kv, keys, pos, vl);
  }
}

__device__ __forceinline__ int fdiv_floor(int x, int y) { return x >= 0 ? x / y : -((-x + y - 1) / y); }

__global__ __launch_bounds__(256) void hyb_build_kernel(HybArgs a) {
  __shared__ int red[4];
  __shared__ unsigned long long cml[kHybChunk];
  __shared__ int cum[kHybChunk];
  if (static_cast<int>(blockIdx.x) >= a.nseq * a.hq) {
    hyb_gather(a, static_cast<int>(blockIdx.x) - a.nseq * a.hq, red);
    return;
  }
  const int r = blockIdx.x, tid = threadIdx.x;
  const int s = r / a.hq, h = r % a.hq;
  // first cache block of s; first gathered tile of list r
  int blk = 0, gb = 0;
  for (int u = tid; u < s; u += 256) blk += (a.cu[u + 1] - a.cu[u] + kBlock - 1) / kBlock;
  for (int u = tid; u < r; u += 256) gb += (list_span(a.off, u, a.n_sel).y + kBlock - 1) / kBlock;
  blk = block_sum256(blk, red);
  gb = min(block_sum256(gb, red), static_cast<int>(a.n_gt));
  const int tok0 = a.cu[s], len = a.cu[s + 1] - tok0;
  const int nk = (len + a.bk - 1) / a.bk, nq = (len + a.bq - 1) / a.bq;
  const int2 sp = list_span(a.off, r, a.n_sel);
  const int start = sp.x;
  const int cnt = min(sp.y, (static_cast<int>(a.n_gt) - gb) * kBlock);
  const int ng = (cnt + kBlock - 1) / kBlock;
  const int cm_base = a.hq * blk + h * nk;
  const int32_t* li = a.idx + start;
  int32_t* dst = reinterpret_cast<int32_t*>(a.trav + a.sel_idx_off) + start;
  if (tid == 0) {
    reinterpret_cast<SelEntry*>(a.trav + a.sel_tab_off)[r] =
        SelEntry{static_cast<uint32_t>(start), static_cast<uint32_t>(cnt), static_cast<uint32_t>(gb),
                 static_cast<uint32_t>(cm_base)};
    if (h == 0)
      reinterpret_cast<SeqEntry*>(a.trav + a.seq_off)[s] =
          SeqEntry{static_cast<uint32_t>(tok0), static_cast<uint32_t>(len), static_cast<uint32_t>(blk),
                   static_cast<uint32_t>(nq)};
    if (r == 0) {
      TravHeader* th = reinterpret_cast<TravHeader*>(a.trav);
      th->magic = TM_TRAV_MAGIC;
      th->version = TM_TRAV_VERSION;
      th->kind = TM_POLICY_HYBRID;
      th->n_items = a.n_items;
      th->max_runs = a.max_runs;
      th->nseq = a.nseq;
      th->hq = a.hq;
      th->hkv = a.hkv;
      th->bq = a.bq;
      th->bk = a.bk;
      th->d = a.d;
      th->nblk = a.nblk;
      th->seq_off = a.seq_off;
      th->item_off = a.item_off;
      th->run_off = a.run_off;
      th->bits_off = 0;
      th->window = a.window;
      th->n_gtiles = a.n_gt;
      th->sel_tab_off = a.sel_tab_off;
      th->sel_idx_off = a.sel_idx_off;
      th->cm_off = a.cm_off;
      th->gh_off = a.gh_off;
      th->gk_off = a.gk_off;
      th->gv_off = a.gv_off;
    }
  }
  if (a.copy_idx)
    for (int e = tid; e < cnt; e += 256) dst[e] = clean_pos(li[e], len);
  // gathered tiles: header {first token, first block, KV head, keys} and 64 positions
  const uint32_t kv = static_cast<uint32_t>(h / (a.hq / a.hkv));
  for (int u = tid; u < ng * kBlock; u += 256) {
    const int t = u / kBlock, k = u % kBlock;
    uint8_t* gh = a.trav + a.gh_off + static_cast<size_t>(gb + t) * kGatherHdr;
    const int keys = min(kBlock, cnt - kBlock * t);
    if (k == 0)
      *reinterpret_cast<GatherEntry*>(gh) =
          GatherEntry{static_cast<uint32_t>(tok0), static_cast<uint32_t>(blk), kv, static_cast<uint32_t>(keys)};
    reinterpret_cast<int32_t*>(gh + 16)[k] = k < keys ? clean_pos(li[kBlock * t + k], len) : INT32_MAX;
  }
  // items at or above level x (query-tile index), over all sequences
  auto items_from = [&](int x) {
    int64_t n = 0;
    for (int u = 0; u < a.nseq; ++u) {
      const int q = (a.cu[u + 1] - a.cu[u] + a.bq - 1) / a.bq;
      if (q > x) n += q - x;
    }
    return n * a.hq;
  };
  uint64_t* cm = reinterpret_cast<uint64_t*>(a.trav + a.cm_off) + cm_base;
  const int W = static_cast<int>(a.window);
  int carry = 0;   // selected keys in the chunks before this one
  for (int j0 = 0; j0 < nk; j0 += kHybChunk) {
    const int jn = min(kHybChunk, nk - j0);
    for (int j = tid; j < kHybChunk; j += 256) cml[j] = 0ull;
    __syncthreads();
    for (int e = tid; e < cnt; e += 256) {
      const int c = li[e];
      const int j = (c >> 6) - j0;
      if (c >= 0 && c < len && j >= 0 && j < jn) atomicOr(&cml[j], 1ull << (c & 63));
    }
    __syncthreads();
    // masks out; inclusive popcount prefix (thread t owns tiles 4t .. 4t+3)
    int pc[4], tsum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = 4 * tid + u;
      const uint64_t m = j < jn ? cml[j] : 0ull;
      if (j < jn) cm[j0 + j] = m;
      pc[u] = __popcll(m);
      tsum += pc[u];
    }
    int ctot;
    int base = block_scan256(tsum, red, &ctot);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      base += pc[u];
      cum[4 * tid + u] = base;
    }
    __syncthreads();
    // the query tiles whose last row falls in this chunk
    for (int i = tid; i < nq; i += 256) {
      const int r0 = i * a.bq, rl = min((i + 1) * a.bq, len) - 1;
      const int jl = (rl >> 6) - j0;
      if (jl < 0 || jl >= jn) continue;
      const uint64_t lowm = (rl & 63) == 63 ? ~0ull : ((1ull << ((rl & 63) + 1)) - 1ull);
      const int vis = carry + (jl > 0 ? cum[jl - 1] : 0) + __popcll(cml[jl] & lowm);
      int rank = 0;
      for (int u = 0; u < s; ++u) rank += (a.cu[u + 1] - a.cu[u] + a.bq - 1) / a.bq > i;
      const uint32_t k = static_cast<uint32_t>(items_from(i + 1) + static_cast<int64_t>(rank) * a.hq + h);
      if (k >= a.n_items) continue;
      const int legal = rl / a.bk + 1;
      const int jfull = min(legal, max(0, fdiv_floor(rl - W, a.bk) + 1));
      const int jedge = W > 0 ? min(jfull, max(0, fdiv_floor(r0 - W - (a.bk - 1), a.bk) + 1)) : jfull;
      const uint32_t ce = static_cast<uint32_t>(jfull - jedge);
      const uint32_t ngi = static_cast<uint32_t>((min(vis, cnt) + kBlock - 1) / kBlock);
      RunEntry* runs = reinterpret_cast<RunEntry*>(a.trav + a.run_off) + static_cast<size_t>(k) * a.max_runs;
      uint32_t nr = 0;
      put_run(runs, nr, static_cast<uint32_t>(jfull), static_cast<uint32_t>(legal - jfull), TM_FP16, a.max_runs);
      put_run(runs, nr, static_cast<uint32_t>(jedge), ce, TM_FP16 | kRunEdge, a.max_runs);
      put_run(runs, nr, static_cast<uint32_t>(jedge), ce, TM_INT8 | kRunEdge, a.max_runs);
      put_run(runs, nr, 0u, static_cast<uint32_t>(jedge), TM_INT8, a.max_runs);
      put_run(runs, nr, static_cast<uint32_t>(gb), ngi, TM_FP16 | kRunGather, a.max_runs);
      ItemEntry* it = reinterpret_cast<ItemEntry*>(a.trav + a.item_off) + k;
      it->seq = static_cast<uint32_t>(s);
      it->head = static_cast<uint32_t>(h);
      it->qtile = static_cast<uint32_t>(i);
      it->nruns = nr;
      it->n8 = ce + static_cast<uint32_t>(jedge);
      it->n4 = 0u;
      it->n16 = static_cast<uint32_t>(legal - jfull) + ce + ngi;
      it->nskip = 0u;
    }
    carry += ctot;
    __syncthreads();
  }
}

hipError_t launch_hybrid_build(const HybArgs& a, bool census, hipStream_t st) {
  const int n_lists = a.nseq * a.hq;
  if (n_lists <= 0) return hipSuccess;
  const unsigned n_wg = static_cast<unsigned>(n_lists) + (a.gk_src != nullptr ? a.n_gt : 0u);
  hipLaunchKernelGGL(hyb_build_kernel, dim3(n_wg), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !census) return e;
  hipLaunchKernelGGL(trav_census_kernel, dim3(1), dim3(256), 0, st, a.trav, a.item_off, a.n_items);
  return hipGetLastError();
}

// Hybrid traversals: fill gathered tile t (its header written by
// hyb_build_kernel) with its selected keys' K rows and V^T.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void gather_rows_kernel(GatherArgs a) {
  __shared__ _Float16 vl[kBlock * (D + 8)];
  const uint32_t t = blockIdx.x;
  const uint8_t* gh = a.trav + a.gh_off + static_cast<size_t>(t) * kGatherHdr;
  const GatherEntry ge = *reinterpret_cast<const GatherEntry*>(gh);
  const int32_t* pos = reinterpret_cast<const int32_t*>(gh + 16);
  gather_rows_tile<D, BF16>(a.trav, a.gk_off, a.gv_off, t, a.k, a.v, a.hkv, ge.tok_start, ge.kv,
                            static_cast<int>(ge.keys), [&](int row) { return pos[row]; }, vl);
}

hipError_t launch_gather_rows(const GatherArgs& a, int d, hipStream_t st) {
  if (a.n_gtiles == 0) return hipSuccess;
  if (d == 128) {
    if (a.bf16) hipLaunchKernelGGL((gather_rows_kernel<128, true>), dim3(a.n_gtiles), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((gather_rows_kernel<128, false>), dim3(a.n_gtiles), dim3(256), 0, st, a);
  } else {
    if (a.bf16) hipLaunchKernelGGL((gather_rows_kernel<64, true>), dim3(a.n_gtiles), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((gather_rows_kernel<64, false>), dim3(a.n_gtiles), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

// Decode selection buffers: fill gathered tile t with its selected keys'
// 16-bit K rows ([64][D]) and fp16 V columns (V^T [D][64], from the cache's
// fp16 V^T copy); slots past the list, and empty slots (position INT32_MAX),
// are zero.
template <int D>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const uint32_t t = blockIdx.x;
  const uint8_t* gh = a.trav + a.gh_off + static_cast<size_t>(t) * kGatherHdr;
  const GatherEntry ge = *reinterpret_cast<const GatherEntry*>(gh);
  const int32_t* pos = reinterpret_cast<const int32_t*>(gh + 16);
  uint16_t* gk = reinterpret_cast<uint16_t*>(a.trav + a.gk_off) + static_cast<size_t>(t) * kBlock * D;
  uint16_t* gv = reinterpret_cast<uint16_t*>(a.trav + a.gv_off) + static_cast<size_t>(t) * D * kBlock;
  // K: 64 rows of D 16-bit values, 16 bytes per thread step
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  for (int u = threadIdx.x; u < kBlock * CPR; u += 256) {
    const int row = u / CPR, ch = u % CPR;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (row < static_cast<int>(ge.keys) && pos[row] != INT32_MAX) {
      const size_t tok = static_cast<size_t>(ge.tok_start) + pos[row];
      v = *reinterpret_cast<const u32x4*>(a.k + (tok * a.hkv + ge.kv) * D + ch * 8);
    }
    *reinterpret_cast<u32x4*>(gk + row * D + ch * 8) = v;
  }
  // V^T: channel rows of 64 slots; thread (slot, channel quarter) copies D/4 channels
  const int slot = threadIdx.x & 63, c0 = threadIdx.x >> 6;
  const bool ok = slot < static_cast<int>(ge.keys) && pos[slot] != INT32_MAX;
  const int key = ok ? pos[slot] : 0;
  const uint16_t* src = a.vt16 + ((static_cast<size_t>(ge.blk_start) + key / kBlock) * a.hkv + ge.kv) * D * kBlock +
                        key % kBlock;
  for (int c = c0; c < D; c += 4) gv[c * kBlock + slot] = ok ? src[c * kBlock] : static_cast<uint16_t>(0);
}

hipError_t launch_gather(const GatherArgs& a, int d, hipStream_t st) {
  if (a.n_gtiles == 0) return hipSuccess;
  if (d == 128) hipLaunchKernelGGL(gather_kernel<128>, dim3(a.n_gtiles), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(gather_kernel<64>, dim3(a.n_gtiles), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_traversal(const TravArgs& a, bool census, hipStream_t st) {
  const unsigned n = max(a.n_items, static_cast<uint32_t>(a.nseq));
  const unsigned blocks = (n + 255) / 256;
  hipLaunchKernelGGL(trav_items_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !census) return e;
  hipLaunchKernelGGL(trav_census_kernel, dim3(1), dim3(256), 0, st, a.trav, a.item_off, a.n_items);
  return hipGetLastError();
}

}  // namespace tmx
