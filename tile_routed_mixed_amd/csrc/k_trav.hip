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
    h->window = a.window;
    h->n_gtiles = a.n_gtiles;
    h->sel_tab_off = a.sel_tab_off;
    h->sel_idx_off = a.sel_idx_off;
    h->cm_off = a.cm_off;
    h->gh_off = a.gh_off;
    h->gk_off = a.gk_off;
    h->gv_off = a.gv_off;
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

  if (a.kind == TM_POLICY_HYBRID) {
    // window classes are contiguous in j: every causal (row, key) pair of key
    // tile j lies within the window from jfull on, none of them before jedge
    const int W = static_cast<int>(a.window);
    const int r0 = qt * a.bq, rl = min((qt + 1) * a.bq, len) - 1;
    auto fdiv = [](int x, int y) { return x >= 0 ? x / y : -((-x + y - 1) / y); };
    const int jfull = min(legal, max(0, fdiv(rl - W, a.bk) + 1));
    const int jedge = W > 0 ? min(jfull, max(0, fdiv(r0 - W - (a.bk - 1), a.bk) + 1)) : jfull;
    const uint32_t ce = static_cast<uint32_t>(jfull - jedge);
    put_run(runs, nr, jfull, static_cast<uint32_t>(legal - jfull), TM_FP16, a.max_runs);
    put_run(runs, nr, jedge, ce, TM_FP16 | kRunEdge, a.max_runs);
    put_run(runs, nr, jedge, ce, TM_INT8 | kRunEdge, a.max_runs);
    put_run(runs, nr, 0, static_cast<uint32_t>(jedge), TM_INT8, a.max_runs);
    // selected keys visible from this query tile (positions <= rl), gathered
    const SelEntry se = reinterpret_cast<const SelEntry*>(a.trav + a.sel_tab_off)[seq * a.hq + head];
    const int32_t* idx = reinterpret_cast<const int32_t*>(a.trav + a.sel_idx_off) + se.start;
    uint32_t lo = 0, hi = se.count;                 // first entry > rl
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if (idx[mid] <= rl) lo = mid + 1; else hi = mid;
    }
    const uint32_t ng = (lo + 63) / 64;
    put_run(runs, nr, se.gbase, ng, TM_FP16 | kRunGather, a.max_runs);
    n16 = static_cast<uint32_t>(legal - jfull) + ce + ng;
    n8 = ce + static_cast<uint32_t>(jedge);
  } else if (a.kind == TM_POLICY_BOUNDARIES) {
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
  it->nskip = a.kind == TM_POLICY_HYBRID ? 0u : static_cast<uint32_t>(legal) - n8 - n4 - n16;
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

// Hybrid policies: fill gathered tile t with its selected keys' 16-bit K rows
// ([64][D]) and fp16 V columns (V^T [D][64]); slots past the list are zero.
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
    if (row < static_cast<int>(ge.keys)) {
      const size_t tok = static_cast<size_t>(ge.tok_start) + pos[row];
      v = *reinterpret_cast<const u32x4*>(a.k + (tok * a.hkv + ge.kv) * D + ch * 8);
    }
    *reinterpret_cast<u32x4*>(gk + row * D + ch * 8) = v;
  }
  // V^T: channel rows of 64 slots; thread (slot, channel quarter) copies D/4 channels
  const int slot = threadIdx.x & 63, c0 = threadIdx.x >> 6;
  const bool ok = slot < static_cast<int>(ge.keys);
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
