// C ABI of libtm: host-side validation, sizing and launches.  Every check runs
// before anything is enqueued, so a nonzero status leaves outputs untouched.
// The entry points follow include/tm.h (which cites the method pages).
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "tm_kernels.h"

using namespace tmx;

namespace {

constexpr int32_t kVersion = (1 << 16) | 0;

struct ShapeInfo {
  int64_t T = 0;
  int64_t nblk = 0;
  int64_t n_items = 0;
  int maxnq = 0;
  int maxnk = 0;
};

tm_status check_shape(const tm_shape* s, bool tiles, ShapeInfo* info) {
  if (s == nullptr || s->cu_seqlens == nullptr) return TM_E_ARG;
  if (s->nseq < 1) return TM_E_SHAPE;
  if (s->d != 64 && s->d != 128) return TM_E_SHAPE;
  if (s->hq < 1 || s->hkv < 1 || s->hq % s->hkv != 0) return TM_E_SHAPE;
  if (s->dtype != TM_F16 && s->dtype != TM_BF16) return TM_E_SHAPE;
  if (tiles) {
    if (s->bk != 64) return TM_E_SHAPE;
    if (s->bq != 64 && s->bq != 128) return TM_E_SHAPE;
  }
  if (s->cu_seqlens[0] != 0) return TM_E_SHAPE;
  ShapeInfo r;
  for (int i = 0; i < s->nseq; ++i) {
    const int64_t a = s->cu_seqlens[i], b = s->cu_seqlens[i + 1];
    if (b < a) return TM_E_SHAPE;
    const int64_t len = b - a;
    r.nblk += (len + 63) / 64;
    if (tiles) {
      const int64_t nq = (len + s->bq - 1) / s->bq;
      r.n_items += nq * s->hq;
      r.maxnq = static_cast<int>(std::max<int64_t>(r.maxnq, nq));
      r.maxnk = static_cast<int>(std::max<int64_t>(r.maxnk, (len + 63) / 64));
    }
  }
  r.T = s->cu_seqlens[s->nseq];
  if (r.T > (int64_t{1} << 30)) return TM_E_SHAPE;
  if (r.n_items > 0x7FFFFFFF) return TM_E_SHAPE;
  if (info) *info = r;
  return TM_OK;
}

tm_status check_qtensor(const tm_qtensor* t, int heads, int layout, int64_t nblk, bool need_t16) {
  if (t == nullptr || t->c8 == nullptr || t->c4 == nullptr || t->s8 == nullptr || t->s4 == nullptr)
    return TM_E_ARG;
  if (need_t16 && t->t16 == nullptr) return TM_E_ARG;
  if (t->heads != heads || t->layout != layout || t->nblk != nblk) return TM_E_SHAPE;
  return TM_OK;
}

float tau_log2e(const tm_shape* s) {
  const float tau = s->softmax_scale > 0.0f ? s->softmax_scale : 1.0f / std::sqrt(static_cast<float>(s->d));
  return tau * kLog2e;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct TravLayout {
  size_t seq_off, item_off, run_off, bytes;
  size_t sel_tab_off = 0, sel_off_off = 0, sel_idx_off = 0, cm_off = 0, gh_off = 0, gk_off = 0, gv_off = 0;
  uint32_t max_runs;
};

// Sizes of a hybrid policy's tables (the tables themselves are built on the
// GPU by hyb_build_kernel).
struct HybridPlan {
  int64_t n_rows = 0, n_sel = 0, n_gt = 0, n_cm = 0;
};

// Lists on the device (sel_idx NULL, both device arrays set): the positions
// are not read on the host.
bool hybrid_dev_lists(const tm_policy* p) {
  return p->sel_idx == nullptr && p->sel_idx_dev != nullptr && p->sel_off_dev != nullptr;
}

tm_status hybrid_plan(const tm_shape* s, const tm_policy* p, HybridPlan* hp) {
  if (p->sel_off == nullptr) return TM_E_ARG;
  if (p->window < 0 || p->sel_off[0] != 0) return TM_E_POLICY;
  const bool dev = hybrid_dev_lists(p);
  const int64_t nr = static_cast<int64_t>(s->nseq) * s->hq;
  int64_t gt = 0, cm = 0;
  for (int sq = 0; sq < s->nseq; ++sq) {
    const int64_t len = s->cu_seqlens[sq + 1] - s->cu_seqlens[sq];
    const int64_t nk = (len + 63) / 64;
    for (int h = 0; h < s->hq; ++h) {
      const int64_t r = static_cast<int64_t>(sq) * s->hq + h;
      const int64_t a = p->sel_off[r], b = p->sel_off[r + 1];
      if (b < a || b - a > len) return TM_E_POLICY;
      if (b > a && p->sel_idx == nullptr && !dev) return TM_E_ARG;
      for (int64_t e = a; !dev && e < b; ++e) {
        const int64_t c = p->sel_idx[e];
        if (c < 0 || c >= len || (e > a && c <= p->sel_idx[e - 1])) return TM_E_POLICY;
      }
      gt += (b - a + 63) / 64;
      cm += nk;
    }
  }
  hp->n_rows = nr;
  hp->n_sel = p->sel_off[nr];
  hp->n_gt = gt;
  hp->n_cm = cm;
  if (hp->n_sel >= (int64_t(1) << 31)) return TM_E_UNSUPPORTED;
  return TM_OK;
}

TravLayout trav_layout(const tm_shape* s, const ShapeInfo& si, const tm_policy* p, const HybridPlan* hp) {
  TravLayout L;
  // boundaries: INT8 band, sink, INT4 band.  Bitmask: at most one run per
  // group.  Four-way: runs split at group edges and, inside code-0 groups, at
  // the three points where the boundary rule changes (sink, INT4, INT8 band).
  // Hybrid: FP16 tiles, FP16 and INT8 parts of the edge tiles, INT8 tiles,
  // gathered tiles.
  const bool grouped = p->kind == TM_POLICY_BITMASK || p->kind == TM_POLICY_FOURWAY;
  const int ngmax = grouped ? (si.maxnk + p->group - 1) / p->group : 0;
  L.max_runs = p->kind == TM_POLICY_BOUNDARIES ? 3u
               : p->kind == TM_POLICY_BITMASK  ? static_cast<uint32_t>(std::max(1, ngmax))
               : p->kind == TM_POLICY_FOURWAY  ? static_cast<uint32_t>(ngmax + 3)
                                               : 5u;
  L.seq_off = TM_TRAV_HEADER_BYTES;
  L.item_off = align256(L.seq_off + sizeof(SeqEntry) * static_cast<size_t>(s->nseq));
  L.run_off = align256(L.item_off + sizeof(ItemEntry) * static_cast<size_t>(si.n_items));
  size_t end = align256(L.run_off + sizeof(RunEntry) * static_cast<size_t>(si.n_items) * L.max_runs);
  if (p->kind == TM_POLICY_HYBRID) {
    const size_t d = static_cast<size_t>(s->d);
    L.sel_tab_off = end;
    end = align256(end + sizeof(SelEntry) * static_cast<size_t>(hp->n_rows));
    L.sel_off_off = end;
    end = align256(end + 4 * static_cast<size_t>(hp->n_rows + 1));
    L.sel_idx_off = end;
    end = align256(end + 4 * static_cast<size_t>(hp->n_sel));
    L.cm_off = end;
    end = align256(end + 8 * static_cast<size_t>(hp->n_cm));
    L.gh_off = end;
    end = align256(end + kGatherHdr * static_cast<size_t>(hp->n_gt));
    L.gk_off = end;
    end = align256(end + static_cast<size_t>(hp->n_gt) * 64 * d * 2);
    L.gv_off = end;
    end = align256(end + static_cast<size_t>(hp->n_gt) * d * 64 * 2);
  }
  L.bytes = end;
  return L;
}

// Words of a bitmask (per_word = 32 one-bit codes) or four-way code map
// (per_word = 16 two-bit codes) for this shape.
int64_t policy_words(const tm_shape* s, int group, int per_word) {
  int64_t w = 0;
  for (int i = 0; i < s->nseq; ++i) {
    const int64_t len = s->cu_seqlens[i + 1] - s->cu_seqlens[i];
    const int64_t nk = (len + s->bk - 1) / s->bk;
    const int64_t ng = (nk + group - 1) / group;
    w += static_cast<int64_t>(s->hq) * ((len + s->bq - 1) / s->bq) * ((ng + per_word - 1) / per_word);
  }
  return w;
}

struct DecodePlan {
  int nsplit;
  size_t ws_bytes;
};

// Decode head classes: the query heads of each KV head, cut into runs of
// consecutive heads with the same cache map (one class per KV head when the
// maps are per KV head, or when a group's per-query-head maps all agree).
struct HeadClass {
  int kv, h0, n, b8, b4;
  bool uni = false;   // a whole group with per-query-head maps (b8, b4 its largest)
  int b8min = 0;      // the group's smallest b8 (uni)
};

// A KV head whose query heads do not all share one map becomes one class
// over its whole group (uni): one wave per split reads the union of the
// heads' bands, each (block, precision) once, and every head drops the blocks
// outside its own bands.  (Beyond kMaxHeadArg query heads the maps do not fit
// the kernel arguments, and such a group is cut into runs of equal maps,
// each read on its own.)
std::vector<HeadClass> head_classes(const tm_shape* s, const tm_dpolicy* p) {
  std::vector<HeadClass> out;
  const int grp = s->hq / s->hkv;
  for (int kv = 0; kv < s->hkv; ++kv) {
    if (p->per_q_head && s->hq <= kMaxHeadArg) {
      int lo8 = INT_MAX, hi8 = 0, hi4 = 0;
      bool same = true;
      for (int h = kv * grp; h < (kv + 1) * grp; ++h) {
        lo8 = std::min(lo8, p->b8[h]);
        hi8 = std::max(hi8, p->b8[h]);
        hi4 = std::max(hi4, p->b4[h]);
        same = same && p->b8[h] == p->b8[kv * grp] && p->b4[h] == p->b4[kv * grp];
      }
      if (!same) {
        HeadClass c{kv, kv * grp, grp, hi8, hi4};
        c.uni = true;
        c.b8min = lo8;
        out.push_back(c);
        continue;
      }
    }
    for (int r = 0; r < grp;) {
      const int h = kv * grp + r;
      const int mi = p->per_q_head ? h : kv;
      int n = 1;
      while (r + n < grp && p->per_q_head && p->b8[h + n] == p->b8[h] && p->b4[h + n] == p->b4[h]) ++n;
      if (!p->per_q_head) n = grp;
      HeadClass c{kv, h, n, p->b8[mi], p->b4[mi]};
      c.b8min = c.b8;
      out.push_back(c);
      r += n;
    }
  }
  return out;
}

DecodePlan decode_plan(const tm_shape* s, const tm_dpolicy* p, const std::vector<HeadClass>& cls) {
  int maxex = 1;
  for (int b = 0; b < s->nseq; ++b) {
    const int L = s->cu_seqlens[b + 1] - s->cu_seqlens[b];
    const int nb = (L + 63) / 64;
    const int jf = p->tail_tokens > 0 ? std::max(0, (L - p->tail_tokens) / 64) : nb;
    for (const HeadClass& c : cls) {
      const int jlo = std::max(0, nb - c.b4);
      const int js = std::min(jlo, jf);
      const int nex = (nb - js) + ((p->sink && js > 0) ? 1 : 0);
      maxex = std::max(maxex, nex);
    }
  }
  // one wave per split, two per SIMD (each computes one unit of cache blocks
  // while the next streams into its registers): about 2048 splits, each
  // walking at least 6 blocks
  const int pairs = s->nseq * static_cast<int>(cls.size());
  int ns = (2048 + pairs - 1) / pairs;
  ns = std::min(ns, std::max(1, maxex / 6));
  ns = std::max(1, std::min(ns, 256));
  DecodePlan d;
  d.nsplit = ns;
  d.ws_bytes = static_cast<size_t>(s->nseq) * s->hq * ns * (s->d + 2) * sizeof(float);
  return d;
}

// Workspace of tm_decode_noalloc: one file-scope device array, 8 MiB on every
// GPU the library runs on, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol): it uses the device address hipGetSymbolAddress returns, taken
// once per device with that device current and kept in g_scratch.
constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// Device address of `scratch` on the device that runs `stream`.
tm_status scratch_for(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return TM_E_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return TM_E_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return TM_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return TM_E_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return TM_E_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return TM_E_HIP;
    if (e != hipSuccess || p == nullptr) return TM_E_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TM_OK;
}

}  // namespace

extern "C" {

const char* tm_status_string(int32_t st) {
  switch (st) {
    case TM_OK: return "TM_OK";
    case TM_E_ARG: return "TM_E_ARG: NULL or out-of-range argument";
    case TM_E_SHAPE: return "TM_E_SHAPE: inconsistent or unsupported shape";
    case TM_E_POLICY: return "TM_E_POLICY: invalid policy";
    case TM_E_SPACE: return "TM_E_SPACE: caller buffer too small";
    case TM_E_UNSUPPORTED: return "TM_E_UNSUPPORTED: not implemented for these arguments";
    case TM_E_HIP: return "TM_E_HIP: HIP launch or copy failed";
    default: return "unknown tm_status";
  }
}

int32_t tm_version(void) { return kVersion; }

int64_t tm_num_blocks(const tm_shape* shape) {
  ShapeInfo si;
  if (check_shape(shape, false, &si) != TM_OK) return -1;
  return si.nblk;
}

tm_status tm_quantize_pack(const tm_shape* shape, const void* x, int32_t heads, tm_qtensor* out, void* stream) {
  ShapeInfo si;
  tm_status st = check_shape(shape, false, &si);
  if (st != TM_OK) return st;
  if (shape->cu_seqlens_dev == nullptr || x == nullptr || out == nullptr || heads < 1) return TM_E_ARG;
  if (out->layout != TM_ROWS && out->layout != TM_COLS) return TM_E_ARG;
  if (out->layout == TM_ROWS && out->t16 != nullptr) return TM_E_ARG;
  if (out->layout == TM_COLS && out->c4x != nullptr) return TM_E_ARG;
  st = check_qtensor(out, heads, out->layout, si.nblk, false);
  if (st != TM_OK) return st;
  if (si.nblk == 0) return TM_OK;
  QuantArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.cu = shape->cu_seqlens_dev;
  a.nseq = shape->nseq;
  a.heads = heads;
  a.nblk = si.nblk;
  a.c8 = out->c8;
  a.c4 = out->c4;
  a.s8 = out->s8;
  a.s4 = out->s4;
  a.t16 = out->t16;
  a.c4x = out->c4x;
  const hipError_t e = launch_quantize(a, shape->d, shape->dtype == TM_BF16, out->layout == TM_COLS,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TM_OK : TM_E_HIP;
}

// tm_build_traversal, and (gk, gv non-null, hybrid policies) the gather of
// tm_gather_selected in the same launch.
static tm_status build_traversal(const tm_shape* shape, const tm_policy* policy, void* trav, size_t* trav_bytes,
                                 tm_census* census, const void* gk, const void* gv, void* stream) {
  ShapeInfo si;
  tm_status st = check_shape(shape, true, &si);
  if (st != TM_OK) return st;
  if (policy == nullptr || trav_bytes == nullptr) return TM_E_ARG;
  const int kind = policy->kind;
  if (kind != TM_POLICY_BOUNDARIES && kind != TM_POLICY_BITMASK && kind != TM_POLICY_FOURWAY &&
      kind != TM_POLICY_HYBRID)
    return TM_E_ARG;
  HybridPlan hp;
  if (kind == TM_POLICY_HYBRID) {
    if ((st = hybrid_plan(shape, policy, &hp)) != TM_OK) return st;
  } else if (kind != TM_POLICY_BITMASK) {   // boundaries, alone or under the four-way codes
    if (policy->b8 == nullptr || policy->b4 == nullptr) return TM_E_ARG;
    if (shape->hq > kMaxHeadsArg) return TM_E_UNSUPPORTED;
    if (policy->sink != 0 && policy->sink != 1) return TM_E_POLICY;
    for (int h = 0; h < shape->hq; ++h) {
      const int b8 = policy->b8[h], b4 = policy->b4[h];
      if (b8 < 0 || b4 < 0 || b8 > b4) return TM_E_POLICY;
      if (b4 == 0 && !policy->sink) return TM_E_POLICY;
    }
  }
  if (kind == TM_POLICY_BITMASK || kind == TM_POLICY_FOURWAY) {   // a packed per-group map
    if (policy->group < 1) return TM_E_POLICY;
    if (policy->n_words < policy_words(shape, policy->group, kind == TM_POLICY_BITMASK ? 32 : 16))
      return TM_E_POLICY;
    if (policy->bits == nullptr && policy->n_words > 0) return TM_E_ARG;
  }
  const TravLayout L = trav_layout(shape, si, policy, &hp);
  if (trav == nullptr) {
    *trav_bytes = L.bytes;
    return TM_OK;
  }
  if (*trav_bytes < L.bytes) return TM_E_SPACE;
  if (shape->cu_seqlens_dev == nullptr) return TM_E_ARG;
  if (L.bytes > 0xFFFFFFFFull) return TM_E_SHAPE;

  TravArgs a;
  std::memset(&a, 0, sizeof(a));
  a.trav = static_cast<uint8_t*>(trav);
  a.cu = shape->cu_seqlens_dev;
  a.bits = policy->bits;
  a.nseq = shape->nseq;
  a.hq = shape->hq;
  a.hkv = shape->hkv;
  a.d = shape->d;
  a.bq = shape->bq;
  a.bk = shape->bk;
  a.kind = policy->kind;
  a.sink = (kind == TM_POLICY_BOUNDARIES || kind == TM_POLICY_FOURWAY) ? policy->sink : 0;
  a.group = (kind == TM_POLICY_BITMASK || kind == TM_POLICY_FOURWAY) ? policy->group : 1;
  a.n_items = static_cast<uint32_t>(si.n_items);
  a.max_runs = L.max_runs;
  a.nblk = static_cast<uint32_t>(si.nblk);
  a.seq_off = static_cast<uint32_t>(L.seq_off);
  a.item_off = static_cast<uint32_t>(L.item_off);
  a.run_off = static_cast<uint32_t>(L.run_off);
  a.bits_off = 0;
  if (kind == TM_POLICY_BOUNDARIES || kind == TM_POLICY_FOURWAY) {
    for (int h = 0; h < shape->hq; ++h) {
      a.b8[h] = policy->b8[h];
      a.b4[h] = policy->b4[h];
    }
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (kind == TM_POLICY_HYBRID) {
    HybArgs y;
    y.trav = a.trav;
    y.cu = shape->cu_seqlens_dev;
    y.nseq = shape->nseq;
    y.hq = shape->hq;
    y.hkv = shape->hkv;
    y.d = shape->d;
    y.bq = shape->bq;
    y.bk = shape->bk;
    y.n_items = a.n_items;
    y.max_runs = L.max_runs;
    y.nblk = a.nblk;
    y.seq_off = a.seq_off;
    y.item_off = a.item_off;
    y.run_off = a.run_off;
    y.window = static_cast<uint32_t>(policy->window);
    y.n_sel = static_cast<uint32_t>(hp.n_sel);
    y.n_gt = static_cast<uint32_t>(hp.n_gt);
    y.sel_tab_off = static_cast<uint32_t>(L.sel_tab_off);
    y.sel_idx_off = static_cast<uint32_t>(L.sel_idx_off);
    y.cm_off = static_cast<uint32_t>(L.cm_off);
    y.gh_off = static_cast<uint32_t>(L.gh_off);
    y.gk_off = static_cast<uint32_t>(L.gk_off);
    y.gv_off = static_cast<uint32_t>(L.gv_off);
    y.gk_src = static_cast<const uint16_t*>(gk);
    y.gv_src = static_cast<const uint16_t*>(gv);
    y.bf16 = shape->dtype == TM_BF16;
    if (hybrid_dev_lists(policy)) {
      // lists in device memory: read (and copied into the traversal) by the kernel, no wait
      y.off = policy->sel_off_dev;
      y.idx = policy->sel_idx_dev;
      y.copy_idx = 1;
    } else {
      // host lists (checked above): stage the offsets and positions into the
      // traversal (pageable host memory: wait for the copies before returning)
      uint8_t* tb = static_cast<uint8_t*>(trav);
      if (hipMemcpyAsync(tb + L.sel_off_off, policy->sel_off, 4 * static_cast<size_t>(hp.n_rows + 1),
                         hipMemcpyHostToDevice, hs) != hipSuccess)
        return TM_E_HIP;
      if (hp.n_sel > 0 && hipMemcpyAsync(tb + L.sel_idx_off, policy->sel_idx, 4 * static_cast<size_t>(hp.n_sel),
                                         hipMemcpyHostToDevice, hs) != hipSuccess)
        return TM_E_HIP;
      if (hipStreamSynchronize(hs) != hipSuccess) return TM_E_HIP;
      y.off = reinterpret_cast<const int32_t*>(tb + L.sel_off_off);
      y.idx = reinterpret_cast<const int32_t*>(tb + L.sel_idx_off);
      y.copy_idx = 0;
    }
    if (launch_hybrid_build(y, census != nullptr, hs) != hipSuccess) return TM_E_HIP;
  } else if (launch_traversal(a, census != nullptr, hs) != hipSuccess) {
    return TM_E_HIP;
  }
  if (census != nullptr) {
    TravHeader h;
    if (hipMemcpyAsync(&h, trav, sizeof(h), hipMemcpyDeviceToHost, hs) != hipSuccess) return TM_E_HIP;
    if (hipStreamSynchronize(hs) != hipSuccess) return TM_E_HIP;
    census->legal = h.census[0];
    census->n_int8 = h.census[1];
    census->n_int4 = h.census[2];
    census->n_fp16 = h.census[3];
    census->n_skip = h.census[4];
    census->n_items = si.n_items;
    census->max_runs = L.max_runs;
  }
  return TM_OK;
}

tm_status tm_build_traversal(const tm_shape* shape, const tm_policy* policy, void* trav, size_t* trav_bytes,
                             tm_census* census, void* stream) {
  return build_traversal(shape, policy, trav, trav_bytes, census, nullptr, nullptr, stream);
}

tm_status tm_build_traversal_gather(const tm_shape* shape, const tm_policy* policy, void* trav, size_t* trav_bytes,
                                    tm_census* census, const void* k, const void* v, void* stream) {
  if (policy == nullptr || policy->kind != TM_POLICY_HYBRID || (trav != nullptr && (k == nullptr || v == nullptr)))
    return TM_E_ARG;
  return build_traversal(shape, policy, trav, trav_bytes, census, k, v, stream);
}

tm_status tm_gather_selected(const tm_shape* shape, const tm_policy* policy, void* trav, const void* k,
                             const void* v, void* stream) {
  ShapeInfo si;
  tm_status st = check_shape(shape, true, &si);
  if (st != TM_OK) return st;
  if (policy == nullptr || trav == nullptr || k == nullptr || v == nullptr || policy->kind != TM_POLICY_HYBRID)
    return TM_E_ARG;
  HybridPlan hp;
  if ((st = hybrid_plan(shape, policy, &hp)) != TM_OK) return st;
  const TravLayout L = trav_layout(shape, si, policy, &hp);
  if (L.bytes > 0xFFFFFFFFull) return TM_E_SHAPE;
  if (hp.n_gt == 0) return TM_OK;
  GatherArgs g;
  g.trav = static_cast<uint8_t*>(trav);
  g.k = static_cast<const uint16_t*>(k);
  g.vt16 = nullptr;
  g.v = static_cast<const uint16_t*>(v);
  g.hkv = shape->hkv;
  g.bf16 = shape->dtype == TM_BF16;
  g.n_gtiles = static_cast<uint32_t>(hp.n_gt);
  g.gh_off = static_cast<uint32_t>(L.gh_off);
  g.gk_off = static_cast<uint32_t>(L.gk_off);
  g.gv_off = static_cast<uint32_t>(L.gv_off);
  return launch_gather_rows(g, shape->d, static_cast<hipStream_t>(stream)) == hipSuccess ? TM_OK : TM_E_HIP;
}

tm_status tm_select_vertical(const tm_shape* shape, const void* q, const void* k, int32_t n_obs,
                             const int32_t* counts, int32_t per_kv_head, float* mass, int32_t* sel_idx, void* ws,
                             size_t* ws_bytes, void* stream) {
  ShapeInfo si;
  tm_status st = check_shape(shape, false, &si);
  if (st != TM_OK) return st;
  if (counts == nullptr || ws_bytes == nullptr) return TM_E_ARG;
  if (n_obs < 1 || n_obs > 64 || (per_kv_head != 0 && per_kv_head != 1)) return TM_E_POLICY;
  const int nl = per_kv_head ? shape->hkv : shape->hq;
  int64_t tiles = 0, sel_total = 0;
  int maxnt = 0;
  std::vector<int32_t> tab(3 * static_cast<size_t>(shape->nseq));
  for (int b = 0; b < shape->nseq; ++b) {
    const int64_t len = shape->cu_seqlens[b + 1] - shape->cu_seqlens[b];
    if (counts[b] < 0 || counts[b] > len) return TM_E_POLICY;
    const int nt = static_cast<int>((len + 63) / 64);
    tab[b] = static_cast<int32_t>(tiles);
    tab[shape->nseq + b] = counts[b];
    tab[2 * shape->nseq + b] = static_cast<int32_t>(sel_total);
    tiles += nt;
    sel_total += static_cast<int64_t>(nl) * counts[b];
    maxnt = std::max(maxnt, nt);
  }
  if (sel_total >= (int64_t(1) << 31)) return TM_E_UNSUPPORTED;
  const size_t part_b = static_cast<size_t>(tiles) * shape->hq * 128 * 4;
  const size_t rows_b = static_cast<size_t>(shape->nseq) * shape->hq * 128 * 4;
  const size_t tab_off = align256(part_b + rows_b);
  const size_t need = align256(tab_off + 4 * tab.size());
  if (ws == nullptr) {
    *ws_bytes = need;
    return TM_OK;
  }
  if (*ws_bytes < need) return TM_E_SPACE;
  if (q == nullptr || k == nullptr || mass == nullptr || shape->cu_seqlens_dev == nullptr) return TM_E_ARG;
  if (maxnt == 0) return TM_OK;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  uint8_t* w = static_cast<uint8_t*>(ws);
  SelectArgs a;
  if (shape->nseq <= kSelInline) {
    // small tables ride in the kernel arguments: no copy, no wait
    a.tab = nullptr;
    std::copy(tab.begin(), tab.end(), a.itab);
  } else {
    if (hipMemcpyAsync(w + tab_off, tab.data(), 4 * tab.size(), hipMemcpyHostToDevice, hs) != hipSuccess)
      return TM_E_HIP;
    if (hipStreamSynchronize(hs) != hipSuccess) return TM_E_HIP;   // tab is freed on return
    a.tab = reinterpret_cast<const int32_t*>(w + tab_off);
  }
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.cu = shape->cu_seqlens_dev;
  a.nseq = shape->nseq;
  a.hq = shape->hq;
  a.hkv = shape->hkv;
  a.n_obs = n_obs;
  a.bf16 = shape->dtype == TM_BF16;
  a.per_kv = per_kv_head;
  a.tau_log2e = tau_log2e(shape);
  a.part = reinterpret_cast<float*>(w);
  a.rows = reinterpret_cast<float*>(w + part_b);
  a.mass = mass;
  a.T = si.T;
  a.sel = sel_idx;
  return launch_select(a, shape->d, maxnt, tiles, hs) == hipSuccess ? TM_OK : TM_E_HIP;
}

tm_status tm_prefill(const tm_shape* shape, const void* trav, int32_t policy_kind, const void* q, const void* k,
                     const tm_qtensor* qq, const tm_qtensor* kq, const tm_qtensor* vq, void* o, int32_t o_dtype,
                     float* lse, int32_t* dbg_qk, const int32_t* dbg_tiles, int32_t n_dbg, void* stream) {
  ShapeInfo si;
  tm_status st = check_shape(shape, true, &si);
  if (st != TM_OK) return st;
  if (trav == nullptr || q == nullptr || k == nullptr || o == nullptr) return TM_E_ARG;
  if (policy_kind != TM_POLICY_BOUNDARIES && policy_kind != TM_POLICY_BITMASK && policy_kind != TM_POLICY_FOURWAY &&
      policy_kind != TM_POLICY_HYBRID)
    return TM_E_ARG;
  if (o_dtype != TM_F32 && o_dtype != TM_F16 && o_dtype != TM_BF16) return TM_E_ARG;
  if (n_dbg < 0 || (n_dbg > 0 && (dbg_qk == nullptr || dbg_tiles == nullptr))) return TM_E_ARG;
  if ((st = check_qtensor(qq, shape->hq, TM_ROWS, si.nblk, false)) != TM_OK) return st;
  if ((st = check_qtensor(kq, shape->hkv, TM_ROWS, si.nblk, false)) != TM_OK) return st;
  if ((st = check_qtensor(vq, shape->hkv, TM_COLS, si.nblk, true)) != TM_OK) return st;
  if (policy_kind == TM_POLICY_BOUNDARIES && kq->c4x == nullptr) return TM_E_ARG;
  // the kernel addresses one (sequence, KV head)'s K and V^T tiles through
  // 32-bit buffer offsets: keep every such range below 2 GiB
  for (int s = 0; s < shape->nseq; ++s) {
    const int64_t len = shape->cu_seqlens[s + 1] - shape->cu_seqlens[s];
    const int64_t nb = (len + 63) / 64;
    const int64_t k16 = len * shape->hkv * shape->d * 2;
    if (nb * shape->hkv * 64 * shape->d * 2 >= (int64_t(1) << 31) || k16 >= (int64_t(1) << 31))
      return TM_E_UNSUPPORTED;
  }
  PrefillArgs a;
  a.trav = static_cast<const uint8_t*>(trav);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.q8 = qq->c8;
  a.q4 = qq->c4;
  a.qs8 = qq->s8;
  a.qs4 = qq->s4;
  a.k8 = kq->c8;
  a.k4 = kq->c4;
  a.k4x = kq->c4x;
  a.ks8 = kq->s8;
  a.ks4 = kq->s4;
  a.vt16 = vq->t16;
  a.o = o;
  a.lse = lse;
  a.dbg_qk = dbg_qk;
  a.dbg_tiles = dbg_tiles;
  a.n_dbg = n_dbg;
  a.o_dtype = o_dtype;
  a.hq = shape->hq;
  a.hkv = shape->hkv;
  a.T = static_cast<int>(si.T);
  a.nblk = si.nblk;
  a.n_items = static_cast<uint32_t>(si.n_items);
  a.tau_log2e = tau_log2e(shape);
  const hipError_t e = launch_prefill(a, shape->d, shape->bq, policy_kind, shape->dtype == TM_BF16,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TM_OK : TM_E_HIP;
}

// Selected decode tokens: per (sequence, KV head) list {first gathered tile,
// keys}, column masks [nblk][hkv], gathered-tile headers, K rows, V^T.
struct DecodeSel {
  std::vector<uint32_t> tab;    // 2 per list
  int64_t n_gt = 0;
  size_t tab_off = 0, cm_off = 0, gh_off = 0, gk_off = 0, gv_off = 0, bytes = 0;
};

// positions: check every listed position (tm_decode_select); the decode step
// itself needs only the list lengths (its reads are bounded by the buffer the
// select call built)
bool decode_dev_lists(const tm_dpolicy* p) {
  return p->sel_idx == nullptr && p->sel_idx_dev != nullptr && p->sel_off_dev != nullptr;
}

tm_status decode_sel_plan(const tm_shape* s, const tm_dpolicy* p, const ShapeInfo& si, DecodeSel* ds,
                          bool positions) {
  if (decode_dev_lists(p)) positions = false;   // device lists are not read on the host
  else if (positions && p->sel_idx == nullptr && p->sel_off[static_cast<size_t>(s->nseq) * s->hkv] > 0)
    return TM_E_ARG;
  if (p->sel_off[0] != 0) return TM_E_POLICY;
  ds->tab.assign(2 * static_cast<size_t>(s->nseq) * s->hkv, 0u);
  int64_t gt = 0;
  for (int b = 0; b < s->nseq; ++b) {
    const int64_t cap = s->cu_seqlens[b + 1] - s->cu_seqlens[b];
    const int64_t L = p->lengths != nullptr ? p->lengths[b] : cap;
    for (int g = 0; g < s->hkv; ++g) {
      const size_t r = static_cast<size_t>(b) * s->hkv + g;
      const int64_t lo = p->sel_off[r], hi = p->sel_off[r + 1];
      if (hi < lo || hi - lo > L) return TM_E_POLICY;
      for (int64_t e = lo; positions && e < hi; ++e) {
        const int64_t c = p->sel_idx[e];
        if (c < 0 || c >= L || (e > lo && c <= p->sel_idx[e - 1])) return TM_E_POLICY;
      }
      ds->tab[2 * r] = static_cast<uint32_t>(gt);
      ds->tab[2 * r + 1] = static_cast<uint32_t>(hi - lo);
      gt += (hi - lo + 63) / 64;
    }
  }
  ds->n_gt = gt;
  const size_t d = static_cast<size_t>(s->d);
  ds->tab_off = 0;
  ds->cm_off = align256(4 * ds->tab.size());
  ds->gh_off = align256(ds->cm_off + 8 * static_cast<size_t>(si.nblk) * s->hkv);
  ds->gk_off = align256(ds->gh_off + kGatherHdr * static_cast<size_t>(gt));
  ds->gv_off = align256(ds->gk_off + static_cast<size_t>(gt) * 64 * d * 2);
  ds->bytes = align256(ds->gv_off + static_cast<size_t>(gt) * d * 64 * 2);
  if (ds->bytes > 0xFFFFFFFFull) return TM_E_UNSUPPORTED;
  return TM_OK;
}

tm_status tm_decode_select(const tm_shape* cache, const tm_dpolicy* policy, const void* k16, const tm_qtensor* vq,
                           void* sel_buf, size_t* sel_bytes, void* stream) {
  ShapeInfo si;
  tm_status st = check_shape(cache, false, &si);
  if (st != TM_OK) return st;
  if (policy == nullptr || policy->sel_off == nullptr || sel_bytes == nullptr) return TM_E_ARG;
  for (int b = 0; b < cache->nseq; ++b) {
    const int64_t cap = cache->cu_seqlens[b + 1] - cache->cu_seqlens[b];
    if (cap < 1) return TM_E_SHAPE;
    if (policy->lengths != nullptr && (policy->lengths[b] < 1 || policy->lengths[b] > cap)) return TM_E_SHAPE;
  }
  DecodeSel ds;
  if ((st = decode_sel_plan(cache, policy, si, &ds, true)) != TM_OK) return st;
  if (sel_buf == nullptr) {
    *sel_bytes = ds.bytes;
    return TM_OK;
  }
  if (*sel_bytes < ds.bytes) return TM_E_SPACE;
  if (k16 == nullptr) return TM_E_ARG;
  if ((st = check_qtensor(vq, cache->hkv, TM_COLS, si.nblk, true)) != TM_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  GatherArgs g;
  g.trav = static_cast<uint8_t*>(sel_buf);
  g.k = static_cast<const uint16_t*>(k16);
  g.vt16 = vq->t16;
  g.v = nullptr;
  g.hkv = cache->hkv;
  g.bf16 = cache->dtype == TM_BF16;
  g.n_gtiles = static_cast<uint32_t>(ds.n_gt);
  g.gh_off = static_cast<uint32_t>(ds.gh_off);
  g.gk_off = static_cast<uint32_t>(ds.gk_off);
  g.gv_off = static_cast<uint32_t>(ds.gv_off);
  if (decode_dev_lists(policy)) {
    // lists in device memory: tables by a kernel, then the gather; no wait
    if (cache->cu_seqlens_dev == nullptr) return TM_E_ARG;
    SelTabArgs t;
    t.buf = static_cast<uint8_t*>(sel_buf);
    t.cu = cache->cu_seqlens_dev;
    t.off = policy->sel_off_dev;
    t.idx = policy->sel_idx_dev;
    t.hkv = cache->hkv;
    t.n_sel = static_cast<uint32_t>(policy->sel_off[static_cast<size_t>(cache->nseq) * cache->hkv]);
    t.n_gt = static_cast<uint32_t>(ds.n_gt);
    t.tab_off = static_cast<uint32_t>(ds.tab_off);
    t.cm_off = static_cast<uint32_t>(ds.cm_off);
    t.gh_off = static_cast<uint32_t>(ds.gh_off);
    if (launch_sel_tables(t, cache->nseq * cache->hkv, hs) != hipSuccess) return TM_E_HIP;
    return launch_gather(g, cache->d, hs) == hipSuccess ? TM_OK : TM_E_HIP;
  }
  // host staging of the list table, the column masks and the tile headers
  std::vector<uint8_t> buf(ds.gk_off, 0);
  std::memcpy(buf.data() + ds.tab_off, ds.tab.data(), 4 * ds.tab.size());
  uint64_t* cm = reinterpret_cast<uint64_t*>(buf.data() + ds.cm_off);
  int64_t blk = 0;
  for (int b = 0; b < cache->nseq; ++b) {
    const int64_t cap = cache->cu_seqlens[b + 1] - cache->cu_seqlens[b];
    for (int g = 0; g < cache->hkv; ++g) {
      const size_t r = static_cast<size_t>(b) * cache->hkv + g;
      const int32_t* idx = policy->sel_idx + policy->sel_off[r];
      const uint32_t n = ds.tab[2 * r + 1];
      for (uint32_t u = 0; u < n; ++u)
        cm[(blk + idx[u] / 64) * cache->hkv + g] |= uint64_t(1) << (idx[u] % 64);
      for (uint32_t t = 0; t * 64 < n; ++t) {
        uint8_t* gh = buf.data() + ds.gh_off + static_cast<size_t>(ds.tab[2 * r] + t) * kGatherHdr;
        const uint32_t keys = std::min<uint32_t>(64, n - 64 * t);
        const GatherEntry ge{static_cast<uint32_t>(cache->cu_seqlens[b]), static_cast<uint32_t>(blk),
                             static_cast<uint32_t>(g), keys};
        std::memcpy(gh, &ge, sizeof(ge));
        int32_t* pos = reinterpret_cast<int32_t*>(gh + 16);
        for (uint32_t k = 0; k < 64; ++k) pos[k] = k < keys ? idx[64 * t + k] : INT32_MAX;
      }
    }
    blk += (cap + 63) / 64;
  }
  if (hipMemcpyAsync(sel_buf, buf.data(), buf.size(), hipMemcpyHostToDevice, hs) != hipSuccess) return TM_E_HIP;
  if (hipStreamSynchronize(hs) != hipSuccess) return TM_E_HIP;
  return launch_gather(g, cache->d, hs) == hipSuccess ? TM_OK : TM_E_HIP;
}

tm_status tm_decode(const tm_shape* cache, const void* q, const tm_qtensor* kq, const tm_qtensor* vq,
                    const void* k16, const tm_dpolicy* policy, void* o, int32_t o_dtype, void* ws,
                    size_t* ws_bytes, void* stream) {
  ShapeInfo si;
  tm_status st = check_shape(cache, false, &si);
  if (st != TM_OK) return st;
  if (cache->hq / cache->hkv > 16 || cache->hkv > kMaxKvArg || cache->hq > kMaxHeadsArg) return TM_E_UNSUPPORTED;
  if (policy == nullptr || policy->b8 == nullptr || policy->b4 == nullptr || ws_bytes == nullptr) return TM_E_ARG;
  if (policy->sink != 0 && policy->sink != 1) return TM_E_POLICY;
  if (policy->tail_tokens < 0) return TM_E_POLICY;
  if (policy->per_q_head != 0 && policy->per_q_head != 1) return TM_E_POLICY;
  const int nmaps = policy->per_q_head ? cache->hq : cache->hkv;
  for (int g = 0; g < nmaps; ++g) {
    const int b8 = policy->b8[g], b4 = policy->b4[g];
    if (b8 < 0 || b4 < 0 || b8 > b4) return TM_E_POLICY;
    if (b4 == 0 && policy->tail_tokens == 0 && !policy->sink) return TM_E_POLICY;
  }
  for (int b = 0; b < cache->nseq; ++b) {
    const int64_t len = cache->cu_seqlens[b + 1] - cache->cu_seqlens[b];
    if (len < 1) return TM_E_SHAPE;
    if (policy->lengths != nullptr && (policy->lengths[b] < 1 || policy->lengths[b] > len)) return TM_E_SHAPE;
    // a sequence's 16-bit rows (and fp16 V copy) must lie within 2 GiB of its first (32-bit offsets)
    if ((len + 63) / 64 * cache->hkv * 64 * cache->d * 2 >= (int64_t(1) << 31)) return TM_E_UNSUPPORTED;
  }
  DecodeSel ds;
  if (policy->sel_off != nullptr && (st = decode_sel_plan(cache, policy, si, &ds, false)) != TM_OK) return st;
  const std::vector<HeadClass> cls = head_classes(cache, policy);
  const DecodePlan plan = decode_plan(cache, policy, cls);
  if (ws == nullptr) {
    *ws_bytes = plan.ws_bytes;
    return TM_OK;
  }
  if (*ws_bytes < plan.ws_bytes) return TM_E_SPACE;
  if (cache->cu_seqlens_dev == nullptr || q == nullptr || k16 == nullptr || o == nullptr) return TM_E_ARG;
  if (policy->sel_off != nullptr && policy->sel_buf == nullptr) return TM_E_ARG;
  if (o_dtype != TM_F32 && o_dtype != TM_F16) return TM_E_ARG;
  if ((st = check_qtensor(kq, cache->hkv, TM_ROWS, si.nblk, false)) != TM_OK) return st;
  if ((st = check_qtensor(vq, cache->hkv, TM_COLS, si.nblk, true)) != TM_OK) return st;
  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(q);
  a.k8 = kq->c8;
  a.k4 = kq->c4;
  a.ks8 = kq->s8;
  a.ks4 = kq->s4;
  a.v8 = vq->c8;
  a.v4 = vq->c4;
  a.vs8 = vq->s8;
  a.vs4 = vq->s4;
  a.vt16 = vq->t16;
  a.k16 = static_cast<const uint16_t*>(k16);
  a.ws = static_cast<float*>(ws);
  a.o = o;
  a.o_dtype = o_dtype;
  a.nseq = cache->nseq;
  a.hq = cache->hq;
  a.hkv = cache->hkv;
  a.nsplit = plan.nsplit;
  a.sink = policy->sink;
  a.tail = policy->tail_tokens;
  a.nblk = si.nblk;
  a.tau_log2e = tau_log2e(cache);
  if (policy->per_q_head && cache->hq <= kMaxHeadArg)   // each query head's map, for union classes
    for (int h = 0; h < cache->hq; ++h) {
      a.hb8[h] = policy->b8[h];
      a.hb4[h] = policy->b4[h];
    }
  if (policy->sel_off != nullptr) {
    a.sel = static_cast<const uint8_t*>(policy->sel_buf);
    a.sel_tab = static_cast<uint32_t>(ds.tab_off);
    a.sel_cm = static_cast<uint32_t>(ds.cm_off);
    a.sel_gk = static_cast<uint32_t>(ds.gk_off);
    a.sel_gv = static_cast<uint32_t>(ds.gv_off);
  }
  bool small = true;
  for (const HeadClass& c : cls) small = small && c.n <= 4;
  // launches of at most kMaxSeqArg sequences, each with its sequences'
  // offsets in the kernel arguments
  const size_t osz = o_dtype == TM_F32 ? 4 : 2;
  int64_t blk = 0;
  for (int s0 = 0; s0 < cache->nseq; s0 += kMaxSeqArg) {
    const int n = std::min(kMaxSeqArg, cache->nseq - s0);
    DecodeArgs c = a;
    c.nseq = n;
    c.seq0 = s0;
    for (int i = 0; i <= n; ++i) c.cu[i] = cache->cu_seqlens[s0 + i];
    for (int i = 0; i < n; ++i) {
      const int32_t cap = cache->cu_seqlens[s0 + i + 1] - cache->cu_seqlens[s0 + i];
      c.len[i] = policy->lengths != nullptr ? policy->lengths[s0 + i] : cap;
      c.blk[i] = static_cast<int32_t>(blk);
      blk += (cap + 63) / 64;
    }
    c.q = a.q + static_cast<size_t>(s0) * cache->hq * cache->d;
    c.o = static_cast<uint8_t*>(o) + static_cast<size_t>(s0) * cache->hq * cache->d * osz;
    c.ws = a.ws + static_cast<size_t>(s0) * cache->hq * plan.nsplit * (cache->d + 2);
    // split launches of at most kMaxClsArg head classes, then one merge
    for (size_t c0 = 0; c0 < cls.size(); c0 += kMaxClsArg) {
      const int nc = static_cast<int>(std::min<size_t>(kMaxClsArg, cls.size() - c0));
      for (int i = 0; i < nc; ++i) {
        const HeadClass& h = cls[c0 + i];
        c.cls[i] = h.kv | (h.h0 << 10) | (h.n << 20) | (static_cast<int32_t>(h.uni) << 30);
        c.b8[i] = h.b8;
        c.b4[i] = h.b4;
        c.b8min[i] = h.b8min;
      }
      if (launch_decode_split(c, nc, small, cache->d, cache->dtype == TM_BF16, static_cast<hipStream_t>(stream)) !=
          hipSuccess)
        return TM_E_HIP;
    }
    if (launch_decode_combine(c, cache->d, static_cast<hipStream_t>(stream)) != hipSuccess) return TM_E_HIP;
  }
  return TM_OK;
}

tm_status tm_cache_append(const tm_shape* cache, const int32_t* lengths, const void* x, int32_t heads,
                          tm_qtensor* out, void* stream) {
  ShapeInfo si;
  tm_status st = check_shape(cache, false, &si);
  if (st != TM_OK) return st;
  if (lengths == nullptr || x == nullptr || out == nullptr || heads < 1) return TM_E_ARG;
  if (out->layout != TM_ROWS && out->layout != TM_COLS) return TM_E_ARG;
  if (out->layout == TM_ROWS && out->t16 != nullptr) return TM_E_ARG;
  if (out->layout == TM_COLS && out->c4x != nullptr) return TM_E_ARG;
  if ((st = check_qtensor(out, heads, out->layout, si.nblk, false)) != TM_OK) return st;
  for (int b = 0; b < cache->nseq; ++b) {
    const int32_t cap = cache->cu_seqlens[b + 1] - cache->cu_seqlens[b];
    if (lengths[b] < 1 || lengths[b] > cap) return TM_E_SHAPE;
  }
  AppendArgs p;
  std::memset(&p, 0, sizeof(p));
  p.q.x = static_cast<const uint16_t*>(x);
  p.q.heads = heads;
  p.q.nblk = si.nblk;
  p.q.c8 = out->c8;
  p.q.c4 = out->c4;
  p.q.s8 = out->s8;
  p.q.s4 = out->s4;
  p.q.t16 = out->t16;
  p.q.c4x = out->c4x;
  int64_t blk = 0;
  for (int s0 = 0; s0 < cache->nseq; s0 += kMaxSeqArg) {
    const int n = std::min(kMaxSeqArg, cache->nseq - s0);
    AppendArgs c = p;
    c.n = n;
    for (int i = 0; i < n; ++i) {
      const int s = s0 + i;
      const int32_t j = (lengths[s] - 1) / 64;   // block of the newest token
      c.blk[i] = static_cast<int32_t>(blk + j);
      c.tok[i] = cache->cu_seqlens[s] + 64 * j;
      c.nvalid[i] = lengths[s] - 64 * j;
      blk += (cache->cu_seqlens[s + 1] - cache->cu_seqlens[s] + 63) / 64;
    }
    const hipError_t e = launch_append(c, cache->d, cache->dtype == TM_BF16, out->layout == TM_COLS,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return TM_E_HIP;
  }
  return TM_OK;
}

tm_status tm_decode_noalloc(const tm_shape* cache, const void* q, const tm_qtensor* kq, const tm_qtensor* vq,
                            const void* k16, const tm_dpolicy* policy, void* o, int32_t o_dtype, void* stream) {
  // size first: a request beyond the scratch array is refused before any HIP call
  size_t need = 0;
  tm_status st = tm_decode(cache, q, kq, vq, k16, policy, o, o_dtype, nullptr, &need, stream);
  if (st != TM_OK) return st;
  if (need > kScratchBytes) return TM_E_SPACE;
  void* ws = nullptr;
  if ((st = scratch_for(static_cast<hipStream_t>(stream), &ws)) != TM_OK) return st;
  size_t cap = kScratchBytes;
  return tm_decode(cache, q, kq, vq, k16, policy, o, o_dtype, ws, &cap, stream);
}

size_t tm_decode_noalloc_max_workspace(void) { return kScratchBytes; }

}  // extern "C"
