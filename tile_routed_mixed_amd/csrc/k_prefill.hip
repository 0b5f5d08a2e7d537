// Fused tile-routed causal prefill for gfx950.
//
// [TriAttention] "TriAttention: Unified Sparse Mixed-Precision Attention for
// Long-Context LLM Inference", abstract: a fused kernel walks the
// precision-grouped traversal, skips omitted tiles and combines the 4-bit and
// 8-bit QK contributions into one normalized attention output.
// [TileMix] "TileMix: Tile-Centric Mixed-Precision Attention for LLM Inference
// Acceleration", abstract: FP16 or INT8 score tiles, both paths updating one
// shared online-softmax state; grouped-query attention; variable lengths.
// [HyQuant] "HyQuant Uses Hybrid Precision to Compress LLM Attention", section
// "How HyQuant works": selected tokens and a sliding window in FP16, the rest
// quantized (the hybrid kind: per-pair masks inside tiles, gathered tiles).
// One specialization per policy kind: boundaries (INT8/INT4), bitmask
// (FP16/INT8), four-way (all three) and hybrid (FP16/INT8 with masks).
//
// Design (gfx950, 64-wide waves):
//  * one workgroup of 4 waves per work item (sequence, query head, query tile
//    of BQ rows); each wave owns BQ/4 query rows for the whole item and keeps
//    their Q operands in registers;
//  * scores are computed transposed, S^T = K Q^T, with 16x16 MFMA tiles:
//    INT8 and INT4 tiles on v_mfma_i32_16x16x64_i8 (INT4 nibbles are widened
//    in registers to int8 holding 16x the code, so the product is exact and
//    256x the code product), FP16 tiles on v_mfma_f32_16x16x32_{f16,bf16};
//    every lane then holds keys of one query row, so the online-softmax
//    bookkeeping is lane-local up to a 4-lane max (two lane-swap VALU ops),
//    and the fp16 probabilities are already in the B-operand layout of PV;
//  * PV runs as O^T += V^T P^T on v_mfma_f32_16x16x32_f16, plus one more MFMA
//    per 32-key chunk with an all-ones A operand that accumulates the row sum
//    of the same fp16 probabilities (no VALU adds; numerator and denominator
//    see identical rounding).  V arrives transposed per 64-token block in fp16
//    (written once by the quantize pass); K rows are fed to the QK MFMA in an
//    interleaved order (sigma) that makes each lane's 8 probabilities per
//    32-key chunk contiguous keys, so one 16-byte LDS read fetches the matching
//    V^T operand;
//  * K and V^T tiles are copied global -> LDS with the direct-to-LDS 16-byte
//    load (no register staging, per-lane source offsets computed once per
//    item) into two buffers: the next tile streams in while the current one is
//    computed, with one barrier per tile.  16-byte chunks are XOR-swizzled by
//    row so the MFMA operand reads are free of bank conflicts;
//  * scores enter exp2 through one FMA, x * scale - m (scale = sq sk tau log2e
//    for integer tiles, tau log2e for FP16 tiles); the running max is updated
//    lazily: probabilities are re-based (O and the sum rescaled) only when a
//    row's max grows by more than 8 in log2 units, so p <= 256;
//  * the item's run list sits one entry per lane and is read with readlane,
//    so advancing the traversal needs no memory access;
//  * workgroups are remapped so the 4 query heads of a GQA group run on the
//    same XCD (dispatch is round-robin over the 8 XCDs) and share K/V in L2.
#include <climits>

#include "k_prefill_common.h"

namespace tmx {

template <int D, int BQ, int KIND, bool BF16, bool DBG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(PrefillArgs a) {
  constexpr int RW = BQ / 4;       // query rows per wave
  constexpr int QB = RW / 16;      // 16-row MFMA blocks per wave
  constexpr int NC8 = D / 64;      // i8 MFMA k-chunks (64 bytes of d each)
  constexpr int NC16 = D / 32;     // f16 MFMA k-chunks
  constexpr int ND = D / 16;       // output channel blocks
  constexpr int KBYTES = KIND == 0 ? kBlock * D : kBlock * 2 * D;   // largest K tile
  constexpr int VBYTES = D * kBlock * 2;
  constexpr int BUF = KBYTES + VBYTES;
  constexpr bool HAS4 = KIND == TM_POLICY_BOUNDARIES || KIND == TM_POLICY_FOURWAY;
  constexpr bool HAS16 = KIND != TM_POLICY_BOUNDARIES;  // bitmask, four-way, hybrid
  constexpr bool HYB = KIND == TM_POLICY_HYBRID;        // per-key precision (see below)
  typedef typename std::conditional<BF16, bf16x8, f16x8>::type q16_t;

  // two tile buffers, at LDS offsets 0 and kBufStride: the next tile streams
  // in while the current one is used; switching buffers flips one address bit
  constexpr int kBufStride = 32768;
  static_assert(BUF <= kBufStride, "tile buffer larger than its slot");
  __shared__ __align__(1024) uint8_t lds[kBufStride + BUF];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const TravHeader* th = reinterpret_cast<const TravHeader*>(a.trav);
  if (th->kind != static_cast<uint32_t>(KIND)) return;   // traversal of another policy kind
  const uint32_t item_idx = remap_block(blockIdx.x, a.n_items);
  const ItemEntry it = reinterpret_cast<const ItemEntry*>(a.trav + th->item_off)[item_idx];
  const SeqEntry se = reinterpret_cast<const SeqEntry*>(a.trav + th->seq_off)[it.seq];
  const RunEntry* runs = reinterpret_cast<const RunEntry*>(a.trav + th->run_off) +
                         static_cast<size_t>(item_idx) * th->max_runs;
  const int head = it.head, kv = head / (a.hq / a.hkv);
  const int len = se.len;
  const int nbs = (len + kBlock - 1) / kBlock;
  const int ntiles = static_cast<int>(it.n8 + it.n4 + it.n16);
  const int qrow0 = it.qtile * BQ + w * RW;
  const int qblk = qrow0 / kBlock;
  const bool qblk_ok = qblk < nbs;
  // codes and scales are block-major ([nblk][heads]...): cache block j of this
  // (sequence, KV head) is entry kv_blk0 + j * hkv
  const size_t qblk_g = (static_cast<size_t>(se.blk_start) + qblk) * a.hq + head;
  const size_t kv_blk0 = static_cast<size_t>(se.blk_start) * a.hkv + kv;
  const uint32_t hkv = static_cast<uint32_t>(a.hkv);
  const uint32_t span = static_cast<uint32_t>(max(nbs, 1) - 1) * hkv + 1;   // entries kv_blk0 .. last block
  const uint32_t kpitch16 = static_cast<uint32_t>(a.hkv) * D * 2;   // bytes between key rows of k
  const float sq8 = qblk_ok ? a.qs8[qblk_g] : 0.0f;
  const float sq4 = (HAS4 && qblk_ok) ? a.qs4[qblk_g] : 0.0f;
  const float tau = a.tau_log2e;

  // buffer resources over this (sequence, KV head): tile j starts at j * hkv * tile bytes
  const __amdgpu_buffer_rsrc_t rs_v =
      make_rsrc(reinterpret_cast<const uint8_t*>(a.vt16) + kv_blk0 * VBYTES, span * VBYTES);
  const __amdgpu_buffer_rsrc_t rs_k8 =
      make_rsrc(reinterpret_cast<const uint8_t*>(a.k8) + kv_blk0 * (kBlock * D), span * (kBlock * D));
  __amdgpu_buffer_rsrc_t rs_k4 = rs_k8, rs_k16 = rs_k8;
  if constexpr (HAS4) rs_k4 = make_rsrc(a.k4 + kv_blk0 * (kBlock * D / 2), span * (kBlock * D / 2));
  if constexpr (HAS16)   // rows past the sequence end fall outside the range and read as zeros
    rs_k16 = make_rsrc(reinterpret_cast<const uint8_t*>(a.k) + (static_cast<size_t>(se.tok_start) * a.hkv + kv) * D * 2,
                       static_cast<uint32_t>(len - 1) * kpitch16 + D * 2);

  TileCopy<D, 8, true> cp_v;
  TileCopy<kBlock, D / 16, false> cp_k8;
  TileCopy<kBlock, D / 32, false> cp_k4;
  TileCopy<kBlock, D / 8, false> cp_k16;
  cp_v.init(w, lane, 128);
  cp_k8.init(w, lane, D);
  if constexpr (HAS4) cp_k4.init(w, lane, D / 2);
  if constexpr (HAS16) cp_k16.init(w, lane, kpitch16);

  // ---- hybrid policies: key c of row r is FP16 if c is selected or r - c <
  // window, else INT8.  Regular tiles mask the selected keys out (one 64-bit
  // column mask per key tile) and, on tiles the window edge crosses, keep
  // only the pairs inside (FP16 pass) or outside (INT8 pass) the window; the
  // selected keys run as gathered FP16 tiles, masked by their positions.
  TileCopy<kBlock, D / 8, false> cp_kg;
  __amdgpu_buffer_rsrc_t rs_kg = rs_v, rs_vg = rs_v;
  const uint64_t* cmask = nullptr;
  int win = 0;
  if constexpr (HYB) {
    win = static_cast<int>(th->window);
    const SelEntry sel = reinterpret_cast<const SelEntry*>(a.trav + th->sel_tab_off)[it.seq * a.hq + head];
    cmask = reinterpret_cast<const uint64_t*>(a.trav + th->cm_off) + sel.cm_base;
    rs_kg = make_rsrc(a.trav + th->gk_off, th->n_gtiles * (kBlock * D * 2));
    rs_vg = make_rsrc(a.trav + th->gv_off, th->n_gtiles * VBYTES);
    cp_kg.init(w, lane, D * 2);
  }

  // ---- per-lane LDS read offsets.  Key rows are read in the order
  // sigma(kb, l16) = sigma(0, l16) + 32 (kb >> 1) + 4 (kb & 1); the swizzle
  // depends on row bits the kb terms leave alone, so every 16-key block kb and
  // both buffers are constant offsets from one per-lane base per 16-byte chunk
  // column; likewise V^T rows db * 16 + l16 for every channel block db.
  const int r0 = sigma(0, l16);
  int kb8[NC8], kb16[NC16], kb4, vb[2];
#pragma unroll
  for (int c = 0; c < NC8; ++c) kb8[c] = lds_off<D / 16, false>(r0, 4 * c + g);
#pragma unroll
  for (int c = 0; c < NC16; ++c) kb16[c] = lds_off<D / 8, false>(r0, 4 * c + g);
  if constexpr (D == 128) kb4 = lds_off<4, false>(r0, g);
  else kb4 = lds_off<2, false>(r0, g >> 1) + (g & 1) * 8;
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) vb[c2] = lds_off<8, true>(l16, 4 * c2 + g);

  // ---- run list: one entry per lane, 64 runs per chunk
  const int nruns = static_cast<int>(it.nruns);
  int run_base = 0;
  RunEntry run_lane = RunEntry{0u, 0u};
  if (lane < nruns) run_lane = runs[lane];

  // ---- tile list: after expand(c), lane L describes executed tile 64c + L of
  // the item: key tile | precision << 24, and its score scale (log2 units).
  uint32_t tl_jp = 0u;
  float tl_cs = 0.0f;
  uint32_t tl_cm0 = 0u, tl_cm1 = 0u;   // hybrid: the tile's column mask
  int rr = 0, rcum = 0;   // first run not wholly consumed, tiles before it
  auto expand = [&](int c) {
    const int t = c * 64 + lane;
    const int cend = c * 64 + 64;
    uint32_t jp = 0u;
    while (rr < nruns && rcum < cend) {
      if (rr - run_base >= 64) {   // next chunk of the run list (items with more than 64 runs)
        run_base += 64;
        run_lane = RunEntry{0u, 0u};
        if (run_base + lane < nruns) run_lane = runs[run_base + lane];
      }
      const uint32_t kt = __builtin_amdgcn_readlane(run_lane.ktile, rr - run_base);
      const uint32_t cp = __builtin_amdgcn_readlane(run_lane.count_prec, rr - run_base);
      const int cnt = static_cast<int>(cp & 0xFFFFFFu);
      if (t >= rcum && t < rcum + cnt) jp = (kt + static_cast<uint32_t>(t - rcum)) | (cp & 0xFF000000u);
      if (rcum + cnt > cend) break;
      rcum += cnt;
      ++rr;
    }
    tl_jp = jp;
    const uint32_t pj = jp >> 24, pc = pj & 3u;
    const size_t kb = kv_blk0 + static_cast<size_t>(jp & 0xFFFFFFu) * hkv;
    float cs = tau;
    if (pc == TM_INT8) cs = (sq8 * a.ks8[kb]) * tau;
    else if (HAS4 && pc == TM_INT4) cs = (sq4 * a.ks4[kb]) * (tau * (1.0f / 256.0f));
    tl_cs = cs;
    if constexpr (HYB) {
      uint64_t m = 0;
      if (pj != 0u && !(pj & kRunGather)) m = cmask[jp & 0xFFFFFFu];
      tl_cm0 = static_cast<uint32_t>(m);
      tl_cm1 = static_cast<uint32_t>(m >> 32);
    }
  };

  // start loading tile j (precision prec) into buffer BUFC
  auto issue = [&](uint32_t j, uint32_t prec, int boff) {
    uint8_t* dst = lds + boff;
    if (HYB && (prec & kRunGather)) {   // gathered tile j: K rows and V^T packed per tile
      cp_v.issue(rs_vg, j * VBYTES, dst + KBYTES, w);
      cp_kg.issue(rs_kg, j * (kBlock * D * 2), dst, w);
      return;
    }
    const uint32_t pc = prec & 3u;
    const uint32_t jh = j * hkv;
    cp_v.issue(rs_v, jh * VBYTES, dst + KBYTES, w);
    if (pc == TM_INT8) cp_k8.issue(rs_k8, jh * (kBlock * D), dst, w);
    else if (HAS4 && pc == TM_INT4) cp_k4.issue(rs_k4, jh * (kBlock * D / 2), dst, w);
    else if (HAS16) cp_k16.issue(rs_k16, j * (kBlock * kpitch16), dst, w);
  };

  uint32_t jp_cur = 0u;
  if (ntiles > 0) {
    expand(0);
    jp_cur = __builtin_amdgcn_readlane(tl_jp, 0);
    issue(jp_cur & 0xFFFFFFu, jp_cur >> 24, 0);
  }

  // ---- resident Q operands (B operand of S^T = K Q^T)
  i32x4 q8[QB][NC8];
  i32x4 q4[QB][NC8];
  q16_t q16[QB][NC16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = qrow0 + qb * 16 + l16;
    const int rb = r % kBlock;
#pragma unroll
    for (int c = 0; c < NC8; ++c)
      q8[qb][c] = qblk_ok ? *reinterpret_cast<const i32x4*>(a.q8 + (qblk_g * kBlock + rb) * D + c * 64 + g * 16)
                          : i32x4{0, 0, 0, 0};
    if constexpr (HAS4) {
      // lane group g holds channels 32g .. 32g+31: packed bytes 16g .. 16g+15
      if constexpr (D == 128) {
        u32x4 p = qblk_ok ? *reinterpret_cast<const u32x4*>(a.q4 + (qblk_g * kBlock + rb) * (D / 2) + g * 16)
                          : u32x4{0, 0, 0, 0};
        q4[qb][0] = widen_nibbles(p[0], p[1]);
        q4[qb][1] = widen_nibbles(p[2], p[3]);
      } else {
        u32x2 p = qblk_ok ? *reinterpret_cast<const u32x2*>(a.q4 + (qblk_g * kBlock + rb) * (D / 2) + g * 8)
                          : u32x2{0, 0};
        q4[qb][0] = widen_nibbles(p[0], p[1]);
      }
    }
    if constexpr (HAS16) {
#pragma unroll
      for (int c = 0; c < NC16; ++c) {
        u32x4 raw = u32x4{0, 0, 0, 0};
        if (r < len)
          raw = *reinterpret_cast<const u32x4*>(a.q + (static_cast<size_t>(se.tok_start + r) * a.hq + head) * D +
                                                 c * 32 + g * 8);
        __builtin_memcpy(&q16[qb][c], &raw, 16);
      }
    }
  }

  f16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<_Float16>(1.0f);
  float m_use[QB];
  f32x4 lacc[QB];                // row sums (all 4 entries equal)
  f32x4 oacc[ND][QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_use[qb] = kNegBig;
    lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One tile: wait for it (and free the other buffer), start the next tile's
  // loads into the other buffer, then compute this one from buffer BUFC.
  int t = 0;
  auto body = [&]() {
    const int boff = (t & 1) * kBufStride;
    wait_vm(0);
    __syncthreads();
    const int j = static_cast<int>(jp_cur & 0xFFFFFFu);
    const uint32_t pflags = jp_cur >> 24, prec = pflags & 3u;
    const float cs = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(tl_cs), t & 63));
    const bool gath = HYB && (pflags & kRunGather);
    const bool edge = HYB && (pflags & kRunEdge);
    uint64_t cm = 0;
    if constexpr (HYB)
      cm = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(tl_cm1, t & 63))) << 32) |
           static_cast<uint32_t>(__builtin_amdgcn_readlane(tl_cm0, t & 63));   // (readlane is signed)
    if (t + 1 < ntiles) {
      if (((t + 1) & 63) == 0) expand((t + 1) >> 6);
      jp_cur = __builtin_amdgcn_readlane(tl_jp, (t + 1) & 63);
      issue(jp_cur & 0xFFFFFFu, jp_cur >> 24, boff ^ kBufStride);
    }

    const uint8_t* kl = lds + boff;
    const uint8_t* vl = kl + KBYTES;
    // need_mmask: pairs to drop from the row maxima too (causal, sequence end,
    // window edge, gathered slots); need_mask: any pair to drop.  Selected
    // keys masked out of a regular tile still count in its maxima: each is a
    // score of the row (computed again in FP16 in a gathered tile).
    const bool need_mmask = (j * kBlock + kBlock - 1 > qrow0) || (j * kBlock + kBlock > len) || gath || edge;
    const bool need_mask = need_mmask || (HYB && cm != 0);
    // hybrid: this tile pass's excluded (row, slot) pairs as one 16-bit mask
    // per row block, bit 4 kb + i for slot sigma(kb, 4g + i)
    uint32_t xmask[QB], mmask[QB];
    if constexpr (HYB) {
      if (need_mask) {
        if (gath) {   // gathered tile: the slots' key positions, compared with the rows
          const int32_t* gp =
              reinterpret_cast<const int32_t*>(a.trav + th->gh_off + static_cast<size_t>(j) * kGatherHdr + 16);
          i32x4 gpos[4];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) gpos[kb] = *reinterpret_cast<const i32x4*>(gp + krow(kb) + 8 * g);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const int row = qrow0 + qb * 16 + l16;
            uint32_t m = 0;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i) m |= static_cast<uint32_t>(gpos[kb][i] > row) << (4 * kb + i);
            xmask[qb] = mmask[qb] = m;
          }
        } else {
          // the selected keys of the lane's slots: bits 8g + {0..7, 32..39} of cm
          const uint64_t t64 = cm >> (8 * g);
          const uint32_t lm = static_cast<uint32_t>(t64 & 0xFFu) | (static_cast<uint32_t>(t64 >> 24) & 0xFF00u);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const int row = qrow0 + qb * 16 + l16;
            uint32_t m = 0;
            if (need_mmask) {
#pragma unroll
              for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int key = j * kBlock + sigma(kb, 4 * g + i);
                  bool x = key > row || key >= len;
                  if (edge) x = x || ((row - key < win) != (prec == TM_FP16));
                  m |= static_cast<uint32_t>(x) << (4 * kb + i);
                }
            }
            mmask[qb] = m;
            xmask[qb] = m | lm;
          }
        }
      }
    }
    // (row block qb, slot) excluded from this tile pass (mx: from the row maxima)
    auto masked = [&](int kb, int i, int qb, bool mx = false) -> bool {
      if constexpr (HYB) {
        return ((mx ? mmask[qb] : xmask[qb]) >> (4 * kb + i)) & 1u;
      } else {
        const int row = qrow0 + qb * 16 + l16;
        const int key = j * kBlock + sigma(kb, 4 * g + i);
        return key > row || key >= len;
      }
    };

    // ---- S^T = K Q^T as fp32 values x (integers converted exactly), score = x * cs
    f32x4 xf[4][QB];
    float tmax[QB];   // the row's largest score in this tile (-inf if none)
    if (HAS16 && prec == TM_FP16) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) xf[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      q16_t av[4][NC16];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int c = 0; c < NC16; ++c) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(kl + krow(kb) * (D * 2) + kb16[c]);
          __builtin_memcpy(&av[kb][c], &raw, 16);
        }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int c = 0; c < NC16; ++c)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            if constexpr (BF16)
              xf[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[kb][c], q16[qb][c], xf[kb][qb], 0, 0, 0);
            else
              xf[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[kb][c], q16[qb][c], xf[kb][qb], 0, 0, 0);
          }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (need_mmask) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (masked(kb, i, qb, true)) xf[kb][qb][i] = -INFINITY;
        }
        float mf = xf[0][qb][0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mf = fmaxf(mf, xf[e >> 2][qb][e & 3]);
        tmax[qb] = max4(mf) * cs;
      }
    } else {
      const bool is8 = !HAS4 || prec == TM_INT8;
      i32x4 acc[4][QB];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[kb][qb] = i32x4{0, 0, 0, 0};
      if (is8) {
        i32x4 av[4][NC8];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int c = 0; c < NC8; ++c)
            av[kb][c] = *reinterpret_cast<const i32x4*>(kl + krow(kb) * D + kb8[c]);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int c = 0; c < NC8; ++c)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              acc[kb][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[kb][c], q8[qb][c], acc[kb][qb], 0, 0, 0);
      } else if constexpr (HAS4) {
        if constexpr (D == 128) {
          u32x4 pk[4];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            pk[kb] = *reinterpret_cast<const u32x4*>(kl + krow(kb) * (D / 2) + kb4);
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const i32x4 a0 = widen_nibbles(pk[kb][0], pk[kb][1]);
            const i32x4 a1 = widen_nibbles(pk[kb][2], pk[kb][3]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              acc[kb][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, q4[qb][0], acc[kb][qb], 0, 0, 0);
              acc[kb][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, q4[qb][1], acc[kb][qb], 0, 0, 0);
            }
          }
        } else {
          // D == 64: rows of 32 packed bytes = 2 chunks; lane group g reads 8 bytes
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const u32x2 p = *reinterpret_cast<const u32x2*>(kl + krow(kb) * (D / 2) + kb4);
            const i32x4 a0 = widen_nibbles(p[0], p[1]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              acc[kb][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, q4[qb][0], acc[kb][qb], 0, 0, 0);
          }
        }
      }
      if constexpr (DBG) {
        for (int e = 0; e < a.n_dbg; ++e) {
          const int32_t* tt = a.dbg_tiles + 4 * e;
          if (tt[0] == static_cast<int>(it.seq) && tt[1] == head && tt[2] == static_cast<int>(it.qtile) && tt[3] == j) {
            int32_t* dst = a.dbg_qk + static_cast<size_t>(e) * BQ * kBlock;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int v = acc[kb][qb][i];
                  dst[(w * RW + qb * 16 + l16) * kBlock + sigma(kb, 4 * g + i)] = is8 ? v : (v >> 8);
                }
          }
        }
      }
      // row maxima on the integer products (cs >= 0 keeps the order); masked
      // keys count as INT_MIN, below every product (|a| <= 2^21)
      int mrow[QB];
      if (need_mmask) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          int mi = INT_MIN;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mi = max(mi, masked(kb, i, qb, true) ? INT_MIN : acc[kb][qb][i]);
          mrow[qb] = mi;
        }
      } else {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          int mi = acc[0][qb][0];
#pragma unroll
          for (int e = 1; e < 16; ++e) mi = max(mi, acc[e >> 2][qb][e & 3]);
          mrow[qb] = mi;
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int mi = max4i(mrow[qb]);
        tmax[qb] = mi == INT_MIN ? -INFINITY : static_cast<float>(mi) * cs;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) xf[kb][qb][i] = static_cast<float>(acc[kb][qb][i]);
      }
    }

    // ---- shared online softmax (log2 domain, lazily re-based): probabilities
    // are taken against m_use, which moves only when a row's max grows by more
    // than 8, so p <= 256.
    f16x8 pb[2][QB];
    bool rebase = false;
    float alpha[QB], nb[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      alpha[qb] = 1.0f;
      if (tmax[qb] > m_use[qb] + 8.0f) {
        alpha[qb] = __builtin_amdgcn_exp2f(m_use[qb] - tmax[qb]);
        m_use[qb] = tmax[qb];
        rebase = true;
      }
      nb[qb] = -m_use[qb];
    }
    if (__any(rebase)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        lacc[qb] *= alpha[qb];
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db][qb] *= alpha[qb];
      }
    }
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float s = __builtin_fmaf(xf[kb][qb][i], cs, nb[qb]);
            pb[kb >> 1][qb][4 * (kb & 1) + i] =
                static_cast<_Float16>(__builtin_amdgcn_exp2f(masked(kb, i, qb) ? -INFINITY : s));
          }
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pb[kb >> 1][qb][4 * (kb & 1) + i] =
                static_cast<_Float16>(__builtin_amdgcn_exp2f(__builtin_fmaf(xf[kb][qb][i], cs, nb[qb])));
    }

    // ---- O^T += V^T P^T; row sums += 1^T P^T.  V^T operands are read one
    // channel block ahead of the MFMAs that use them (pinned below, which also
    // keeps the scheduler from hoisting every read and running out of VGPRs).
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[c2][qb], lacc[qb], 0, 0, 0);
    f16x8 va[2][2];
    auto read_v = [&](int db, f16x8* dst) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(vl + db * 2048 + vb[c2]);
        __builtin_memcpy(&dst[c2], &raw, 16);
      }
    };
    read_v(0, va[0]);
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      if (db + 1 < ND) read_v(db + 1, va[(db + 1) & 1]);
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[db & 1][c2], pb[c2][qb], oacc[db][qb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * QB, 0);
#pragma unroll
    for (int db = 1; db < ND; ++db) {
      if (db + 1 < ND) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * QB, 0);
    }
  };

  for (; t < ntiles; ++t) body();

  // ---- epilogue: O = O / l, lse
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = lacc[qb][0];
    const int r = qrow0 + qb * 16 + l16;
    if (r >= len) continue;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const size_t tok = static_cast<size_t>(se.tok_start) + r;
    const size_t obase = (tok * a.hq + head) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const f32x4 v = oacc[db][qb] * inv;
      const size_t off = obase + db * 16 + 4 * g;
      if (a.o_dtype == TM_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + off) = v;
      } else if (a.o_dtype == TM_F16) {
        f16x4 hv = {static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1]), static_cast<_Float16>(v[2]),
                    static_cast<_Float16>(v[3])};
        *reinterpret_cast<f16x4*>(static_cast<_Float16*>(a.o) + off) = hv;
      } else {
        u32x2 bv;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          uint32_t lo = __float_as_uint(v[2 * e]), hi = __float_as_uint(v[2 * e + 1]);
          lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
          hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
          bv[e] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.o) + off) = bv;
      }
    }
    if (a.lse != nullptr && g == 0)
      a.lse[static_cast<size_t>(head) * a.T + tok] = (m_use[qb] + __builtin_amdgcn_logf(lt)) * kLn2;
  }
}

template <int D, int BQ, int KIND, bool BF16>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  if (a.n_dbg > 0)
    hipLaunchKernelGGL((prefill_kernel<D, BQ, KIND, BF16, true>), dim3(a.n_items), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, BQ, KIND, BF16, false>), dim3(a.n_items), dim3(256), 0, st, a);
  return hipGetLastError();
}

// (boundary policies run prefill_pipe_kernel, k_prefill_pipe.hip)
template <int D, int BQ>
static hipError_t launch_prefill_k(const PrefillArgs& a, int kind, bool bf16, hipStream_t st) {
  if (kind == TM_POLICY_BITMASK)
    return bf16 ? launch_prefill_t<D, BQ, 1, true>(a, st) : launch_prefill_t<D, BQ, 1, false>(a, st);
  if (kind == TM_POLICY_FOURWAY)
    return bf16 ? launch_prefill_t<D, BQ, 2, true>(a, st) : launch_prefill_t<D, BQ, 2, false>(a, st);
  return bf16 ? launch_prefill_t<D, BQ, 3, true>(a, st) : launch_prefill_t<D, BQ, 3, false>(a, st);
}

hipError_t launch_prefill(const PrefillArgs& a, int d, int bq, int kind, bool bf16, hipStream_t st) {
  if (a.n_items == 0) return hipSuccess;
  if (kind == TM_POLICY_BOUNDARIES) return launch_prefill_pipe(a, d, bq, st);
  if (d == 128) {
    if (bq == 128) return launch_prefill_k<128, 128>(a, kind, bf16, st);
    return launch_prefill_k<128, 64>(a, kind, bf16, st);
  }
  if (bq == 128) return launch_prefill_k<64, 128>(a, kind, bf16, st);
  return launch_prefill_k<64, 64>(a, kind, bf16, st);
}

}  // namespace tmx
