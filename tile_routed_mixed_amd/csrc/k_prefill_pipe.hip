// Software-pipelined tile-routed prefill for boundary policies (INT8 and INT4
// score tiles).
//
// [TriAttention] "TriAttention: Unified Sparse Mixed-Precision Attention for
// Long-Context LLM Inference", abstract: two diagonal-distance boundaries per
// head route each query-key tile to 8-bit, 4-bit or no computation; the
// traversal lists the executed tiles grouped by precision, skipped tiles are
// never touched, and one fused kernel merges both QK precisions into one
// normalized output.  [TileMix] "TileMix: Tile-Centric Mixed-Precision
// Attention for LLM Inference Acceleration", abstract: every executed tile
// updates one shared online-softmax state.
//
// Same work decomposition, operand layouts and numerics as prefill_kernel
// (k_prefill.hip): one workgroup of 4 waves per (sequence, query head, query
// tile), S^T = K Q^T on the int8 matrix cores, O^T += V^T P^T on the fp16
// ones with P rounded to fp16, row sums on a ones-MFMA, a lazily re-based
// running maximum.  What differs is the schedule and the VALU work per score,
// made for gfx950, where a wave's VALU work competes with its own matrix-core
// issue and hides under it only when the two are interleaved and independent:
//
//  * iteration t runs three phases.  Phase A issues the QK MFMAs of tile t+1
//    and, between them, the exponentials of tile t's first 32 keys (scale
//    FMA, exp2, fp16 pack); phase B1 issues the PV MFMAs of those 32 keys
//    and, between them, the exponentials of the last 32; phase B2 issues the
//    PV MFMAs of the last 32 keys and, between them, the integer row maxima
//    of tile t+1.  No phase waits on its own results;
//  * scores accumulate onto the bit pattern of 1.5 * 2^23, so they are read
//    as floats with no conversion instruction (see sm_half);
//  * INT4 tiles read K's INT4 codes from their one-byte copy (quantize pass),
//    so INT4 and INT8 tiles are the same i8 MFMA work with different Q
//    operands (Q's INT4 codes widened to 16 x code) and scales;
//  * LDS holds two K slots and two V slots: iteration t reads K(t+1) and
//    V(t), and issues the direct-to-LDS copies of K(t+2) and V(t+1) right
//    after its one barrier, a whole iteration ahead of their use;
//  * the at most BQ/64 tiles that cross the diagonal or the sequence end (the
//    only ones that need masks) run first, through masked variants of the
//    phases; the rest of the item runs unmasked.
#include <type_traits>

#include "k_prefill_common.h"

namespace tmx {

typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));

// 16 packed INT4 codes (two dwords; code 2i in the low nibble of byte i, code
// 2i + 1 in the high one) -> 16 bytes, byte k holding 16 x code k.  Each
// result dword spreads one packed byte pair (b, b') to b, b, b', b' and keeps
// the low nibble (shifted up) of bytes 0 and 2 and the high nibble of bytes 1
// and 3.
__device__ __forceinline__ i32x4 widen_in_order(uint32_t p0, uint32_t p1) {
  auto pair = [](uint32_t p, uint32_t sel) {
    const uint32_t x = __builtin_amdgcn_perm(p, p, sel);
    return static_cast<int>(((x << 4) & 0x00F000F0u) | (x & 0xF000F000u));
  };
  return i32x4{pair(p0, 0x01010000u), pair(p0, 0x03030202u), pair(p1, 0x01010000u), pair(p1, 0x03030202u)};
}

template <int D, int BQ, bool DBG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_pipe_kernel(PrefillArgs a) {
  constexpr int RW = BQ / 4;       // query rows per wave
  constexpr int QB = RW / 16;      // 16-row MFMA blocks per wave
  constexpr int NC8 = D / 64;      // i8 MFMA k-chunks (64 bytes of d each)
  constexpr int ND = D / 16;       // output channel blocks
  constexpr int KB = kBlock * D;   // bytes of a K tile (INT8 codes or one-byte INT4 codes)
  constexpr int VB = D * kBlock * 2;   // bytes of a V^T tile (fp16)
  constexpr int VS0 = 2 * KB;      // K slots at [0, KB), [KB, 2KB); V slots from VS0
  __shared__ __align__(1024) uint8_t lds[2 * KB + 2 * VB];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const TravHeader* th = reinterpret_cast<const TravHeader*>(a.trav);
  if (th->kind != static_cast<uint32_t>(TM_POLICY_BOUNDARIES)) return;
  const uint32_t item_idx = remap_block(blockIdx.x, a.n_items);
  const ItemEntry it = reinterpret_cast<const ItemEntry*>(a.trav + th->item_off)[item_idx];
  const SeqEntry se = reinterpret_cast<const SeqEntry*>(a.trav + th->seq_off)[it.seq];
  const RunEntry* runs = reinterpret_cast<const RunEntry*>(a.trav + th->run_off) +
                         static_cast<size_t>(item_idx) * th->max_runs;
  const int head = it.head, kv = head / (a.hq / a.hkv);
  const int len = se.len;
  const int nbs = (len + kBlock - 1) / kBlock;
  const int qrow0 = it.qtile * BQ + w * RW;
  const int qblk = qrow0 / kBlock;
  const bool qblk_ok = qblk < nbs;
  // codes and scales are block-major ([nblk][heads]...): cache block j of this
  // (sequence, KV head) is entry kv_blk0 + j * hkv
  const size_t qblk_g = (static_cast<size_t>(se.blk_start) + qblk) * a.hq + head;
  const size_t kv_blk0 = static_cast<size_t>(se.blk_start) * a.hkv + kv;
  const uint32_t hkv = static_cast<uint32_t>(a.hkv);
  const uint32_t span = static_cast<uint32_t>(max(nbs, 1) - 1) * hkv + 1;   // entries kv_blk0 .. last block
  const float sq8 = qblk_ok ? a.qs8[qblk_g] : 0.0f;
  const float sq4 = qblk_ok ? a.qs4[qblk_g] : 0.0f;
  const float tau = a.tau_log2e;

  // buffer resources over this (sequence, KV head): tile j starts at j * hkv * tile bytes
  const __amdgpu_buffer_rsrc_t rs_v =
      make_rsrc(reinterpret_cast<const uint8_t*>(a.vt16) + kv_blk0 * VB, span * VB);
  // K tile bases: INT8 codes, and the one-byte INT4 codes as an offset from them
  const uintptr_t kbase8 = reinterpret_cast<uintptr_t>(a.k8 + kv_blk0 * KB);
  const uintptr_t kdelta4 = reinterpret_cast<uintptr_t>(a.k4x + kv_blk0 * KB) - kbase8;
  TileCopy<D, 8, true> cp_v;
  TileCopy<kBlock, D / 16, false> cp_k;
  cp_v.init(w, lane, 128);
  cp_k.init(w, lane, D);

  // per-lane LDS read offsets (see prefill_kernel): K rows in sigma order,
  // V^T rows db * 16 + l16
  const int r0 = sigma(0, l16);
  int kb8[NC8], vb[2];
#pragma unroll
  for (int c = 0; c < NC8; ++c) kb8[c] = lds_off<D / 16, false>(r0, 4 * c + g);
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) vb[c2] = lds_off<8, true>(l16, 4 * c2 + g);

  // ---- the item's tiles.  Key tiles from jd on cross the diagonal (or the
  // sequence end) and need masks; they are the last tiles of their runs and at
  // most BQ/64 of them.  They run first; the others follow in run order, from
  // the runs cut off at jd.
  const int jd = (static_cast<int>(it.qtile) * BQ) / kBlock;
  const int jend = (min((static_cast<int>(it.qtile) + 1) * BQ, len) + kBlock - 1) / kBlock;
  const int nruns = static_cast<int>(it.nruns);
  int n_m = 0, n_u = 0;
  uint32_t mj0 = 0u, mj1 = 0u;   // masked tiles: key tile | precision << 24
  for (int r = 0; r < nruns; ++r) {
    const RunEntry re = runs[r];
    const int kt = static_cast<int>(re.ktile), cnt = static_cast<int>(re.count_prec & 0xFFFFFFu);
    const uint32_t pr = re.count_prec & 0xFF000000u;
    n_u += min(max(jd - kt, 0), cnt);
    for (int j = max(kt, jd); j < min(kt + cnt, jend); ++j) {
      if (n_m == 0) mj0 = static_cast<uint32_t>(j) | pr;
      else mj1 = static_cast<uint32_t>(j) | pr;
      ++n_m;
    }
  }
  const int n = n_m + n_u;

  // scale of a tile, in log2 units per unit of its integer product (INT4: the
  // Q operand holds 16 x code), rounded to 22 significant bits (a relative
  // change below 2^-22) so that 1.5 * 2^23 times it is exact in binary32
  auto scale_of = [&](uint32_t jp) -> float {
    const size_t kb = kv_blk0 + static_cast<size_t>(jp & 0xFFFFFFu) * hkv;
    const float cs = (jp >> 24) == TM_INT8 ? (sq8 * a.ks8[kb]) * tau : (sq4 * a.ks4[kb]) * (tau * (1.0f / 16.0f));
    return __uint_as_float((__float_as_uint(cs) + 2u) & ~3u);
  };
  // unmasked tiles, 64 at a time: after expand(c), lane L holds tile 64c + L.
  // Each run is walked from its highest key tile down, so after the diagonal
  // every item of a query tile steps down from the diagonal at the same pace
  // whatever its bands: the four query heads of a KV head (adjacent items on
  // one XCD) read the same K/V tiles at about the same time and share them
  // in that XCD's L2 (long sequences: 35.2 -> 34.4 ms at 128K against the
  // ascending walk).
  uint32_t tl_jp = 0u;
  float tl_cs = 0.0f;
  int rr = 0, rcum = 0;   // first run not wholly listed, tiles before it
  auto expand = [&](int c) {
    const int t = c * 64 + lane, cend = c * 64 + 64;
    uint32_t jp = 0u;
    while (rr < nruns && rcum < cend) {
      const RunEntry re = runs[rr];
      const int kt = static_cast<int>(re.ktile);
      const int cnt = min(max(jd - kt, 0), static_cast<int>(re.count_prec & 0xFFFFFFu));
      if (t >= rcum && t < rcum + cnt) jp = static_cast<uint32_t>(kt + cnt - 1 - (t - rcum)) | (re.count_prec & 0xFF000000u);
      if (rcum + cnt > cend) break;
      rcum += cnt;
      ++rr;
    }
    tl_jp = jp;
    tl_cs = scale_of(jp);
  };
  // tile t >= n_m of the item's order (an unmasked one; calls come in order
  // of t, so each chunk of the list is expanded once, when its first tile is
  // asked for)
  auto entry_u = [&](int t, uint32_t& jp, float& cs) {
    const int u = t - n_m;
    if ((u & 63) == 0) expand(u >> 6);
    jp = __builtin_amdgcn_readlane(tl_jp, u & 63);
    cs = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(tl_cs), u & 63));
  };

  // (the base is computed, not chosen between two captured variables: the
  // compiler turns such a choice into a load through a selected address,
  // which keeps the captures, and everything the copy touches, in per-lane
  // memory, and the copies then take waterfall loops)
  auto issue_k = [&](uint32_t jp, int slot) {
    const uint32_t soff = (jp & 0xFFFFFFu) * hkv * KB;
    const uintptr_t base = kbase8 + ((jp >> 24) == TM_INT8 ? uintptr_t(0) : kdelta4);
    cp_k.issue(make_rsrc(reinterpret_cast<const void*>(base), span * KB), soff, lds + slot * KB, w);
  };
  auto issue_v = [&](uint32_t jp, int slot) {
    const uint32_t j = jp & 0xFFFFFFu;
    cp_v.issue(rs_v, j * hkv * VB, lds + VS0 + slot * VB, w);
  };

  // ---- Q operands (B operand of S^T = K Q^T), one set in registers: the
  // INT8 codes, or the INT4 codes widened to 16 x code, loaded again
  // whenever the precision of the tiles changes (at most three times per item
  // for boundary traversals; the codes come from L2)
  i32x4 qop[QB][NC8];
  auto load_q = [&](bool is8) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int rb = (qrow0 + qb * 16 + l16) % kBlock;
      if (is8) {
#pragma unroll
        for (int c = 0; c < NC8; ++c)
          qop[qb][c] = qblk_ok ? *reinterpret_cast<const i32x4*>(a.q8 + (qblk_g * kBlock + rb) * D + c * 64 + g * 16)
                               : i32x4{0, 0, 0, 0};
      } else {
        // the channels of the K operand (chunk c, lane group g: 64 c + 16 g
        // onwards, one byte each): 8 packed bytes at 32 c + 8 g
#pragma unroll
        for (int c = 0; c < NC8; ++c) {
          const u32x2 p = qblk_ok ? *reinterpret_cast<const u32x2*>(a.q4 + (qblk_g * kBlock + rb) * (D / 2) + c * 32 + g * 8)
                                  : u32x2{0, 0};
          qop[qb][c] = widen_in_order(p[0], p[1]);
        }
      }
    }
  };

  // Q operands for a tile of precision is8, loaded only when the operands in
  // registers are of the other precision: an item's tiles change precision
  // at most three times, and each load is a memory round trip the first
  // tiles would otherwise wait for.  (Uniform: the precision comes from the
  // wave's scalar run entries.)
  int q_prec = -1;
  auto need_q = [&](bool is8) {
    if (q_prec != static_cast<int>(is8)) {
      load_q(is8);
      q_prec = static_cast<int>(is8);
    }
  };

  // ---- softmax state.  The i8 products accumulate onto the bit pattern of
  // 1.5 * 2^23, so a score's int32 bits, read as a float, are exactly
  // 1.5 * 2^23 + product (|product| < 2^21 for INT8 codes and for 16 x INT4
  // codes at d <= 128); integer order is value order, so the row maxima stay
  // integer and no conversion runs per score.  Two score buffers alternate
  // with the parity of the tile index (tile t's scores in sc[t & 1]), so QK of
  // tile t+1 and the exponentials of tile t use different registers, without
  // copies.
  constexpr int KMAG = 0x4B400000;
  constexpr float KMAGF = 12582912.0f;
  constexpr int LA = 3;   // LDS operand reads issued this many chunks ahead
  f32x4 oacc[ND][QB];
  f32x4 lacc[QB];         // row sums: every element of lacc[qb] sums row l16's probabilities
  float m_use[QB];        // running base, integer-valued
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_use[qb] = kNegBig;
    lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  i32x4 sc[2][4][QB];
  uint32_t xm[QB];        // excluded (row, key) pairs of a masked tile: bit 4 kb + i
  i32x4 kmag = {KMAG, KMAG, KMAG, KMAG};
  f16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<_Float16>(1.0f);
  // (kept in VGPRs for the whole item: otherwise the compiler rebuilds them
  // from scalar registers with VALU moves at every use)
  asm volatile("" : "+v"(kmag), "+v"(ones));
  // masked products enter the maxima as this biased value: below every real
  // one (|product| < 2^21), and its float view is tiny, so the lane maximum
  // of an all-masked lane comes out near -1.5 * 2^23 cs
  constexpr int KMASK = KMAG - (1 << 30);

  constexpr int NA = 4 * NC8;   // phase A chunks: one K operand, QB QK MFMAs
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T_ = std::true_type;
  using F_ = std::false_type;

  // exponentials of scores 2 hh, 2 hh + 1 of block (qb, kb) of s: with
  // nb = -(1.5 * 2^23 cs + m_use) (exact: cs has at most 22 significant bits
  // and m_use is an integer, so the sum is representable), fma(bits, cs, nb)
  // rounds product * cs - m_use once, as fma(float(product), cs, -m_use)
  // would.  One packed fp16 pair into pb (the B-operand layout of PV).
  auto sm_half = [&](auto masked, const i32x4 (&s)[4][QB], float cs, const float (&nb)[QB], int qb, int kb, int hh,
                     u32x4 (&pb)[2][QB]) {
    float e[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 2 * hh + u;
      float x = __builtin_fmaf(__int_as_float(s[kb][qb][i]), cs, nb[qb]);
      if constexpr (decltype(masked)::value)
        if ((xm[qb] >> (4 * kb + i)) & 1u) x = -INFINITY;
      e[u] = __builtin_amdgcn_exp2f(x);
    }
    f16x2v h;
    h[0] = static_cast<_Float16>(e[0]);
    h[1] = static_cast<_Float16>(e[1]);
    uint32_t wd = __builtin_bit_cast(uint32_t, h);
    // (pins the half-block here: pure arithmetic carries no ordering of its
    // own, and instruction selection would otherwise gather it elsewhere)
    asm volatile("" : "+v"(wd));
    pb[kb >> 1][qb][2 * (kb & 1) + hh] = wd;
  };

  // block (qb, kb) of s into the running lane maxima mp (masked pairs
  // excluded, their bits collected in xm)
  auto mc_block = [&](auto masked, const i32x4 (&s)[4][QB], int qb, int kb, uint32_t jp, int (&mp)[QB]) {
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = s[kb][qb][i];
    if constexpr (decltype(masked)::value) {
      const int row = qrow0 + qb * 16 + l16;
      const int key0 = static_cast<int>(jp & 0xFFFFFFu) * kBlock;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + sigma(kb, 4 * g + i);
        const bool x = key > row || key >= len;
        xm[qb] |= static_cast<uint32_t>(x) << (4 * kb + i);
        if (x) v[i] = KMASK;
      }
    }
    mp[qb] = max(max(mp[qb], v[0]), v[1]);
    mp[qb] = max(max(mp[qb], v[2]), v[3]);
    asm volatile("" : "+v"(mp[qb]));
  };

  // phase A of iteration t (scores of tile t in sc[P]): the QK MFMAs of tile
  // t+1 (if QK; K slot 1 - P) into sc[1 - P], chunk by chunk with the
  // exponentials of key blocks 0 and 1 of tile t.  Each chunk: one K operand
  // (read LA chunks ahead), QB MFMAs and its share of the half-blocks; nothing
  // moves across chunks.
  auto phase_a = [&](auto P, auto masked, auto with_qk, float cs, const float (&nb)[QB], u32x4 (&pb)[2][QB]) {
    constexpr int p = decltype(P)::value;
    constexpr bool QK = decltype(with_qk)::value;
    constexpr int NH = 4 * QB;   // half-blocks: (kb 0..1) x (qb) x 2
    const uint8_t* kl = lds + (1 - p) * KB;
    i32x4 av[NA];
    // (chunk i = key block i % 4, k-chunk i / 4: the two products of one
    // accumulator are four chunks apart)
    auto rd = [&](int i) { av[i] = *reinterpret_cast<const i32x4*>(kl + krow(i % 4) * D + kb8[i / 4]); };
    if constexpr (QK) {
#pragma unroll
      for (int i = 0; i < LA && i < NA; ++i) rd(i);
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if constexpr (QK) {
        if (i + LA < NA) rd(i + LA);
        const int kb = i % 4, c = i / 4;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sc[1 - p][kb][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[i], qop[qb][c], c == 0 ? kmag : sc[1 - p][kb][qb],
                                                                    0, 0, 0);
      }
#pragma unroll
      for (int j = i * NH / NA; j < (i + 1) * NH / NA; ++j)
        sm_half(masked, sc[p], cs, nb, (j >> 1) % QB, (j >> 1) / QB, j & 1, pb);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // phase B, half H of iteration t: the PV MFMAs of tile t's keys 32 H ..
  // 32 H + 31 (V slot P, probabilities pb[H]) and their row-sum MFMA against
  // ones, chunk by chunk with (if VW) the exponentials of key blocks 2 and 3
  // of tile t (H = 0) or the maxima of tile t+1's scores sc[1 - P] (H = 1, key
  // tile jp).  Each chunk: one channel block's V^T operand (read LA chunks
  // ahead) and QB MFMAs.
  auto phase_b = [&](auto P, auto H, auto masked, auto with_vw, u32x4 (&pb)[2][QB], float cs, const float (&nb)[QB],
                     uint32_t jp, int (&mp)[QB]) {
    constexpr int p = decltype(P)::value, h = decltype(H)::value;
    constexpr bool VW = decltype(with_vw)::value;
    constexpr int NV = h == 0 ? 4 * QB : 4 * QB;   // half-blocks (H = 0) or blocks (H = 1)
    const uint8_t* vl = lds + VS0 + p * VB;
    f16x8 va[ND];
    auto rd = [&](int db) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(vl + db * 2048 + vb[h]);
      va[db] = __builtin_bit_cast(f16x8, raw);
    };
#pragma unroll
    for (int i = 0; i < LA && i < ND; ++i) rd(i);
    if constexpr (h == 1 && VW) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        mp[qb] = KMASK;
        if constexpr (decltype(masked)::value) xm[qb] = 0u;
      }
    }
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      if (db + LA < ND) rd(db + LA);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[db], __builtin_bit_cast(f16x8, pb[h][qb]), oacc[db][qb],
                                                              0, 0, 0);
      if (db == 0) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, __builtin_bit_cast(f16x8, pb[h][qb]), lacc[qb], 0, 0, 0);
      }
      if constexpr (VW) {
#pragma unroll
        for (int j = db * NV / ND; j < (db + 1) * NV / ND; ++j) {
          if constexpr (h == 0) sm_half(masked, sc[p], cs, nb, (j >> 1) % QB, 2 + (j >> 1) / QB, j & 1, pb);
          else mc_block(masked, sc[1 - p], j % QB, j / QB, jp, mp);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // lane maxima -> log2-domain maxima of the lane's scores (scale cs)
  // (one FMA on the float view: -1.5 * 2^23 cs is exact, as in sm_half)
  auto lane_max = [&](const int (&mp)[QB], float cs, float (&tl)[QB]) {
    const float b = -KMAGF * cs;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) tl[qb] = __builtin_fmaf(__int_as_float(mp[qb]), cs, b);
  };

  // QK of tile 0 (K slot 0) into sc[0] and its maxima (the first tile of an item)
  auto qk_alone = [&](auto masked, float cs, uint32_t jp, float (&tl)[QB]) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int kb = i / NC8, c = i % NC8;
      const i32x4 av = *reinterpret_cast<const i32x4*>(lds + krow(kb) * D + kb8[c]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        sc[0][kb][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, qop[qb][c], c == 0 ? kmag : sc[0][kb][qb], 0, 0, 0);
    }
    int mp[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      mp[qb] = KMASK;
      if constexpr (decltype(masked)::value) xm[qb] = 0u;
    }
#pragma unroll
    for (int j = 0; j < 4 * QB; ++j) mc_block(masked, sc[0], j % QB, j / QB, jp, mp);
    lane_max(mp, cs, tl);
  };

  // lazy re-base: probabilities are taken against m_use, which moves only when
  // a row's maximum exceeds it by more than 8 (log2 units), so p <= 256.  The
  // test runs on each lane's own maximum; the row maximum over the row's four
  // lanes is formed only when some lane of the wave passes it.  m_use moves to
  // the row maximum rounded up to an integer.
  auto rebase = [&](const float (&tl)[QB]) {
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) need |= tl[qb] > m_use[qb] + 8.0f;
    if (__any(need)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float rm = max4(tl[qb]);
        float alpha = 1.0f;
        if (rm > m_use[qb] + 8.0f) {
          const float nm = __builtin_ceilf(rm);
          alpha = __builtin_amdgcn_exp2f(m_use[qb] - nm);
          m_use[qb] = nm;
        }
        lacc[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db][qb] *= alpha;
      }
    }
  };

  // raw integer products of listed tiles (tests): INT4 tiles in code units
  auto capture = [&](uint32_t jp, const i32x4 (&s)[4][QB]) {
    if constexpr (DBG) {
      const int j = static_cast<int>(jp & 0xFFFFFFu);
      const bool is8 = (jp >> 24) == TM_INT8;
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
                const int v = s[kb][qb][i] - KMAG;
                dst[(w * RW + qb * 16 + l16) * kBlock + sigma(kb, 4 * g + i)] = is8 ? v : (v >> 4);
              }
        }
      }
    }
  };

  if (n > 0) {
    uint32_t e0 = 0u, e1 = 0u, e2 = 0u;   // tiles t, t + 1, t + 2
    float c0 = 0.0f, c1 = 0.0f, c2 = 0.0f;
    // tiles 0 and 1 (masked tiles are at most two, so tiles from 2 on come
    // from the unmasked list)
    if (n_m > 0) {
      e0 = mj0;
      c0 = scale_of(mj0);
    } else {
      entry_u(0, e0, c0);
    }
    if (n > 1) {
      if (n_m > 1) {
        e1 = mj1;
        c1 = scale_of(mj1);
      } else {
        entry_u(1, e1, c1);
      }
    }

    // prologue: K(0), V(0), K(1) and tile 0's Q operands, all in flight
    // together; scores and maxima of tile 0
    issue_k(e0, 0);
    issue_v(e0, 0);
    if (n > 1) issue_k(e1, 1);
    need_q((e0 >> 24) == TM_INT8);
    wait_vm(0);
    __syncthreads();
    {
      float tl[QB];
      if (n_m > 0) qk_alone(T_{}, c0, e0, tl);
      else qk_alone(F_{}, c0, e0, tl);
      capture(e0, sc[0]);
      rebase(tl);
    }

    // iteration t (parity P = t & 1): exponentials and PV of tile t, QK and
    // maxima of tile t+1.  MA: tile t is masked; MB: tile t+1 may be (the
    // masked code is also correct for unmasked tiles, whose exclusion bits
    // come out zero).  qop holds the Q operands of tile t+1's precision.
    auto iteration = [&](int t, auto P, auto MA, auto MB) {
      constexpr int p = decltype(P)::value;
      wait_vm(0);
      __syncthreads();
      if (t + 2 < n) {
        entry_u(t + 2, e2, c2);
        issue_k(e2, p);
      }
      issue_v(e1, 1 - p);
      float nb[QB], tl[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) nb[qb] = __builtin_fmaf(-KMAGF, c0, -m_use[qb]);
      u32x4 pb[2][QB];
      int mp[QB];
      phase_a(P, MA, T_{}, c0, nb, pb);
      capture(e1, sc[1 - p]);
      phase_b(P, I0{}, MA, T_{}, pb, c0, nb, e1, mp);
      phase_b(P, I1{}, MB, T_{}, pb, c0, nb, e1, mp);
      lane_max(mp, c1, tl);
      rebase(tl);
      e0 = e1;
      c0 = c1;
      e1 = e2;
      c1 = c2;
    };
    int t = 0;
    if (n_m > 0 && n > 1) {   // the masked tiles (at most two)
      need_q((e1 >> 24) == TM_INT8);
      iteration(0, I0{}, T_{}, T_{});
      t = 1;
      if (n_m > 1 && n > 2) {
        need_q((e1 >> 24) == TM_INT8);
        iteration(1, I1{}, T_{}, T_{});
        t = 2;
      }
    }
    // the rest in stretches of one precision of tile t+1 (the runs of a
    // boundary traversal change precision at most three times per item), two
    // iterations (both parities) per trip
    while (t + 1 < n) {
      const uint32_t pr = e1 >> 24;
      need_q(pr == TM_INT8);
      if (t & 1) {
        iteration(t, I1{}, F_{}, F_{});
        ++t;
      }
      while (t + 1 < n && (e1 >> 24) == pr) {
        iteration(t, I0{}, F_{}, F_{});
        ++t;
        if (!(t + 1 < n && (e1 >> 24) == pr)) break;
        iteration(t, I1{}, F_{}, F_{});
        ++t;
      }
    }

    // the last tile: its exponentials and PV
    wait_vm(0);
    __syncthreads();
    auto last = [&](auto P) {
      float nb[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) nb[qb] = __builtin_fmaf(-KMAGF, c0, -m_use[qb]);
      u32x4 pb[2][QB];
      int mp[QB];
      if (n - 1 < n_m) {
        phase_a(P, T_{}, F_{}, c0, nb, pb);
        phase_b(P, I0{}, T_{}, T_{}, pb, c0, nb, e0, mp);
      } else {
        phase_a(P, F_{}, F_{}, c0, nb, pb);
        phase_b(P, I0{}, F_{}, T_{}, pb, c0, nb, e0, mp);
      }
      phase_b(P, I1{}, F_{}, F_{}, pb, c0, nb, e0, mp);
    };
    if ((n - 1) & 1) last(I1{});
    else last(I0{});
  }

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

template <int D, int BQ>
static hipError_t launch_pipe_t(const PrefillArgs& a, hipStream_t st) {
  if (a.n_dbg > 0)
    hipLaunchKernelGGL((prefill_pipe_kernel<D, BQ, true>), dim3(a.n_items), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_pipe_kernel<D, BQ, false>), dim3(a.n_items), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prefill_pipe(const PrefillArgs& a, int d, int bq, hipStream_t st) {
  if (a.n_items == 0) return hipSuccess;
  if (d == 128) return bq == 128 ? launch_pipe_t<128, 128>(a, st) : launch_pipe_t<128, 64>(a, st);
  return bq == 128 ? launch_pipe_t<64, 128>(a, st) : launch_pipe_t<64, 64>(a, st);
}

}  // namespace tmx
