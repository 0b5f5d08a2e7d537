// Decode over the compressed KV cache (gfx950).
//
// [TriAttention] "TriAttention: Unified Sparse Mixed-Precision Attention for
// Long-Context LLM Inference", abstract: the K/V codes made during prefill are
// reused as a compressed KV cache for decoding, cutting repeated reads of the
// prompt.  [HyQuant] "HyQuant Uses Hybrid Precision to Compress LLM
// Attention", section "How HyQuant works": the recent window stays FP16, the
// rest is quantized, and dequantization is fused with the attention math.
// [TileMix] abstract: grouped-query attention and INT8 K/V caches.
//
// The step is bound by HBM bytes (every cached code is read once per step).
// One wave (64 lanes) per (split, head class, sequence): a split is an even
// share of one (sequence, KV head)'s cache blocks, and a head class is a run
// of query heads of that KV head with one cache map; the class's query heads
// are the columns of 16x16 fp16 MFMAs:
//   S^T = K Q^T   (v_mfma_f32_16x16x32_f16),   O^T += V^T P^T (same shape).
// Codes stream from HBM straight into registers, one unit (an INT8 block, or
// two INT4 blocks, the same bytes) at a time, double-buffered: the next
// unit's loads are in flight while the current one is computed.  No LDS.
// Codes enter the MFMAs as fp16 subnormals: the byte b = c + 128 (INT8) or
// the nibble n = c + 8 (INT4) placed in the low bits of a zero-exponent fp16
// is exactly b * 2^-24, so two perms (or a mask) per pair of codes build an
// operand, with no arithmetic.  The offsets come back out exactly where they
// are cheap: for scores, 2^24 S' - off * sum(q) in the FMA that scales them;
// for outputs, one extra MFMA per block accumulates off * 2^-24 * sum(p) per
// head, subtracted once at the end.  MFMA products and sums of these values
// are exact fp32 (no flush of fp16 subnormals on this path).
// FP16 window blocks read the 16-bit keys and the fp16 V^T copy.  Selected
// tokens (when given) are masked out of their blocks and read in FP16 from
// gathered tiles, shared among the splits.
// A second kernel merges the splits' (max, sum, O) by log-sum-exp.
#include "tm_kernels.h"

namespace tmx {

// Eight 16-bit values (fp16, or bf16 narrowed to fp16: exact for magnitudes
// in [2^-14, 65504], the range of normal fp16 numbers, and saturated beyond
// it) as an fp16 MFMA operand.
template <bool BF16>
__device__ __forceinline__ f16x8 to_f16x8(u32x4 raw) {
  f16x8 v;
  if constexpr (BF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = to_f16_sat(__uint_as_float(raw[e] << 16));
      v[2 * e + 1] = to_f16_sat(__uint_as_float(raw[e] & 0xFFFF0000u));
    }
  } else {
    __builtin_memcpy(&v, &raw, 16);
  }
  return v;
}

// Four INT8 codes (one dword) -> four fp16 (c + 128) * 2^-24, in order.
__device__ __forceinline__ u32x2 sub_i8x4(uint32_t c) {
  const uint32_t t = c ^ 0x80808080u;
  return u32x2{__builtin_amdgcn_perm(t, t, 0x0c010c00u), __builtin_amdgcn_perm(t, t, 0x0c030c02u)};
}

// Eight INT4 codes (one dword, element 2t in the low nibble of byte t) ->
// eight fp16 (c + 8) * 2^-24, in order.
__device__ __forceinline__ u32x4 sub_i4x8(uint32_t c) {
  const uint32_t t = c ^ 0x88888888u;
  const uint32_t lo = t & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6
  const uint32_t hi = (t >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
  return u32x4{__builtin_amdgcn_perm(hi, lo, 0x0c040c00u), __builtin_amdgcn_perm(hi, lo, 0x0c050c01u),
               __builtin_amdgcn_perm(hi, lo, 0x0c060c02u), __builtin_amdgcn_perm(hi, lo, 0x0c070c03u)};
}

// Four INT4 codes (16 bits) -> four fp16 (c + 8) * 2^-24, in order.
__device__ __forceinline__ u32x2 sub_i4x4(uint32_t x) {
  const uint32_t y = x >> 8;
  const uint32_t t0 = x | (x << 12), t1 = y | (y << 12);   // nibbles 0, 1 (2, 3) at bits 0 and 16
  return u32x2{(t0 & 0x000F000Fu) ^ 0x00080008u, (t1 & 0x000F000Fu) ^ 0x00080008u};
}

template <typename T, typename S>
__device__ __forceinline__ T as(const S& s) {
  T t;
  __builtin_memcpy(&t, &s, sizeof(T));
  return t;
}

// Key that feeds MFMA row m of 16-key block kb (kb = 0..3 of a 64-key cache
// block): lane group g of every block kb holds keys 16g + 4kb + i, so a lane
// group owns keys 16g .. 16g+15 of the block, and for the 32-key chunk c2 of
// the PV product it holds keys 16g + 8c2 .. 16g + 8c2 + 7, the B-operand slice
// (chunk c2's k index e maps to key 16 (e / 8) + 8 c2 + e % 8).
__device__ __forceinline__ int dsig(int kb, int m) { return 16 * (m >> 2) + 4 * kb + (m & 3); }

// One unit of streamed codes in a lane's registers: one INT8 block, or two
// consecutive INT4 blocks, which take the same bytes and the same load
// instructions (so the loads never sit under a precision branch).
//  K: 8 pieces of KW bytes.  INT8: piece 2 kb + h = channels DG g + (KW h) ..
//     of key row dsig(kb, l16).  INT4: piece 4 bb + kb = the lane's DG/2
//     bytes (DG channels) of key row dsig(kb, l16) of block bb.
//  V: 2 ND pieces of 8 bytes.  INT8: piece 2 db + h = keys 16g + 8h .. +7 of
//     V^T row 16 db + l16.  INT4: piece 2 db + bb = keys 16g .. 16g+15 of
//     that row of block bb.
template <int D>
struct UnitRegs {
  u32x4 k[8];
  u32x2 v[D / 8];
  float sk[2], sv[2];
  uint64_t xm[2];   // selected-token masks of the unit's blocks (scalar)
};

// Cross-lane moves within rows of 16 lanes (DPP): lane i of a row takes the
// value of lane i - n (shr), i + n (shl) or (i - n) mod 16 (ror); lanes of
// banks (groups of 4 lanes of a row) outside bank_mask keep `old`.
template <int CTRL, int BANKS>
__device__ __forceinline__ float dpp_f(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, 0xF, BANKS, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t src) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(src), CTRL, 0xF, 0xF, false));
}
constexpr int kRowShr = 0x110, kRowShl = 0x100, kRowRor = 0x120;

// SMALLG: at most 4 query heads per KV head.  The QK product leaves head
// l16's scores in lanes l16 < 4 only (16 values a lane); they are first moved
// four to a lane, so that the softmax works on every lane and on a quarter of
// the values.  SEL: the step reads selected tokens (a.sel).
// Cache policy of the streamed code loads (INT8 and INT4 blocks):
// non-temporal.  Each code is read once per step, and the read set of a long
// cache exceeds the last-level cache; measured at 16 x 32K: 85.3 us per step
// against 90.2 us with the default policy.  (The FP16 window's strided key
// rows measured slower with it, so they keep the default.)
constexpr int kStream = 2;

template <int D, bool BF16, bool SMALLG, bool SEL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_split_kernel(DecodeArgs a) {
  constexpr int NC = D / 32;          // k-chunks of the QK MFMA (lane group g owns channels DG*g ..)
  constexpr int ND = D / 16;          // output channel blocks
  constexpr int DG = D / 4;
  constexpr int KW = D / 8;           // bytes of one K piece (INT8: half a lane's row slice)
  constexpr float kTwo24 = 16777216.0f;
  typedef UnitRegs<D> Regs;

  const int lane = threadIdx.x, l16 = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, cl = blockIdx.y, b = blockIdx.z;
  // head class: grp consecutive query heads from h0, all reading KV head kv
  const int cls = a.cls[cl];
  const int kv = cls & 1023, h0 = (cls >> 10) & 1023, grp = (cls >> 20) & 1023;
  const bool uni = (cls >> 30) & 1;   // the KV head's whole group, one map per query head

  // this sequence's extent (kernel-argument tables: scalar loads)
  const int tok0 = a.cu[b];
  const int L = a.len[b];
  const int blk0 = a.blk[b];
  // this class's bands, in 64-token blocks
  const int nb = (L + kBlock - 1) / kBlock;
  const int jf = a.tail > 0 ? max(0, (L - a.tail) / kBlock) : nb;    // FP16 window [jf, nb)
  const int jst = min(max(0, nb - a.b4[cl]), jf);                    // delta < b4 from here
  const int j8lo = min(max(jst, nb - a.b8[cl]), jf);                 // INT8 band [j8lo, jf)
  const bool sinkb = a.sink && j8lo > 0;                             // block 0 INT8, ahead of the bands
  const int j4lo = (sinkb && jst == 0) ? 1 : jst;                    // INT4 band [j4lo, j4hi)
  // (a group of query heads with their own maps: the union of their bands,
  // INT4 up to the last head's INT8 band start, each block read once at each
  // precision some head needs; every lane then drops the blocks outside its
  // own head's bands)
  const int j4hi = uni ? min(max(jst, nb - a.b8min[cl]), jf) : j8lo;
  int lj4lo = 0, lj8lo = 0;
  if (uni) {
    const int col = SMALLG ? (l16 & 3) : l16;   // this lane's query head (column) in the class
    const int hl = h0 + min(col, grp - 1);
    const int lst = min(max(0, nb - a.hb4[hl]), jf);
    lj8lo = min(max(lst, nb - a.hb8[hl]), jf);
    lj4lo = (a.sink && lj8lo > 0 && lst == 0) ? 1 : lst;
  }
  // Each split takes an even share of the INT4 band and an even share of the
  // rest ([j8lo, nb): the INT8 band, then the FP16 window, whose blocks count
  // as kW16 INT8 blocks: twice the bytes, read without look-ahead), so every
  // split carries the same mix of work; split 0 also takes the sink.
  constexpr int kW16 = 3;
  const int ns = a.nsplit;
  const int i4a = j4lo + (j4hi - j4lo) * split / ns, i4b = j4lo + (j4hi - j4lo) * (split + 1) / ns;
  const int n8 = jf - j8lo, wt = n8 + kW16 * (nb - jf);
  auto tail_at = [&](int s) {   // first tail entry of split s: INT8 entries [0, n8), then FP16
    const int t = wt * s / ns;
    return t <= n8 ? t : n8 + (t - n8 + kW16 - 1) / kW16;
  };
  const int ta = tail_at(split), tb = tail_at(split + 1);
  const int i8a = j8lo + min(ta, n8), i8b = j8lo + min(tb, n8);         // INT8 blocks
  const int ifa = jf + max(ta - n8, 0), ifb = jf + max(tb - n8, 0);     // FP16 blocks
  // codes and scales are block-major ([nblk][hkv]...): cache block j of this
  // (sequence, KV head) is entry kvb0 + j * hkv
  const size_t kvb0 = static_cast<size_t>(blk0) * a.hkv + kv;
  const uint32_t hkv = static_cast<uint32_t>(a.hkv);

  // Q^T operand: column l16 = query head h0 + l16 (zero past the class).
  // Chunk c of lane group g holds 8 channels; the K operands use the same
  // channel map.  INT4 / 16-bit K: channels DG g + 8c ..  INT8 K: channels
  // (D/2) h + KW g + 8 sub .. with c = h (KW/8) + sub, so the four lane groups
  // of a row read one contiguous span per load.  qsum: the head's sum of q
  // (for the code offsets).
  // (rows past the group lie outside the resource and read as zeros)
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(a.q + (static_cast<size_t>(b) * a.hq + h0) * D, static_cast<uint32_t>(grp * D * 2));
  auto q_operand = [&](bool map8, f16x8 (&qop)[NC]) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = map8 ? (D / 2) * (c / (KW / 8)) + KW * g + 8 * (c % (KW / 8)) : DG * g + 8 * c;
      const u32x4 raw = as<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(rq, static_cast<uint32_t>((l16 * D + ch) * 2), 0, 0));
      qop[c] = to_f16x8<BF16>(raw);
    }
  };
  // qsum: sum over all d channels of the head's q (either channel map holds
  // each channel once per lane column), taken from the first phase's operand
  float qsum = 0.0f;
  bool have_qsum = false;
  auto take_qsum = [&](const f16x8 (&qop)[NC]) {
    float t = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) t += static_cast<float>(qop[c][e]);
    const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    t = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    qsum = __uint_as_float(y[0]) + __uint_as_float(y[1]);
    if constexpr (SMALLG) {   // the compacted softmax holds head l16 & 3 in lane l16
      float qc = qsum;
      qc = dpp_f<kRowShr + 4, 0x2>(qc, qsum);
      qc = dpp_f<kRowShr + 8, 0x4>(qc, qsum);
      qc = dpp_f<kRowShr + 12, 0x8>(qc, qsum);
      qsum = qc;
    }
    have_qsum = true;
  };

  // buffer resources over this (sequence, KV head)'s blocks (a unit's second
  // INT4 block may lie past the last block: such loads return zeros and the
  // block is not computed)
  const uint32_t span = static_cast<uint32_t>(max(nb, 1) - 1) * hkv + 1;   // entries kvb0 .. last block
  const int8_t* const k8p = pin_sgpr(a.k8 + kvb0 * (kBlock * D));
  const int8_t* const v8p = pin_sgpr(a.v8 + kvb0 * (kBlock * D));
  const uint8_t* const k4p = pin_sgpr(a.k4 + kvb0 * (kBlock * D / 2));
  const uint8_t* const v4p = pin_sgpr(a.v4 + kvb0 * (kBlock * D / 2));
  const float* const ks8 = pin_sgpr(a.ks8 + kvb0);
  const float* const vs8 = pin_sgpr(a.vs8 + kvb0);
  const float* const ks4 = pin_sgpr(a.ks4 + kvb0);
  const float* const vs4 = pin_sgpr(a.vs4 + kvb0);
  // selected tokens: block j's mask is entry kvb0 + j * hkv of [nblk][hkv]
  const uint64_t* const xmp = SEL ? pin_sgpr(reinterpret_cast<const uint64_t*>(a.sel + a.sel_cm) + kvb0) : nullptr;
  const uint32_t kb8 = static_cast<uint32_t>(dsig(0, l16) * D + KW * g);
  const uint32_t kb4 = static_cast<uint32_t>(dsig(0, l16) * (D / 2) + (DG / 2) * g);
  const uint32_t vb8 = static_cast<uint32_t>(l16 * 64 + 16 * g);
  const uint32_t vb4 = static_cast<uint32_t>(l16 * 32 + 8 * g);

  // Start loading the unit at block j (an INT4 pair j, j+1 when FOUR, the
  // pair ending before jend) into r.  Each cache block of the unit gets a
  // buffer resource of its own (scalar registers), sized 0 when the block
  // does not exist (valid false, or the second block of an INT4 pair at
  // jend), so its loads return zeros without touching memory; the per-lane
  // offsets are loop-invariant and the piece offsets immediate, so no vector
  // register is written between a unit's loads.  Every unit is loaded by the
  // same instruction sequence, whether or not it exists: the loads never sit
  // under a branch, so the count of loads in flight is the same on every path
  // and computing one unit waits only for that unit's loads.
  auto load = [&](int jj, bool valid, int jend, auto tag, Regs& r) {
    constexpr bool FOUR = decltype(tag)::value;
    const int j = valid ? jj : 0;
    const size_t jo = static_cast<size_t>(j) * hkv;   // entry offset of block j
    if constexpr (!FOUR) {
      const uint32_t nr = valid ? kBlock * D : 0u;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(k8p + jo * (kBlock * D), nr);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(v8p + jo * (kBlock * D), nr);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t o = kb8 + static_cast<uint32_t>(dsig(i >> 1, 0) * D + (i & 1) * (D / 2));
        if constexpr (KW == 16) {
          r.k[i] = as<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, kStream));
        } else {
          const u32x2 x = as<u32x2>(__builtin_amdgcn_raw_buffer_load_b64(rk, o, 0, kStream));
          r.k[i] = u32x4{x[0], x[1], 0u, 0u};
        }
      }
#pragma unroll
      for (int db = 0; db < ND; ++db) {   // keys 16g .. 16g+15 of V^T row 16 db + l16: one 16-byte load
        const u32x4 x = as<u32x4>(
            __builtin_amdgcn_raw_buffer_load_b128(rv, vb8 + static_cast<uint32_t>(db * 1024), 0, kStream));
        r.v[2 * db] = u32x2{x[0], x[1]};
        r.v[2 * db + 1] = u32x2{x[2], x[3]};
      }
      r.sk[0] = sload(ks8, jo);
      r.sv[0] = sload(vs8, jo);
      if constexpr (SEL) r.xm[0] = sload64(xmp, jo);
    } else {
      const bool two = valid && j + 1 < jend;
      const uint32_t nr0 = valid ? kBlock * D / 2 : 0u, nr1 = two ? kBlock * D / 2 : 0u;
      const size_t jo1 = two ? jo + hkv : jo;
      const __amdgpu_buffer_rsrc_t rk0 = make_rsrc(k4p + jo * (kBlock * D / 2), nr0);
      const __amdgpu_buffer_rsrc_t rk1 = make_rsrc(k4p + jo1 * (kBlock * D / 2), nr1);
      const __amdgpu_buffer_rsrc_t rv0 = make_rsrc(v4p + jo * (kBlock * D / 2), nr0);
      const __amdgpu_buffer_rsrc_t rv1 = make_rsrc(v4p + jo1 * (kBlock * D / 2), nr1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t o = kb4 + static_cast<uint32_t>(dsig(i & 3, 0) * (D / 2));
        if constexpr (KW == 16) {
          r.k[i] = as<u32x4>(__builtin_amdgcn_raw_buffer_load_b128((i >> 2) ? rk1 : rk0, o, 0, kStream));
        } else {
          const u32x2 x = as<u32x2>(__builtin_amdgcn_raw_buffer_load_b64((i >> 2) ? rk1 : rk0, o, 0, kStream));
          r.k[i] = u32x4{x[0], x[1], 0u, 0u};
        }
      }
#pragma unroll
      for (int i = 0; i < 2 * ND; ++i)
        r.v[i] = as<u32x2>(__builtin_amdgcn_raw_buffer_load_b64((i & 1) ? rv1 : rv0,
                                                                vb4 + static_cast<uint32_t>((i >> 1) * 512), 0, kStream));
      r.sk[0] = sload(ks4, jo);
      r.sv[0] = sload(vs4, jo);
      r.sk[1] = sload(ks4, jo1);
      r.sv[1] = sload(vs4, jo1);
      if constexpr (SEL) {
        r.xm[0] = sload64(xmp, jo);
        r.xm[1] = sload64(xmp, jo1);
      }
    }
  };

  float m_run = kNegBig, l_run = 0.0f;   // per lane: head l16, the keys of lane group g
  f32x4 oacc[ND], ocorr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Online softmax over one 64-key block given its S^T accumulators (16 per
  // lane), score = acc * m1 + m0; key slot k stands for key kbase + k, and
  // keys at index >= klim, or whose bit of xm is set, are dropped.  Leaves
  // the fp16 P^T operands (p * sv) of the two 32-key chunks in pb.
  auto softmax = [&](const f32x4 (&acc)[4], float m1, float m0, float sv, int kbase, int klim, uint64_t xm,
                     f16x8 (&pb)[2]) {
    if constexpr (SMALLG) {
      // lane (4a + h, g) takes head h's keys 16g + 4a + i (i = 0..3): the
      // values acc[a][i] of lane (h, g)
      const int a4 = l16 >> 2;
      float c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = acc[0][i];
        c[i] = dpp_f<kRowShr + 4, 0x2>(c[i], acc[1][i]);
        c[i] = dpp_f<kRowShr + 8, 0x4>(c[i], acc[2][i]);
        c[i] = dpp_f<kRowShr + 12, 0x8>(c[i], acc[3][i]);
      }
      const bool tail = kbase + kBlock > klim;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = __builtin_fmaf(c[i], m1, m0);
        if (tail && kbase + dsig(a4, 4 * g + i) >= klim) c[i] = -INFINITY;
        if (SEL && xm != 0 && ((xm >> dsig(a4, 4 * g + i)) & 1u)) c[i] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3]));
      mx = fmaxf(mx, dpp_f<kRowRor + 4, 0xF>(mx, mx));   // over the 4 banks of the row
      mx = fmaxf(mx, dpp_f<kRowRor + 8, 0xF>(mx, mx));
      {   // over the 4 rows (lane groups)
        const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
        const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
      }
      const bool up = mx > m_run;
      if (__any(up)) {
        const float mn = up ? mx + 2.0f : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
        m_run = mn;
        l_run *= alpha;
        ocorr *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db] *= alpha;
      }
      _Float16 ph[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(c[i] - m_run);
        l_run += p;
        ph[i] = static_cast<_Float16>(p * sv);
      }
      const uint32_t w0 = as<uint16_t>(ph[0]) | (static_cast<uint32_t>(as<uint16_t>(ph[1])) << 16);
      const uint32_t w1 = as<uint16_t>(ph[2]) | (static_cast<uint32_t>(as<uint16_t>(ph[3])) << 16);
      // back to the B-operand slices of lane (h, g): keys 16g + 8c2 + e live
      // in lane 4 (2c2 + e/4) + h, value e % 4
      pb[0] = as<f16x8>(u32x4{w0, w1, dpp_u<kRowShl + 4>(w0), dpp_u<kRowShl + 4>(w1)});
      pb[1] = as<f16x8>(u32x4{dpp_u<kRowShl + 8>(w0), dpp_u<kRowShl + 8>(w1), dpp_u<kRowShl + 12>(w0),
                              dpp_u<kRowShl + 12>(w1)});
      return;
    }
    float s[4][4];
    const bool tail = kbase + kBlock > klim;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[kb][i] = __builtin_fmaf(acc[kb][i], m1, m0);
        if (tail && kbase + dsig(kb, 4 * g + i) >= klim) s[kb][i] = -INFINITY;
        if (SEL && xm != 0 && ((xm >> dsig(kb, 4 * g + i)) & 1u)) s[kb][i] = -INFINITY;
      }
    float mx = s[0][0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e >> 2][e & 3]);
    {   // max over the 4 lane groups of the head (lanes l, l^16, l^32, l^48)
      const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
      const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
    }
    // re-base when a head's max passes m_run, to 2 above it: p <= 1/4, so
    // p * sv stays inside the fp16 range, and small later rises need no re-base
    const bool up = mx > m_run;
    if (__any(up)) {
      const float mn = up ? mx + 2.0f : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_run *= alpha;
      ocorr *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db) oacc[db] *= alpha;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[kb][i] - m_run);
        l_run += p;
        pb[kb >> 1][4 * (kb & 1) + i] = static_cast<_Float16>(p * sv);
      }
  };

  // one quantized block of a unit: bb = which block of an INT4 pair
  auto compute = [&](const Regs& r, auto tag, int bb, int j, const f16x8 (&qop)[NC]) {
    constexpr bool four = decltype(tag)::value;
    f32x4 acc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        f16x8 kop;
        if constexpr (!four) {   // piece h = c / (KW / 8) of the lane's row, dwords of sub = c % (KW / 8)
          const u32x4 w4 = r.k[2 * kb + (KW == 16 ? c >> 1 : c)];
          const int d0 = KW == 16 ? 2 * (c & 1) : 0;
          const u32x2 lo = sub_i8x4(w4[d0]), hi = sub_i8x4(w4[d0 + 1]);
          kop = as<f16x8>(u32x4{lo[0], lo[1], hi[0], hi[1]});
        } else {
          kop = as<f16x8>(sub_i4x8(r.k[4 * bb + kb][c]));
        }
        acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[c], acc[kb], 0, 0, 0);
      }
    }
    // score = tau log2e sk (2^24 acc - off sum(q)), off = 128 (INT8) or 8 (INT4)
    const float cs = a.tau_log2e * r.sk[bb];
    // (a union group: a block outside this lane's head's band at this
    // precision drops all its keys)
    int klim = L;
    if (uni && !(four ? (j >= lj4lo && j < lj8lo) : (j >= lj8lo || (a.sink && j == 0)))) klim = j * kBlock;
    f16x8 pb[2];
    softmax(acc, cs * kTwo24, -(four ? 8.0f : 128.0f) * qsum * cs, r.sv[bb], j * kBlock, klim,
            SEL ? r.xm[bb] : 0ull, pb);
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        f16x8 va;
        if constexpr (!four) {
          const u32x2 lo = sub_i8x4(r.v[2 * db + c2][0]), hi = sub_i8x4(r.v[2 * db + c2][1]);
          va = as<f16x8>(u32x4{lo[0], lo[1], hi[0], hi[1]});
        } else {
          va = as<f16x8>(sub_i4x8(r.v[2 * db + bb][c2]));
        }
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[c2], oacc[db], 0, 0, 0);
      }
    // every row of this A operand is off * 2^-24: accumulates the offsets' share
    const uint32_t o2 = four ? 0x00080008u : 0x00800080u;
    const f16x8 offa = as<f16x8>(u32x4{o2, o2, o2, o2});
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) ocorr = __builtin_amdgcn_mfma_f32_16x16x32_f16(offa, pb[c2], ocorr, 0, 0, 0);
  };

  // ---- quantized units, registers double-buffered: the next unit's loads are
  // in flight while the current one is computed.  A split runs up to three
  // phases of one precision each (sink block, its INT4 share, its INT8
  // share), so the loads and the dequantization are specialized per phase.
  auto phase = [&](auto tag, int ja, int jb) {
    constexpr int U = decltype(tag)::value ? 2 : 1;   // blocks per unit
    if (ja >= jb) return;
    Regs ra, rb;
    int j = ja;
    load(j, true, jb, tag, ra);   // the first unit's loads go out before q is read
    f16x8 qop[NC];
    q_operand(!decltype(tag)::value, qop);
    if (!have_qsum) take_qsum(qop);
    while (true) {
      const int na = min(U, jb - j), j2 = j + na;
      load(j2, j2 < jb, jb, tag, rb);
      __builtin_amdgcn_sched_barrier(0);   // the next unit's loads go out before this unit's math
      compute(ra, tag, 0, j, qop);
      if (na == 2) compute(ra, tag, 1, j + 1, qop);
      j = j2;
      if (j >= jb) break;
      const int nb2 = min(U, jb - j), j3 = j + nb2;
      load(j3, j3 < jb, jb, tag, ra);
      __builtin_amdgcn_sched_barrier(0);
      compute(rb, tag, 0, j, qop);
      if (nb2 == 2) compute(rb, tag, 1, j + 1, qop);
      j = j3;
      if (j >= jb) break;
    }
  };
  {
    typedef std::integral_constant<bool, false> Int8;
    typedef std::integral_constant<bool, true> Int4;
    if (sinkb && split == 0) phase(Int8{}, 0, 1);
    phase(Int4{}, i4a, i4b);
    phase(Int8{}, i8a, i8b);
  }
  // back to value units: O = 2^24 (O' - offsets)
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[db][i] = (oacc[db][i] - ocorr[i]) * kTwo24;

  // ---- FP16 blocks: 16-bit K rows (row kr0 + k of rk, `pitch` bytes apart,
  // for key slot k) and fp16 V^T (rows of 64 slots from byte vo of rt), all
  // of a block's loads issued before its first product; rows past the K
  // range read as zeros (their scores are dropped by klim)
  auto fp16_block = [&](const __amdgpu_buffer_rsrc_t& rk, uint32_t kr0, uint32_t pitch,
                        const __amdgpu_buffer_rsrc_t& rt, uint32_t vo, int kbase, int klim, uint64_t xm,
                        const f16x8 (&qop)[NC]) {
    u32x4 kraw[4][NC], vraw[ND][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint32_t row = kr0 + static_cast<uint32_t>(dsig(kb, l16));   // K row of MFMA row l16
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kraw[kb][c] = as<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(
            rk, row * pitch + static_cast<uint32_t>((DG * g + 8 * c) * 2), 0, 0));
    }
    const uint32_t vl = vo + static_cast<uint32_t>(l16 * kBlock * 2 + 32 * g);
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)   // V^T row 16 db + l16, keys 16g + 8c2 ..
        vraw[db][c2] = as<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(
            rt, vl + static_cast<uint32_t>(db * 16 * kBlock * 2 + 16 * c2), 0, 0));
    f32x4 acc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c)
        acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(to_f16x8<BF16>(kraw[kb][c]), qop[c], acc[kb], 0, 0, 0);
    }
    f16x8 pb[2];
    softmax(acc, a.tau_log2e, 0.0f, 1.0f, kbase, klim, xm, pb);
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as<f16x8>(vraw[db][c2]), pb[c2], oacc[db], 0, 0, 0);
  };

  // the FP16 window: 16-bit keys of this sequence and the fp16 V^T copy
  int ga = 0, gb = 0;
  uint32_t gbase = 0, gkeys = 0;
  if constexpr (SEL) {   // this split's share of the gathered selected tokens
    const uint32_t* te = reinterpret_cast<const uint32_t*>(a.sel + a.sel_tab) +
                         2 * (static_cast<size_t>(a.seq0 + b) * a.hkv + kv);
    gbase = te[0];
    gkeys = te[1];
    const int ng = static_cast<int>((gkeys + kBlock - 1) / kBlock);
    ga = ng * split / ns;
    gb = ng * (split + 1) / ns;
  }
  if (ifa < ifb || ga < gb) {
    f16x8 qop[NC];
    q_operand(false, qop);
    if (ifa < ifb) {
      const uint32_t pitch = hkv * (D * 2);   // bytes between key rows of k16
      const __amdgpu_buffer_rsrc_t rk16 = make_rsrc(a.k16 + (static_cast<size_t>(tok0) * hkv + kv) * D,
                                                    static_cast<uint32_t>(L - 1) * pitch + D * 2);
      const __amdgpu_buffer_rsrc_t rt16 = make_rsrc(a.vt16 + kvb0 * (D * kBlock), span * (D * kBlock * 2));
      for (int j = ifa; j < ifb; ++j)
        fp16_block(rk16, static_cast<uint32_t>(j * kBlock), pitch, rt16,
                   static_cast<uint32_t>(j) * hkv * (D * kBlock * 2), j * kBlock, L,
                   SEL ? sload64(xmp, static_cast<size_t>(j) * hkv) : 0ull, qop);
    }
    if constexpr (SEL) {
      for (int t = ga; t < gb; ++t) {
        const size_t tile = gbase + static_cast<uint32_t>(t);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(
            reinterpret_cast<const uint16_t*>(a.sel + a.sel_gk) + tile * (kBlock * D), kBlock * D * 2);
        const __amdgpu_buffer_rsrc_t rt = make_rsrc(
            reinterpret_cast<const uint16_t*>(a.sel + a.sel_gv) + tile * (D * kBlock), D * kBlock * 2);
        fp16_block(rk, 0u, D * 2, rt, 0u, 0, static_cast<int>(gkeys) - t * kBlock, 0ull, qop);
      }
    }
  }

  // ---- the split's (m, l, O) per query head
  float lt = l_run;
  if constexpr (SMALLG) {   // head h's sums sit in the 4 banks of every row
    lt += dpp_f<kRowRor + 4, 0xF>(lt, lt);
    lt += dpp_f<kRowRor + 8, 0xF>(lt, lt);
  }
  {
    const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(lt), __float_as_uint(lt), false, false);
    lt = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(lt), __float_as_uint(lt), false, false);
    lt = __uint_as_float(y[0]) + __uint_as_float(y[1]);
  }
  if (l16 < grp) {
    float* dst = a.ws + ((static_cast<size_t>(b) * a.hq + h0 + l16) * a.nsplit + split) * (D + 2);
    if (g == 0) {
      dst[0] = m_run;
      dst[1] = lt;
    }
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[2 + db * 16 + 4 * g + i] = oacc[db][i];
  }
}

// Merge of one query head's split results by log-sum-exp: one workgroup of
// kCombWaves waves per head, wave w folding splits w, w + kCombWaves, ...
// (a sequence alone on the GPU has hundreds of splits per head, so one wave
// would wait on each group of loads in turn), then the waves' states merged
// through LDS.  Splits are taken 16 at a time per wave with every load of a
// group (their maxima and sums through scalar loads, the lane's output
// channels through vector loads) in flight together, and folded into a
// running (max, sum, O) state.
constexpr int kCombWaves = 4;
template <int D>
__global__ __launch_bounds__(64 * kCombWaves) void decode_combine_kernel(DecodeArgs a) {
  constexpr int PER = D / 64, G = 16;
  const int bh = blockIdx.x, lane = threadIdx.x & 63, ns = a.nsplit;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const float* const src = pin_sgpr(a.ws + static_cast<size_t>(bh) * ns * (D + 2));
  float M = kNegBig, lsum = 0.0f, ov[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) ov[p] = 0.0f;
  for (int c0 = w * G; c0 < ns; c0 += kCombWaves * G) {
    float m[G], l[G], x[G][PER];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int c = min(c0 + u, ns - 1);
      m[u] = c0 + u < ns ? sload(src, static_cast<size_t>(c) * (D + 2)) : kNegBig;
      l[u] = sload(src, static_cast<size_t>(c) * (D + 2) + 1);
#pragma unroll
      for (int p = 0; p < PER; ++p) x[u][p] = src[c * (D + 2) + 2 + 64 * p + lane];
    }
    float mc = m[0];
#pragma unroll
    for (int u = 1; u < G; ++u) mc = fmaxf(mc, m[u]);
    const float mn = fmaxf(M, mc);
    const float sc = __builtin_amdgcn_exp2f(M - mn);
    lsum *= sc;
#pragma unroll
    for (int p = 0; p < PER; ++p) ov[p] *= sc;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const float f = c0 + u < ns ? __builtin_amdgcn_exp2f(m[u] - mn) : 0.0f;
      lsum += l[u] * f;
#pragma unroll
      for (int p = 0; p < PER; ++p) ov[p] += x[u][p] * f;
    }
    M = mn;
  }
  // the waves' states, merged by wave 0 (a wave with no split keeps
  // M = kNegBig and zero sums, which weigh nothing)
  __shared__ float sm[kCombWaves], sl[kCombWaves], so[kCombWaves][D];
  if (lane == 0) {
    sm[w] = M;
    sl[w] = lsum;
  }
#pragma unroll
  for (int p = 0; p < PER; ++p) so[w][64 * p + lane] = ov[p];
  __syncthreads();
  if (w != 0) return;
  float mx = sm[0];
#pragma unroll
  for (int u = 1; u < kCombWaves; ++u) mx = fmaxf(mx, sm[u]);
  lsum = 0.0f;
#pragma unroll
  for (int p = 0; p < PER; ++p) ov[p] = 0.0f;
#pragma unroll
  for (int u = 0; u < kCombWaves; ++u) {
    const float f = __builtin_amdgcn_exp2f(sm[u] - mx);
    lsum += sl[u] * f;
#pragma unroll
    for (int p = 0; p < PER; ++p) ov[p] += so[u][64 * p + lane] * f;
  }
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const float r = lsum > 0.0f ? ov[p] / lsum : 0.0f;
    const size_t off = static_cast<size_t>(bh) * D + 64 * p + lane;
    if (a.o_dtype == TM_F32) static_cast<float*>(a.o)[off] = r;
    else static_cast<_Float16*>(a.o)[off] = static_cast<_Float16>(r);
  }
}

template <int D, bool BF16>
static void launch_split(bool small, dim3 grid, const DecodeArgs& a, hipStream_t st) {
  if (a.sel != nullptr) {
    if (small) hipLaunchKernelGGL((decode_split_kernel<D, BF16, true, true>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((decode_split_kernel<D, BF16, false, true>), grid, dim3(64), 0, st, a);
  } else {
    if (small) hipLaunchKernelGGL((decode_split_kernel<D, BF16, true, false>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((decode_split_kernel<D, BF16, false, false>), grid, dim3(64), 0, st, a);
  }
}

// Splits of `ncls` head classes (a.cls) over a.nseq sequences; small: every
// class has at most 4 heads (the compacted softmax).
hipError_t launch_decode_split(const DecodeArgs& a, int ncls, bool small, int d, bool bf16, hipStream_t st) {
  dim3 grid(a.nsplit, ncls, a.nseq);
  if (d == 128) {
    if (bf16) launch_split<128, true>(small, grid, a, st);
    else launch_split<128, false>(small, grid, a, st);
  } else {
    if (bf16) launch_split<64, true>(small, grid, a, st);
    else launch_split<64, false>(small, grid, a, st);
  }
  return hipGetLastError();
}

hipError_t launch_decode_combine(const DecodeArgs& a, int d, hipStream_t st) {
  if (d == 128) hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(a.nseq * a.hq), dim3(64 * kCombWaves), 0, st, a);
  else hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(a.nseq * a.hq), dim3(64 * kCombWaves), 0, st, a);
  return hipGetLastError();
}

}  // namespace tmx
