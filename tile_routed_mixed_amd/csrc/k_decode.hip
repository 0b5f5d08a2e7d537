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
// One workgroup of 4 waves walks a split of one (sequence, KV head)'s cache
// blocks; the blocks stream global -> LDS through a 4-deep ring of direct
// (buffer-to-LDS) loads, so three blocks are in flight while one is used, and
// each wave scores 16 keys of the current block against the (up to 16) GQA
// query heads, which are the columns of 16x16 fp16 MFMAs:
//   S^T = K Q^T   (v_mfma_f32_16x16x32_f16),   O^T += V^T P^T (16x16x16).
// Codes enter the MFMAs as fp16 subnormals: the byte b = c + 128 (INT8) or
// the nibble n = c + 8 (INT4) placed in the low bits of a zero-exponent fp16
// is exactly b * 2^-24, so two perms (or a mask) per pair of codes build an
// operand, with no arithmetic.  The offsets come back out exactly where they
// are cheap: for scores, 2^24 S' - off * sum(q) in the FMA that scales them;
// for outputs, one extra MFMA per block accumulates off * 2^-24 * sum(p) per
// head, subtracted once at the end.  MFMA products and sums of these values
// are exact fp32 (no flush of fp16 subnormals on this path).
// A second kernel merges the splits' (max, sum, O) by log-sum-exp.
#include "tm_kernels.h"

namespace tmx {

// Eight 16-bit values (fp16, or bf16 widened to fp16: exact for magnitudes in
// [2^-14, 65504], the range of normal fp16 numbers) as an fp16 MFMA operand.
template <bool BF16>
__device__ __forceinline__ f16x8 to_f16x8(u32x4 raw) {
  f16x8 v;
  if constexpr (BF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = static_cast<_Float16>(__uint_as_float(raw[e] << 16));
      v[2 * e + 1] = static_cast<_Float16>(__uint_as_float(raw[e] & 0xFFFF0000u));
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

// Cache blocks of one (sequence, KV head), in the order a split walks them:
// the sink block (when it lies outside the band), then blocks jstart .. nb-1
// in ascending order: the INT4 band, the INT8 band, then the FP16 window.
struct DecodeList {
  int nb, jstart, jf, b8, sink, sink_extra, n_ex;
  __device__ __forceinline__ int block(int e) const {
    return sink_extra ? (e == 0 ? 0 : jstart + e - 1) : jstart + e;
  }
  // HBM cost of entries [0, e) in units of an INT4 block (INT8 2, FP16 4)
  __device__ __forceinline__ int64_t weight(int e) const {
    int64_t wsum = 0;
    if (sink_extra && e > 0) {
      wsum += 2;
      --e;
    }
    const int hi = jstart + e;                        // blocks [jstart, hi)
    const int qend = min(hi, jf);                     // quantized part [jstart, qend)
    const int n16 = max(0, hi - max(jf, jstart));
    int n8 = max(0, qend - max(jstart, nb - b8));
    int n4 = max(0, qend - jstart) - n8;
    if (sink && jstart == 0 && qend > 0 && nb - b8 > 0) {   // block 0 inside the INT4 range is INT8
      ++n8;
      --n4;
    }
    return wsum + 2 * n8 + n4 + 4 * n16;
  }
  // first entry e with weight(e) * parts >= total * c
  __device__ __forceinline__ int split(int c, int parts) const {
    const int64_t target = weight(n_ex) * c;
    int lo = 0, hi = n_ex;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (weight(mid) * parts >= target) hi = mid;
      else lo = mid + 1;
    }
    return lo;
  }
  // list index of the first FP16 block (n_ex if none)
  __device__ __forceinline__ int first_fp16() const {
    return jf < nb ? (sink_extra ? 1 : 0) + (jf - jstart) : n_ex;
  }
};

// Swizzle of the 16-byte chunk columns of a block's rows in LDS.  K rows (NCH
// chunks, 16/NCH rows per 256 bytes of banks) are read 16 at a time at one
// logical chunk, so the chunk moves with the row's position in the bank
// cycle; V^T rows are read 16 at a time at one key offset.
template <int NCH>
__device__ __forceinline__ int kswz(int row) {
  return NCH >= 16 ? row & 15 : (row >> (NCH == 8 ? 1 : NCH == 4 ? 2 : 3)) & (NCH - 1);
}
template <int NCH>
__device__ __forceinline__ int vswz(int row) { return NCH >= 4 ? (row >> 2) & 3 : (row >> 3) & 1; }

// Direct-to-LDS copy of a contiguous region of ROWS rows of NCH chunks with
// the chunk columns of row r permuted (load n fills LDS bytes
// [n*1024, n*1024+1024), lane L lands at n*1024 + 16L and fetches the chunk
// that belongs there); wave w issues loads n = 4i + w.
template <int ROWS, int NCH, bool VT>
struct BlockCopy {
  static constexpr int NI = ROWS * NCH / 64;
  static constexpr int PER = (NI + 3) / 4;
  uint32_t voff[PER];
  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int off = (i * 4 + w) * 1024 + lane * 16;
      const int r = off / (NCH * 16), slot = (off / 16) % NCH;
      const int sw = VT ? vswz<NCH>(r) : kswz<NCH>(r);
      voff[i] = static_cast<uint32_t>(r * NCH * 16 + ((slot ^ sw) << 4));
    }
  }
  __device__ __forceinline__ static constexpr int count(int w) {
    return NI % 4 == 0 ? PER : (w < NI % 4 ? PER : PER - 1);
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, uint32_t soff, uint8_t* dst, int w) const {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (NI % 4 == 0 || i * 4 + w < NI) lds_dma16(rs, dst + (i * 4 + w) * 1024, voff[i], soff);
  }
};

template <int D, bool BF16>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int NC = D / 32;          // k-chunks of the QK MFMA (lane group g owns channels DG*g ..)
  constexpr int ND = D / 16;          // output channel blocks
  constexpr int DG = D / 4;
  constexpr int SLOT = 128 * D;       // bytes of one INT8 block: K rows, then V^T rows
  constexpr int S = 4;                // ring depth: S - 1 blocks stream in while one is used
  constexpr int NCK8 = D / 16, NCK4 = D / 32;   // 16-byte chunks per K row
  constexpr float kTwo24 = 16777216.0f;
  __shared__ __align__(1024) uint8_t lds[S * SLOT];

  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunk = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int grp = a.hq / a.hkv;

  const int tok0 = a.cu[b];
  const int L = a.cu[b + 1] - tok0;
  const int blk0 = __builtin_amdgcn_readfirstlane(seq_blk_start(a.cu, b));
  DecodeList dl;
  dl.nb = (L + kBlock - 1) / kBlock;
  dl.b8 = __builtin_amdgcn_readfirstlane(a.b8[kv]);
  dl.sink = a.sink;
  dl.jf = a.tail > 0 ? max(0, (L - a.tail) / kBlock) : dl.nb;                                    // first FP16 block
  dl.jstart = min(max(0, dl.nb - __builtin_amdgcn_readfirstlane(a.b4[kv])), dl.jf);             // delta < b4
  dl.sink_extra = (a.sink && dl.jstart > 0) ? 1 : 0;
  dl.n_ex = (dl.nb - dl.jstart) + dl.sink_extra;
  const int e0 = dl.split(chunk, a.nsplit), e1 = dl.split(chunk + 1, a.nsplit);
  const int eF = max(e0, min(e1, dl.first_fp16()));
  const int nI = eF - e0;                                                                        // quantized blocks
  const size_t kvb0 = static_cast<size_t>(kv) * a.nblk + blk0;

  // Q^T operand: column l16 = query head kv*grp + l16 (zero past the group);
  // qsum: the head's sum of q over all channels (for the code offsets)
  f16x8 qop[NC];
  float qsum = 0.0f;
  {
    const bool ok = l16 < grp;
    const uint16_t* qs = a.q + (static_cast<size_t>(b) * a.hq + kv * grp + (ok ? l16 : 0)) * D + DG * g;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 raw = ok ? *reinterpret_cast<const u32x4*>(qs + 8 * c) : u32x4{0, 0, 0, 0};
      qop[c] = to_f16x8<BF16>(raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) qsum += static_cast<float>(qop[c][e]);
    }
    const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(qsum), __float_as_uint(qsum), false, false);
    qsum = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(qsum), __float_as_uint(qsum), false, false);
    qsum = __uint_as_float(y[0]) + __uint_as_float(y[1]);
  }

  // buffer resources over this (sequence, KV head)'s blocks
  const uint32_t nbs = static_cast<uint32_t>(dl.nb);
  const __amdgpu_buffer_rsrc_t rk8 = make_rsrc(a.k8 + kvb0 * (kBlock * D), nbs * (kBlock * D));
  const __amdgpu_buffer_rsrc_t rv8 = make_rsrc(a.v8 + kvb0 * (kBlock * D), nbs * (kBlock * D));
  const __amdgpu_buffer_rsrc_t rk4 = make_rsrc(a.k4 + kvb0 * (kBlock * D / 2), nbs * (kBlock * D / 2));
  const __amdgpu_buffer_rsrc_t rv4 = make_rsrc(a.v4 + kvb0 * (kBlock * D / 2), nbs * (kBlock * D / 2));
  BlockCopy<kBlock, NCK8, false> ck8;
  BlockCopy<D, 4, true> cv8;
  BlockCopy<kBlock, NCK4, false> ck4;
  BlockCopy<D, 2, true> cv4;
  ck8.init(w, lane);
  cv8.init(w, lane);
  ck4.init(w, lane);
  cv4.init(w, lane);
  // Every block costs each wave the same number of vector-memory
  // instructions: INT4 blocks pad with re-reads of their first KiB into the
  // slot space INT4 leaves unused, so the ring's waits are constants.
  const int n8 = ck8.count(w) + cv8.count(w);
  const int npad = n8 - (ck4.count(w) + cv4.count(w));

  // list entry e -> cache block j; quantized entries are INT4 or INT8
  const int eS = dl.sink_extra;
  const int j4hi = min(dl.nb - dl.b8, dl.jf);
  auto jof = [&](int e) { return e < eS ? 0 : dl.jstart + (e - eS); };
  auto is4 = [&](int j) { return j >= dl.jstart && j < j4hi && !(dl.sink && j == 0); };
  auto issue = [&](int t) {
    const int j = jof(e0 + t);
    uint8_t* dst = lds + (t & (S - 1)) * SLOT;
    if (!is4(j)) {
      ck8.issue(rk8, j * (kBlock * D), dst, w);
      cv8.issue(rv8, j * (kBlock * D), dst + kBlock * D, w);
    } else {
      ck4.issue(rk4, j * (kBlock * D / 2), dst, w);
      cv4.issue(rv4, j * (kBlock * D / 2), dst + kBlock * D, w);
      // (distinct sources and targets, so the compiler cannot fold them:
      // the ring's wait counts rely on every one being issued)
      for (int k = 0; k < npad; ++k)
        lds_dma16(rk4, dst + (k == 0 ? kBlock * D / 2 : kBlock * D + kBlock * D / 2) + (w % (D / 32)) * 1024,
                  k * 1024 + lane * 16, j * (kBlock * D / 2));
    }
  };
  // scale factors of a quantized block (scalar loads, fetched one block ahead)
  const float* const ks8 = pin_sgpr(a.ks8 + kvb0);
  const float* const vs8 = pin_sgpr(a.vs8 + kvb0);
  const float* const ks4 = pin_sgpr(a.ks4 + kvb0);
  const float* const vs4 = pin_sgpr(a.vs4 + kvb0);
  auto scales = [&](int t, float& sk, float& sv) {
    const int j = jof(e0 + t);
    const bool four = is4(j);
    sk = sload(four ? ks4 : ks8, j);
    sv = sload(four ? vs4 : vs8, j);
  };

  // per-lane LDS read offsets inside a ring slot: K row 16w + l16 (the chunks
  // of lane group g), V^T rows l16 + 16 db at keys 16w + 4g (db adds a constant)
  const int krow = 16 * w + l16;
  int k8off[NC / 2 > 0 ? NC / 2 : 1];
#pragma unroll
  for (int c2 = 0; c2 < NC / 2; ++c2) k8off[c2] = krow * D + ((((DG / 16) * g + c2) ^ kswz<NCK8>(krow)) << 4);
  const int k4off = D == 128 ? krow * (D / 2) + ((g ^ kswz<NCK4>(krow)) << 4)
                             : krow * (D / 2) + (((g >> 1) ^ kswz<NCK4>(krow)) << 4) + 8 * (g & 1);
  const int v8off = kBlock * D + l16 * 64 + ((w ^ vswz<4>(l16)) << 4) + 4 * g;
  const int v4off = kBlock * D + l16 * 32 + (((w >> 1) ^ vswz<2>(l16)) << 4) + 8 * (w & 1) + 2 * g;

  float m_run = kNegBig, l_run = 0.0f;   // per lane: head l16, keys of lane group g
  f32x4 oacc[ND], ocorr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One block's keys 16w .. 16w+15: s holds the lane's 4 scores (log2 units)
  // of head l16 for keys 4g + i.  Returns the fp16 P^T operand (p * sv).
  auto softmax = [&](float (&s)[4], float sv) {
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
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
    f16x4 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(s[i] - m_run);
      l_run += p;
      pb[i] = static_cast<_Float16>(p * sv);
    }
    return pb;
  };

  float sk_n = 0.0f, sv_n = 0.0f;
  if (nI > 0) scales(0, sk_n, sv_n);

  // ---- quantized blocks through the LDS ring
#pragma unroll
  for (int t = 0; t < S - 1; ++t)
    if (t < nI) issue(t);
  for (int t = 0; t < nI; ++t) {
    // wait for block t (loads complete in order; each later block in flight
    // holds n8 loads of this wave), then a barrier so every wave's share landed
    // and block t-1's slot (the next issue's target) is free
    const int ahead = min(S - 2, nI - 1 - t);
    if (ahead >= 2) wait_vm(2 * n8);
    else if (ahead == 1) wait_vm(n8);
    else wait_vm(0);
    lds_barrier();
    if (t + S - 1 < nI) issue(t + S - 1);
    const float sk = sk_n, sv = sv_n;
    if (t + 1 < nI) scales(t + 1, sk_n, sv_n);

    const int j = jof(e0 + t);
    const bool four = is4(j);
    const uint8_t* sl0 = lds + (t & (S - 1)) * SLOT;
    f16x8 kop[NC];
    f16x4 va[ND];
    if (!four) {
#pragma unroll
      for (int c2 = 0; c2 < NC / 2; ++c2) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(sl0 + k8off[c2]);
        kop[2 * c2] = as<f16x8>(u32x4{sub_i8x4(raw[0])[0], sub_i8x4(raw[0])[1], sub_i8x4(raw[1])[0],
                                      sub_i8x4(raw[1])[1]});
        kop[2 * c2 + 1] = as<f16x8>(u32x4{sub_i8x4(raw[2])[0], sub_i8x4(raw[2])[1], sub_i8x4(raw[3])[0],
                                          sub_i8x4(raw[3])[1]});
      }
#pragma unroll
      for (int db = 0; db < ND; ++db)
        va[db] = as<f16x4>(sub_i8x4(*reinterpret_cast<const uint32_t*>(sl0 + v8off + db * 1024)));
    } else {
      if constexpr (D == 128) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(sl0 + k4off);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) kop[e2] = as<f16x8>(sub_i4x8(raw[e2]));
      } else {
        const u32x2 raw = *reinterpret_cast<const u32x2*>(sl0 + k4off);
        kop[0] = as<f16x8>(sub_i4x8(raw[0]));
        kop[1] = as<f16x8>(sub_i4x8(raw[1]));
      }
#pragma unroll
      for (int db = 0; db < ND; ++db)
        va[db] = as<f16x4>(sub_i4x4(*reinterpret_cast<const uint16_t*>(sl0 + v4off + db * 512)));
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[c], qop[c], acc, 0, 0, 0);
    // score = tau log2e sk (2^24 acc - off sum(q)), off = 128 (INT8) or 8 (INT4)
    const float cs = a.tau_log2e * sk;
    const float m1 = cs * kTwo24, m0 = -(four ? 8.0f : 128.0f) * qsum * cs;
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = __builtin_fmaf(acc[i], m1, m0);
    if (j * kBlock + kBlock > L) {   // partial last block (no FP16 window)
      const int kbase = j * kBlock + 16 * w + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (kbase + i >= L) s[i] = -INFINITY;
    }
    const f16x4 pb = softmax(s, sv);
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(va[db], pb, oacc[db], 0, 0, 0);
    // every row of this A operand is off * 2^-24: accumulates the offsets' share
    const f16x4 offa = as<f16x4>(u32x2{four ? 0x00080008u : 0x00800080u, four ? 0x00080008u : 0x00800080u});
    ocorr = __builtin_amdgcn_mfma_f32_16x16x16f16(offa, pb, ocorr, 0, 0, 0);
  }
  // back to value units: O = 2^24 (O' - offsets)
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[db][i] = (oacc[db][i] - ocorr[i]) * kTwo24;

  // ---- FP16 window blocks: 16-bit K rows and the fp16 V^T copy, from global memory
  for (int e = eF; e < e1; ++e) {
    const int j = dl.block(e);
    const size_t kblk = kvb0 + j;
    const int key = j * kBlock + 16 * w + l16;   // K row of this lane (MFMA row l16)
    f16x8 kop[NC];
    {
      const uint16_t* src = a.k16 + (static_cast<size_t>(tok0 + (key < L ? key : 0)) * a.hkv + kv) * D + DG * g;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u32x4 raw = key < L ? *reinterpret_cast<const u32x4*>(src + 8 * c) : u32x4{0, 0, 0, 0};
        kop[c] = to_f16x8<BF16>(raw);
      }
    }
    f16x4 va[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int d = db * 16 + l16;
      const u32x2 raw = *reinterpret_cast<const u32x2*>(a.vt16 + (kblk * D + d) * kBlock + 16 * w + 4 * g);
      va[db] = as<f16x4>(raw);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[c], qop[c], acc, 0, 0, 0);
    float s[4];
    const int kbase = j * kBlock + 16 * w + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = kbase + i < L ? acc[i] * a.tau_log2e : -INFINITY;
    const f16x4 pb = softmax(s, 1.0f);
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(va[db], pb, oacc[db], 0, 0, 0);
  }

  // ---- merge the 4 waves (reusing the ring), write the split's (m, l, O) per query head
  __syncthreads();
  float* sm = reinterpret_cast<float*>(lds);            // [4][16]
  float* sl = sm + 64;                                  // [4][16]
  float* so = sl + 64;                                  // [4][16][D + 1]
  float lt = l_run;
  {
    const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(lt), __float_as_uint(lt), false, false);
    lt = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(lt), __float_as_uint(lt), false, false);
    lt = __uint_as_float(y[0]) + __uint_as_float(y[1]);
  }
  if (g == 0) {
    sm[w * 16 + l16] = m_run;
    sl[w * 16 + l16] = lt;
  }
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) so[(w * 16 + l16) * (D + 1) + db * 16 + 4 * g + i] = oacc[db][i];
  __syncthreads();
  for (int x = tid; x < grp * D; x += 256) {
    const int qh = x / D, dv = x % D;
    float M = kNegBig;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm[ww * 16 + qh]);
    float lsum = 0.0f, ov = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = __builtin_amdgcn_exp2f(sm[ww * 16 + qh] - M);
      lsum += sl[ww * 16 + qh] * f;
      ov += so[(ww * 16 + qh) * (D + 1) + dv] * f;
    }
    float* dst = a.ws + ((static_cast<size_t>(b) * a.hq + kv * grp + qh) * a.nsplit + chunk) * (D + 2);
    dst[2 + dv] = ov;
    if (dv == 0) {
      dst[0] = M;
      dst[1] = lsum;
    }
  }
}

template <int D>
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const float* src = a.ws + static_cast<size_t>(bh) * a.nsplit * (D + 2);
  float M = kNegBig;
  for (int c = 0; c < a.nsplit; ++c) M = fmaxf(M, src[c * (D + 2)]);
  for (int dv = threadIdx.x; dv < D; dv += blockDim.x) {
    float lsum = 0.0f, ov = 0.0f;
    for (int c = 0; c < a.nsplit; ++c) {
      const float f = __builtin_amdgcn_exp2f(src[c * (D + 2)] - M);
      lsum += src[c * (D + 2) + 1] * f;
      ov += src[c * (D + 2) + 2 + dv] * f;
    }
    const float r = lsum > 0.0f ? ov / lsum : 0.0f;
    const size_t off = static_cast<size_t>(bh) * D + dv;
    if (a.o_dtype == TM_F32) static_cast<float*>(a.o)[off] = r;
    else static_cast<_Float16*>(a.o)[off] = static_cast<_Float16>(r);
  }
}

hipError_t launch_decode(const DecodeArgs& a, int d, bool bf16, hipStream_t st) {
  dim3 grid(a.nsplit, a.hkv, a.nseq);
  if (d == 128) {
    if (bf16) hipLaunchKernelGGL((decode_split_kernel<128, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((decode_split_kernel<128, false>), grid, dim3(256), 0, st, a);
  } else {
    if (bf16) hipLaunchKernelGGL((decode_split_kernel<64, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((decode_split_kernel<64, false>), grid, dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (d == 128) hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(a.nseq * a.hq), dim3(128), 0, st, a);
  else hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(a.nseq * a.hq), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace tmx
