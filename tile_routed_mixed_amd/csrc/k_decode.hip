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
// The step is bound by HBM bytes (each cached code is read once per step), so
// the kernel streams blocks straight from global memory into MFMA operand
// registers without LDS.  Work: one workgroup of 4 waves per
// (sequence, KV head, chunk of executed cache blocks); each wave owns whole
// 64-token blocks.  The GQA query heads of the KV head are the (up to 16)
// columns of v_mfma_f32_16x16x32_f16:
//   S^T = Kcodes Q^T   (codes widened exactly to fp16, per-block scale applied
//                       to the fp32 scores),
//   O^T += sv * (Vcodes^T P^T)   (V codes stored transposed per block).
// INT8 codes widen with the exponent trick: byte u = c ^ 0x80 placed under
// the fp16 exponent of 1024 gives 1024 + u exactly, and one packed subtract of
// 1152 returns c.  INT4 nibbles use 1024 + (n ^ 8) - 1032.
// A second kernel merges the chunks' (max, sum, O) by log-sum-exp.
#include "tm_kernels.h"

namespace tmx {


// Key row of block kb / MFMA row m such that lane group g of the PV product
// sees keys 16g .. 16g+15 (8 per 32-key chunk).
__device__ __forceinline__ int dsigma(int kb, int m) {
  return 16 * (m >> 2) + 8 * (kb >> 1) + 4 * (kb & 1) + (m & 3);
}

__device__ __forceinline__ u32x2 widen_i8x4(uint32_t c) {
  const uint32_t t = c ^ 0x80808080u;
  u32x2 r;
  r[0] = __builtin_amdgcn_perm(0x64646464u, t, 0x07010600u);   // bytes: t0, 64, t1, 64
  r[1] = __builtin_amdgcn_perm(0x64646464u, t, 0x07030602u);   // bytes: t2, 64, t3, 64
  return r;
}

__device__ __forceinline__ f16x8 fix_i8(u32x2 a, u32x2 b) {
  f16x8 v;
  u32x4 raw = {a[0], a[1], b[0], b[1]};
  __builtin_memcpy(&v, &raw, 16);
  const f16x8 off = {1152, 1152, 1152, 1152, 1152, 1152, 1152, 1152};
  return v - off;
}

// 8 nibbles (elements 2t low / 2t+1 high of byte t) -> 8 fp16 values in order.
__device__ __forceinline__ f16x8 widen_i4x8(uint32_t c) {
  const uint32_t t = c ^ 0x88888888u;
  const uint32_t lo = t & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6
  const uint32_t hi = (t >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
  u32x4 raw;
  raw[0] = __builtin_amdgcn_perm(hi, lo, 0x0c040c00u) | 0x64006400u;
  raw[1] = __builtin_amdgcn_perm(hi, lo, 0x0c050c01u) | 0x64006400u;
  raw[2] = __builtin_amdgcn_perm(hi, lo, 0x0c060c02u) | 0x64006400u;
  raw[3] = __builtin_amdgcn_perm(hi, lo, 0x0c070c03u) | 0x64006400u;
  f16x8 v;
  __builtin_memcpy(&v, &raw, 16);
  const f16x8 off = {1032, 1032, 1032, 1032, 1032, 1032, 1032, 1032};
  return v - off;
}

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

// Cache blocks of one (sequence, KV head), in the order a split walks them:
// the sink block (when it lies outside the band), then blocks jstart .. nb-1
// in ascending order: the INT4 band, the INT8 band, then the FP16 window.
struct DecodeList {
  int nb, jstart, jf, b8, sink, sink_extra, n_ex;
  __device__ __forceinline__ int block(int e) const {
    return sink_extra ? (e == 0 ? 0 : jstart + e - 1) : jstart + e;
  }
  __device__ __forceinline__ int prec(int j) const {
    if (j >= jf) return TM_FP16;
    if ((sink && j == 0) || nb - 1 - j < b8) return TM_INT8;
    return TM_INT4;
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

// Swizzle of 16-byte chunk columns in the LDS copies of a block: K rows of
// NCH chunks (rows read 16 at a time by one lane group) and V^T rows (16
// channel rows read together at one key offset).
template <int NCH>
__device__ __forceinline__ int kswz(int row) { return row & (NCH - 1) & 7; }
template <int NCH>
__device__ __forceinline__ int vswz(int row) { return NCH >= 4 ? (row >> 2) & 3 : (row >> 3) & 1; }

// Direct-to-LDS copy of a contiguous region of ROWS rows of NCH chunks with
// the chunk columns of row r permuted by SW(r) (see TileCopy in the prefill).
template <int ROWS, int NCH, int SWK>
struct BlockCopy {
  static constexpr int NI = ROWS * NCH / 64;            // 1 KiB loads per region
  static constexpr int PER = (NI + 3) / 4;
  uint32_t voff[PER];
  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int off = (i * 4 + w) * 1024 + lane * 16;
      const int r = off / (NCH * 16), slot = (off / 16) % NCH;
      const int sw = SWK == 0 ? kswz<NCH>(r) : vswz<NCH>(r);
      voff[i] = static_cast<uint32_t>(r * NCH * 16 + ((slot ^ sw) << 4));
    }
  }
  __device__ __forceinline__ static int count(int w) { return w < NI % 4 || NI % 4 == 0 ? PER : PER - 1; }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, uint32_t soff, uint8_t* dst, int w) const {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (i * 4 + w < NI) lds_dma16(rs, dst + (i * 4 + w) * 1024, voff[i], soff);
  }
};

template <int D, bool BF16>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int NC = D / 32;          // k-chunks of the QK MFMA (lane group g owns channels DG*g ..)
  constexpr int ND = D / 16;          // output channel blocks
  constexpr int DG = D / 4;
  constexpr int SLOT = 128 * D;       // bytes of one INT8 block: K rows then V^T rows
  constexpr int S = 4;                // ring depth: S - 1 blocks stream in while one is used
  constexpr int NCK8 = D / 16, NCK4 = D / 32;   // 16-byte chunks per K row
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
  dl.jf = a.tail > 0 ? max(0, (L - a.tail) / kBlock) : dl.nb;            // first FP16 block
  dl.jstart = min(max(0, dl.nb - __builtin_amdgcn_readfirstlane(a.b4[kv])), dl.jf);                     // first block with delta < b4
  dl.sink_extra = (a.sink && dl.jstart > 0) ? 1 : 0;
  dl.n_ex = (dl.nb - dl.jstart) + dl.sink_extra;
  const int e0 = dl.split(chunk, a.nsplit), e1 = dl.split(chunk + 1, a.nsplit);
  const int eF = max(e0, min(e1, dl.first_fp16()));
  const int nI = eF - e0;                                                 // quantized blocks of this split
  const size_t kvb0 = static_cast<size_t>(kv) * a.nblk + blk0;

  // Q^T operand: column l16 = query head kv*grp + l16 (zero past the group)
  f16x8 qop[NC];
  {
    const bool ok = l16 < grp;
    const uint16_t* qs = a.q + (static_cast<size_t>(b) * a.hq + kv * grp + (ok ? l16 : 0)) * D + DG * g;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 raw = ok ? *reinterpret_cast<const u32x4*>(qs + 8 * c) : u32x4{0, 0, 0, 0};
      qop[c] = to_f16x8<BF16>(raw);
    }
  }

  // buffer resources over this (sequence, KV head)'s blocks
  const uint32_t nbs = static_cast<uint32_t>(dl.nb);
  const __amdgpu_buffer_rsrc_t rk8 = make_rsrc(a.k8 + kvb0 * (kBlock * D), nbs * (kBlock * D));
  const __amdgpu_buffer_rsrc_t rv8 = make_rsrc(a.v8 + kvb0 * (kBlock * D), nbs * (kBlock * D));
  const __amdgpu_buffer_rsrc_t rk4 = make_rsrc(a.k4 + kvb0 * (kBlock * D / 2), nbs * (kBlock * D / 2));
  const __amdgpu_buffer_rsrc_t rv4 = make_rsrc(a.v4 + kvb0 * (kBlock * D / 2), nbs * (kBlock * D / 2));
  BlockCopy<kBlock, NCK8, 0> ck8;
  BlockCopy<D, 4, 1> cv8;
  BlockCopy<kBlock, NCK4, 0> ck4;
  BlockCopy<D, 2, 1> cv4;
  ck8.init(w, lane);
  cv8.init(w, lane);
  ck4.init(w, lane);
  cv4.init(w, lane);
  // list entry e -> cache block j, and whether it is an INT4 block (entries
  // before eF are INT8 or INT4; see DecodeList)
  const int eS = dl.sink_extra;
  const int j4hi = min(dl.nb - dl.b8, dl.jf);
  auto jof = [&](int e) { return e < eS ? 0 : dl.jstart + (e - eS); };
  auto is4 = [&](int j) { return j >= dl.jstart && j < j4hi && !(dl.sink && j == 0); };
  auto loads_of = [&](bool four) {   // vector-memory instructions this wave issues for one block
    return four ? decltype(ck4)::count(w) + decltype(cv4)::count(w)
                : decltype(ck8)::count(w) + decltype(cv8)::count(w);
  };
  auto issue = [&](int t) {
    const int j = jof(e0 + t);
    uint8_t* dst = lds + (t & (S - 1)) * SLOT;
    if (!is4(j)) {
      ck8.issue(rk8, j * (kBlock * D), dst, w);
      cv8.issue(rv8, j * (kBlock * D), dst + kBlock * D, w);
    } else {
      ck4.issue(rk4, j * (kBlock * D / 2), dst, w);
      cv4.issue(rv4, j * (kBlock * D / 2), dst + kBlock * D, w);
    }
  };

  // per-lane LDS read offsets inside a ring slot: K row 16w + l16 (chunks of
  // lane group g), V^T rows l16 + 16 db at keys 16w + 4g (db adds a constant)
  const int krow = 16 * w + l16;
  int k8off[NC / 2 > 0 ? NC / 2 : 1];
#pragma unroll
  for (int c2 = 0; c2 < NC / 2; ++c2) k8off[c2] = krow * D + ((((DG / 16) * g + c2) ^ kswz<NCK8>(krow)) << 4);
  const int k4off = D == 128 ? krow * (D / 2) + ((g ^ kswz<NCK4>(krow)) << 4)
                             : krow * (D / 2) + (((g >> 1) ^ kswz<NCK4>(krow)) << 4) + 8 * (g & 1);
  const int v8off = kBlock * D + l16 * 64 + ((w ^ vswz<4>(l16)) << 4) + 4 * g;
  const int v4off = kBlock * D + l16 * 32 + (((w >> 1) ^ vswz<2>(l16)) << 4) + 8 * (w & 1) + 2 * g;

  float m_run = kNegBig, l_run = 0.0f;   // per lane: head l16, keys of lane group g
  f32x4 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One block's keys 16w .. 16w+15 given S^T scores (already scaled, log2
  // units) in lane (g, head) for keys 4g + i, and the V^T operands.
  auto softmax_pv = [&](float (&s)[4], const f16x4 (&va)[ND], float sv) {
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
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(va[db], pb, oacc[db], 0, 0, 0);
  };

  // scale factors of a quantized block: cs = tau log2e sk, sv (scalar loads,
  // fetched one block ahead)
  auto scales = [&](int t, float& cs, float& sv) {
    const int j = jof(e0 + t);
    const size_t kblk = kvb0 + j;
    if (!is4(j)) {
      cs = sload(a.ks8, kblk);
      sv = sload(a.vs8, kblk);
    } else {
      cs = sload(a.ks4, kblk);
      sv = sload(a.vs4, kblk);
    }
  };
  float cs_n = 0.0f, sv_n = 0.0f;
  if (nI > 0) scales(0, cs_n, sv_n);

  // ---- quantized blocks through the LDS ring
#pragma unroll
  for (int t = 0; t < S - 1; ++t)
    if (t < nI) issue(t);
  for (int t = 0; t < nI; ++t) {
    // wait for block t: only this wave's loads of blocks t+1 .. t+S-2 may remain
    int younger = 0;
#pragma unroll
    for (int u = 1; u <= S - 2; ++u)
      if (t + u < nI) younger += loads_of(is4(jof(e0 + t + u)));
    wait_vm(younger);
    lds_barrier();   // block t landed for every wave; block t-1's slot is free
    if (t + S - 1 < nI) issue(t + S - 1);
    const float cs = a.tau_log2e * cs_n, sv = sv_n;
    if (t + 1 < nI) scales(t + 1, cs_n, sv_n);

    const int j = jof(e0 + t);
    const uint8_t* sl0 = lds + (t & (S - 1)) * SLOT;
    f16x8 kop[NC];
    f16x4 va[ND];
    if (!is4(j)) {
#pragma unroll
      for (int c2 = 0; c2 < NC / 2; ++c2) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(sl0 + k8off[c2]);
        kop[2 * c2] = fix_i8(widen_i8x4(raw[0]), widen_i8x4(raw[1]));
        kop[2 * c2 + 1] = fix_i8(widen_i8x4(raw[2]), widen_i8x4(raw[3]));
      }
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const uint32_t raw = *reinterpret_cast<const uint32_t*>(sl0 + v8off + db * 1024);
        const u32x2 h = widen_i8x4(raw);
        f16x4 v;
        __builtin_memcpy(&v, &h, 8);
        const f16x4 off = {1152, 1152, 1152, 1152};
        va[db] = v - off;
      }
    } else {
      if constexpr (D == 128) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(sl0 + k4off);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) kop[e2] = widen_i4x8(raw[e2]);
      } else {
        const u32x2 raw = *reinterpret_cast<const u32x2*>(sl0 + k4off);
        kop[0] = widen_i4x8(raw[0]);
        kop[1] = widen_i4x8(raw[1]);
      }
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const uint32_t raw = *reinterpret_cast<const uint16_t*>(sl0 + v4off + db * 512);
        const f16x8 v8 = widen_i4x8(raw);
        va[db] = f16x4{v8[0], v8[1], v8[2], v8[3]};
      }
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[c], qop[c], acc, 0, 0, 0);
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = acc[i] * cs;
    if (j * kBlock + kBlock > L) {   // partial last block (no FP16 window)
      const int kbase = j * kBlock + 16 * w + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (kbase + i >= L) s[i] = -INFINITY;
    }
    softmax_pv(s, va, sv);
  }

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
      __builtin_memcpy(&va[db], &raw, 8);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[c], qop[c], acc, 0, 0, 0);
    float s[4];
    const int kbase = j * kBlock + 16 * w + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = kbase + i < L ? acc[i] * a.tau_log2e : -INFINITY;
    softmax_pv(s, va, 1.0f);
  }

  // ---- merge the 4 waves (reusing the ring), write the split's (m, l, O) per query head
  __syncthreads();
  float* sm = reinterpret_cast<float*>(lds);            // [4][16]
  float* sl = sm + 64;                                  // [4][16]
  float* so = sl + 64;                                  // [4][16][D + 1]
  float lt = l_run + __shfl_xor(l_run, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
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
