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

template <int D, bool BF16>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int NC = D / 32;      // f16 MFMA k-chunks over d
  constexpr int ND = D / 16;      // output channel blocks
  constexpr int DG = D / 4;       // channels per lane group in the QK operand
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int chunk = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int grp = a.hq / a.hkv;

  const int tok0 = a.cu[b];
  const int L = a.cu[b + 1] - tok0;
  const int blk0 = seq_blk_start(a.cu, b);
  const int nb = (L + kBlock - 1) / kBlock;
  const int b8 = a.b8[kv], b4 = a.b4[kv];
  const int jf = a.tail > 0 ? max(0, (L - a.tail) / kBlock) : nb;    // first FP16 block
  const int jlo = max(0, nb - b4);                                   // first block with delta < b4
  const int jstart = min(jlo, jf);
  const bool sink_extra = a.sink && jstart > 0;
  const int n_ex = (nb - jstart) + (sink_extra ? 1 : 0);
  const int e0 = static_cast<int>(static_cast<int64_t>(chunk) * n_ex / a.nsplit);
  const int e1 = static_cast<int>(static_cast<int64_t>(chunk + 1) * n_ex / a.nsplit);

  // Q^T operand: column l16 = query head kv*grp + l16 (zero past the group).
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

  float m_run = kNegBig, l_run = 0.0f;
  f32x4 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int e = e0 + w; e < e1; e += 4) {
    const int j = sink_extra ? (e == 0 ? 0 : jstart + e - 1) : jstart + e;
    int prec;
    if (j >= jf) prec = TM_FP16;
    else if ((a.sink && j == 0) || (nb - 1 - j) < b8) prec = TM_INT8;
    else prec = TM_INT4;
    const size_t kblk = static_cast<size_t>(kv) * a.nblk + blk0 + j;

    // ---- K operands (A of S^T = K Q^T): lane (g, m) holds key dsigma(kb, m), channels DG*g ..
    f16x8 kop[4][NC];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = dsigma(kb, l16);
      if (prec == TM_INT8) {
        const int8_t* src = a.k8 + (kblk * kBlock + key) * D + DG * g;
#pragma unroll
        for (int c2 = 0; c2 < NC / 2; ++c2) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(src + 16 * c2);
          kop[kb][2 * c2] = fix_i8(widen_i8x4(raw[0]), widen_i8x4(raw[1]));
          kop[kb][2 * c2 + 1] = fix_i8(widen_i8x4(raw[2]), widen_i8x4(raw[3]));
        }
      } else if (prec == TM_INT4) {
        const uint8_t* src = a.k4 + (kblk * kBlock + key) * (D / 2) + (DG / 2) * g;
#pragma unroll
        for (int c4 = 0; c4 < NC / 4; ++c4) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(src + 16 * c4);
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) kop[kb][4 * c4 + e2] = widen_i4x8(raw[e2]);
        }
        if constexpr (NC % 4 != 0) {
          const u32x2 raw = *reinterpret_cast<const u32x2*>(src + 16 * (NC / 4));
          kop[kb][NC - 2] = widen_i4x8(raw[0]);
          kop[kb][NC - 1] = widen_i4x8(raw[1]);
        }
      } else {
        const int tk = j * kBlock + key;
        const uint16_t* src = a.k16 + (static_cast<size_t>(tok0 + (tk < L ? tk : 0)) * a.hkv + kv) * D + DG * g;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          u32x4 raw = tk < L ? *reinterpret_cast<const u32x4*>(src + 8 * c) : u32x4{0, 0, 0, 0};
          kop[kb][c] = to_f16x8<BF16>(raw);
        }
      }
    }
    // ---- V^T operands (A of O^T = V^T P^T): lane (g, dv) holds keys 16g .. 16g+15
    f16x8 vop[ND][2];
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int dv = db * 16 + l16;
      if (prec == TM_INT8) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(a.v8 + (kblk * D + dv) * kBlock + 16 * g);
        vop[db][0] = fix_i8(widen_i8x4(raw[0]), widen_i8x4(raw[1]));
        vop[db][1] = fix_i8(widen_i8x4(raw[2]), widen_i8x4(raw[3]));
      } else if (prec == TM_INT4) {
        const u32x2 raw = *reinterpret_cast<const u32x2*>(a.v4 + (kblk * D + dv) * (kBlock / 2) + 8 * g);
        vop[db][0] = widen_i4x8(raw[0]);
        vop[db][1] = widen_i4x8(raw[1]);
      } else {
        const uint16_t* src = a.vt16 + (kblk * D + dv) * kBlock + 16 * g;
        u32x4 r0 = *reinterpret_cast<const u32x4*>(src);
        u32x4 r1 = *reinterpret_cast<const u32x4*>(src + 8);
        __builtin_memcpy(&vop[db][0], &r0, 16);
        __builtin_memcpy(&vop[db][1], &r1, 16);
      }
    }

    // ---- scores
    f32x4 acc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[kb][c], qop[c], acc[kb], 0, 0, 0);
    }
    float cs = a.tau_log2e, vsc = 1.0f;
    if (prec == TM_INT8) {
      cs *= a.ks8[kblk];
      vsc = a.vs8[kblk];
    } else if (prec == TM_INT4) {
      cs *= a.ks4[kblk];
      vsc = a.vs4[kblk];
    }
    float s[4][4];
    const bool tailblk = j * kBlock + kBlock > L;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = acc[kb][i] * cs;
        if (tailblk && j * kBlock + dsigma(kb, 4 * g + i) >= L) x = -INFINITY;
        s[kb][i] = x;
      }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
    m_run = mn;
    float ps = 0.0f;
    f16x8 pb[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[kb][i] - mn);
        ps += p;
        pb[kb >> 1][4 * (kb & 1) + i] = static_cast<_Float16>(p);
      }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
      t = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[db][0], pb[0], t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[db][1], pb[1], t, 0, 0, 0);
      oacc[db] = oacc[db] * alpha + t * vsc;
    }
  }

  // ---- merge the 4 waves, write the chunk's partial (m, l, O) per query head
  __shared__ float sm[4][16], sl[4][16];
  __shared__ float so[4][16][D + 1];
  float lt = l_run + __shfl_xor(l_run, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (g == 0) {
    sm[w][l16] = m_run;
    sl[w][l16] = lt;
  }
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) so[w][l16][db * 16 + 4 * g + i] = oacc[db][i];
  __syncthreads();
  for (int x = tid; x < grp * D; x += 256) {
    const int qh = x / D, dv = x % D;
    float M = fmaxf(fmaxf(sm[0][qh], sm[1][qh]), fmaxf(sm[2][qh], sm[3][qh]));
    float lsum = 0.0f, ov = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = __builtin_amdgcn_exp2f(sm[ww][qh] - M);
      lsum += sl[ww][qh] * f;
      ov += so[ww][qh][dv] * f;
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
