// Quantize/pack kernel: symmetric per-(head, 64-token block) scales, INT8 codes,
// INT4 nibble-packed codes, and (transposed layout) an fp16 copy of the block.
//
// [TriAttention] "TriAttention: Unified Sparse Mixed-Precision Attention for
// Long-Context LLM Inference", abstract: keys and values are quantized during
// prefill and reused as the compressed decode cache; QK tiles run at 4 or 8
// bits.  The pages give no formula; the library defines the symmetric block
// quantizer documented in include/tm.h (binary32 division, round half to even).
//
// One workgroup (256 threads) per (block, head).  The pass is HBM-bound: each
// input element is read once (2 B) and its codes written once (1.5 B, plus 2 B
// for the fp16 copy in the transposed layout).
#include "tm_kernels.h"

namespace tmx {


__device__ __forceinline__ int8_t quant_code(float x, float s, float qmax) {
  if (!(s > 0.0f)) return 0;
  float c = __builtin_rintf(__fdiv_rn(x, s));   // IEEE division, round half to even
  c = fminf(fmaxf(c, -qmax), qmax);
  return static_cast<int8_t>(c);
}

// The same code from y = RN(1/s), with the IEEE division only near an edge.
// q0 = RN(x y) is within |x/s| (2^-23 + 2^-48) of x/s.  When q0 lies more
// than |q0| 2^-20 + 2^-22 inside the half-integer edges around c = rint(q0),
// x/s lies farther than 2^-24 (|x/s| + 1) inside them, more than half an ulp
// of either edge, so the IEEE quotient RN(x/s) stays strictly between the
// edges and its code is c as well.  The caller passes base = 0.5 - 2^-22 and
// y = RN(1/s) for s >= 2^-100 (normal, and the residual argument holds), else
// base = -1, which sends every element to quant_code.
__device__ __forceinline__ int8_t quant_code_recip(float x, float s, float y, float base, float qmax) {
  const float q0 = x * y;
  const float c = __builtin_rintf(q0);
  const float t = __builtin_fmaf(-fabsf(q0), 0x1p-20f, base);
  if (!(fabsf(q0 - c) <= t)) return quant_code(x, s, qmax);
  return static_cast<int8_t>(fminf(fmaxf(c, -qmax), qmax));
}

// Quantize cache block b (global index) of head h: its first token is row
// tok_first of x, and its first nvalid rows are valid (the rest count as 0).
template <int D, bool BF16, bool COLS>
__device__ __forceinline__ void quant_block(const QuantArgs& a, int b, int h, size_t tok_first, int nvalid) {
  constexpr int EPT = D / 4;            // elements per thread (one quarter row)
  const int tid = threadIdx.x;
  const int row = tid >> 2;
  const int col0 = (tid & 3) * EPT;

  float xv[EPT];
  if (row < nvalid) {
    const size_t tok = tok_first + row;
    const uint16_t* src = a.x + (tok * a.heads + h) * D + col0;
#pragma unroll
    for (int v = 0; v < EPT / 8; ++v) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(src + v * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = raw[e];
        const uint16_t lo = static_cast<uint16_t>(w & 0xFFFFu), hi = static_cast<uint16_t>(w >> 16);
        xv[v * 8 + 2 * e] = BF16 ? bf16_bits_to_f32(lo) : f16_bits_to_f32(lo);
        xv[v * 8 + 2 * e + 1] = BF16 ? bf16_bits_to_f32(hi) : f16_bits_to_f32(hi);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) xv[e] = 0.0f;
  }

  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) am = fmaxf(am, fabsf(xv[e]));
  am = wave_max(am);
  __shared__ float red[4];
  if ((tid & 63) == 0) red[tid >> 6] = am;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc8 = __fdiv_rn(amax, 127.0f);
  const float sc4 = __fdiv_rn(amax, 7.0f);
  const size_t blk = static_cast<size_t>(b) * a.heads + h;   // block-major: [nblk][heads]
  if (tid == 0) {
    a.s8[blk] = sc8;
    a.s4[blk] = sc4;
  }

  const bool f8 = sc8 >= 0x1p-100f, f4 = sc4 >= 0x1p-100f;   // (false for a zero scale)
  const float y8 = f8 ? __fdiv_rn(1.0f, sc8) : 0.0f, y4 = f4 ? __fdiv_rn(1.0f, sc4) : 0.0f;
  const float base8 = f8 ? 0.5f - 0x1p-22f : -1.0f, base4 = f4 ? 0.5f - 0x1p-22f : -1.0f;
  int8_t c8v[EPT], c4v[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    c8v[e] = quant_code_recip(xv[e], sc8, y8, base8, 127.0f);
    c4v[e] = quant_code_recip(xv[e], sc4, y4, base4, 7.0f);
  }

  if constexpr (!COLS) {
    // rows layout: c8 [nblk][heads][64][D], c4 [nblk][heads][64][D/2]
    int8_t* d8 = a.c8 + (blk * kBlock + row) * D + col0;
#pragma unroll
    for (int v = 0; v < EPT / 16; ++v) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int o = v * 16 + e * 4;
        pk[e] = (static_cast<uint32_t>(static_cast<uint8_t>(c8v[o]))) |
                (static_cast<uint32_t>(static_cast<uint8_t>(c8v[o + 1])) << 8) |
                (static_cast<uint32_t>(static_cast<uint8_t>(c8v[o + 2])) << 16) |
                (static_cast<uint32_t>(static_cast<uint8_t>(c8v[o + 3])) << 24);
      }
      *reinterpret_cast<u32x4*>(d8 + v * 16) = pk;
    }
    if (a.c4x != nullptr) {   // the INT4 codes again, one per byte, in the INT8 codes' layout
      int8_t* dx = a.c4x + (blk * kBlock + row) * D + col0;
#pragma unroll
      for (int v = 0; v < EPT / 16; ++v) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int o = v * 16 + e * 4;
          pk[e] = (static_cast<uint32_t>(static_cast<uint8_t>(c4v[o]))) |
                  (static_cast<uint32_t>(static_cast<uint8_t>(c4v[o + 1])) << 8) |
                  (static_cast<uint32_t>(static_cast<uint8_t>(c4v[o + 2])) << 16) |
                  (static_cast<uint32_t>(static_cast<uint8_t>(c4v[o + 3])) << 24);
        }
        *reinterpret_cast<u32x4*>(dx + v * 16) = pk;
      }
    }
    uint8_t* d4 = a.c4 + (blk * kBlock + row) * (D / 2) + col0 / 2;
#pragma unroll
    for (int v = 0; v < EPT / 16; ++v) {
      u32x2 pk;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        uint32_t wv = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int o = v * 16 + e * 8 + 2 * t;
          const uint32_t byte = (static_cast<uint32_t>(c4v[o]) & 0xFu) |
                                ((static_cast<uint32_t>(c4v[o + 1]) & 0xFu) << 4);
          wv |= byte << (8 * t);
        }
        pk[e] = wv;
      }
      *reinterpret_cast<u32x2*>(d4 + v * 8) = pk;
    }
  } else {
    // transposed layout: stage the block in LDS, then write columns.
    __shared__ int8_t s_c8[kBlock][D + 4];
    __shared__ int8_t s_c4[kBlock][D + 4];
    __shared__ _Float16 s_h[kBlock][D + 2];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      s_c8[row][col0 + e] = c8v[e];
      s_c4[row][col0 + e] = c4v[e];
      s_h[row][col0 + e] = to_f16_sat(xv[e]);
    }
    __syncthreads();
    constexpr int TPR = 256 / D;          // threads per output row (channel)
    constexpr int TOK = kBlock / TPR;     // tokens per thread: 32 (D=128) or 16 (D=64)
    const int ch = tid / TPR;
    const int t0 = (tid % TPR) * TOK;
    int8_t* d8 = a.c8 + (blk * D + ch) * kBlock + t0;
#pragma unroll
    for (int v = 0; v < TOK / 16; ++v) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t wv = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          wv |= static_cast<uint32_t>(static_cast<uint8_t>(s_c8[t0 + v * 16 + e * 4 + t][ch])) << (8 * t);
        pk[e] = wv;
      }
      *reinterpret_cast<u32x4*>(d8 + v * 16) = pk;
    }
    uint8_t* d4 = a.c4 + (blk * D + ch) * (kBlock / 2) + t0 / 2;
#pragma unroll
    for (int v = 0; v < TOK / 16; ++v) {
      u32x2 pk;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        uint32_t wv = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int tok = t0 + v * 16 + e * 8 + 2 * t;
          const uint32_t byte = (static_cast<uint32_t>(s_c4[tok][ch]) & 0xFu) |
                                ((static_cast<uint32_t>(s_c4[tok + 1][ch]) & 0xFu) << 4);
          wv |= byte << (8 * t);
        }
        pk[e] = wv;
      }
      *reinterpret_cast<u32x2*>(d4 + v * 8) = pk;
    }
    if (a.t16 != nullptr) {
      uint16_t* dh = a.t16 + (blk * D + ch) * kBlock + t0;
#pragma unroll
      for (int v = 0; v < TOK / 8; ++v) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          _Float16 lo = s_h[t0 + v * 8 + 2 * e][ch], hi = s_h[t0 + v * 8 + 2 * e + 1][ch];
          uint16_t lb16, hb16;
          __builtin_memcpy(&lb16, &lo, 2);
          __builtin_memcpy(&hb16, &hi, 2);
          pk[e] = static_cast<uint32_t>(lb16) | (static_cast<uint32_t>(hb16) << 16);
        }
        *reinterpret_cast<u32x4*>(dh + v * 8) = pk;
      }
    }
  }
}

template <int D, bool BF16, bool COLS>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
  const int b = blockIdx.x, h = blockIdx.y;
  const SeqOfBlock so = find_block_seq(a.cu, a.nseq, b);
  const int lb = b - so.blk_start;
  quant_block<D, BF16, COLS>(a, b, h, static_cast<size_t>(so.tok_start) + lb * kBlock,
                             min(kBlock, so.len - lb * kBlock));
}

// Cache append: workgroup (i, h) re-quantizes the block that holds sequence
// i's newest token, over the sequence's current length (codes and scales of
// a partial block cover its valid rows, as tm_quantize_pack would).
template <int D, bool BF16, bool COLS>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs p) {
  const int i = blockIdx.x, h = blockIdx.y;
  quant_block<D, BF16, COLS>(p.q, p.blk[i], h, static_cast<size_t>(p.tok[i]), p.nvalid[i]);
}

template <int D, bool BF16, bool COLS>
static hipError_t launch_append_t(const AppendArgs& p, hipStream_t st) {
  hipLaunchKernelGGL((append_kernel<D, BF16, COLS>), dim3(p.n, p.q.heads), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& p, int d, bool bf16, bool cols, hipStream_t st) {
  if (p.n == 0) return hipSuccess;
  if (d == 128) {
    if (bf16) return cols ? launch_append_t<128, true, true>(p, st) : launch_append_t<128, true, false>(p, st);
    return cols ? launch_append_t<128, false, true>(p, st) : launch_append_t<128, false, false>(p, st);
  }
  if (bf16) return cols ? launch_append_t<64, true, true>(p, st) : launch_append_t<64, true, false>(p, st);
  return cols ? launch_append_t<64, false, true>(p, st) : launch_append_t<64, false, false>(p, st);
}

template <int D, bool BF16, bool COLS>
static hipError_t launch_quant_t(const QuantArgs& a, hipStream_t st) {
  dim3 grid(static_cast<unsigned>(a.nblk), static_cast<unsigned>(a.heads));
  hipLaunchKernelGGL((quantize_kernel<D, BF16, COLS>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, int d, bool bf16, bool cols, hipStream_t st) {
  if (a.nblk == 0) return hipSuccess;
  if (d == 128) {
    if (bf16) return cols ? launch_quant_t<128, true, true>(a, st) : launch_quant_t<128, true, false>(a, st);
    return cols ? launch_quant_t<128, false, true>(a, st) : launch_quant_t<128, false, false>(a, st);
  }
  if (bf16) return cols ? launch_quant_t<64, true, true>(a, st) : launch_quant_t<64, true, false>(a, st);
  return cols ? launch_quant_t<64, false, true>(a, st) : launch_quant_t<64, false, false>(a, st);
}

}  // namespace tmx
