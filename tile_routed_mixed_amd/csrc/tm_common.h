// Internal definitions shared by the HIP sources of libtm (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tm.h"

namespace tmx {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kBlock = 64;            // quantization block = key tile (tokens)
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;   // finite "minus infinity" for running maxima

// Traversal header field offsets (bytes), mirrored in include/tm.h.
struct TravHeader {
  uint32_t magic, version, kind, n_items, max_runs, nseq, hq, hkv, bq, bk, d, nblk;
  uint32_t seq_off, item_off, run_off, bits_off;
  uint32_t pad[16];
  int64_t census[8];  // legal, int8, int4, fp16, skip
  int64_t pad2[8];
};
static_assert(sizeof(TravHeader) == TM_TRAV_HEADER_BYTES, "traversal header size");

struct SeqEntry { uint32_t tok_start, len, blk_start, nq; };
struct ItemEntry { uint32_t seq, head, qtile, nruns, n8, n4, n16, nskip; };
struct RunEntry { uint32_t ktile, count_prec; };

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return static_cast<float>(h);
}

// Wave-wide reductions over 64 lanes.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// First block index and block count of sequence `s`, and the sequence that
// owns global block `b`, from cu_seqlens on the device.  One wave scans 64
// sequences per step with a lane prefix sum.
struct SeqOfBlock { int seq, blk_start, tok_start, len; };

__device__ inline SeqOfBlock find_block_seq(const int32_t* __restrict__ cu, int nseq, int b) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int s0 = 0; s0 < nseq; s0 += 64) {
    const int s = s0 + lane;
    int nb = 0, st = 0, ln = 0;
    if (s < nseq) {
      st = cu[s];
      ln = cu[s + 1] - st;
      nb = (ln + kBlock - 1) / kBlock;
    }
    int incl = nb;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    const int excl = incl - nb;
    const bool hit = (s < nseq) && (b >= base + excl) && (b < base + incl);
    const unsigned long long m = __ballot(hit);
    if (m) {
      const int src = __ffsll(static_cast<long long>(m)) - 1;
      SeqOfBlock r;
      r.seq = s0 + src;
      r.blk_start = base + __shfl(excl, src, 64);
      r.tok_start = __shfl(st, src, 64);
      r.len = __shfl(ln, src, 64);
      return r;
    }
    base += __shfl(incl, 63, 64);
  }
  SeqOfBlock r{-1, 0, 0, 0};
  return r;
}

// Block start of sequence `seq` (sum of ceil(len/64) over earlier sequences).
__device__ inline int seq_blk_start(const int32_t* __restrict__ cu, int seq) {
  const int lane = threadIdx.x & 63;
  int acc = 0;
  for (int s0 = 0; s0 < seq; s0 += 64) {
    const int s = s0 + lane;
    int nb = 0;
    if (s < seq) nb = (cu[s + 1] - cu[s] + kBlock - 1) / kBlock;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) nb += __shfl_xor(nb, o, 64);
    acc += nb;
  }
  return acc;
}

}  // namespace tmx
