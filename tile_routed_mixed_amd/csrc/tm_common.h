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
  // hybrid policies: window (tokens), gathered tiles, table offsets (bytes)
  uint32_t window, n_gtiles, sel_tab_off, sel_idx_off, cm_off, gh_off, gk_off, gv_off;
  uint32_t pad[8];
  int64_t census[8];  // legal, int8, int4, fp16, skip
  int64_t pad2[8];
};
static_assert(sizeof(TravHeader) == TM_TRAV_HEADER_BYTES, "traversal header size");

struct SeqEntry { uint32_t tok_start, len, blk_start, nq; };
struct ItemEntry { uint32_t seq, head, qtile, nruns, n8, n4, n16, nskip; };
struct RunEntry { uint32_t ktile, count_prec; };
// hybrid: one per (sequence, query head) list; one header per gathered tile
struct SelEntry { uint32_t start, count, gbase, cm_base; };
struct GatherEntry { uint32_t tok_start, blk_start, kv, keys; };
constexpr int kGatherHdr = 512;     // bytes per gathered tile header: entry + int32[64] positions
// hybrid run precisions: the compute precision in bits 0-1, edge and gathered flags
constexpr uint32_t kRunEdge = 4u, kRunGather = 8u;

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

// A widened 16-bit input as fp16, saturated: a bf16 value beyond the fp16
// range takes the nearest finite fp16 value (+-65504) instead of becoming
// infinite; NaN stays NaN (its comparison is false).  Every fp16 copy of a
// 16-bit input (the V^T copy, decode's q and FP16-window operands) goes
// through it.
__device__ __forceinline__ _Float16 to_f16_sat(float x) {
  return static_cast<_Float16>(__builtin_fabsf(x) > 65504.0f ? __builtin_copysignf(65504.0f, x) : x);
}

// s_waitcnt vmcnt(n) with the other counters left alone (n <= 15).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
    case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
    case 15: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

// 16-byte buffer load of each lane straight into LDS: lane L's bytes land at
// dst + 16 L (dst is wave-uniform); the source is rs at voff (per lane) + soff.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, void* dst, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)   // (the host pass never runs device bodies)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst), 16, voff, soff, 0, 0);
#endif
}

// A uniform pointer pinned in scalar registers: the empty asm hides where it
// came from, so the compiler keeps it instead of reloading it from the kernel
// arguments (and waiting on that load) inside a loop.
template <typename T>
__device__ __forceinline__ T* pin_sgpr(T* p) {
  asm volatile("" : "+s"(p));
  return p;
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads it
// does not wait for outstanding global or LDS-DMA loads (callers wait for the
// loads they need with wait_vm first), so deeper load pipelines survive it.
// (The barrier is written as inline asm because the compiler puts a full
// s_waitcnt in front of every s_barrier it emits on this target.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Scalar (constant address space) load of a uniform float: counted by
// lgkmcnt, so the vector-memory counts of tile copies stay exact.
__device__ __forceinline__ float sload(const float* p, size_t i) {
  typedef const __attribute__((address_space(4))) float cfloat;
  return ((cfloat*)(p))[i];
}

// The same for a uniform 64-bit word.
__device__ __forceinline__ uint64_t sload64(const uint64_t* p, size_t i) {
  typedef const __attribute__((address_space(4))) uint64_t cu64;
  return ((cu64*)(p))[i];
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
