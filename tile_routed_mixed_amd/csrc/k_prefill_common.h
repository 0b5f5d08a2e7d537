// Pieces shared by the prefill kernels (gfx950): the key order inside a tile,
// the LDS swizzle, the direct-to-LDS tile copy, lane-group maxima and the
// XCD-aware workgroup order.
#pragma once

#include "tm_kernels.h"

namespace tmx {

// Key row (0..63) of a 64-key tile that feeds row m of 16-key MFMA block kb.
__device__ __forceinline__ int sigma(int kb, int m) {
  return 32 * (kb >> 1) + 8 * (m >> 2) + 4 * (kb & 1) + (m & 3);
}

// sigma(kb, m) - sigma(0, m): the part of the key row that depends on kb only.
__host__ __device__ constexpr int krow(int kb) { return 32 * (kb >> 1) + 4 * (kb & 1); }

// Swizzle key of a row for a tile whose rows hold NCH 16-byte chunks: rows read
// together by 8 lanes (sigma rows base+{0..3, 8..11} for K, consecutive rows
// for V^T) land in distinct chunk columns.
template <int NCH, bool VT>
__device__ __forceinline__ int swz(int row) {
  if constexpr (VT) return row & (NCH - 1) & 7;
  if constexpr (NCH >= 8) return (row & 3) | (((row >> 3) & 1) << 2);
  if constexpr (NCH == 4) return ((row >> 1) & 1) | (((row >> 3) & 1) << 1);
  return (row >> 1) & 1;
}

// Byte offset in LDS of 16-byte chunk c of row `row` (rows of NCH chunks).
template <int NCH, bool VT>
__device__ __forceinline__ int lds_off(int row, int c) {
  return row * NCH * 16 + ((c ^ swz<NCH, VT>(row)) << 4);
}

// 8 packed INT4 codes (one dword) -> two dwords of int8 holding 16 * code.
__device__ __forceinline__ i32x4 widen_nibbles(uint32_t p0, uint32_t p1) {
  i32x4 r;
  r[0] = static_cast<int>((p0 << 4) & 0xF0F0F0F0u);
  r[1] = static_cast<int>(p0 & 0xF0F0F0F0u);
  r[2] = static_cast<int>((p1 << 4) & 0xF0F0F0F0u);
  r[3] = static_cast<int>(p1 & 0xF0F0F0F0u);
  return r;
}

// max over the 4 lanes {l, l^16, l^32, l^48} (the lane groups of one row).
__device__ __forceinline__ float max4(float v) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// the same for int32 values
__device__ __forceinline__ int max4i(int v) {
  const auto s = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v), false, false);
  const int m = max(static_cast<int>(s[0]), static_cast<int>(s[1]));
  const auto r = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(m), static_cast<uint32_t>(m), false, false);
  return max(static_cast<int>(r[0]), static_cast<int>(r[1]));
}

__device__ __forceinline__ uint32_t remap_block(uint32_t b, uint32_t n) {
  constexpr uint32_t kXcd = 8, kGroup = 4, kChunk = kXcd * kGroup;
  const uint32_t full = (n / kChunk) * kChunk;
  if (b >= full) return b;
  const uint32_t c = b / kChunk, r = b % kChunk;
  return c * kChunk + (r % kXcd) * kGroup + r / kXcd;
}

// Per-lane layout of a direct-to-LDS tile copy: a region of ROWS rows x NCH
// 16-byte chunks is moved by ROWS*NCH/64 buffer loads of 1 KiB; load n fills
// LDS bytes [n*1024, n*1024+1024) and lane L lands at n*1024 + 16L, which is
// row (n*1024 + 16L) / (16 NCH), swizzled slot L mod NCH, i.e. it must fetch
// logical chunk slot ^ swz(row).  Wave w issues loads n = 4i + w.  The lane's
// source offset inside a tile is fixed for the whole item; the tile's own
// offset goes in the scalar offset of the load.
template <int ROWS, int NCH, bool VT>
struct TileCopy {
  static constexpr int NI = ROWS * NCH / 64;
  static constexpr int PER = NI >= 4 ? NI / 4 : 1;
  static_assert(NI < 4 || NI % 4 == 0, "tile regions are whole multiples of 4 KiB");
  uint32_t voff[PER];
  __device__ __forceinline__ void init(int w, int lane, uint32_t pitch) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int n = i * 4 + w;
      const int off = n * 1024 + lane * 16;
      const int r = off / (NCH * 16);
      const int slot = (off / 16) % NCH;
      voff[i] = static_cast<uint32_t>(r) * pitch + static_cast<uint32_t>((slot ^ swz<NCH, VT>(r)) * 16);
    }
  }
  // tile at byte `soff` of `rs` -> LDS [dst, dst + ROWS * NCH * 16)
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, uint32_t soff, uint8_t* dst, int w) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (NI < 4 && w >= NI) break;
      lds_dma16(rs, dst + (i * 4 + w) * 1024, voff[i], soff);
    }
  }
};

// sum over the 4 lanes {l, l^16, l^32, l^48}
__device__ __forceinline__ float sum4(float v) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace tmx
