// Vertical-line token selection for the hybrid policies.
//
// [HyQuant] "HyQuant Uses Hybrid Precision to Compress LLM Attention",
// sections "The observation behind the method" and "How HyQuant works": a
// small set of key positions is attended by many queries (vertical lines in
// the attention map), and a lightweight pass over attention-pattern signals
// picks those tokens to keep in FP16.  The signal here is the attention mass
// each key receives from the last n_obs query rows of its sequence (16-bit
// scores, fp32 arithmetic); the k keys of largest mass are selected.
//
// Passes 1 and 3 run one workgroup per (run of key tiles of 64, sequence, KV
// head, up to 4 of its query heads): the query heads of a KV head share each
// key tile, staged once through LDS.  The probe scores come from the matrix
// cores (recomputed in pass 3, cheaper than storing them):
//   1. probe scores of the tile's keys -> per probe row a partial (max, sum);
//   2. (one workgroup per (sequence, head)) partials -> each row's (m, l);
//   3. probe scores again -> mass of each key, sum over the probe rows of
//      exp(s - m) / l.
// Then a top-k pass per list: an MSB-first radix select on the (non-negative)
// float bits finds the k-th largest mass; keys above it, and the lowest
// positions among those equal to it, are written in ascending order.  Masses
// are stored head-major ([hq][T]): pass 3 stores a tile's 64 keys in one
// coalesced write and a list's keys are contiguous for the top-k.
#include "tm_kernels.h"

namespace tmx {

constexpr int kProbe = 64;   // most probe rows per sequence

struct ProbeSeq {
  int tok0, len, nobs, r0;
};

__device__ __forceinline__ ProbeSeq probe_seq(const SelectArgs& a, int b) {
  ProbeSeq p;
  p.tok0 = a.cu[b];
  p.len = a.cu[b + 1] - p.tok0;
  p.nobs = min(a.n_obs, p.len);
  p.r0 = p.len - p.nobs;
  return p;
}

// Work split of passes 1 and 3.  A workgroup of 4 waves takes QB query heads
// of one KV head (they share its keys) and a.tw consecutive key tiles of one
// sequence; each wave computes QB blocks of 16 probe rows of one head, so a
// head's 64 probe rows span 4 / QB waves.  Each key tile is staged once
// through LDS for all the waves, double-buffered: the next tile's loads are
// in flight while the current one is multiplied.
constexpr int kProbeThreads = 256;

template <int D>
struct KTile {
  static constexpr int PITCH = 2 * D + 16;               // bytes per key row: the padding puts the
                                                          // 16 rows of an operand read in distinct banks
  static constexpr int CPR = D / 8;                      // 16-byte chunks per row
  static constexpr int PER = 64 * CPR / kProbeThreads;   // chunks per thread
  static constexpr int BYTES = 64 * PITCH;
};

// loads of key tile j (keys past the sequence end read as zeros)
template <int D>
__device__ __forceinline__ void ktile_load(const SelectArgs& a, const ProbeSeq& ps, int kv, int j,
                                           u32x4 (&r)[KTile<D>::PER]) {
#pragma unroll
  for (int u = 0; u < KTile<D>::PER; ++u) {
    const int i = static_cast<int>(threadIdx.x) + kProbeThreads * u;
    const int row = i / KTile<D>::CPR, col = i % KTile<D>::CPR, key = j * kBlock + row;
    r[u] = u32x4{0u, 0u, 0u, 0u};
    if (key < ps.len)
      r[u] = *reinterpret_cast<const u32x4*>(a.k + (static_cast<size_t>(ps.tok0 + key) * a.hkv + kv) * D + 8 * col);
  }
}

template <int D>
__device__ __forceinline__ void ktile_store(uint8_t* buf, const u32x4 (&r)[KTile<D>::PER]) {
#pragma unroll
  for (int u = 0; u < KTile<D>::PER; ++u) {
    const int i = static_cast<int>(threadIdx.x) + kProbeThreads * u;
    *reinterpret_cast<u32x4*>(buf + (i / KTile<D>::CPR) * KTile<D>::PITCH + 16 * (i % KTile<D>::CPR)) = r[u];
  }
}

// A wave's probe-row operands: rows 16 (qb0 + q) + l16, q < QB, of head h
// (rows past the probe are zeros), loaded once for all the wave's tiles.
template <int D, bool BF16, int QB>
struct ProbeQ {
  typedef typename std::conditional<BF16, bf16x8, f16x8>::type op_t;
  static constexpr int NC = D / 32;
  op_t q[QB][NC];
};

template <int D, bool BF16, int QB>
__device__ __forceinline__ void probe_q(const SelectArgs& a, const ProbeSeq& ps, int h, int qb0,
                                        ProbeQ<D, BF16, QB>& pq) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int row = 16 * (qb0 + q) + l16;
#pragma unroll
    for (int c = 0; c < ProbeQ<D, BF16, QB>::NC; ++c) {
      u32x4 raw = u32x4{0u, 0u, 0u, 0u};
      if (row < ps.nobs)
        raw = *reinterpret_cast<const u32x4*>(a.q + (static_cast<size_t>(ps.tok0 + ps.r0 + row) * a.hq + h) * D +
                                              32 * c + 8 * g);
      __builtin_memcpy(&pq.q[q][c], &raw, 16);
    }
  }
}

// One wave's raw probe products (no scale, no mask) with the staged key tile,
// on the matrix cores (v_mfma_f32_16x16x32_{f16,bf16}).  The same registers
// serve as either operand, so the product comes in either orientation:
//   TRANS: S^T = K Q^T, lane (l16, g) holds probe row 16 (qb0 + q) + l16 and
//          keys 16 kb + 4 g + i in s[kb][q][i] (a row's keys in the lane: row
//          statistics reduce in registers);
//   else:  S = Q K^T, lane (l16, g) holds key 16 kb + l16 and probe rows
//          16 (qb0 + q) + 4 g + i (a key's rows in the lane: column sums
//          reduce in registers).
template <int D, bool BF16, int QB, bool TRANS>
__device__ __forceinline__ void probe_raw(const uint8_t* buf, const ProbeQ<D, BF16, QB>& pq, f32x4 (&s)[4][QB]) {
  typedef typename ProbeQ<D, BF16, QB>::op_t op_t;
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int q = 0; q < QB; ++q) s[kb][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the next block of 16 keys' operands is read from LDS while the current
  // block's products run
  constexpr int NC = ProbeQ<D, BF16, QB>::NC;
  const uint8_t* base = buf + l16 * KTile<D>::PITCH + 16 * g;
  u32x4 kr[2][NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) kr[0][c] = *reinterpret_cast<const u32x4*>(base + 64 * c);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    if (kb + 1 < 4) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kr[(kb + 1) & 1][c] = *reinterpret_cast<const u32x4*>(base + 16 * (kb + 1) * KTile<D>::PITCH + 64 * c);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      op_t kop;
      __builtin_memcpy(&kop, &kr[kb & 1][c], 16);
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const op_t& x = TRANS ? kop : pq.q[q][c];
        const op_t& y = TRANS ? pq.q[q][c] : kop;
        if constexpr (BF16) s[kb][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, s[kb][q], 0, 0, 0);
        else s[kb][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, s[kb][q], 0, 0, 0);
      }
    }
  }
}

// A key tile needs the (row, key) mask when some of its keys lie after the
// first probe row or past the sequence end, or the probe is shorter than 64
// rows; the other tiles are whole for every probe row.
__device__ __forceinline__ bool probe_tile_masked(const ProbeSeq& ps, int j) {
  return j * kBlock + kBlock - 1 > ps.r0 || j * kBlock + kBlock > ps.len || ps.nobs < kProbe;
}

// max and sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (one row's lane groups)
__device__ __forceinline__ float probe_max4(float v) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float probe_sum4(float v) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// sum of the QB per-row-block partial sums, as a tree
template <int QB>
__device__ __forceinline__ float probe_tree(const float (&x)[QB]) {
  if constexpr (QB == 4) return (x[0] + x[1]) + (x[2] + x[3]);
  else if constexpr (QB == 2) return x[0] + x[1];
  else return x[0];
}

// The workgroup's place: sequence b, KV head kv, the wave's head h and first
// row block qb0, its tiles [j0, jn).  Returns false for a workgroup past the
// sequence's tiles.
struct ProbeWork {
  int b, kv, h, qb0, j0, jn;
  ProbeSeq ps;
};
template <int QB>
__device__ __forceinline__ bool probe_work(const SelectArgs& a, ProbeWork& pw) {
  const int grp = a.hq / a.hkv, wph = 4 / QB, w = threadIdx.x >> 6;
  pw.b = blockIdx.z;
  pw.kv = blockIdx.y / (grp / QB);
  pw.h = pw.kv * grp + (blockIdx.y % (grp / QB)) * QB + w / wph;
  pw.qb0 = (w % wph) * QB;
  pw.ps = probe_seq(a, pw.b);
  pw.j0 = blockIdx.x * a.tw;
  pw.jn = min(pw.j0 + a.tw, (pw.ps.len + kBlock - 1) / kBlock);
  return pw.j0 < pw.jn;
}

// pass 1: per (row, tile) partial max and sum (log2 units), from S^T
template <int D, bool BF16, int QB>
__global__ __launch_bounds__(kProbeThreads, 2) void probe_partial_kernel(SelectArgs a) {
  ProbeWork pw;
  if (!probe_work<QB>(a, pw)) return;   // whole workgroup
  const ProbeSeq& ps = pw.ps;
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][KTile<D>::BYTES];
  // the probe rows' loads go first: the wait before the first tile's LDS
  // store then covers them, and no load in the loop waits behind them
  ProbeQ<D, BF16, QB> pq;
  probe_q<D, BF16, QB>(a, ps, pw.h, pw.qb0, pq);
  u32x4 pre[KTile<D>::PER];
  ktile_load<D>(a, ps, pw.kv, pw.j0, pre);
  ktile_store<D>(kbuf[0], pre);
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
  const float tau = a.tau_log2e;
  // (uniform: kept in scalar registers, so no vector load in the loop waits
  // on the next tile's loads)
  const int tile0 = __builtin_amdgcn_readfirstlane(sel_tab(a, 0, pw.b));
  for (int j = pw.j0; j < pw.jn; ++j) {
    __syncthreads();   // tile j staged; every wave is done with the other buffer
    const bool more = j + 1 < pw.jn;
    if (more) ktile_load<D>(a, ps, pw.kv, j + 1, pre);
    f32x4 s[4][QB];
    probe_raw<D, BF16, QB, true>(kbuf[(j - pw.j0) & 1], pq, s);
    if (probe_tile_masked(ps, j)) {
      // (an opaque statement keeps this a branch taken by the few boundary
      // tiles, instead of selects executed on every tile)
      __asm__ volatile("");
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int q = 0; q < QB; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * (pw.qb0 + q) + l16, key = j * kBlock + 16 * kb + 4 * g + i;
            if (!(row < ps.nobs && key <= ps.r0 + row && key < ps.len)) s[kb][q][i] = -INFINITY;
          }
    }
    float* dst = a.part + ((static_cast<size_t>(tile0) + j) * a.hq + pw.h) * (2 * kProbe);
    // row 16 (qb0 + q) + l16: 16 products in the lane, the rest in lanes
    // l16 + 16, 32, 48.  The row blocks are independent (no branch between
    // them) and each sum runs in 4 partial chains, for instruction-level
    // parallelism.
    float mrow[QB], lrow[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      float m4[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) m4[kb] = fmaxf(fmaxf(s[kb][q][0], s[kb][q][1]), fmaxf(s[kb][q][2], s[kb][q][3]));
      mrow[q] = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) mrow[q] = probe_max4(mrow[q]) * tau;   // (tau > 0: the maximum of the scaled scores)
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      // a row with no visible key (-inf) sums exp2(-inf) = 0 against offset 0
      const float off = mrow[q] > -INFINITY ? -mrow[q] : 0.0f;
      float l4[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        l4[kb] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][q][0], tau, off));
#pragma unroll
        for (int i = 1; i < 4; ++i) l4[kb] += __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][q][i], tau, off));
      }
      lrow[q] = (l4[0] + l4[1]) + (l4[2] + l4[3]);
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) lrow[q] = probe_sum4(lrow[q]);
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int row = 16 * (pw.qb0 + q) + l16;
      if (lane < 16 && row < ps.nobs) {
        dst[2 * row] = mrow[q];
        dst[2 * row + 1] = lrow[q];
      }
    }
    if (more) ktile_store<D>(kbuf[(j + 1 - pw.j0) & 1], pre);
  }
}

// pass 2: each probe row's (m, l) over all tiles; thread (row, q) merges the
// tiles q, q + 16, ..., then the 16 parts are merged through LDS.  Stored as
// (m, log2 l), the pair pass 3 subtracts.
constexpr int kRowParts = 16;
__global__ __launch_bounds__(64 * kRowParts) void probe_rows_kernel(SelectArgs a) {
  const int b = blockIdx.y, h = blockIdx.x;
  const int r = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int len = a.cu[b + 1] - a.cu[b];
  const int nt = (len + kBlock - 1) / kBlock;
  const float* base = a.part + (static_cast<size_t>(sel_tab(a, 0, b)) * a.hq + h) * (2 * kProbe) + 2 * r;
  const size_t tstride = static_cast<size_t>(a.hq) * (2 * kProbe);
  float M = -INFINITY, L = 0.0f;
  auto merge = [&](float m, float l) {
    if (!(m > -INFINITY)) return;   // (rows past the probe, and tiles after the row, stay -inf)
    const float mn = fmaxf(M, m);
    L = L * __builtin_amdgcn_exp2f(M - mn) + l * __builtin_amdgcn_exp2f(m - mn);
    M = mn;
  };
  int j = q;
  for (; j + 3 * kRowParts < nt; j += 4 * kRowParts) {   // four loads in flight
    float2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float2*>(base + (j + u * kRowParts) * tstride);
#pragma unroll
    for (int u = 0; u < 4; ++u) merge(v[u].x, v[u].y);
  }
  for (; j < nt; j += kRowParts) {
    const float2 v = *reinterpret_cast<const float2*>(base + j * tstride);
    merge(v.x, v.y);
  }
  __shared__ float sm[kRowParts][64], sl[kRowParts][64];
  sm[q][r] = M;
  sl[q][r] = L;
  __syncthreads();
  if (q == 0) {
    M = -INFINITY;
    L = 0.0f;
#pragma unroll
    for (int u = 0; u < kRowParts; ++u) merge(sm[u][r], sl[u][r]);
    float* dst = a.rows + (static_cast<size_t>(b) * a.hq + h) * (2 * kProbe) + 2 * r;
    dst[0] = M;
    dst[1] = M > -INFINITY ? __builtin_amdgcn_logf(L) : 0.0f;
  }
}

// pass 3: mass of each key of tile j, the sum over the probe rows of
// exp2(tau s - m - log2 l), from S = Q K^T: a lane holds one key's products
// with 4 QB of the rows, summed in registers, then over the 4 lane groups;
// with QB < 4 the 4 / QB waves of a head add their sums through LDS
template <int D, bool BF16, int QB>
__global__ __launch_bounds__(kProbeThreads, 2) void probe_mass_kernel(SelectArgs a) {
  ProbeWork pw;
  if (!probe_work<QB>(a, pw)) return;   // whole workgroup
  const ProbeSeq& ps = pw.ps;
  constexpr int wph = 4 / QB;
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][KTile<D>::BYTES];
  __shared__ float part[wph > 1 ? 4 : 1][64];
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4, w = threadIdx.x >> 6;
  // the lane's rows 16 (qb0 + q) + 4 g + i: bias -(m + log2 l), -inf past the probe
  float bias[QB][4];
  const float* st = a.rows + (static_cast<size_t>(pw.b) * a.hq + pw.h) * (2 * kProbe);
#pragma unroll
  for (int q = 0; q < QB; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * (pw.qb0 + q) + 4 * g + i;
      bias[q][i] = -INFINITY;
      if (row < ps.nobs) {
        const float2 ml = *reinterpret_cast<const float2*>(st + 2 * row);
        bias[q][i] = -(ml.x + ml.y);
      }
    }
  ProbeQ<D, BF16, QB> pq;
  probe_q<D, BF16, QB>(a, ps, pw.h, pw.qb0, pq);
  u32x4 pre[KTile<D>::PER];
  ktile_load<D>(a, ps, pw.kv, pw.j0, pre);
  ktile_store<D>(kbuf[0], pre);   // (the wait before it covers the loads above)
  const float tau = a.tau_log2e;
  for (int j = pw.j0; j < pw.jn; ++j) {
    __syncthreads();   // tile j staged; every wave is done with the other buffer and the sums
    const bool more = j + 1 < pw.jn;
    if (more) ktile_load<D>(a, ps, pw.kv, j + 1, pre);
    f32x4 s[4][QB];
    probe_raw<D, BF16, QB, false>(kbuf[(j - pw.j0) & 1], pq, s);
    float p[4];
    if (j * kBlock + kBlock - 1 > ps.r0) {
      // keys after the first probe row: row 16 (qb0 + q) + 4 g + i sees key c
      // when c <= r0 + row (rows past the probe have bias -inf)
      __asm__ volatile("");   // (a branch for the boundary tiles, as in pass 1)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int lim = j * kBlock + 16 * kb + l16 - ps.r0 - 4 * g - 16 * pw.qb0;   // visible: 16 q + i >= lim
        float acc[QB];
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          acc[q] = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][q][i], tau, bias[q][i]));
            acc[q] += 16 * q + i >= lim ? e : 0.0f;
          }
        }
        p[kb] = probe_tree<QB>(acc);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float acc[QB];
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          acc[q] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][q][0], tau, bias[q][0]));
#pragma unroll
          for (int i = 1; i < 4; ++i) acc[q] += __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][q][i], tau, bias[q][i]));
        }
        p[kb] = probe_tree<QB>(acc);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) p[kb] = probe_sum4(p[kb]);
    // every lane group holds the 64 sums; group g takes keys 16 g + l16
    float v = g == 0 ? p[0] : g == 1 ? p[1] : g == 2 ? p[2] : p[3];
    const int key = j * kBlock + 16 * g + l16;
    if constexpr (wph > 1) {
      part[w][lane] = v;
      __syncthreads();
      if (w % wph == 0) {
#pragma unroll
        for (int u = 1; u < wph; ++u) v += part[w + u][lane];
        if (key < ps.len) a.mass[static_cast<size_t>(pw.h) * a.T + ps.tok0 + key] = v;
      }
    } else {
      if (key < ps.len) a.mass[static_cast<size_t>(pw.h) * a.T + ps.tok0 + key] = v;
    }
    if (more) ktile_store<D>(kbuf[(j + 1 - pw.j0) & 1], pre);
  }
}

// Inclusive prefix sum over the 64 lanes of a wave, on the DPP cross-lane
// paths: shifts by 1, 2, 4, 8 lanes within each row of 16 (lanes whose source
// lies outside the row add 0), then the last lane of row 0 (row 2) is
// broadcast into row 1 (row 3), and lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31, rows 2 and 3
  return x;
}

// Block-wide exclusive prefix sums of two values per thread (NT threads);
// sets the totals.  Uses its LDS once per kernel.
template <int NT>
__device__ __forceinline__ int2 block_scan2(int x, int y, int2* total) {
  __shared__ int2 wtot[NT / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ix = wave_incl_scan(x), iy = wave_incl_scan(y);
  if (lane == 63) wtot[w] = make_int2(ix, iy);
  __syncthreads();
  int2 base = make_int2(0, 0), tot = make_int2(0, 0);
#pragma unroll
  for (int u = 0; u < NT / 64; ++u) {
    const int2 t = wtot[u];
    if (u < w) {
      base.x += t.x;
      base.y += t.y;
    }
    tot.x += t.x;
    tot.y += t.y;
  }
  *total = tot;
  return make_int2(base.x + ix - x, base.y + iy - y);
}

// top-k of one list, (sequence b, list head g): the mass of query head g, or
// the sum over KV head g's query heads.  Thread t owns the list positions
// [t per, (t + 1) per).  The k-th largest value is found by an MSB-first
// radix select on the float bits (non-negative, so the bits order as the
// values) in three digits: bits 30..20, 19..10, 9..0; each digit's histogram
// of the keys that match the digits found so far is built with LDS atomics,
// and wave 0 finds the digit where the count from the top reaches k.  Then
// the keys above the threshold and the lowest positions among those equal to
// it are written in ascending order.  PER > 0: lists of up to PER x 1024
// keys, held in registers; PER = 0: any length, re-read from global memory.
constexpr int kTopkThreads = 1024;
constexpr int kTopkPer = 12;
template <int PER>
__device__ __forceinline__ void topk_list(const SelectArgs& a, const float* src, int nsum, int len, int k,
                                          int32_t* out) {
  constexpr int NT = kTopkThreads;
  const int lane = threadIdx.x & 63;
  const int per = (len + NT - 1) / NT;
  const int c_lo = min(len, static_cast<int>(threadIdx.x) * per);
  const int n_mine = min(len, c_lo + per) - c_lo;
  auto value = [&](int c) -> uint32_t {
    float v = 0.0f;
    for (int u = 0; u < nsum; ++u) v += src[static_cast<size_t>(u) * a.T + c];
    return __float_as_uint(fmaxf(v, 0.0f));
  };
  uint32_t rv[PER > 0 ? PER : 1];
  if constexpr (PER > 0) {
    // every load issued before the first add: one memory latency per head
    float acc[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) acc[u] = 0.0f;
    for (int hh = 0; hh < nsum; ++hh) {
      const float* p = src + static_cast<size_t>(hh) * a.T + c_lo;
      float x[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) x[u] = u < n_mine ? p[u] : 0.0f;
#pragma unroll
      for (int u = 0; u < PER; ++u) acc[u] += x[u];
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) rv[u] = __float_as_uint(fmaxf(acc[u], 0.0f));
  }
  // calls f(position, bits) for the thread's keys
  auto each = [&](auto&& f) {
    if constexpr (PER > 0) {
#pragma unroll
      for (int u = 0; u < PER; ++u)
        if (u < n_mine) f(c_lo + u, rv[u]);
    } else {
      for (int u = 0; u < n_mine; ++u) f(c_lo + u, value(c_lo + u));
    }
  };
  __shared__ int hist[2048 + 1024 + 1024];
  __shared__ int pick_d, pick_above;
  for (int i = threadIdx.x; i < 4096; i += NT) hist[i] = 0;
  __syncthreads();
  uint32_t prefix = 0, pmask = 0;
  int want = k;   // rank (from the top) of the k-th largest among the keys matching prefix
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : pass == 1 ? 10 : 0;
    const int nb = pass == 0 ? 2048 : 1024;
    int* h = hist + (pass == 0 ? 0 : pass == 1 ? 2048 : 3072);
    // runs of equal digits among the thread's consecutive keys are added at
    // once (clustered masses share few digits: fewer atomics on one address)
    int run_bin = 0, run_n = 0;
    each([&](int, uint32_t v) {
      if ((v & pmask) == prefix) {
        const int bin = static_cast<int>((v >> shift) & static_cast<uint32_t>(nb - 1));
        if (run_n > 0 && bin != run_bin) {
          atomicAdd(&h[run_bin], run_n);
          run_n = 0;
        }
        run_bin = bin;
        ++run_n;
      }
    });
    if (run_n > 0) atomicAdd(&h[run_bin], run_n);
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l holds the digits top - u, u < B (descending); the sum is read
      // in a lane-rotated order so the lanes' reads fall in different banks
      const int B = nb >> 6, top = nb - 1 - B * lane;
      int t = 0;
      for (int u = 0; u < B; ++u) t += h[top - ((u + lane) & (B - 1))];
      const int incl = wave_incl_scan(t);
      int acc = incl - t;
      if (acc < want && incl >= want) {   // the one lane where the count from the top reaches want
        // (its counts read at once, then searched in registers)
        constexpr int BM = 2048 / 64;
        int cnt[BM];
#pragma unroll
        for (int u = 0; u < BM; ++u) cnt[u] = u < B ? h[top - u] : 0;
        bool found = false;
#pragma unroll
        for (int u = 0; u < BM; ++u) {
          if (!found && u < B && acc + cnt[u] >= want) {
            found = true;
            pick_d = top - u;
            pick_above = acc;
          }
          acc += cnt[u];
        }
      }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(pick_d) << shift;
    pmask |= static_cast<uint32_t>(nb - 1) << shift;
    want -= pick_above;
  }
  const uint32_t thr = prefix;   // the k-th largest value's bits; want = how many keys equal to it to take
  int ngt = 0, neq = 0;
  each([&](int, uint32_t v) {
    ngt += v > thr;
    neq += v == thr;
  });
  int2 tot;
  const int2 ex = block_scan2<NT>(ngt, neq, &tot);
  int pos = ex.x + min(ex.y, want), eq_rank = ex.y;
  each([&](int c, uint32_t v) {
    bool take = v > thr;
    if (v == thr) take = eq_rank++ < want;
    if (take) {
      if (pos < k) out[pos] = c;
      ++pos;
    }
  });
}

__global__ __launch_bounds__(1024) void topk_kernel(SelectArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int tok0 = a.cu[b], len = a.cu[b + 1] - tok0;
  const int k = sel_tab(a, 1, b);
  if (k <= 0) return;
  int32_t* out = a.sel + sel_tab(a, 2, b) + static_cast<size_t>(g) * k;
  const int grp = a.hq / a.hkv;
  const float* src = a.mass + static_cast<size_t>(a.per_kv ? g * grp : g) * a.T + tok0;
  if (len <= kTopkPer * kTopkThreads) topk_list<kTopkPer>(a, src, a.per_kv ? grp : 1, len, k, out);
  else topk_list<0>(a, src, a.per_kv ? grp : 1, len, k, out);
}

template <int D, bool BF16, int QB>
static hipError_t launch_select_t(const SelectArgs& a0, int maxnt, int64_t tiles, hipStream_t st) {
  SelectArgs a = a0;
  // tiles per workgroup: enough workgroups for two per compute unit where
  // the sequences allow it, up to 8 tiles each
  const int64_t wg1 = tiles * a.hkv * (a.hq / a.hkv / QB);
  a.tw = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(8, wg1 / 512)));
  const dim3 g3((maxnt + a.tw - 1) / a.tw, a.hkv * (a.hq / a.hkv / QB), a.nseq);
  hipLaunchKernelGGL((probe_partial_kernel<D, BF16, QB>), g3, dim3(kProbeThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(probe_rows_kernel, dim3(a.hq, a.nseq), dim3(64 * kRowParts), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((probe_mass_kernel<D, BF16, QB>), g3, dim3(kProbeThreads), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.sel != nullptr) {
    hipLaunchKernelGGL(topk_kernel, dim3(a.per_kv ? a.hkv : a.hq, a.nseq), dim3(kTopkThreads), 0, st, a);
    e = hipGetLastError();
  }
  return e;
}

template <int D, bool BF16>
static hipError_t launch_select_qb(const SelectArgs& a, int maxnt, int64_t tiles, hipStream_t st) {
  // query heads per workgroup: 4 when the KV head's group allows, else 2 or 1
  const int grp = a.hq / a.hkv;
  if (grp % 4 == 0) return launch_select_t<D, BF16, 4>(a, maxnt, tiles, st);
  if (grp % 2 == 0) return launch_select_t<D, BF16, 2>(a, maxnt, tiles, st);
  return launch_select_t<D, BF16, 1>(a, maxnt, tiles, st);
}

hipError_t launch_select(const SelectArgs& a, int d, int maxnt, int64_t tiles, hipStream_t st) {
  if (d == 128)
    return a.bf16 ? launch_select_qb<128, true>(a, maxnt, tiles, st) : launch_select_qb<128, false>(a, maxnt, tiles, st);
  return a.bf16 ? launch_select_qb<64, true>(a, maxnt, tiles, st) : launch_select_qb<64, false>(a, maxnt, tiles, st);
}

}  // namespace tmx
