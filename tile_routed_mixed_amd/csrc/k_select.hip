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
// Passes 1 and 3 run one wave per (key tile of 64, sequence, query head), so a
// sequence of S tokens spreads over S/64 x hq waves; their probe scores come
// from the matrix cores (recomputed in pass 3, cheaper than storing them):
//   1. probe scores of the tile's keys -> per probe row a partial (max, sum);
//   2. (one workgroup per (sequence, head)) partials -> each row's (m, l);
//   3. probe scores again -> mass of each key, sum over the probe rows of
//      exp(s - m) / l.
// Then a top-k pass per list: an MSB-first radix select on the (non-negative)
// float bits finds the k-th largest mass; keys above it, and the lowest
// positions among those equal to it, are written in ascending order.
#include "tm_kernels.h"

namespace tmx {

constexpr int kProbe = 64;   // most probe rows per sequence

// One wave's probe scores: all probe rows of (sequence b, head h) against the
// 64 keys of tile j, on the matrix cores, S^T = K Q^T with
// v_mfma_f32_16x16x32_{f16,bf16}.  The Q operands (the probe rows, B columns)
// are loaded once per wave by probe_q and serve every tile the wave takes;
// the tile's 4 blocks of 16 keys are the A rows, loaded straight from global
// memory.  Lane (l16, g) gets probe row 16qb + l16 and key 16kb + 4g + i in
// s[kb][qb][i] (log2 units); keys past the row (causal) or the sequence end,
// and rows past the probe, score -inf.
template <int D, bool BF16>
struct ProbeQ {
  typedef typename std::conditional<BF16, bf16x8, f16x8>::type op_t;
  static constexpr int NC = D / 32;
  op_t q[4][NC];
};

struct ProbeSeq {
  int tok0, len, nobs, r0, kv;
};

__device__ __forceinline__ ProbeSeq probe_seq(const SelectArgs& a, int b, int h) {
  ProbeSeq p;
  p.tok0 = a.cu[b];
  p.len = a.cu[b + 1] - p.tok0;
  p.nobs = min(a.n_obs, p.len);
  p.r0 = p.len - p.nobs;
  p.kv = h / (a.hq / a.hkv);
  return p;
}

template <int D, bool BF16>
__device__ __forceinline__ void probe_q(const SelectArgs& a, const ProbeSeq& ps, int h, ProbeQ<D, BF16>& pq) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int row = 16 * qb + l16;
#pragma unroll
    for (int c = 0; c < ProbeQ<D, BF16>::NC; ++c) {
      u32x4 raw = u32x4{0u, 0u, 0u, 0u};
      if (row < ps.nobs)
        raw = *reinterpret_cast<const u32x4*>(a.q + (static_cast<size_t>(ps.tok0 + ps.r0 + row) * a.hq + h) * D +
                                              32 * c + 8 * g);
      __builtin_memcpy(&pq.q[qb][c], &raw, 16);
    }
  }
}

template <int D, bool BF16>
__device__ __forceinline__ void probe_scores(const SelectArgs& a, const ProbeSeq& ps, const ProbeQ<D, BF16>& pq, int j,
                                             f32x4 (&s)[4][4]) {
  typedef typename ProbeQ<D, BF16>::op_t op_t;
  constexpr int NC = ProbeQ<D, BF16>::NC;
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
  u32x4 kraw[4][NC];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int key = j * kBlock + 16 * kb + l16;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kraw[kb][c] = u32x4{0u, 0u, 0u, 0u};
      if (key < ps.len)
        kraw[kb][c] = *reinterpret_cast<const u32x4*>(a.k + (static_cast<size_t>(ps.tok0 + key) * a.hkv + ps.kv) * D +
                                                      32 * c + 8 * g);
    }
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      op_t kop;
      __builtin_memcpy(&kop, &kraw[kb][c], 16);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        if constexpr (BF16) s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, pq.q[qb][c], s[kb][qb], 0, 0, 0);
        else s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, pq.q[qb][c], s[kb][qb], 0, 0, 0);
      }
    }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * qb + l16, key = j * kBlock + 16 * kb + 4 * g + i;
        const bool ok = row < ps.nobs && key <= ps.r0 + row && key < ps.len;
        s[kb][qb][i] = ok ? s[kb][qb][i] * a.tau_log2e : -INFINITY;
      }
}

// Passes 1 and 3 give each wave kTilesPerWave consecutive key tiles (the
// probe rows' operands are loaded once for all of them): workgroup x covers
// tiles 4 kTilesPerWave x onwards of (sequence z, head y).
constexpr int kProbeWaves = 4;
constexpr int kTilesPerWave = 2;

// pass 1: per (row, tile) partial max and sum (log2 units)
template <int D, bool BF16>
__global__ __launch_bounds__(256) void probe_partial_kernel(SelectArgs a) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int j0 = (blockIdx.x * kProbeWaves + (threadIdx.x >> 6)) * kTilesPerWave;
  const ProbeSeq ps = probe_seq(a, b, h);
  if (j0 * kBlock >= ps.len) return;   // whole wave
  ProbeQ<D, BF16> pq;
  probe_q<D, BF16>(a, ps, h, pq);
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  for (int j = j0; j < j0 + kTilesPerWave && j * kBlock < ps.len; ++j) {
    f32x4 s[4][4];
    probe_scores<D, BF16>(a, ps, pq, j, s);
    float* dst = a.part + ((static_cast<size_t>(sel_tab(a, 0, b)) + j) * a.hq + h) * (2 * kProbe);
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      // row 16qb + l16: 16 keys in the lane, the rest in lanes l16 + 16, 32, 48
      float m = s[0][qb][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) m = fmaxf(m, s[e >> 2][qb][e & 3]);
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      float l = 0.0f;
      if (m > -INFINITY) {
#pragma unroll
        for (int e = 0; e < 16; ++e) l += __builtin_amdgcn_exp2f(s[e >> 2][qb][e & 3] - m);
      }
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
      const int row = 16 * qb + l16;
      if (lane < 16 && row < ps.nobs) {
        dst[2 * row] = m;
        dst[2 * row + 1] = l;
      }
    }
  }
}

// pass 2: each probe row's (m, l) over all tiles; thread (row, q) merges the
// tiles q, q + 16, ..., then the 16 parts are merged through LDS
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
    dst[1] = L;
  }
}

// pass 3: mass of each key of tile j: the sum over the probe rows of
// exp2(s - m) / l, first over the lane's 4 rows, then across the 16 lanes of
// each lane group
template <int D, bool BF16>
__global__ __launch_bounds__(256) void probe_mass_kernel(SelectArgs a) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int j0 = (blockIdx.x * kProbeWaves + (threadIdx.x >> 6)) * kTilesPerWave;
  const ProbeSeq ps = probe_seq(a, b, h);
  if (j0 * kBlock >= ps.len) return;   // whole wave
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
  float m[4], inv[4];
  const float* st = a.rows + (static_cast<size_t>(b) * a.hq + h) * (2 * kProbe);
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int row = 16 * qb + l16;
    m[qb] = 0.0f;
    inv[qb] = 0.0f;
    if (row < ps.nobs) {
      m[qb] = st[2 * row];
      inv[qb] = 1.0f / st[2 * row + 1];
    }
  }
  ProbeQ<D, BF16> pq;
  probe_q<D, BF16>(a, ps, h, pq);
  for (int j = j0; j < j0 + kTilesPerWave && j * kBlock < ps.len; ++j) {
    f32x4 s[4][4];
    probe_scores<D, BF16>(a, ps, pq, j, s);
    float p[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float acc = 0.0f;
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const float x = s[e >> 2][qb][e & 3];
        acc += x > -INFINITY ? __builtin_amdgcn_exp2f(x - m[qb]) * inv[qb] : 0.0f;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) acc += __shfl_xor(acc, o, 64);
      p[e] = acc;
    }
    if (l16 == 0) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = j * kBlock + 16 * kb + 4 * g + i;
          if (key < ps.len) a.mass[(static_cast<size_t>(ps.tok0) + key) * a.hq + h] = p[4 * kb + i];
        }
    }
  }
}

// Block-wide exclusive prefix sum of one value per thread (NT threads);
// returns the prefix and sets *total.
template <int NT>
__device__ __forceinline__ int block_scan(int v, int* total) {
  __shared__ int warp_tot[NT / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) warp_tot[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int u = 0; u < NT / 64; ++u) {
    if (u < w) base += warp_tot[u];
    tot += warp_tot[u];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// top-k of one list: (sequence b, list head g): the mass of query head g, or
// the sum over KV head g's query heads
constexpr int kTopkThreads = 1024;
constexpr int kTopkLds = 12288;   // keys of a list held in LDS (48 KiB)
__global__ __launch_bounds__(1024) void topk_kernel(SelectArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int tok0 = a.cu[b], len = a.cu[b + 1] - a.cu[b];
  const int k = sel_tab(a, 1, b);
  int32_t* out = a.sel + sel_tab(a, 2, b) + static_cast<size_t>(g) * k;
  const int grp = a.hq / a.hkv;
  auto value = [&](int c) -> uint32_t {
    float v;
    if (a.per_kv) {
      v = 0.0f;
      for (int u = 0; u < grp; ++u) v += a.mass[(static_cast<size_t>(tok0) + c) * a.hq + g * grp + u];
    } else {
      v = a.mass[(static_cast<size_t>(tok0) + c) * a.hq + g];
    }
    return __float_as_uint(fmaxf(v, 0.0f));   // non-negative: the bits order as the values
  };
  if (k <= 0) return;
  constexpr int NT = kTopkThreads;
  const int lane = threadIdx.x & 63;
  // a list of up to kTopkLds keys is read from global memory once and kept
  // in LDS for the radix passes and the compaction
  __shared__ uint32_t sv[kTopkLds];
  const bool in_lds = len <= kTopkLds;
  if (in_lds) {
    for (int c = threadIdx.x; c < len; c += NT) sv[c] = value(c);
    __syncthreads();
  }
  auto get = [&](int c) -> uint32_t { return in_lds ? sv[c] : value(c); };
  // radix select of the k-th largest, 8 bits at a time from the top
  __shared__ int hist[256];
  __shared__ int pick, above;
  uint32_t prefix = 0, pmask = 0;
  int want = k;   // rank (1-based, from the top) of the k-th largest among values matching prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) hist[threadIdx.x] = 0;
    __syncthreads();
    for (int c0 = 0; c0 < len; c0 += 4 * NT) {
      uint32_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * NT + static_cast<int>(threadIdx.x);
        v[u] = c < len ? get(c) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * NT + static_cast<int>(threadIdx.x);
        bool pend = c < len && (v[u] & pmask) == prefix;
        const uint32_t bin = (v[u] >> shift) & 255u;
        // lanes that share the first pending lane's digit add once (masses
        // cluster in a few digits, which would serialize the LDS atomics);
        // two rounds, then one atomic per remaining lane
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const uint64_t act = __ballot(pend);
          if (act == 0) break;
          const int leader = __builtin_ctzll(act);
          const uint32_t lb = static_cast<uint32_t>(__shfl(static_cast<int>(bin), leader, 64));
          const bool same = pend && bin == lb;
          const uint64_t mm = __ballot(same);
          if (lane == leader) atomicAdd(&hist[lb], __popcll(mm));
          if (same) pend = false;
        }
        if (pend) atomicAdd(&hist[bin], 1);
      }
    }
    __syncthreads();
    // digit d: the largest with count(digits >= d) >= want.  Lane l of wave 0
    // holds digits 255 - 4l .. 252 - 4l (descending); a scan over the lanes
    // gives the count above each lane, and the lowest lane whose digits reach
    // want holds d (digit 0 when none of 255..1 does)
    if (threadIdx.x < 64) {
      int c[4], t = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        c[u] = hist[255 - 4 * lane - u];
        t += c[u];
      }
      int incl = t;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      int acc = incl - t, fd = -1, fa = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = 255 - 4 * lane - u;
        if (d == 0) break;
        if (fd < 0 && acc + c[u] >= want) {
          fd = d;
          fa = acc;
        }
        acc += c[u];
      }
      const uint64_t found = __ballot(fd >= 0);
      if (found == 0) {
        if (lane == 63) {   // acc = count of digits 255..1
          pick = 0;
          above = acc;
        }
      } else if (lane == __builtin_ctzll(found)) {
        pick = fd;
        above = fa;
      }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(pick) << shift;
    pmask |= 255u << shift;
    want -= above;
    __syncthreads();
  }
  const uint32_t thr = prefix;   // the k-th largest value's bits
  // keys above the threshold, then the first `want` equal ones, in position
  // order: thread t owns the contiguous positions [t per, (t + 1) per)
  const int per = (len + NT - 1) / NT;
  const int c_lo = min(len, static_cast<int>(threadIdx.x) * per), c_hi = min(len, c_lo + per);
  int ngt = 0, neq = 0;
  for (int c = c_lo; c < c_hi; ++c) {
    const uint32_t v = get(c);
    ngt += v > thr;
    neq += v == thr;
  }
  int eq_tot;
  int eq_rank = block_scan<NT>(neq, &eq_tot);   // equal keys before this thread's range
  const int ntake = ngt + max(0, min(neq, want - eq_rank));
  int take_tot;
  int pos = block_scan<NT>(ntake, &take_tot);
  for (int c = c_lo; c < c_hi; ++c) {
    const uint32_t v = get(c);
    bool take = v > thr;
    if (v == thr) take = eq_rank++ < want;
    if (take) {
      if (pos < k) out[pos] = c;
      ++pos;
    }
  }
}

template <int D, bool BF16>
static hipError_t launch_select_t(const SelectArgs& a, int maxnt, hipStream_t st) {
  const dim3 g3((maxnt + kProbeWaves * kTilesPerWave - 1) / (kProbeWaves * kTilesPerWave), a.hq, a.nseq);
  hipLaunchKernelGGL((probe_partial_kernel<D, BF16>), g3, dim3(64 * kProbeWaves), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(probe_rows_kernel, dim3(a.hq, a.nseq), dim3(64 * kRowParts), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((probe_mass_kernel<D, BF16>), g3, dim3(64 * kProbeWaves), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.sel != nullptr) {
    hipLaunchKernelGGL(topk_kernel, dim3(a.per_kv ? a.hkv : a.hq, a.nseq), dim3(kTopkThreads), 0, st, a);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_select(const SelectArgs& a, int d, int maxnt, hipStream_t st) {
  if (d == 128) return a.bf16 ? launch_select_t<128, true>(a, maxnt, st) : launch_select_t<128, false>(a, maxnt, st);
  return a.bf16 ? launch_select_t<64, true>(a, maxnt, st) : launch_select_t<64, false>(a, maxnt, st);
}

}  // namespace tmx
