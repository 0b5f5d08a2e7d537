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
// Passes 1 and 3 run one workgroup per (key tile of 64, sequence, query
// head), so a sequence of S tokens spreads over S/64 x hq workgroups; their
// probe scores come from the matrix cores (recomputed in pass 3, cheaper than
// storing them):
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

// Scores of the probe rows x the 64 keys of tile j, for (sequence b, head h),
// on the matrix cores: S^T = K Q^T with v_mfma_f32_16x16x32_{f16,bf16}, wave w
// taking probe rows 16w .. 16w+15 (the B columns) and the tile's 4 blocks of
// 16 keys (the A rows), operands loaded straight from global memory.  Lane
// (l16, g) gets row 16w + l16 and keys 16kb + 4g + i in s[4kb + i] (log2
// units); keys past the row (causal) or the sequence end, and rows past the
// probe, score -inf.
template <int D, bool BF16>
__device__ __forceinline__ void probe_scores(const SelectArgs& a, int b, int h, int j, float (&s)[16], int& row,
                                             int& nobs) {
  typedef typename std::conditional<BF16, bf16x8, f16x8>::type op_t;
  constexpr int NC = D / 32;
  const int tok0 = a.cu[b], len = a.cu[b + 1] - a.cu[b];
  nobs = min(a.n_obs, len);
  const int r0 = len - nobs;   // first probe row
  const int kv = h / (a.hq / a.hkv);
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4, w = threadIdx.x >> 6;
  row = 16 * w + l16;
  op_t qop[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    u32x4 raw = u32x4{0u, 0u, 0u, 0u};
    if (row < nobs)
      raw = *reinterpret_cast<const u32x4*>(a.q + (static_cast<size_t>(tok0 + r0 + row) * a.hq + h) * D + 32 * c + 8 * g);
    __builtin_memcpy(&qop[c], &raw, 16);
  }
  f32x4 acc[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int key = j * kBlock + 16 * kb + l16;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 raw = u32x4{0u, 0u, 0u, 0u};
      if (key < len)
        raw = *reinterpret_cast<const u32x4*>(a.k + (static_cast<size_t>(tok0 + key) * a.hkv + kv) * D + 32 * c + 8 * g);
      op_t kop;
      __builtin_memcpy(&kop, &raw, 16);
      if constexpr (BF16) acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[c], acc[kb], 0, 0, 0);
      else acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[c], acc[kb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = j * kBlock + 16 * kb + 4 * g + i;
      const bool ok = row < nobs && key <= r0 + row && key < len;
      s[4 * kb + i] = ok ? acc[kb][i] * a.tau_log2e : -INFINITY;
    }
}

// pass 1: per (row, tile) partial max and sum (log2 units)
template <int D, bool BF16>
__global__ __launch_bounds__(256) void probe_partial_kernel(SelectArgs a) {
  const int j = blockIdx.x, b = blockIdx.z, h = blockIdx.y;
  const int len = a.cu[b + 1] - a.cu[b];
  if (j * kBlock >= len) return;
  float s[16];
  int row, nobs;
  probe_scores<D, BF16>(a, b, h, j, s, row, nobs);
  // the row's 64 keys: 16 in the lane, the rest in lanes l16 + 16, 32, 48
  float m = s[0];
#pragma unroll
  for (int e = 1; e < 16; ++e) m = fmaxf(m, s[e]);
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  float l = 0.0f;
  if (m > -INFINITY) {
#pragma unroll
    for (int e = 0; e < 16; ++e) l += __builtin_amdgcn_exp2f(s[e] - m);
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if ((threadIdx.x & 63) < 16 && row < nobs) {
    float* dst = a.part + ((static_cast<size_t>(a.tile0[b]) + j) * a.hq + h) * (2 * kProbe) + 2 * row;
    dst[0] = m;
    dst[1] = l;
  }
}

// pass 2: each probe row's (m, l) over all tiles; thread (row, q) merges the
// tiles q, q + 4, ..., then the four quarters are merged across lanes
__global__ __launch_bounds__(256) void probe_rows_kernel(SelectArgs a) {
  const int b = blockIdx.y, h = blockIdx.x;
  const int r = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int len = a.cu[b + 1] - a.cu[b];
  const int nt = (len + kBlock - 1) / kBlock;
  float M = -INFINITY, L = 0.0f;
  for (int j = q; j < nt; j += 4) {
    const float* p = a.part + ((static_cast<size_t>(a.tile0[b]) + j) * a.hq + h) * (2 * kProbe) + 2 * r;
    const float m = p[0], l = p[1];
    if (!(m > -INFINITY)) continue;   // (rows past the probe, and tiles after the row, stay -inf)
    const float mn = fmaxf(M, m);
    L = L * __builtin_amdgcn_exp2f(M - mn) + l * __builtin_amdgcn_exp2f(m - mn);
    M = mn;
  }
  __shared__ float sm[4][64], sl[4][64];
  sm[q][r] = M;
  sl[q][r] = L;
  __syncthreads();
  if (q == 0) {
    float Mt = -INFINITY, Lt = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float m = sm[u][r], l = sl[u][r];
      if (!(m > -INFINITY)) continue;
      const float mn = fmaxf(Mt, m);
      Lt = Lt * __builtin_amdgcn_exp2f(Mt - mn) + l * __builtin_amdgcn_exp2f(m - mn);
      Mt = mn;
    }
    float* dst = a.rows + (static_cast<size_t>(b) * a.hq + h) * (2 * kProbe) + 2 * r;
    dst[0] = Mt;
    dst[1] = Lt;
  }
}

// pass 3: mass of each key of tile j
template <int D, bool BF16>
__global__ __launch_bounds__(256) void probe_mass_kernel(SelectArgs a) {
  const int j = blockIdx.x, b = blockIdx.z, h = blockIdx.y;
  const int len = a.cu[b + 1] - a.cu[b];
  if (j * kBlock >= len) return;
  __shared__ float mass[kBlock];
  if (threadIdx.x < kBlock) mass[threadIdx.x] = 0.0f;
  __syncthreads();
  float s[16];
  int row, nobs;
  probe_scores<D, BF16>(a, b, h, j, s, row, nobs);
  float m = 0.0f, inv = 0.0f;
  if (row < nobs) {
    const float* st = a.rows + (static_cast<size_t>(b) * a.hq + h) * (2 * kProbe) + 2 * row;
    m = st[0];
    inv = 1.0f / st[1];
  }
  float p[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    p[e] = s[e] > -INFINITY ? __builtin_amdgcn_exp2f(s[e] - m) * inv : 0.0f;
    // sum over the wave's 16 rows (lanes l16 of the lane group)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) p[e] += __shfl_xor(p[e], o, 64);
  }
  if ((threadIdx.x & 15) == 0) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&mass[16 * kb + 4 * g + i], p[4 * kb + i]);
  }
  __syncthreads();
  const int c = threadIdx.x;
  if (c < kBlock && j * kBlock + c < len)
    a.mass[(static_cast<size_t>(a.cu[b]) + j * kBlock + c) * a.hq + h] = mass[c];
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
__global__ __launch_bounds__(1024) void topk_kernel(SelectArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int tok0 = a.cu[b], len = a.cu[b + 1] - a.cu[b];
  const int k = a.kcount[b];
  const int nlist = a.per_kv ? a.hkv : a.hq;
  int32_t* out = a.sel + a.sel_base[b] + static_cast<size_t>(g) * k;
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
  (void)nlist;
  if (k <= 0) return;
  // radix select of the k-th largest, 8 bits at a time from the top
  __shared__ int hist[256];
  constexpr int NT = kTopkThreads;
  uint32_t prefix = 0, pmask = 0;
  int want = k;   // rank (1-based, from the top) of the k-th largest among values matching prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) hist[threadIdx.x] = 0;
    __syncthreads();
    for (int c = threadIdx.x; c < len; c += NT) {
      const uint32_t v = value(c);
      if ((v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & 255u], 1);
    }
    __syncthreads();
    // digit d: the largest with count(digits >= d) >= want
    __shared__ int pick, above;
    if (threadIdx.x == 0) {
      int acc = 0, d = 255;
      for (; d > 0; --d) {
        if (acc + hist[d] >= want) break;
        acc += hist[d];
      }
      pick = d;
      above = acc;
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(pick) << shift;
    pmask |= 255u << shift;
    want -= above;
    __syncthreads();
  }
  const uint32_t thr = prefix;   // the k-th largest value's bits
  // keys above the threshold, then the first `want` equal ones, in position order
  int eq_seen = 0, written = 0;
  for (int c0 = 0; c0 < len; c0 += NT) {
    const int c = c0 + threadIdx.x;
    const uint32_t v = c < len ? value(c) : 0u;
    const int gt = c < len && v > thr, eq = c < len && v == thr;
    int eq_tot;
    const int eq_rank = eq_seen + block_scan<NT>(eq, &eq_tot);
    const int take = gt || (eq && eq_rank < want);
    int take_tot;
    const int pos = written + block_scan<NT>(take, &take_tot);
    if (take && pos < k) out[pos] = c;
    eq_seen += eq_tot;
    written += take_tot;
  }
}

template <int D, bool BF16>
static hipError_t launch_select_t(const SelectArgs& a, int maxnt, hipStream_t st) {
  const dim3 g3(maxnt, a.hq, a.nseq);
  hipLaunchKernelGGL((probe_partial_kernel<D, BF16>), g3, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(probe_rows_kernel, dim3(a.hq, a.nseq), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((probe_mass_kernel<D, BF16>), g3, dim3(256), 0, st, a);
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
