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
// Three passes over (key tile of 64, sequence, query head), one workgroup
// each, so a sequence of S tokens spreads over S/64 x hq workgroups:
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

// Scores of probe rows x the 64 keys of tile j, for (sequence b, head h):
// thread t takes rows 4 (t / 16) + u and keys (t % 16) + 16 i (u, i = 0..3),
// s[4u + i]; per channel it reads 4 Q and 4 K values from LDS for 16 FMAs.
// Keys past the row (causal) or the sequence end score -inf.
template <int D>
__device__ __forceinline__ void probe_scores(const SelectArgs& a, int b, int h, int j, float (&s)[16], int& row0,
                                             int& nobs) {
  __shared__ float qs[kProbe][D + 1];
  __shared__ float ks[kBlock][D + 1];
  const int tok0 = a.cu[b], len = a.cu[b + 1] - a.cu[b];
  nobs = min(a.n_obs, len);
  const int r0 = len - nobs;   // first probe row
  const int kv = h / (a.hq / a.hkv);
  for (int u = threadIdx.x; u < kProbe * D; u += 256) {
    const int r = u / D, c = u % D;
    float x = 0.0f;
    if (r < nobs) {
      const uint16_t v = a.q[(static_cast<size_t>(tok0 + r0 + r) * a.hq + h) * D + c];
      x = a.bf16 ? bf16_bits_to_f32(v) : f16_bits_to_f32(v);
    }
    qs[r][c] = x;
  }
  for (int u = threadIdx.x; u < kBlock * D; u += 256) {
    const int r = u / D, c = u % D;
    const int key = j * kBlock + r;
    float x = 0.0f;
    if (key < len) {
      const uint16_t v = a.k[(static_cast<size_t>(tok0 + key) * a.hkv + kv) * D + c];
      x = a.bf16 ? bf16_bits_to_f32(v) : f16_bits_to_f32(v);
    }
    ks[r][c] = x;
  }
  __syncthreads();
  const int rg = threadIdx.x >> 4, kc = threadIdx.x & 15;
  row0 = 4 * rg;
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  for (int c = 0; c < D; ++c) {
    float qv[4], kvv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) qv[u] = qs[row0 + u][c];
#pragma unroll
    for (int i = 0; i < 4; ++i) kvv[i] = ks[kc + 16 * i][c];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[4 * u + i] = __builtin_fmaf(qv[u], kvv[i], acc[4 * u + i]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = row0 + u, key = j * kBlock + kc + 16 * i;
      const bool ok = rr < nobs && key <= r0 + rr && key < len;
      s[4 * u + i] = ok ? acc[4 * u + i] * a.tau_log2e : -INFINITY;
    }
}

// pass 1: per (row, tile) partial max and sum (log2 units)
template <int D>
__global__ __launch_bounds__(256) void probe_partial_kernel(SelectArgs a) {
  const int j = blockIdx.x, b = blockIdx.z, h = blockIdx.y;
  const int len = a.cu[b + 1] - a.cu[b];
  if (j * kBlock >= len) return;
  float s[16];
  int row0, nobs;
  probe_scores<D>(a, b, h, j, s, row0, nobs);
#pragma unroll
  for (int u = 0; u < 4; ++u) {   // row row0 + u: its 64 keys sit in the 16 lanes of this key group
    float m = fmaxf(fmaxf(s[4 * u], s[4 * u + 1]), fmaxf(s[4 * u + 2], s[4 * u + 3]));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float l = 0.0f;
    if (m > -INFINITY) {
#pragma unroll
      for (int i = 0; i < 4; ++i) l += __builtin_amdgcn_exp2f(s[4 * u + i] - m);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) l += __shfl_xor(l, o, 64);
    const int row = row0 + u;
    if ((threadIdx.x & 15) == 0 && row < nobs) {
      float* dst = a.part + ((static_cast<size_t>(a.tile0[b]) + j) * a.hq + h) * (2 * kProbe) + 2 * row;
      dst[0] = m;
      dst[1] = l;
    }
  }
}

// pass 2: each probe row's (m, l) over all tiles
__global__ __launch_bounds__(64) void probe_rows_kernel(SelectArgs a) {
  const int b = blockIdx.y, h = blockIdx.x, r = threadIdx.x;
  const int len = a.cu[b + 1] - a.cu[b];
  const int nt = (len + kBlock - 1) / kBlock;
  float M = -INFINITY, L = 0.0f;
  for (int j = 0; j < nt; ++j) {
    const float* p = a.part + ((static_cast<size_t>(a.tile0[b]) + j) * a.hq + h) * (2 * kProbe) + 2 * r;
    const float m = p[0], l = p[1];
    if (!(m > -INFINITY)) continue;   // (rows past the probe, and tiles after the row, stay -inf)
    const float mn = fmaxf(M, m);
    L = L * __builtin_amdgcn_exp2f(M - mn) + l * __builtin_amdgcn_exp2f(m - mn);
    M = mn;
  }
  float* dst = a.rows + (static_cast<size_t>(b) * a.hq + h) * (2 * kProbe) + 2 * r;
  dst[0] = M;
  dst[1] = L;
}

// pass 3: mass of each key of tile j
template <int D>
__global__ __launch_bounds__(256) void probe_mass_kernel(SelectArgs a) {
  const int j = blockIdx.x, b = blockIdx.z, h = blockIdx.y;
  const int len = a.cu[b + 1] - a.cu[b];
  if (j * kBlock >= len) return;
  __shared__ float mass[kBlock];
  if (threadIdx.x < kBlock) mass[threadIdx.x] = 0.0f;
  float s[16];
  int row0, nobs;
  probe_scores<D>(a, b, h, j, s, row0, nobs);   // (its barrier also orders the clear above)
  float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};     // this thread's 4 keys, summed over its 4 rows
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (row0 + u >= nobs) continue;
    const float* st = a.rows + (static_cast<size_t>(b) * a.hq + h) * (2 * kProbe) + 2 * (row0 + u);
    const float m = st[0], inv = 1.0f / st[1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (s[4 * u + i] > -INFINITY) part[i] += __builtin_amdgcn_exp2f(s[4 * u + i] - m) * inv;
  }
  const int kc = threadIdx.x & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (part[i] != 0.0f) atomicAdd(&mass[kc + 16 * i], part[i]);
  __syncthreads();
  const int c = threadIdx.x;
  if (c < kBlock && j * kBlock + c < len)
    a.mass[(static_cast<size_t>(a.cu[b]) + j * kBlock + c) * a.hq + h] = mass[c];
}

// Block-wide exclusive prefix sum of one value per thread (256 threads);
// returns the prefix and sets *total.
__device__ __forceinline__ int block_scan(int v, int* total) {
  __shared__ int warp_tot[4];
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
  for (int u = 0; u < 4; ++u) {
    if (u < w) base += warp_tot[u];
    tot += warp_tot[u];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// top-k of one list: (sequence b, list head g): the mass of query head g, or
// the sum over KV head g's query heads
__global__ __launch_bounds__(256) void topk_kernel(SelectArgs a) {
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
  uint32_t prefix = 0, pmask = 0;
  int want = k;   // rank (1-based, from the top) of the k-th largest among values matching prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[threadIdx.x] = 0;
    __syncthreads();
    for (int c = threadIdx.x; c < len; c += 256) {
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
  for (int c0 = 0; c0 < len; c0 += 256) {
    const int c = c0 + threadIdx.x;
    const uint32_t v = c < len ? value(c) : 0u;
    const int gt = c < len && v > thr, eq = c < len && v == thr;
    int eq_tot;
    const int eq_rank = eq_seen + block_scan(eq, &eq_tot);
    const int take = gt || (eq && eq_rank < want);
    int take_tot;
    const int pos = written + block_scan(take, &take_tot);
    if (take && pos < k) out[pos] = c;
    eq_seen += eq_tot;
    written += take_tot;
  }
}

template <int D>
static hipError_t launch_select_t(const SelectArgs& a, int maxnt, hipStream_t st) {
  const dim3 g3(maxnt, a.hq, a.nseq);
  hipLaunchKernelGGL(probe_partial_kernel<D>, g3, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(probe_rows_kernel, dim3(a.hq, a.nseq), dim3(64), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(probe_mass_kernel<D>, g3, dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.sel != nullptr) {
    hipLaunchKernelGGL(topk_kernel, dim3(a.per_kv ? a.hkv : a.hq, a.nseq), dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_select(const SelectArgs& a, int d, int maxnt, hipStream_t st) {
  return d == 128 ? launch_select_t<128>(a, maxnt, st) : launch_select_t<64>(a, maxnt, st);
}

}  // namespace tmx
