// Hardware ceilings of one MI355X (gfx950), measured: the rates the
// roofline fractions of the attention kernels are read against.
//
//  * MFMA issue rate of the three contractions the kernels use
//    (v_mfma_i32_16x16x64_i8, v_mfma_f32_16x16x32_{f16,bf16}), one and two
//    waves per SIMD, with the shader clock read from s_memtime against the
//    100 MHz s_memrealtime;
//  * how much VALU work (plain FMA, exp, conversions, integer max) one or two
//    waves per SIMD hide under MFMA issue, per 16x16 and 32x32 MFMA shape
//    (the "mix", "split" and "bundle" tables);
//  * LDS read bandwidth (ds_read_b128) per CU;
//  * HBM streaming read and copy bandwidth.
//
// Usage: tm_ceiling            full tables (text)
//        tm_ceiling --summary  MFMA rates, LDS and HBM bandwidth as one JSON line
//        tm_ceiling --bundles  the MFMA + VALU bundle table
// Every kernel touches only its own buffers, indexed within the launch grid.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <vector>
#include <cstdint>
#include <algorithm>
#include <cstring>

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

#define CHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); exit(1);} } while (0)

struct Clk { unsigned long long t0, t1, r0, r1; };

__device__ __forceinline__ void clk_begin(Clk* c) {
  if (blockIdx.x == 0 && threadIdx.x == 0) { c->t0 = __builtin_amdgcn_s_memtime(); c->r0 = __builtin_amdgcn_s_memrealtime(); }
}
__device__ __forceinline__ void clk_end(Clk* c) {
  if (blockIdx.x == 0 && threadIdx.x == 0) { c->t1 = __builtin_amdgcn_s_memtime(); c->r1 = __builtin_amdgcn_s_memrealtime(); }
}

// KIND 0: i8 16x16x64, 1: f16 16x16x32, 2: bf16 16x16x32.  NACC independent accumulators.
template <int KIND, int NACC>
__global__ __launch_bounds__(256) void mfma_rate(float* out, Clk* clk, int iters) {
  clk_begin(clk);
  const int t = threadIdx.x;
  i32x4 ai = {t, t * 3, t * 5, t * 7};
  f16x8 ah, bh;
  bf16x8 ab, bb;
  for (int e = 0; e < 8; ++e) {
    ah[e] = (_Float16)(0.001f * (t + e));
    bh[e] = (_Float16)(0.002f * (t - e));
    ab[e] = (__bf16)(0.001f * (t + e));
    bb[e] = (__bf16)(0.002f * (t - e));
  }
  i32x4 acci[NACC];
  f32x4 accf[NACC];
  for (int j = 0; j < NACC; ++j) { acci[j] = i32x4{0, 0, 0, 0}; accf[j] = f32x4{0, 0, 0, 0}; }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NACC; ++j) {
      if constexpr (KIND == 0) acci[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, ai, acci[j], 0, 0, 0);
      else if constexpr (KIND == 1) accf[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, accf[j], 0, 0, 0);
      else accf[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bb, accf[j], 0, 0, 0);
    }
  }
  float s = 0;
  for (int j = 0; j < NACC; ++j) s += (float)acci[j][0] + accf[j][0] + accf[j][3];
  out[blockIdx.x * 256 + t] = s;
  clk_end(clk);
}

// 4 f16 MFMAs (independent accumulators) + NV VALU ops per iteration,
// interleaved MFMA, NV/4 VALU, MFMA, ...  OP 0: v_fma_f32, 1: v_exp_f32,
// 2: v_cvt_f32_i32, 3: v_cvt_pk_f16_f32 (via two floats -> half2), 4: v_max_i32
template <int NV, int OP, bool MF>
__global__ __launch_bounds__(256) void mix(float* out, Clk* clk, int iters) {
  clk_begin(clk);
  const int t = threadIdx.x;
  f16x8 ah, bh;
  for (int e = 0; e < 8; ++e) {
    ah[e] = (_Float16)(0.001f * (t + e));
    bh[e] = (_Float16)(0.002f * (t - e));
  }
  f32x4 acc[4];
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0, 0, 0, 0};
  float x[16];
  int xi[16];
  for (int v = 0; v < 16; ++v) { x[v] = 0.5f + 0.01f * v + 1e-4f * t; xi[v] = t + v; }
  const float c1 = 0.999f + 1e-7f * t, c2 = 1e-3f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (MF) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc[j], 0, 0, 0);
#pragma unroll
      for (int v = 0; v < NV / 4; ++v) {
        const int r = (j * (NV / 4) + v) & 15;
        if constexpr (OP == 0) x[r] = __builtin_fmaf(x[r], c1, c2);
        else if constexpr (OP == 1) x[r] = __builtin_amdgcn_exp2f(-x[r]);
        else if constexpr (OP == 2) { x[r] = (float)xi[r]; xi[r] = __float_as_int(x[r]) ^ it; }
        else if constexpr (OP == 3) {
          auto h = __builtin_amdgcn_cvt_pkrtz(x[r], x[(r + 1) & 15]);
          x[r] = __builtin_bit_cast(float, h);
        } else xi[r] = max(xi[r], xi[(r + 5) & 15] ^ it);
      }
      if constexpr (MF) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (OP == 1) __builtin_amdgcn_sched_group_barrier(0x400, NV / 4, 0);
      else __builtin_amdgcn_sched_group_barrier(0x002, NV / 4, 0);
    }
  }
  float s = 0;
  for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][3];
  for (int v = 0; v < 16; ++v) s += x[v] + (float)xi[v];
  out[blockIdx.x * 256 + t] = s;
  clk_end(clk);
}


typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// Bundles: per iteration 4 MFMAs of kind MK (4 independent accumulators), each
// followed by NF/4 FMAs and NE/4 exps (16 FMA chains, 8 exp chains).
// MK 0: f16 16x16x32, 1: f16 32x32x16, 2: i8 16x16x64, 3: i8 32x32x32, -1: none.
template <int MK, int NF, int NE>
__global__ __launch_bounds__(256) void bundle(float* out, Clk* clk, int iters) {
  clk_begin(clk);
  const int t = threadIdx.x;
  f16x8 ah, bh;
  for (int e = 0; e < 8; ++e) {
    ah[e] = (_Float16)(0.001f * (t + e));
    bh[e] = (_Float16)(0.002f * (t - e));
  }
  const i32x4 ai = {t, t * 3, t * 5, t * 7};
  f32x4 a4[4];
  i32x4 i4[4];
  f32x16 a16[4];
  i32x16 i16[4];
  for (int j = 0; j < 4; ++j) {
    a4[j] = f32x4{0, 0, 0, 0};
    i4[j] = i32x4{0, 0, 0, 0};
    for (int e = 0; e < 16; ++e) { a16[j][e] = 0; i16[j][e] = 0; }
  }
  float x[16], y[8];
  for (int v = 0; v < 16; ++v) x[v] = 0.5f + 0.01f * v + 1e-4f * t;
  for (int v = 0; v < 8; ++v) y[v] = 0.25f + 0.01f * v + 1e-4f * t;
  const float c1 = 0.999f + 1e-7f * t, c2 = 1e-3f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (MK == 0) a4[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, a4[j], 0, 0, 0);
      else if constexpr (MK == 1) a16[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, a16[j], 0, 0, 0);
      else if constexpr (MK == 2) i4[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, ai, i4[j], 0, 0, 0);
      else if constexpr (MK == 3) i16[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ai, ai, i16[j], 0, 0, 0);
#pragma unroll
      for (int v = 0; v < NF / 4; ++v) {
        const int r = (j * (NF / 4) + v) & 15;
        x[r] = __builtin_fmaf(x[r], c1, c2);
      }
#pragma unroll
      for (int v = 0; v < NE / 4; ++v) {
        const int r = (j * (NE / 4) + v) & 7;
        y[r] = __builtin_amdgcn_exp2f(-y[r]);
      }
      if constexpr (MK >= 0) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (NF > 0) __builtin_amdgcn_sched_group_barrier(0x002, NF / 4, 0);
      if constexpr (NE > 0) __builtin_amdgcn_sched_group_barrier(0x400, NE / 4, 0);
    }
  }
  float s = 0;
  for (int j = 0; j < 4; ++j) {
    s += a4[j][0] + (float)i4[j][1];
    for (int e = 0; e < 16; e += 5) s += a16[j][e] + (float)i16[j][e];
  }
  for (int v = 0; v < 16; ++v) s += x[v];
  for (int v = 0; v < 8; ++v) s += y[v];
  out[blockIdx.x * 256 + t] = s;
  clk_end(clk);
}

// 8 waves per workgroup: waves 0-3 run MFMAs only, waves 4-7 VALU only (OP as
// in mix; NV ops per MFMA-iteration equivalent).  Waves w and w+4 share a SIMD.
template <int OP>
__global__ __launch_bounds__(512) void split(float* out, Clk* clk, int iters_m, int iters_v) {
  clk_begin(clk);
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  float s = 0;
  if (w < 4) {
    f16x8 ah, bh;
    for (int e = 0; e < 8; ++e) {
      ah[e] = (_Float16)(0.001f * (t + e));
      bh[e] = (_Float16)(0.002f * (t - e));
    }
    f32x4 acc[4];
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0, 0, 0, 0};
    for (int it = 0; it < iters_m; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc[j], 0, 0, 0);
    }
    for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][3];
  } else {
    float x[16];
    for (int v = 0; v < 16; ++v) x[v] = 0.5f + 0.01f * v + 1e-4f * t;
    const float c1 = 0.999f + 1e-7f * t, c2 = 1e-3f;
    for (int it = 0; it < iters_v; ++it) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        if constexpr (OP == 0) x[v] = __builtin_fmaf(x[v], c1, c2);
        else x[v] = __builtin_amdgcn_exp2f(-x[v]);
      }
    }
    for (int v = 0; v < 16; ++v) s += x[v];
  }
  out[blockIdx.x * 512 + t] = s;
  clk_end(clk);
}

// LDS reads: 8 ds_read_b128 per asm block (waited inside the block), 64 KiB region.
__global__ __launch_bounds__(256) void lds_read(float* out, Clk* clk, int iters) {
  __shared__ __align__(16) unsigned char lds[65536];
  clk_begin(clk);
  const int t = threadIdx.x;
  for (int i = t; i < 65536 / 4; i += 256) reinterpret_cast<unsigned*>(lds)[i] = i * 2654435761u;
  __syncthreads();
  const int w = t >> 6, lane = t & 63;
  unsigned acc = 0;
  // wave w reads 8 KiB at [w * 8 KiB + i * 1 KiB + lane * 16] (mod 64 KiB) per block
  unsigned addr = static_cast<unsigned>(reinterpret_cast<uintptr_t>(lds)) + (w * 8192 + lane * 16);
  for (int it = 0; it < iters; ++it) {
    u32x4 r0, r1, r2, r3, r4, r5, r6, r7;
    const unsigned a = addr + ((it * 32768) & 32767);
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\t"
        "ds_read_b128 %3, %8 offset:3072\n\t"
        "ds_read_b128 %4, %8 offset:4096\n\t"
        "ds_read_b128 %5, %8 offset:5120\n\t"
        "ds_read_b128 %6, %8 offset:6144\n\t"
        "ds_read_b128 %7, %8 offset:7168\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3), "=v"(r4), "=v"(r5), "=v"(r6), "=v"(r7)
        : "v"(a)
        : "memory");
    acc ^= r0[0] ^ r1[1] ^ r2[2] ^ r3[3] ^ r4[0] ^ r5[1] ^ r6[2] ^ r7[3];
  }
  out[blockIdx.x * 256 + t] = (float)acc;
  clk_end(clk);
}

// HBM streaming read: n16 16-byte elements, grid-stride.
__global__ __launch_bounds__(256) void hbm_read(const u32x4* __restrict__ src, size_t n16, float* out) {
  unsigned acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[blockIdx.x * 256 + threadIdx.x] = (float)acc;
}

__global__ __launch_bounds__(256) void hbm_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

template <typename F>
static float time_ms(F f, int reps) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  f();
  CHECK(hipDeviceSynchronize());
  std::vector<float> ts;
  for (int r = 0; r < reps; ++r) {
    CHECK(hipEventRecord(a));
    f();
    CHECK(hipEventRecord(b));
    CHECK(hipEventSynchronize(b));
    float ms;
    CHECK(hipEventElapsedTime(&ms, a, b));
    ts.push_back(ms);
  }
  std::sort(ts.begin(), ts.end());
  return ts[ts.size() / 2];
}

// One JSON line: MFMA rates (two waves per SIMD, eight independent
// accumulators), LDS read bandwidth (two workgroups per CU) and the best HBM
// read and copy bandwidth over a few grid sizes.
static int run_summary(int ncu, float* out, Clk* clk) {
  const int iters = 20000;
  const int nb = ncu * 2;
  const double waves = nb * 4.0;
  auto ghz_of = [&]() {
    Clk hc;
    CHECK(hipMemcpy(&hc, clk, sizeof(Clk), hipMemcpyDeviceToHost));
    return (double)(hc.t1 - hc.t0) / (double)(hc.r1 - hc.r0) * 0.1;
  };
  float ms_i8 = time_ms([&] { hipLaunchKernelGGL((mfma_rate<0, 8>), dim3(nb), dim3(256), 0, 0, out, clk, iters); }, 3);
  const double g_i8 = ghz_of();
  float ms_f16 = time_ms([&] { hipLaunchKernelGGL((mfma_rate<1, 8>), dim3(nb), dim3(256), 0, 0, out, clk, iters); }, 3);
  const double g_f16 = ghz_of();
  float ms_bf16 = time_ms([&] { hipLaunchKernelGGL((mfma_rate<2, 8>), dim3(nb), dim3(256), 0, 0, out, clk, iters); }, 3);
  const double g_bf16 = ghz_of();
  const double ops_i8 = waves * iters * 8 * 16.0 * 16 * 64 * 2, ops_f16 = waves * iters * 8 * 16.0 * 16 * 32 * 2;
  const int lit = 20000;
  float ms_lds = time_ms([&] { hipLaunchKernelGGL(lds_read, dim3(nb), dim3(256), 0, 0, out, clk, lit); }, 3);
  const double g_lds = ghz_of();
  const double lds_bytes = (double)nb * 4 * lit * 8 * 1024;
  const size_t nbytes = size_t(4) << 30;
  u32x4 *a, *b;
  CHECK(hipMalloc(&a, nbytes));
  CHECK(hipMalloc(&b, nbytes / 2));
  CHECK(hipMemset(a, 1, nbytes));
  CHECK(hipMemset(b, 0, nbytes / 2));
  float rd = 1e30f, cp = 1e30f;
  for (int g : {ncu * 4, ncu * 8}) {
    rd = std::min(rd, time_ms([&] { hipLaunchKernelGGL(hbm_read, dim3(g), dim3(256), 0, 0, a, nbytes / 16, out); }, 5));
    cp = std::min(cp, time_ms([&] { hipLaunchKernelGGL(hbm_copy, dim3(g), dim3(256), 0, 0, a, b, nbytes / 32); }, 5));
  }
  CHECK(hipFree(a));
  CHECK(hipFree(b));
  printf("{\"mfma_i8_16x16x64_TOPs\": %.1f, \"mfma_f16_16x16x32_TFLOPs\": %.1f, \"mfma_bf16_16x16x32_TFLOPs\": %.1f, "
         "\"shader_clock_GHz_under_mfma\": [%.3f, %.3f, %.3f], \"lds_read_B_per_clk_per_CU\": %.1f, "
         "\"hbm_read_TBps\": %.3f, \"hbm_copy_TBps_read_plus_write\": %.3f, "
         "\"note\": \"tm_ceiling --summary: two waves per SIMD, eight independent accumulators; LDS: ds_read_b128, "
         "two workgroups per CU; HBM: best of two grid sizes over a 4 GiB read and a 2 GiB copy\"}\n",
         ops_i8 / ms_i8 / 1e9, ops_f16 / ms_f16 / 1e9, ops_f16 / ms_bf16 / 1e9, g_i8, g_f16, g_bf16,
         lds_bytes / ncu / (ms_lds * 1e-3 * g_lds * 1e9), nbytes / rd / 1e9, nbytes / cp / 1e9);
  fflush(stdout);
  CHECK(hipFree(out));
  CHECK(hipFree(clk));
  return 0;
}

int main(int argc, char** argv) {
  bool summary = false, bundles = false;
  for (int i = 1; i < argc; ++i) {
    if (!strcmp(argv[i], "--summary")) summary = true;
    else if (!strcmp(argv[i], "--bundles")) bundles = true;
    else { fprintf(stderr, "usage: tm_ceiling [--summary | --bundles]\n"); return 2; }
  }
  hipDeviceProp_t p;
  CHECK(hipGetDeviceProperties(&p, 0));
  const int ncu = p.multiProcessorCount;
  printf("device %s, %d CUs, clockRate %d kHz, memClock %d kHz, bus %d bits, LDS/block %zu\n", p.gcnArchName, ncu,
         p.clockRate, p.memoryClockRate, p.memoryBusWidth, p.sharedMemPerBlock);
  fflush(stdout);
  float* out;
  Clk* clk;
  const int maxblk = ncu * 8;
  CHECK(hipMalloc(&out, sizeof(float) * maxblk * 256));
  CHECK(hipMalloc(&clk, sizeof(Clk)));
  Clk hc;
  auto clkinfo = [&](double* ghz) {
    CHECK(hipMemcpy(&hc, clk, sizeof(Clk), hipMemcpyDeviceToHost));
    const double dt = (double)(hc.t1 - hc.t0), dr = (double)(hc.r1 - hc.r0);
    *ghz = dt / dr * 0.1;   // memrealtime at 100 MHz
  };


  // ---- bundles: ns per iteration per SIMD (4 MFMAs + NF FMA + NE exp per wave-iteration)
  if (summary) return run_summary(ncu, out, clk);
  if (bundles) {
    const int bit = 10000;
    auto run_b = [&](auto kern, const char* name, int wps) {
      const int nb = ncu * wps;
      float ms = time_ms([&] { hipLaunchKernelGGL(kern, dim3(nb), dim3(256), 0, 0, out, clk, bit); }, 3);
      printf("bundle %-28s wps=%d: %.3f ms, %.2f ns per wave-iteration per SIMD\n", name, wps, ms,
             ms * 1e6 / (bit * (double)wps));
      fflush(stdout);
    };
    for (int wps = 1; wps <= 2; ++wps) {
      run_b(bundle<-1, 16, 0>, "none + 16 fma", wps);
      run_b(bundle<-1, 0, 8>, "none + 8 exp", wps);
      run_b(bundle<-1, 8, 8>, "none + 8 fma + 8 exp", wps);
      run_b(bundle<0, 0, 0>, "f16 16x16x32", wps);
      run_b(bundle<0, 16, 0>, "f16 16x16x32 + 16 fma", wps);
      run_b(bundle<0, 8, 0>, "f16 16x16x32 + 8 fma", wps);
      run_b(bundle<0, 8, 8>, "f16 16x16x32 + 8 fma + 8 exp", wps);
      run_b(bundle<1, 0, 0>, "f16 32x32x16", wps);
      run_b(bundle<1, 16, 0>, "f16 32x32x16 + 16 fma", wps);
      run_b(bundle<1, 32, 0>, "f16 32x32x16 + 32 fma", wps);
      run_b(bundle<1, 16, 16>, "f16 32x32x16 + 16 fma + 16 exp", wps);
      run_b(bundle<2, 0, 0>, "i8 16x16x64", wps);
      run_b(bundle<2, 16, 0>, "i8 16x16x64 + 16 fma", wps);
      run_b(bundle<3, 0, 0>, "i8 32x32x32", wps);
      run_b(bundle<3, 32, 0>, "i8 32x32x32 + 32 fma", wps);
      run_b(bundle<3, 16, 16>, "i8 32x32x32 + 16 fma + 16 exp", wps);
    }
    printf("done\n");
    return 0;
  }

  // ---- MFMA rates, 1 and 2 waves per SIMD
  const int iters = 20000;
  for (int wps = 1; wps <= 2; ++wps) {
    const int nb = ncu * wps;
    const double waves = nb * 4.0;
    double ghz;
    float ms;
    ms = time_ms([&] { hipLaunchKernelGGL((mfma_rate<0, 8>), dim3(nb), dim3(256), 0, 0, out, clk, iters); }, 3);
    clkinfo(&ghz);
    double ops = waves * iters * 8 * 16.0 * 16 * 64 * 2;
    printf("mfma i8 16x16x64   wps=%d: %.3f ms  %.1f TOP/s  memtime/realtime clock %.3f GHz  cycles/MFMA/SIMD %.2f\n", wps,
           ms, ops / ms / 1e9, ghz, ms * 1e-3 * ghz * 1e9 / (iters * 8.0 * wps));
    ms = time_ms([&] { hipLaunchKernelGGL((mfma_rate<1, 8>), dim3(nb), dim3(256), 0, 0, out, clk, iters); }, 3);
    clkinfo(&ghz);
    ops = waves * iters * 8 * 16.0 * 16 * 32 * 2;
    printf("mfma f16 16x16x32  wps=%d: %.3f ms  %.1f TFLOP/s  clock %.3f GHz  cycles/MFMA/SIMD %.2f\n", wps, ms,
           ops / ms / 1e9, ghz, ms * 1e-3 * ghz * 1e9 / (iters * 8.0 * wps));
    ms = time_ms([&] { hipLaunchKernelGGL((mfma_rate<2, 8>), dim3(nb), dim3(256), 0, 0, out, clk, iters); }, 3);
    clkinfo(&ghz);
    printf("mfma bf16 16x16x32 wps=%d: %.3f ms  %.1f TFLOP/s  clock %.3f GHz  cycles/MFMA/SIMD %.2f\n", wps, ms,
           ops / ms / 1e9, ghz, ms * 1e-3 * ghz * 1e9 / (iters * 8.0 * wps));
    fflush(stdout);
  }
  // dependent chains: 4 and 2 accumulators
  {
    double ghz;
    float ms = time_ms([&] { hipLaunchKernelGGL((mfma_rate<1, 2>), dim3(ncu), dim3(256), 0, 0, out, clk, iters * 4); }, 3);
    clkinfo(&ghz);
    printf("mfma f16 2 chains wps=1: cycles/MFMA %.2f\n", ms * 1e-3 * ghz * 1e9 / (iters * 8.0));
    ms = time_ms([&] { hipLaunchKernelGGL((mfma_rate<1, 4>), dim3(ncu), dim3(256), 0, 0, out, clk, iters * 2); }, 3);
    clkinfo(&ghz);
    printf("mfma f16 4 chains wps=1: cycles/MFMA %.2f\n", ms * 1e-3 * ghz * 1e9 / (iters * 8.0));
    fflush(stdout);
  }

  // ---- MFMA + VALU mixes: cycles per iteration (4 MFMAs + NV VALU) per wave slot
  const int mit = 10000;
  const char* opn[5] = {"fma_f32", "exp_f32", "cvt_f32_i32", "cvt_pkrtz", "max_i32"};
  auto run_mix = [&](auto kern, const char* name, int nv, int wps) {
    const int nb = ncu * wps;
    double ghz;
    float ms = time_ms([&] { hipLaunchKernelGGL(kern, dim3(nb), dim3(256), 0, 0, out, clk, mit); }, 3);
    clkinfo(&ghz);
    printf("%-12s NV=%2d wps=%d: %.3f ms, SIMD cycles per iteration-wave %.1f (4 MFMA = %.0f at 16)\n", name, nv, wps,
           ms, ms * 1e-3 * ghz * 1e9 / (mit * (double)wps), 64.0);
    fflush(stdout);
  };
  for (int wps = 1; wps <= 2; ++wps) {
    run_mix(mix<16, 0, true>, "mfma+fma", 16, wps);
    run_mix(mix<16, 0, false>, "fma only", 16, wps);
    run_mix(mix<32, 0, true>, "mfma+fma", 32, wps);
    run_mix(mix<32, 0, false>, "fma only", 32, wps);
    run_mix(mix<8, 1, true>, "mfma+exp", 8, wps);
    run_mix(mix<8, 1, false>, "exp only", 8, wps);
    run_mix(mix<16, 1, true>, "mfma+exp", 16, wps);
    run_mix(mix<16, 1, false>, "exp only", 16, wps);
    run_mix(mix<16, 2, false>, "cvt_f32_i32", 16, wps);
    run_mix(mix<16, 3, false>, "cvt_pkrtz", 16, wps);
    run_mix(mix<16, 4, false>, "max_i32", 16, wps);
    run_mix(mix<16, 4, true>, "mfma+max_i32", 16, wps);
    run_mix(mix<4, 0, true>, "mfma only", 4, wps);
  }

  // ---- cross-wave co-execution: MFMA waves and VALU waves sharing SIMDs
  {
    const int im = 10000;   // 40000 MFMAs per MFMA wave
    const int ivf = 10000;  // 160000 fma per VALU wave (= 4 per MFMA)
    const int ive = 5000;   // 80000 exp per VALU wave (= 2 per MFMA)
    double ghz;
    auto cyc = [&](float ms) { return ms * 1e-3 * ghz * 1e9; };
    float m_only = time_ms([&] { hipLaunchKernelGGL((split<0>), dim3(ncu), dim3(512), 0, 0, out, clk, im, 0); }, 3);
    clkinfo(&ghz);
    printf("split: MFMA waves only (40000 MFMA/wave): %.0f cycles (%.2f per MFMA)\n", cyc(m_only), cyc(m_only) / 40000);
    float vf = time_ms([&] { hipLaunchKernelGGL((split<0>), dim3(ncu), dim3(512), 0, 0, out, clk, 0, ivf); }, 3);
    clkinfo(&ghz);
    printf("split: fma waves only (160000 fma/wave): %.0f cycles (%.2f per fma)\n", cyc(vf), cyc(vf) / 160000);
    float bf = time_ms([&] { hipLaunchKernelGGL((split<0>), dim3(ncu), dim3(512), 0, 0, out, clk, im, ivf); }, 3);
    clkinfo(&ghz);
    printf("split: MFMA + fma waves together: %.0f cycles\n", cyc(bf));
    float ve = time_ms([&] { hipLaunchKernelGGL((split<1>), dim3(ncu), dim3(512), 0, 0, out, clk, 0, ive); }, 3);
    clkinfo(&ghz);
    printf("split: exp waves only (80000 exp/wave): %.0f cycles (%.2f per exp)\n", cyc(ve), cyc(ve) / 80000);
    float be = time_ms([&] { hipLaunchKernelGGL((split<1>), dim3(ncu), dim3(512), 0, 0, out, clk, im, ive); }, 3);
    clkinfo(&ghz);
    printf("split: MFMA + exp waves together: %.0f cycles\n", cyc(be));
    fflush(stdout);
  }

  // ---- LDS read bandwidth (bytes per clock per CU)
  for (int wgs = 1; wgs <= 2; ++wgs) {
    const int nb = ncu * wgs;
    const int lit = 20000;
    double ghz;
    float ms = time_ms([&] { hipLaunchKernelGGL(lds_read, dim3(nb), dim3(256), 0, 0, out, clk, lit); }, 3);
    clkinfo(&ghz);
    const double bytes = (double)nb * 4 * lit * 8 * 1024;
    printf("lds ds_read_b128 wg/CU=%d: %.3f ms, %.1f TB/s, %.1f B/clk/CU\n", wgs, ms, bytes / ms / 1e9,
           bytes / ncu / (ms * 1e-3 * ghz * 1e9));
    fflush(stdout);
  }

  // ---- HBM
  const size_t nbytes = size_t(4) << 30;
  u32x4 *a, *b;
  CHECK(hipMalloc(&a, nbytes));
  CHECK(hipMalloc(&b, nbytes / 2));
  CHECK(hipMemset(a, 1, nbytes));
  CHECK(hipMemset(b, 0, nbytes / 2));
  for (int g : {ncu * 2, ncu * 4, ncu * 8}) {
    float ms = time_ms([&] { hipLaunchKernelGGL(hbm_read, dim3(g), dim3(256), 0, 0, a, nbytes / 16, out); }, 5);
    printf("hbm read 4 GiB, %d blocks: %.3f ms, %.2f TB/s\n", g, ms, nbytes / ms / 1e9);
    fflush(stdout);
  }
  for (int g : {ncu * 4, ncu * 8}) {
    float ms = time_ms([&] { hipLaunchKernelGGL(hbm_copy, dim3(g), dim3(256), 0, 0, a, b, nbytes / 32); }, 5);
    printf("hbm copy 2 GiB -> 2 GiB, %d blocks: %.3f ms, %.2f TB/s (read + write)\n", g, ms, nbytes / ms / 1e9);
    fflush(stdout);
  }
  CHECK(hipFree(a));
  CHECK(hipFree(b));
  CHECK(hipFree(out));
  CHECK(hipFree(clk));
  printf("done\n");
  return 0;
}
