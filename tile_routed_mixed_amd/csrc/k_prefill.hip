// Fused tile-routed causal prefill for gfx950.
//
// [TriAttention] "TriAttention: Unified Sparse Mixed-Precision Attention for
// Long-Context LLM Inference", abstract: a fused kernel walks the
// precision-grouped traversal, skips omitted tiles and combines the 4-bit and
// 8-bit QK contributions into one normalized attention output.
// [TileMix] "TileMix: Tile-Centric Mixed-Precision Attention for LLM Inference
// Acceleration", abstract: FP16 or INT8 score tiles, both paths updating one
// shared online-softmax state; grouped-query attention; variable lengths.
//
// Design (gfx950, 64-wide waves):
//  * one workgroup of 4 waves per work item (sequence, query head, query tile
//    of BQ rows); each wave owns BQ/4 query rows for the whole item;
//  * scores are computed transposed, S^T = K Q^T, with 16x16 MFMA tiles:
//    INT8 and INT4 tiles on v_mfma_i32_16x16x64_i8 (INT4 nibbles are widened
//    in registers to int8 holding 16x the code, so the product is exact and
//    256x the code product), FP16 tiles on v_mfma_f32_16x16x32_{f16,bf16};
//    the transposed layout leaves every lane with keys of a single query row,
//    so the running max/sum/rescale of the online softmax are lane-local up to
//    a 4-lane reduction, and the fp16 probabilities are already in the
//    register layout of the B operand of the PV product;
//  * PV runs as O^T += V^T P^T on v_mfma_f32_16x16x32_f16; V arrives already
//    transposed per 64-token block in fp16 (written once by the quantize
//    pass), so LDS staging is a plain copy;
//  * K rows are fed to the QK MFMA in an interleaved order (sigma below) that
//    makes each lane's 8 probabilities per 32-key chunk contiguous keys, so
//    one 16-byte LDS read fetches the matching V^T operand;
//  * the next tile's K/V are fetched from global memory into registers while
//    the current tile is computed, then stored to LDS;
//  * workgroups are remapped so the 4 query heads of a GQA group run on the
//    same XCD (dispatch is round-robin over the 8 XCDs) and share K/V in L2.
#include "tm_kernels.h"

namespace tmx {


// Key row (0..63) of a 64-key tile that feeds row m of 16-key MFMA block kb.
__device__ __forceinline__ int sigma(int kb, int m) {
  return 32 * (kb >> 1) + 8 * (m >> 2) + 4 * (kb & 1) + (m & 3);
}

// 8 packed INT4 codes (one dword) -> two dwords of int8 holding 16 * code.
__device__ __forceinline__ i32x4 widen_nibbles(u32x2 p) {
  i32x4 r;
  r[0] = static_cast<int>((p[0] << 4) & 0xF0F0F0F0u);
  r[1] = static_cast<int>(p[0] & 0xF0F0F0F0u);
  r[2] = static_cast<int>((p[1] << 4) & 0xF0F0F0F0u);
  r[3] = static_cast<int>(p[1] & 0xF0F0F0F0u);
  return r;
}

__device__ __forceinline__ uint32_t remap_block(uint32_t b, uint32_t n) {
  constexpr uint32_t kXcd = 8, kGroup = 4, kChunk = kXcd * kGroup;
  const uint32_t full = (n / kChunk) * kChunk;
  if (b >= full) return b;
  const uint32_t c = b / kChunk, r = b % kChunk;
  return c * kChunk + (r % kXcd) * kGroup + r / kXcd;
}

template <int D, int BQ, bool BF16, bool DBG>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  constexpr int RW = BQ / 4;       // query rows per wave
  constexpr int QB = RW / 16;      // 16-row MFMA blocks per wave
  constexpr int NC8 = D / 64;      // i8 MFMA k-chunks
  constexpr int NC16 = D / 32;     // f16 MFMA k-chunks
  constexpr int ND = D / 16;       // output channel blocks
  constexpr int KROW8 = D + 16;    // LDS row pitch (bytes) per K precision
  constexpr int KROW4 = D / 2 + 16;
  constexpr int KROW16 = 2 * D + 16;
  constexpr int VROW = 2 * kBlock + 16;
  constexpr int VCH = D * kBlock * 2 / 16 / 256;   // 16-byte V chunks per thread
  constexpr int KCH = 2 * D * kBlock / 16 / 256;   // max K chunks per thread (fp16)
  typedef typename std::conditional<BF16, bf16x8, f16x8>::type q16_t;

  __shared__ __align__(16) uint8_t lds_k[kBlock * KROW16];
  __shared__ __align__(16) uint8_t lds_v[D * VROW];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const TravHeader* th = reinterpret_cast<const TravHeader*>(a.trav);
  const uint32_t item_idx = remap_block(blockIdx.x, a.n_items);
  const ItemEntry it = reinterpret_cast<const ItemEntry*>(a.trav + th->item_off)[item_idx];
  const SeqEntry se = reinterpret_cast<const SeqEntry*>(a.trav + th->seq_off)[it.seq];
  const RunEntry* runs = reinterpret_cast<const RunEntry*>(a.trav + th->run_off) +
                         static_cast<size_t>(item_idx) * th->max_runs;
  const int head = it.head, kv = head / (a.hq / a.hkv);
  const int len = se.len;
  const int nbs = (len + kBlock - 1) / kBlock;          // blocks of this sequence
  const int qrow0 = it.qtile * BQ + w * RW;             // first sequence row of the wave
  const int qblk = qrow0 / kBlock;
  const bool qblk_ok = qblk < nbs;
  const size_t qblk_g = static_cast<size_t>(head) * a.nblk + se.blk_start + qblk;

  // ---- resident Q operands (B operand of S^T = K Q^T)
  i32x4 q8[QB][NC8];
  i32x4 q4[QB][NC8];
  q16_t q16[QB][NC16];
  const bool has16 = th->kind == TM_POLICY_BITMASK;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = qrow0 + qb * 16 + l16;
    const int rb = r % kBlock;
#pragma unroll
    for (int c = 0; c < NC8; ++c) {
      if (qblk_ok) {
        q8[qb][c] = *reinterpret_cast<const i32x4*>(a.q8 + (qblk_g * kBlock + rb) * D + c * 64 + g * 16);
        q4[qb][c] = widen_nibbles(
            *reinterpret_cast<const u32x2*>(a.q4 + (qblk_g * kBlock + rb) * (D / 2) + c * 32 + g * 8));
      } else {
        q8[qb][c] = i32x4{0, 0, 0, 0};
        q4[qb][c] = i32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int c = 0; c < NC16; ++c) {
      if (has16 && r < len) {
        const uint16_t* src = a.q + (static_cast<size_t>(se.tok_start + r) * a.hq + head) * D + c * 32 + g * 8;
        u32x4 raw = *reinterpret_cast<const u32x4*>(src);
        __builtin_memcpy(&q16[qb][c], &raw, 16);
      } else {
        u32x4 z = {0, 0, 0, 0};
        __builtin_memcpy(&q16[qb][c], &z, 16);
      }
    }
  }
  const float sq8 = qblk_ok ? a.qs8[qblk_g] : 0.0f;
  const float sq4 = qblk_ok ? a.qs4[qblk_g] : 0.0f;

  float m_run[QB], l_run[QB];
  f32x4 oacc[ND][QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegBig;
    l_run[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- tile iterator over the runs
  const int nruns = static_cast<int>(it.nruns);
  int ri = 0, roff = 0;
  uint32_t r_first = 0, r_count = 0, r_prec = 0;
  if (nruns > 0) {
    r_first = runs[0].ktile;
    r_count = runs[0].count_prec & 0xFFFFFFu;
    r_prec = runs[0].count_prec >> 24;
  }

  // global -> register prefetch of one tile's K and V^T
  u32x4 pk[KCH], pv[VCH];
  auto fetch = [&](int j, uint32_t prec) {
    const size_t kblk = static_cast<size_t>(kv) * a.nblk + se.blk_start + j;
    const uint16_t* vsrc = a.vt16 + kblk * D * kBlock;
#pragma unroll
    for (int i = 0; i < VCH; ++i)
      pv[i] = *reinterpret_cast<const u32x4*>(vsrc + (i * 256 + tid) * 8);
    if (prec == TM_INT8) {
      constexpr int n = kBlock * D / 16;
      const int8_t* src = a.k8 + kblk * kBlock * D;
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int ci = i * 256 + tid;
        if (ci < n) pk[i] = *reinterpret_cast<const u32x4*>(src + ci * 16);
      }
    } else if (prec == TM_INT4) {
      constexpr int n = kBlock * D / 2 / 16;
      const uint8_t* src = a.k4 + kblk * kBlock * (D / 2);
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int ci = i * 256 + tid;
        if (ci < n) pk[i] = *reinterpret_cast<const u32x4*>(src + ci * 16);
      }
    } else {
      constexpr int n = kBlock * D * 2 / 16;
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int ci = i * 256 + tid;
        if (ci < n) {
          const int row = (ci * 16) / (2 * D), col = (ci * 16) % (2 * D);
          const int key = j * kBlock + row;
          if (key < len) {
            const uint8_t* src = reinterpret_cast<const uint8_t*>(a.k) +
                                 (static_cast<size_t>(se.tok_start + key) * a.hkv + kv) * D * 2 + col;
            pk[i] = *reinterpret_cast<const u32x4*>(src);
          } else {
            pk[i] = u32x4{0, 0, 0, 0};
          }
        }
      }
    }
  };
  auto stash = [&](uint32_t prec) {
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int off = (i * 256 + tid) * 16;
      *reinterpret_cast<u32x4*>(lds_v + (off / 128) * VROW + off % 128) = pv[i];
    }
    const int n = prec == TM_INT8 ? kBlock * D / 16 : prec == TM_INT4 ? kBlock * D / 32 : kBlock * D / 8;
    const int rowb = prec == TM_INT8 ? D : prec == TM_INT4 ? D / 2 : 2 * D;
    const int pitch = prec == TM_INT8 ? KROW8 : prec == TM_INT4 ? KROW4 : KROW16;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ci = i * 256 + tid;
      if (ci < n) {
        const int off = ci * 16;
        *reinterpret_cast<u32x4*>(lds_k + (off / rowb) * pitch + off % rowb) = pk[i];
      }
    }
  };

  int cur_j = static_cast<int>(r_first);
  uint32_t cur_p = r_prec;
  bool have = nruns > 0;
  if (have) fetch(cur_j, cur_p);

  while (have) {
    // advance the iterator to the next tile
    int nxt_j = -1;
    uint32_t nxt_p = 0;
    {
      ++roff;
      if (roff >= static_cast<int>(r_count)) {
        ++ri;
        roff = 0;
        if (ri < nruns) {
          r_first = runs[ri].ktile;
          r_count = runs[ri].count_prec & 0xFFFFFFu;
          r_prec = runs[ri].count_prec >> 24;
        }
      }
      if (ri < nruns) {
        nxt_j = static_cast<int>(r_first) + roff;
        nxt_p = r_prec;
      }
    }
    __syncthreads();               // previous tile's LDS reads are done
    stash(cur_p);
    __syncthreads();
    if (nxt_j >= 0) fetch(nxt_j, nxt_p);

    const int j = cur_j;
    const uint32_t prec = cur_p;
    const size_t kblk = static_cast<size_t>(kv) * a.nblk + se.blk_start + j;

    // ---- S^T = K Q^T for the wave's rows
    float s[4][QB][4];
    if (prec == TM_FP16) {
      f32x4 acc[4][QB];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint8_t* krow = lds_k + sigma(kb, l16) * KROW16;
#pragma unroll
        for (int c = 0; c < NC16; ++c) {
          q16_t av;
          u32x4 raw = *reinterpret_cast<const u32x4*>(krow + (c * 32 + g * 8) * 2);
          __builtin_memcpy(&av, &raw, 16);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            if constexpr (BF16)
              acc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, q16[qb][c], acc[kb][qb], 0, 0, 0);
            else
              acc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, q16[qb][c], acc[kb][qb], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[kb][qb][i] = acc[kb][qb][i] * a.tau_log2e;
    } else {
      const bool is8 = prec == TM_INT8;
      i32x4 acc[4][QB];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[kb][qb] = i32x4{0, 0, 0, 0};
      if (is8) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const uint8_t* krow = lds_k + sigma(kb, l16) * KROW8;
#pragma unroll
          for (int c = 0; c < NC8; ++c) {
            const i32x4 av = *reinterpret_cast<const i32x4*>(krow + c * 64 + g * 16);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              acc[kb][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, q8[qb][c], acc[kb][qb], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const uint8_t* krow = lds_k + sigma(kb, l16) * KROW4;
#pragma unroll
          for (int c = 0; c < NC8; ++c) {
            const i32x4 av = widen_nibbles(*reinterpret_cast<const u32x2*>(krow + c * 32 + g * 8));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              acc[kb][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, q4[qb][c], acc[kb][qb], 0, 0, 0);
          }
        }
      }
      if constexpr (DBG) {
        for (int e = 0; e < a.n_dbg; ++e) {
          const int32_t* t = a.dbg_tiles + 4 * e;
          if (t[0] == static_cast<int>(it.seq) && t[1] == head && t[2] == static_cast<int>(it.qtile) && t[3] == j) {
            int32_t* dst = a.dbg_qk + static_cast<size_t>(e) * BQ * kBlock;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int row = w * RW + qb * 16 + l16;
                  const int key = sigma(kb, 4 * g + i);
                  dst[row * kBlock + key] = is8 ? acc[kb][qb][i] : (acc[kb][qb][i] >> 8);
                }
          }
        }
      }
      const float sk = is8 ? a.ks8[kblk] : a.ks4[kblk];
      const float cs = is8 ? (sq8 * sk) * a.tau_log2e : (sq4 * sk) * (a.tau_log2e * (1.0f / 256.0f));
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[kb][qb][i] = static_cast<float>(acc[kb][qb][i]) * cs;
    }

    // ---- causal / sequence-end mask (only tiles reaching past the wave's first row)
    if (j * kBlock + kBlock - 1 > qrow0 || j * kBlock + kBlock > len) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = j * kBlock + sigma(kb, 4 * g + i);
            const int row = qrow0 + qb * 16 + l16;
            if (key > row || key >= len) s[kb][qb][i] = -INFINITY;
          }
    }

    // ---- shared online softmax update (log2 domain)
    float alpha[QB];
    bool rescale = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][qb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m_run[qb], mx);
      alpha[qb] = __builtin_amdgcn_exp2f(m_run[qb] - mn);
      rescale |= mn != m_run[qb];
      m_run[qb] = mn;
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(s[kb][qb][i] - mn);
          s[kb][qb][i] = p;
          ps += p;
        }
      l_run[qb] = l_run[qb] * alpha[qb] + ps;
    }
    if (__any(rescale)) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] *= alpha[qb];
    }

    // ---- P^T operands (fp16, round to nearest even)
    f16x8 pb[2][QB];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[c2][qb][i] = static_cast<_Float16>(s[2 * c2][qb][i]);
          pb[c2][qb][4 + i] = static_cast<_Float16>(s[2 * c2 + 1][qb][i]);
        }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const uint8_t* vrow = lds_v + (db * 16 + l16) * VROW;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        f16x8 va;
        u32x4 raw = *reinterpret_cast<const u32x4*>(vrow + (32 * c2 + 8 * g) * 2);
        __builtin_memcpy(&va, &raw, 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[c2][qb], oacc[db][qb], 0, 0, 0);
      }
    }

    have = nxt_j >= 0;
    cur_j = nxt_j;
    cur_p = nxt_p;
  }

  // ---- epilogue: O = O / l, lse
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float lt = l_run[qb] + __shfl_xor(l_run[qb], 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int r = qrow0 + qb * 16 + l16;
    if (r >= len) continue;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const size_t tok = static_cast<size_t>(se.tok_start) + r;
    const size_t obase = (tok * a.hq + head) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const f32x4 v = oacc[db][qb] * inv;
      const size_t off = obase + db * 16 + 4 * g;
      if (a.o_dtype == TM_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + off) = v;
      } else if (a.o_dtype == TM_F16) {
        f16x4 hv = {static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1]), static_cast<_Float16>(v[2]),
                    static_cast<_Float16>(v[3])};
        *reinterpret_cast<f16x4*>(static_cast<_Float16*>(a.o) + off) = hv;
      } else {
        u32x2 bv;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          uint32_t lo = __float_as_uint(v[2 * e]), hi = __float_as_uint(v[2 * e + 1]);
          lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
          hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
          bv[e] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.o) + off) = bv;
      }
    }
    if (a.lse != nullptr && g == 0)
      a.lse[static_cast<size_t>(head) * a.T + tok] = (m_run[qb] + __builtin_amdgcn_logf(lt)) * kLn2;
  }
}

template <int D, int BQ, bool BF16>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  if (a.n_dbg > 0)
    hipLaunchKernelGGL((prefill_kernel<D, BQ, BF16, true>), dim3(a.n_items), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, BQ, BF16, false>), dim3(a.n_items), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int d, int bq, bool bf16, hipStream_t st) {
  if (a.n_items == 0) return hipSuccess;
  if (d == 128) {
    if (bq == 128) return bf16 ? launch_prefill_t<128, 128, true>(a, st) : launch_prefill_t<128, 128, false>(a, st);
    return bf16 ? launch_prefill_t<128, 64, true>(a, st) : launch_prefill_t<128, 64, false>(a, st);
  }
  if (bq == 128) return bf16 ? launch_prefill_t<64, 128, true>(a, st) : launch_prefill_t<64, 128, false>(a, st);
  return bf16 ? launch_prefill_t<64, 64, true>(a, st) : launch_prefill_t<64, 64, false>(a, st);
}

}  // namespace tmx
