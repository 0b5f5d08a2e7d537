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
//    of BQ rows); each wave owns BQ/4 query rows for the whole item and keeps
//    their Q operands in registers;
//  * scores are computed transposed, S^T = K Q^T, with 16x16 MFMA tiles:
//    INT8 and INT4 tiles on v_mfma_i32_16x16x64_i8 (INT4 nibbles are widened
//    in registers to int8 holding 16x the code, so the product is exact and
//    256x the code product), FP16 tiles on v_mfma_f32_16x16x32_{f16,bf16};
//    every lane then holds keys of one query row, so the online-softmax max,
//    sum and rescale are lane-local up to a 4-lane reduction, and the fp16
//    probabilities are already in the B-operand layout of the PV product;
//  * PV runs as O^T += V^T P^T on v_mfma_f32_16x16x32_f16.  V arrives
//    transposed per 64-token block in fp16 (written once by the quantize
//    pass), K rows are fed to the QK MFMA in an interleaved order (sigma) that
//    makes each lane's 8 probabilities per 32-key chunk contiguous keys, so a
//    single 16-byte LDS read fetches the matching V^T operand;
//  * K and V^T tiles are copied global -> LDS with the direct-to-LDS 16-byte
//    load (no register staging) into two buffers: the next tile streams in
//    while the current one is computed, with one barrier per tile.  16-byte
//    chunks are XOR-swizzled by row so the MFMA operand reads are free of
//    bank conflicts;
//  * the running max is updated lazily: the probabilities are re-based (and O
//    and the sum rescaled) only when a row's max grows by more than 8 in log2
//    units, so p <= 256 stays exact enough in fp16 and rescales are rare;
//  * row maxima of integer tiles are taken on the int32 accumulators (the
//    per-row scale is positive), before any conversion;
//  * workgroups are remapped so the 4 query heads of a GQA group run on the
//    same XCD (dispatch is round-robin over the 8 XCDs) and share K/V in L2.
#include "tm_kernels.h"

namespace tmx {

// Key row (0..63) of a 64-key tile that feeds row m of 16-key MFMA block kb.
__device__ __forceinline__ int sigma(int kb, int m) {
  return 32 * (kb >> 1) + 8 * (m >> 2) + 4 * (kb & 1) + (m & 3);
}

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

__device__ __forceinline__ uint32_t remap_block(uint32_t b, uint32_t n) {
  constexpr uint32_t kXcd = 8, kGroup = 4, kChunk = kXcd * kGroup;
  const uint32_t full = (n / kChunk) * kChunk;
  if (b >= full) return b;
  const uint32_t c = b / kChunk, r = b % kChunk;
  return c * kChunk + (r % kXcd) * kGroup + r / kXcd;
}

// Copy a tile region of ROWS rows x NCH 16-byte chunks from global memory into
// swizzled LDS with direct-to-LDS loads.  Instruction n (of ROWS*NCH/64) moves
// LDS bytes [n*1024, n*1024+1024); lane L lands at n*1024 + 16*L, which is row
// (n*1024 + 16L) / (16 NCH), swizzled slot (L mod NCH): it loads the logical
// chunk slot ^ swz(row).  `src(row)` gives the row's global address.
template <int ROWS, int NCH, bool VT, typename SrcFn>
__device__ __forceinline__ void load_tile(uint8_t* lds, int w, int lane, SrcFn src) {
  constexpr int NI = ROWS * NCH / 64;   // 1 KiB instructions for the region
  auto one = [&](int n) {
    const int off = n * 1024 + lane * 16;
    const int row = off / (NCH * 16);
    const int slot = (off / 16) % NCH;
    const int c = slot ^ swz<NCH, VT>(row);
    const uint8_t* g = src(row) + c * 16;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(g), reinterpret_cast<void*>(lds + n * 1024),
                                     16, 0, 0);
  };
  if constexpr (NI >= 4) {
    static_assert(NI % 4 == 0, "tile regions are whole multiples of 4 KiB");
#pragma unroll
    for (int i = 0; i < NI / 4; ++i) one(i * 4 + w);
  } else {
    if (w < NI) one(w);
  }
}

template <int D, int BQ, int KIND, bool BF16, bool DBG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(PrefillArgs a) {
  constexpr int RW = BQ / 4;       // query rows per wave
  constexpr int QB = RW / 16;      // 16-row MFMA blocks per wave
  constexpr int NC8 = D / 64;      // i8 MFMA k-chunks (64 bytes of d each)
  constexpr int NC16 = D / 32;     // f16 MFMA k-chunks
  constexpr int ND = D / 16;       // output channel blocks
  constexpr int KBYTES = KIND == 0 ? kBlock * D : kBlock * 2 * D;   // largest K tile
  constexpr int VBYTES = D * kBlock * 2;
  constexpr int BUF = KBYTES + VBYTES;
  constexpr bool HAS4 = KIND == TM_POLICY_BOUNDARIES;
  constexpr bool HAS16 = KIND == TM_POLICY_BITMASK;
  typedef typename std::conditional<BF16, bf16x8, f16x8>::type q16_t;

  __shared__ __align__(1024) uint8_t lds[2 * BUF];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const TravHeader* th = reinterpret_cast<const TravHeader*>(a.trav);
  if (th->kind != static_cast<uint32_t>(KIND)) return;   // traversal of another policy kind
  const uint32_t item_idx = remap_block(blockIdx.x, a.n_items);
  const ItemEntry it = reinterpret_cast<const ItemEntry*>(a.trav + th->item_off)[item_idx];
  const SeqEntry se = reinterpret_cast<const SeqEntry*>(a.trav + th->seq_off)[it.seq];
  const RunEntry* runs = reinterpret_cast<const RunEntry*>(a.trav + th->run_off) +
                         static_cast<size_t>(item_idx) * th->max_runs;
  const int head = it.head, kv = head / (a.hq / a.hkv);
  const int len = se.len;
  const int nbs = (len + kBlock - 1) / kBlock;
  const int qrow0 = it.qtile * BQ + w * RW;
  const int qblk = qrow0 / kBlock;
  const bool qblk_ok = qblk < nbs;
  const size_t qblk_g = static_cast<size_t>(head) * a.nblk + se.blk_start + qblk;
  const size_t kv_blk0 = static_cast<size_t>(kv) * a.nblk + se.blk_start;

  // ---- tile iterator over the runs (uniform across the workgroup)
  const int nruns = static_cast<int>(it.nruns);
  int ri = 0, roff = 0;
  int r_first = 0, r_count = 0, r_prec = 0;
  if (nruns > 0) {
    const RunEntry r0 = runs[0];
    r_first = static_cast<int>(r0.ktile);
    r_count = static_cast<int>(r0.count_prec & 0xFFFFFFu);
    r_prec = static_cast<int>(r0.count_prec >> 24);
  }

  // Start loading tile j into `buf` and fetch its K scale (read after the next
  // barrier, when every load of the tile has been waited for).
  auto issue = [&](int j, int prec, uint8_t* buf, float& sk) {
    const size_t kb = kv_blk0 + j;
    sk = prec == TM_INT8 ? a.ks8[kb] : ((HAS4 && prec == TM_INT4) ? a.ks4[kb] : 0.0f);
    uint8_t* kl = buf;
    uint8_t* vl = buf + KBYTES;
    const uint8_t* vsrc = reinterpret_cast<const uint8_t*>(a.vt16) + kb * VBYTES;
    load_tile<D, 8, true>(vl, w, lane, [&](int row) { return vsrc + row * 128; });
    if (prec == TM_INT8) {
      const uint8_t* ks = reinterpret_cast<const uint8_t*>(a.k8) + kb * kBlock * D;
      load_tile<kBlock, D / 16, false>(kl, w, lane, [&](int row) { return ks + row * D; });
    } else if (HAS4 && prec == TM_INT4) {
      const uint8_t* ks = a.k4 + kb * kBlock * (D / 2);
      load_tile<kBlock, D / 32, false>(kl, w, lane, [&](int row) { return ks + row * (D / 2); });
    } else if (HAS16) {
      const int last = len - 1 - j * kBlock;   // clamp rows past the sequence end (masked later)
      const uint8_t* ks = reinterpret_cast<const uint8_t*>(a.k) +
                          (static_cast<size_t>(se.tok_start + j * kBlock) * a.hkv + kv) * D * 2;
      const size_t pitch = static_cast<size_t>(a.hkv) * D * 2;
      load_tile<kBlock, D / 8, false>(kl, w, lane, [&](int row) { return ks + min(row, last) * pitch; });
    }
  };

  // issue the first tile before the Q loads so both are in flight together
  float sk_cur = 0.0f, sk_nxt = 0.0f;
  if (nruns > 0) issue(r_first, r_prec, lds, sk_nxt);

  // ---- resident Q operands (B operand of S^T = K Q^T)
  i32x4 q8[QB][NC8];
  i32x4 q4[QB][NC8];
  q16_t q16[QB][NC16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = qrow0 + qb * 16 + l16;
    const int rb = r % kBlock;
#pragma unroll
    for (int c = 0; c < NC8; ++c)
      q8[qb][c] = qblk_ok ? *reinterpret_cast<const i32x4*>(a.q8 + (qblk_g * kBlock + rb) * D + c * 64 + g * 16)
                          : i32x4{0, 0, 0, 0};
    if constexpr (HAS4) {
      // lane group g holds channels 32g .. 32g+31: packed bytes 16g .. 16g+15
      if constexpr (D == 128) {
        u32x4 p = qblk_ok ? *reinterpret_cast<const u32x4*>(a.q4 + (qblk_g * kBlock + rb) * (D / 2) + g * 16)
                          : u32x4{0, 0, 0, 0};
        q4[qb][0] = widen_nibbles(p[0], p[1]);
        q4[qb][1] = widen_nibbles(p[2], p[3]);
      } else {
        u32x2 p = qblk_ok ? *reinterpret_cast<const u32x2*>(a.q4 + (qblk_g * kBlock + rb) * (D / 2) + g * 8)
                          : u32x2{0, 0};
        q4[qb][0] = widen_nibbles(p[0], p[1]);
      }
    }
    if constexpr (HAS16) {
#pragma unroll
      for (int c = 0; c < NC16; ++c) {
        u32x4 raw = u32x4{0, 0, 0, 0};
        if (r < len)
          raw = *reinterpret_cast<const u32x4*>(a.q + (static_cast<size_t>(se.tok_start + r) * a.hq + head) * D +
                                                 c * 32 + g * 8);
        __builtin_memcpy(&q16[qb][c], &raw, 16);
      }
    }
  }
  const float sq8 = qblk_ok ? a.qs8[qblk_g] : 0.0f;
  const float sq4 = (HAS4 && qblk_ok) ? a.qs4[qblk_g] : 0.0f;

  float m_use[QB], l_run[QB];
  f32x4 oacc[ND][QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_use[qb] = kNegBig;
    l_run[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  int cur_j = r_first, cur_p = r_prec;
  bool have = nruns > 0;
  int buf = 0;
  while (have) {
    // next tile of the traversal
    int nxt_j = -1, nxt_p = 0;
    if (++roff >= r_count) {
      ++ri;
      roff = 0;
      if (ri < nruns) {
        const RunEntry rr = runs[ri];
        r_first = static_cast<int>(rr.ktile);
        r_count = static_cast<int>(rr.count_prec & 0xFFFFFFu);
        r_prec = static_cast<int>(rr.count_prec >> 24);
      }
    }
    if (ri < nruns) {
      nxt_j = r_first + roff;
      nxt_p = r_prec;
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of the current tile have landed
    __syncthreads();                 // ... and everyone's; the other buffer is free
    sk_cur = sk_nxt;
    if (nxt_j >= 0) issue(nxt_j, nxt_p, lds + (buf ^ 1) * BUF, sk_nxt);

    const uint8_t* kl = lds + buf * BUF;
    const uint8_t* vl = kl + KBYTES;
    const int j = cur_j;
    const int prec = cur_p;
    const bool need_mask = (j * kBlock + kBlock - 1 > qrow0) || (j * kBlock + kBlock > len);

    // ---- S^T = K Q^T, then scores in log2 units
    float s[4][QB][4];
    float mx[QB];
    if (HAS16 && prec == TM_FP16) {
      f32x4 acc[4][QB];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int row = sigma(kb, l16);
#pragma unroll
        for (int c = 0; c < NC16; ++c) {
          q16_t av;
          const u32x4 raw = *reinterpret_cast<const u32x4*>(kl + lds_off<D / 8, false>(row, 4 * c + g));
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
      for (int qb = 0; qb < QB; ++qb) {
        mx[qb] = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = acc[kb][qb][i] * a.tau_log2e;
            if (need_mask) {
              const int key = j * kBlock + sigma(kb, 4 * g + i);
              if (key > qrow0 + qb * 16 + l16 || key >= len) x = -INFINITY;
            }
            s[kb][qb][i] = x;
            mx[qb] = fmaxf(mx[qb], x);
          }
      }
    } else {
      const bool is8 = !HAS4 || prec == TM_INT8;
      i32x4 acc[4][QB];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[kb][qb] = i32x4{0, 0, 0, 0};
      if (is8) {
        i32x4 av[4][NC8];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int c = 0; c < NC8; ++c)
            av[kb][c] = *reinterpret_cast<const i32x4*>(kl + lds_off<D / 16, false>(sigma(kb, l16), 4 * c + g));
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int c = 0; c < NC8; ++c)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              acc[kb][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[kb][c], q8[qb][c], acc[kb][qb], 0, 0, 0);
      } else if constexpr (HAS4) {
        if constexpr (D == 128) {
          u32x4 pk[4];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            pk[kb] = *reinterpret_cast<const u32x4*>(kl + lds_off<4, false>(sigma(kb, l16), g));
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const i32x4 a0 = widen_nibbles(pk[kb][0], pk[kb][1]);
            const i32x4 a1 = widen_nibbles(pk[kb][2], pk[kb][3]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              acc[kb][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, q4[qb][0], acc[kb][qb], 0, 0, 0);
              acc[kb][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, q4[qb][1], acc[kb][qb], 0, 0, 0);
            }
          }
        } else {
          // D == 64: rows of 32 packed bytes = 2 chunks; lane group g reads 8 bytes
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const int row = sigma(kb, l16);
            const u32x2 p = *reinterpret_cast<const u32x2*>(kl + lds_off<2, false>(row, g >> 1) + (g & 1) * 8);
            const i32x4 a0 = widen_nibbles(p[0], p[1]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              acc[kb][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, q4[qb][0], acc[kb][qb], 0, 0, 0);
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
                for (int i = 0; i < 4; ++i)
                  dst[(w * RW + qb * 16 + l16) * kBlock + sigma(kb, 4 * g + i)] =
                      is8 ? acc[kb][qb][i] : (acc[kb][qb][i] >> 8);
          }
        }
      }
      const float cs = is8 ? (sq8 * sk_cur) * a.tau_log2e : (sq4 * sk_cur) * (a.tau_log2e * (1.0f / 256.0f));
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          mx[qb] = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = j * kBlock + sigma(kb, 4 * g + i);
              float x = static_cast<float>(acc[kb][qb][i]) * cs;
              if (key > qrow0 + qb * 16 + l16 || key >= len) x = -INFINITY;
              s[kb][qb][i] = x;
              mx[qb] = fmaxf(mx[qb], x);
            }
        }
      } else {
        // scale >= 0: the row max of the scores is the scaled max of the integers
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          int im = acc[0][qb][0];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              im = max(im, acc[kb][qb][i]);
              s[kb][qb][i] = static_cast<float>(acc[kb][qb][i]) * cs;
            }
          mx[qb] = static_cast<float>(im) * cs;
        }
      }
    }

    // ---- shared online softmax (log2 domain, lazily re-based)
    bool rebase = false;
    float alpha[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m = fmaxf(mx[qb], __shfl_xor(mx[qb], 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      alpha[qb] = 1.0f;
      if (m > m_use[qb] + 8.0f) {
        alpha[qb] = __builtin_amdgcn_exp2f(m_use[qb] - m);
        m_use[qb] = m;
        rebase = true;
      }
    }
    if (__any(rebase)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        l_run[qb] *= alpha[qb];
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db][qb] *= alpha[qb];
      }
    }
    f16x8 pb[2][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(s[kb][qb][i] - m_use[qb]);
          ps += p;
          pb[kb >> 1][qb][4 * (kb & 1) + i] = static_cast<_Float16>(p);
        }
      l_run[qb] += ps;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int dv = db * 16 + l16;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        f16x8 va;
        const u32x4 raw = *reinterpret_cast<const u32x4*>(vl + lds_off<8, true>(dv, 4 * c2 + g));
        __builtin_memcpy(&va, &raw, 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[c2][qb], oacc[db][qb], 0, 0, 0);
      }
    }

    buf ^= 1;
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
      a.lse[static_cast<size_t>(head) * a.T + tok] = (m_use[qb] + __builtin_amdgcn_logf(lt)) * kLn2;
  }
}

template <int D, int BQ, int KIND, bool BF16>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  if (a.n_dbg > 0)
    hipLaunchKernelGGL((prefill_kernel<D, BQ, KIND, BF16, true>), dim3(a.n_items), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, BQ, KIND, BF16, false>), dim3(a.n_items), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int BQ>
static hipError_t launch_prefill_k(const PrefillArgs& a, int kind, bool bf16, hipStream_t st) {
  if (kind == TM_POLICY_BOUNDARIES)
    return bf16 ? launch_prefill_t<D, BQ, 0, true>(a, st) : launch_prefill_t<D, BQ, 0, false>(a, st);
  return bf16 ? launch_prefill_t<D, BQ, 1, true>(a, st) : launch_prefill_t<D, BQ, 1, false>(a, st);
}

hipError_t launch_prefill(const PrefillArgs& a, int d, int bq, int kind, bool bf16, hipStream_t st) {
  if (a.n_items == 0) return hipSuccess;
  if (d == 128) {
    if (bq == 128) return launch_prefill_k<128, 128>(a, kind, bf16, st);
    return launch_prefill_k<128, 64>(a, kind, bf16, st);
  }
  if (bq == 128) return launch_prefill_k<64, 128>(a, kind, bf16, st);
  return launch_prefill_k<64, 64>(a, kind, bf16, st);
}

}  // namespace tmx
