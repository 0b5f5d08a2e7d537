#!/usr/bin/env python3
"""Benchmark of the tile-routed mixed-precision attention hot path on one GPU.

One step = one pass of the whole path over one batch of synthetic input that
is already resident in HBM:
  tm_quantize_pack(Q), tm_quantize_pack(K), tm_quantize_pack(V, transposed +
  fp16 copy), tm_build_traversal, tm_prefill, and tm_decode of one new query
  per sequence over the compressed cache the prefill just quantized.

Headline workload: the largest one-GPU configuration, one 131072-token
sequence, 32 query / 8 KV heads, d = 128, bf16, 128x64 tiles, K with 4 outlier
channels x10, per-head diagonal-distance boundaries giving about 60 % skipped,
25 % INT4 and 15 % INT8 tiles, key tile 0 kept INT8.  ``value`` is the
effective dense-causal prefill rate of the whole step: 4*d*hq*S^2/2 FLOPs per
step over the measured step time.

Beside it, each with its own roofline object: the decode sub-benchmark (16
sequences x 32768 cached tokens, three caches rotated so the read set exceeds
the last-level cache), the other prefill workloads (toy 512, 8K, varlen 32K,
8K hybrid), the error of every workload against unquantized float64 attention
(reported, not gated), measured hardware ceilings, and the CPU oracle timed on
a bounded sample.

Prints one JSON line.  --gpus N > 1 is refused: this path runs on one GPU.
"""
import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective prefill attn TFLOP/s (dense-causal) + MFMA util; decode KV GB/s"
PEAK_F16 = 2.5e15     # MI355X dense MFMA, fp16/bf16 (FLOP/s)
PEAK_I8 = 5.0e15      # MI355X dense MFMA, int8 (OP/s)
PEAK_HBM = 8.0e12     # MI355X HBM3E (B/s)
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "tile_routed_mixed_amd", "csrc")
HEADLINE = "long128k"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def describe(w, hybrid=None, fourway=False):
    if hybrid is not None:
        pol = (f"hybrid: {hybrid[0] * 100:.0f} % of keys per head selected by the vertical-line pass (attention "
               f"mass from the last 64 rows), {hybrid[1]}-token window in FP16, the rest INT8")
    elif fourway:
        pol = ("four-way: per-head diagonal-distance boundaries plus a 2-bit code per group of 4 key tiles "
               "(0 = the boundaries with probability 1/2, else INT4, INT8 or FP16)")
    elif w.policy == "boundaries":
        pol = "per-head diagonal-distance boundaries"
    else:
        pol = f"packed bitmask, {w.group} key tiles per bit, P(FP16)={w.p_fp16}"
    seqs = w.seqlens if len(w.seqlens) <= 4 else f"{len(w.seqlens)}x{w.seqlens[0]}"
    return (f"{w.name}: seqs {seqs}, {w.hq}/{w.hkv} heads, d={w.d}, {w.dtype}, {w.bq}x{w.bk} tiles, {pol}"
            + (", key tile 0 INT8" if (w.sink or fourway) and hybrid is None else "")
            + (f", K outliers {w.outliers}x{w.outlier_scale:g}" if w.outliers else ""))


def dense_causal_flops(w):
    return sum(4.0 * w.d * w.hq * S * S / 2.0 for S in w.seqlens)


def decode_policy_for(S):
    """Cache tags for the decode step after a prefill of S tokens: the toy
    workload's bands (INT8 below 2/8, INT4 below 5/8 of the blocks) scaled to the
    cache, first block INT8, last 128 tokens FP16."""
    nb = -(-S // 64)
    b8 = max(1, nb // 4)
    return b8, max(b8, (nb * 5) // 8)


def src_sha(*names):
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(CSRC, n), "rb").read())
    return h.hexdigest()


def pmc_traffic(summary, sources):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when it is absent or was taken on other kernel sources."""
    try:
        s = json.load(open(os.path.join(PROFILES, summary)))
    except (OSError, ValueError):
        return None
    if s.get("kernel_source_sha256") != src_sha(*sources):
        return None
    return s.get("hbm_bytes_per_launch")


def prefill_kernel_of(w, hybrid=False, fourway=False):
    """The prefill kernel a workload's policy runs, and its source files:
    boundary policies run the software-pipelined kernel, the other kinds
    (bitmask, four-way, hybrid) prefill_kernel."""
    if w.policy == "boundaries" and not hybrid and not fourway:
        return "prefill_pipe_kernel", ("k_prefill_pipe.hip", "k_prefill_common.h")
    return "prefill_kernel", ("k_prefill.hip", "k_prefill_common.h")


def prefill_roofline(w, census, t_ms, traffic=None, hybrid=False, fourway=False):
    """Roofline of the prefill kernel: executed ops (both contractions of every
    executed tile, masked elements included) over the measured launch time,
    against the precision-weighted MFMA peak of this workload's tiles (INT8
    and INT4 QK at the int8 rate, FP16 QK and every PV at the fp16 rate)."""
    qk = pv = 2.0 * w.bq * w.bk * w.d
    n_int = census["int8"] + census["int4"]
    n16 = census["fp16"]
    ops = (n_int + n16) * (qk + pv)
    t_peak = n_int * qk / PEAK_I8 + n16 * qk / PEAK_F16 + (n_int + n16) * pv / PEAK_F16
    achieved = ops / (t_ms * 1e-3) / 1e12
    peak = ops / t_peak / 1e12
    return {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
            "traffic": traffic, "kernel": prefill_kernel_of(w, hybrid, fourway)[0], "ops_per_launch": ops,
            "peak_note": "precision-weighted: INT8/INT4 QK at 5.0 POP/s, FP16 QK and every PV at 2.5 PFLOP/s, "
                         "over the executed tiles of this workload"}


def events_ms(fn, n, queue_ahead=False):
    """Per-call times (ms) of n calls of fn, from HIP events recorded on the
    current stream (the stream the library's kernels are launched on).
    queue_ahead: a spin kernel keeps the GPU busy while the host enqueues the
    n calls, so that calls shorter than their host-side launch cost are timed
    on the device (back to back, as behind a long prefill) rather than at the
    host's pace."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    if queue_ahead:
        torch.cuda._sleep(5_000_000)
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def stats(ms):
    s = sorted(ms)
    return {"mean": sum(s) / len(s), "median": s[len(s) // 2], "min": s[0]}


# ----------------------------------------------------------------------------- error against unquantized fp64

def sample_rows(w, n, seed=7):
    """Seeded (seq, head, row) triples: first and last rows, block edges and
    random rows, at most n."""
    import numpy as np
    rng = np.random.default_rng(seed)
    out = set()
    for s, S in enumerate(w.seqlens):
        for r in (0, 63, 64, S // 2, S - 1):
            if 0 <= r < S:
                out.add((s, int(rng.integers(0, w.hq)), r))
    while len(out) < n:
        s = int(rng.integers(0, len(w.seqlens)))
        out.add((s, int(rng.integers(0, w.hq)), int(rng.integers(0, w.seqlens[s]))))
    return sorted(out)[:max(n, 1)]


def err_stats(a, b):
    import numpy as np
    e = np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))
    return {"max_abs": float(e.max()), "mean_abs": float(e.mean())}


def prefill_fp64_error(w, pol, pp, q, k, v, n_rows):
    """GPU fp32 prefill output on sampled rows against float64 attention on
    the unquantized inputs, with the policy's skips (same_skip: quantization
    error alone) and without (dense: plus the skipped tiles)."""
    import numpy as np
    import torch
    import tile_routed_mixed_amd as T
    from oracle import attention as OA
    rows = sample_rows(w, n_rows) if w.total_tokens * w.hq > n_rows else \
        [(s, h, r) for s, S in enumerate(w.seqlens) for h in range(w.hq) for r in range(S)]
    o32 = torch.empty((w.total_tokens, w.hq, w.d), dtype=torch.float32, device="cuda:0")
    T._binding.tm_prefill(pp.shape, pp.trav, pp.policy.kind, pp.q, pp.k, pp.qq, pp.kq, pp.vq, o=o32,
                          o_dtype=T.TM_F32)
    cu = w.cu_seqlens
    ti = torch.tensor([int(cu[s]) + r for s, h, r in rows], device="cuda:0")
    hi = torch.tensor([h for s, h, r in rows], device="cuda:0")
    got = o32[ti, hi].cpu().numpy()
    del o32
    torch.cuda.empty_cache()
    args = (w.seqlens, w.hq, w.hkv, w.d, w.bq, w.bk, pol, q[1], k[1], v[1])
    same = OA.prefill_unquantized(*args, rows=rows, compact=True)
    dense = OA.prefill_unquantized(*args, rows=rows, compact=True, dense=True)
    return {"rows": len(rows), "same_skip": err_stats(got, same), "dense": err_stats(got, dense),
            "note": "fp32 GPU output vs float64 softmax attention on the unquantized 16-bit inputs; reported, "
                    "not gated"}


# ----------------------------------------------------------------------------- prefill lines

def prefill_line(name, steps=10, warmup=2, hybrid=None, fp64_rows=48, fourway=False):
    """Prefill alone on one workload: time per launch (HIP events on the
    launch stream), effective dense-causal rate, roofline against the
    precision-weighted MFMA peak of its executed tiles, and its error against
    unquantized attention.  hybrid = (fraction selected, window): the
    workload's shape under the token-granular policy, with the selected keys
    picked on the GPU by the vertical-line pass (tm_select_vertical).
    fourway: the workload's boundaries plus seeded 2-bit group codes."""
    import torch
    import tile_routed_mixed_amd as T
    import workloads as W
    w = W.get(name)
    q, k, v = W.make_qkv(w)
    pol = W.make_policy(w) if hybrid is None else W.make_selection(w, hybrid[0], hybrid[1])
    if fourway:
        pol = W.make_fourway_policy(w)
    pp = T.PrefillPipeline(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, pol)
    pp.upload(q[0], k[0], v[0])
    pp.quantize()
    sel = trv = None
    if hybrid is not None:
        # the lists stay in device memory: selection, traversal and gather run
        # back to back with no copy to the host and no wait
        pol = pp.vertical_policy(hybrid[0], hybrid[1], on_device=True)
        torch.cuda.synchronize()
        sel = stats(events_ms(lambda: pp.vertical_policy(hybrid[0], hybrid[1], on_device=True), 7,
                              queue_ahead=True)[2:])
        pp.set_policy(pol)
        pp.traversal()
        torch.cuda.synchronize()
        trv = stats(events_ms(lambda: pp.traversal(), 7, queue_ahead=True)[2:])
        n_sel = int(pol["sel_off"][-1])
        pol_host = dict(kind=pol["kind"], window=pol["window"], sel_off=pol["sel_off"],
                        sel_idx=pol["sel_idx_dev"][:n_sel].cpu().numpy())   # for the oracle, untimed
    census = pp.traversal(census=True)
    o_dtype = T.TM_BF16 if w.dtype == "bf16" else T.TM_F16
    for _ in range(warmup):
        pp.prefill(o_dtype)
    torch.cuda.synchronize()
    t = stats(events_ms(lambda: pp.prefill(o_dtype), steps))
    roof = prefill_roofline(w, census, t["mean"],
                            pmc_traffic(f"prefill_{name}_pmc.json", prefill_kernel_of(w)[1])
                            if hybrid is None and not fourway else None,
                            hybrid=hybrid is not None, fourway=fourway)
    res = {"workload": describe(w, hybrid, fourway), "prefill_ms": t["mean"], "prefill_ms_median": t["median"],
           "prefill_ms_min": t["min"],
           "effective_tflops_dense_causal": dense_causal_flops(w) / (t["mean"] * 1e-3) / 1e12,
           "roofline": roof, "census": census}
    if sel is not None:
        res["selection_ms"] = sel["mean"]
        res["hybrid_traversal_ms"] = trv["mean"]
        res["selection_plus_traversal_frac_of_prefill"] = (sel["mean"] + trv["mean"]) / t["mean"]
        res["selection_note"] = ("tm_select_vertical (lists left in device memory), then "
                                 "tm_build_traversal_gather on those lists (tables and gathered rows in one "
                                 "launch): no host copy, no stream wait; event-timed "
                                 "on the launch stream, enqueued behind a spin kernel so that the device time "
                                 "is measured, not the host's launch pace")
        pol = pol_host
    if fp64_rows:
        res["fp64_error"] = prefill_fp64_error(w, pol, pp, q, k, v, fp64_rows)
    del pp
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- decode

def decode_block_counts(L, b8, b4, sink, tail):
    """Blocks of each precision that one decode step reads for a cache of L
    tokens (the query at L - 1): blocks reaching into the last `tail` tokens
    are FP16, block 0 is INT8 under a sink, and block j otherwise sits at
    distance last - j from the query's block (INT8 below b8, INT4 below b4,
    else skipped).  Byte accounting for the bench line only."""
    nb = -(-L // 64)
    last = (L - 1) // 64
    first_tail = max(0, (L - tail) // 64) if tail > 0 else nb   # first block reaching the tail
    c = {"int8": 0, "int4": 0, "fp16": nb - first_tail, "skip": 0}
    for j in range(first_tail):
        if sink and j == 0:
            c["int8"] += 1
            continue
        dl = last - j
        c["int8" if dl < b8 else ("int4" if dl < b4 else "skip")] += 1
    return c


def decode_bytes(w, dpol, d):
    """Algorithmic bytes of one decode step: codes and the two scales of every
    INT block read (K and V), 16-bit K and V^T of every FP16 block, per
    (sequence, KV head); q and o are negligible.  Per-query-head maps: a
    (sequence, KV head) reads each block once at every precision some query
    head of its group needs it in (the distinct (block, precision) pairs)."""
    per = {"int8": 64 * d * 2 + 8, "int4": 64 * d + 8, "fp16": 64 * d * 2 * 2, "skip": 0}
    counts = {"int8": 0, "int4": 0, "fp16": 0, "skip": 0}
    grp = w.hq // w.hkv
    for L in w.seqlens:
        for g in range(w.hkv):
            if not dpol.get("per_q_head", 0):
                for t, n in decode_block_counts(L, int(dpol["b8"][g]), int(dpol["b4"][g]), dpol["sink"],
                                                dpol["tail"]).items():
                    counts[t] += n
                continue
            # (b8, b4) bands of the group's heads: a block is INT8 for some head
            # if its distance is below the largest b8, INT4 for some head if it
            # lies in [b8_h, b4_h) for one of them
            maps = [(int(dpol["b8"][h]), int(dpol["b4"][h])) for h in range(g * grp, (g + 1) * grp)]
            nb = -(-L // 64)
            last = (L - 1) // 64
            first_tail = max(0, (L - dpol["tail"]) // 64) if dpol["tail"] > 0 else nb
            counts["fp16"] += nb - first_tail
            for j in range(first_tail):
                if dpol["sink"] and j == 0:
                    counts["int8"] += 1
                    continue
                dl = last - j
                i8 = any(dl < b8 for b8, _ in maps)
                i4 = any(b8 <= dl < b4 for b8, b4 in maps)
                counts["int8"] += int(i8)
                counts["int4"] += int(i4)
                counts["skip"] += int(not i8 and not i4)
    return sum(per[t] * n for t, n in counts.items()), counts


def decode_bench(steps, rotate=3, select_frac=None, tags=None, fp64_pairs=0, per_q_head=False):
    """Decode over a 16 x 32768-token compressed cache; returns timing, bytes
    and the HBM roofline.  select_frac: that fraction of every (sequence, KV
    head)'s tokens (seeded) is kept in FP16 as selected tokens.  per_q_head:
    every query head with its own seeded (b8, b4) around the workload's."""
    import numpy as np
    import torch
    import tile_routed_mixed_amd as T
    import workloads as W
    w = W.get("decode16x32k")
    dpol = W.make_decode_policy(w)
    if tags is not None:   # another reading of the cache tags: (b8, b4) in blocks
        dpol = dict(dpol, b8=np.full(w.hkv, tags[0], np.int32), b4=np.full(w.hkv, tags[1], np.int32))
    if per_q_head:
        dpol = W.make_decode_policy_per_q_head(w)
    _, k, v = W.make_qkv(w)
    dq = W.make_decode_query(w)
    caches = []
    for c in range(rotate):
        p = T.DecodePipeline(w.seqlens, w.hq, w.hkv, w.d, dpol, dtype=w.dtype)
        p.upload(dq[0], k[0], v[0])
        p.build_cache()
        if select_frac is not None:
            p.select(*W.make_decode_selection(w, select_frac))
        caches.append(p)
    torch.cuda.synchronize()
    nbytes, counts = decode_bytes(w, dpol, w.d)
    n_sel = 0
    if select_frac is not None:
        # selected tokens: their 16-bit K row and fp16 V column, plus one 8-byte
        # mask per read block (their codes are still read with their blocks)
        n_sel = int(caches[0].dpol.sel_idx.size)
        nbytes += n_sel * w.d * 2 * 2 + 8 * (counts["int8"] + counts["int4"] + counts["fp16"])
    for i in range(5):
        caches[i % rotate].decode()
    torch.cuda.synchronize()
    # back-to-back steps, each on the next cache, between one pair of events on
    # the launch stream: the mean is whole-job time per step (every kernel of
    # the call and the gaps between launches); per-step events give the spread
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        caches[i % rotate].decode()
    ev1.record()
    torch.cuda.synchronize()
    mean = ev0.elapsed_time(ev1) / steps
    single = stats(_rotating(caches, steps))
    b8t, b4t = int(dpol["b8"][0]), int(dpol["b4"][0])
    desc = describe(w) + f", cache tags (b8, b4) = ({b8t}, {b4t if b4t < 1 << 20 else 'never'}) blocks, " \
                         f"last 128 tokens FP16"
    if per_q_head:
        desc = describe(w) + (f", per-query-head cache tags: b8 {int(dpol['b8'].min())}-{int(dpol['b8'].max())}, "
                              f"b4 {int(dpol['b4'].min())}-{int(dpol['b4'].max())} blocks (seeded per head), "
                              f"last 128 tokens FP16; bytes count each (block, precision) a KV group needs once")
    if select_frac is not None:
        desc += f", {select_frac * 100:g} % of tokens per (sequence, KV head) selected and read in FP16 ({n_sel} in all)"
    gbs = nbytes / (mean * 1e-3) / 1e9
    traffic = pmc_traffic("decode16x32k_pmc.json", ("k_decode.hip",)) \
        if (select_frac is None and tags is None and not per_q_head) else None
    res = {"workload": desc, "bytes_per_step": nbytes, "ms_mean": mean, "ms_median_single": single["median"],
           "ms_min_single": single["min"], "GBps": gbs, "hbm_frac": gbs * 1e9 / PEAK_HBM,
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                        "frac": gbs * 1e9 / PEAK_HBM, "traffic": traffic, "kernel": "tm_decode (all its kernels)"},
           "blocks": counts, "rotated_caches": rotate}
    if fp64_pairs:
        res["fp64_error"] = decode_fp64_error(w, dpol, caches[0], k, v, dq, fp64_pairs)
    del caches
    torch.cuda.empty_cache()
    return res


def _rotating(caches, steps):
    """Per-step event times of `steps` decode calls on the rotated caches."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        caches[i % len(caches)].decode()
        ev[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def decode_fp64_error(w, dpol, p, k, v, dq, n_pairs):
    """GPU decode output (fp32) on sampled (sequence, query head) pairs
    against one-query float64 attention on the unquantized cache: over the
    keys the tags read (same_skip) and over every key (dense)."""
    import numpy as np
    import torch
    from oracle import attention as OA
    rng = np.random.default_rng(11)
    pairs = sorted(set((int(rng.integers(0, len(w.seqlens))), int(rng.integers(0, w.hq)))
                       for _ in range(n_pairs)))
    o = p.decode()
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    got = np.stack([o[b, h] for b, h in pairs])
    args = (w.seqlens, w.hq, w.hkv, w.d, dq[1], k[1], v[1], dpol)
    same = OA.decode_unquantized(*args, pairs=set(pairs))
    dense = OA.decode_unquantized(*args, pairs=set(pairs), dense=True)
    return {"pairs": len(pairs), "same_skip": err_stats(got, np.stack([same[b, h] for b, h in pairs])),
            "dense": err_stats(got, np.stack([dense[b, h] for b, h in pairs])),
            "note": "fp32 GPU output vs float64 one-query attention on the unquantized cache; reported, not gated"}


def decode_loop_bench(steps=64):
    """Generation loop over the 16 x 32768-token workload: the caches start
    `steps` tokens short of 32768 and every step decodes one query per
    sequence, then appends that step's token (tm_cache_append for K and V,
    the new rows already in device memory).  Returns time per step twice:
    device-paced (the steps enqueued behind a spin kernel, so they run back
    to back on the GPU whatever the host's launch pace) and host-paced (the
    loop as the host drives it, launch cost included)."""
    import time as _time
    import numpy as np
    import torch
    import tile_routed_mixed_amd as T
    import workloads as W
    from tile_routed_mixed_amd import _binding as B
    w = W.get("decode16x32k")
    dpol = W.make_decode_policy(w)
    _, k, v = W.make_qkv(w)
    dq = W.make_decode_query(w)
    p = T.DecodePipeline(w.seqlens, w.hq, w.hkv, w.d, dpol, dtype=w.dtype)
    p.upload(dq[0], k[0], v[0])
    del k, v
    L0 = np.array(w.seqlens, np.int64) - steps
    lens = [L0 + i for i in range(steps + 1)]

    def run(spin_cycles):
        p.start(L0)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if spin_cycles:
            torch.cuda._sleep(spin_cycles)
        t0 = _time.perf_counter()
        ev0.record()
        for i in range(steps):
            p.decode()
            p.dpol.set_lengths(lens[i + 1])
            B.tm_cache_append(p.shape, lens[i + 1], p.k, p.kq)
            B.tm_cache_append(p.shape, lens[i + 1], p.v, p.vq)
        ev1.record()
        t_enq = _time.perf_counter() - t0
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps, t_enq

    host_ms, t_enq = run(0)
    # spin length: the spin kernel's rate measured once, then enough cycles to
    # cover twice the host's enqueue time of the loop
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(1_000_000)
    e1.record()
    torch.cuda.synchronize()
    cyc_per_ms = 1_000_000 / max(e0.elapsed_time(e1), 1e-3)
    dev_ms, _ = run(int(min(2.0 * t_enq * 1e3 * cyc_per_ms, 2e9)))
    return {"workload": "decode16x32k generation loop: decode + K/V cache append per step, lengths "
                        f"{int(L0[0])} -> {int(lens[-1][0])}", "steps": steps, "ms_per_step": dev_ms,
            "tokens_per_s": len(w.seqlens) / (dev_ms * 1e-3), "ms_per_step_host_paced": host_ms,
            "note": "ms_per_step: the steps enqueued behind a spin kernel and run back to back on the GPU; "
                    "ms_per_step_host_paced: the same loop at the host's launch pace"}


# ----------------------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(w, q, k, v, pol, seconds):
    """The oracle (numpy float64) on a bounded, seeded sample of whole
    (sequence, head, query tile) items of the same workload, timed on this
    host's cores; the codes of the sampled query blocks and of K are made by
    the oracle's quantizer first (not timed)."""
    import numpy as np
    from oracle import attention as OA
    from oracle import quant as OQ
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    rng = np.random.default_rng(12345)
    items = [(s, h, i) for s, S in enumerate(w.seqlens) for h in range(w.hq) for i in range(-(-S // w.bq))]
    order = [items[n] for n in rng.permutation(len(items))[:512]]
    blocks = set()
    for s, h, i in order:
        for x in range(0, w.bq, 64):
            if i * w.bq + x < w.seqlens[s]:
                blocks.add((s, (i * w.bq + x) // 64))
    qq = OQ.quantize_blocks(q[1], w.seqlens, blocks)
    kq = OQ.quantize(k[1], w.seqlens)
    q64, k64, v64 = (x[1].astype(np.float64) for x in (q, k, v))
    done, flops, t0 = 0, 0.0, time.perf_counter()
    for s, h, i in order:
        OA.prefill(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.bk, pol, q64, k64, v64, qq, kq, qtiles=[(s, h, i)],
                   compact=True)
        r0, r1 = i * w.bq, min((i + 1) * w.bq, w.seqlens[s])
        flops += sum(4.0 * w.d * (r + 1) for r in range(r0, r1))
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    cpu = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{w.name}: {done} of {len(items)} (sequence, head, query tile) items drawn with seed 12345, "
                      f"{dt:.1f} s; attention rows only (codes precomputed); dense-causal FLOPs of those rows; "
                      f"{cpu}, os.cpu_count() = {os.cpu_count()}, BLAS threads = {int(threads)}"}


# ----------------------------------------------------------------------------- hardware ceilings

def ceilings():
    """Measured MFMA and HBM ceilings from the tm_ceiling microbenchmarks (a
    child process), or None if it is not built."""
    exe = os.path.join(ROOT, "tile_routed_mixed_amd", "tm_ceiling")
    if not os.path.exists(exe):
        return None
    r = subprocess.run([exe, "--summary"], capture_output=True, text=True, timeout=120)
    for line in reversed(r.stdout.splitlines()):
        if line.startswith("{"):
            return json.loads(line)
    return None


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-bench", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the prefill lines of the toy, 8K, varlen and hybrid workloads")
    ap.add_argument("--no-fp64-error", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="only run the decode sub-benchmark (16 x 32768-token cache) and print its JSON")
    ap.add_argument("--prefill-only", metavar="WORKLOAD",
                    help="only run the prefill line of one workload and print its JSON")
    ap.add_argument("--hybrid", type=float, default=None, metavar="FRAC",
                    help="with --prefill-only: the hybrid policy with FRAC of the keys selected by the "
                         "vertical-line pass and a 128-token window")
    ap.add_argument("--fourway", action="store_true",
                    help="with --prefill-only: the workload's boundaries plus seeded four-way group codes")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain elementwise copy of BYTES bytes (read BYTES, write BYTES) 5 times, "
                         "to scale HBM byte counters; prints nothing else")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(5):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "launches": 5}), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this hot path runs on one GPU; --gpus N > 1 is not supported (see DESIGN.md for "
              "how it would shard)", file=sys.stderr)
        sys.exit(2)
    if args.decode_only:
        print(json.dumps(decode_bench(max(5, args.steps))), flush=True)
        return
    if args.prefill_only:
        hyb = None if args.hybrid is None else (args.hybrid, 128)
        print(json.dumps(prefill_line(args.prefill_only, steps=max(3, args.steps), warmup=args.warmup,
                                      hybrid=hyb, fp64_rows=8, fourway=args.fourway)), flush=True)
        return

    import torch
    import tile_routed_mixed_amd as T
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    T.lib()
    w = W.get(args.workload)
    log(f"[bench] workload {describe(w)}")
    q, k, v = W.make_qkv(w)
    pol = W.make_policy(w)
    pp = T.PrefillPipeline(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, pol)
    pp.upload(q[0], k[0], v[0])
    pp.quantize()
    census = pp.traversal(census=True)
    b8, b4 = decode_policy_for(w.seqlens[0])
    dpol = dict(b8=[b8] * w.hkv, b4=[b4] * w.hkv, sink=1, tail=128)
    dq = W.make_decode_query(w)
    dp = T.DecodePipeline.from_prefill(pp, dpol, dq[0])
    o_dtype = T.TM_BF16 if w.dtype == "bf16" else T.TM_F16
    log(f"[bench] census {census}")

    E = lambda: torch.cuda.Event(enable_timing=True)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        pp.quantize()
        if ev is not None:
            ev[1].record()
        pp.traversal(False)
        if ev is not None:
            ev[2].record()
        pp.prefill(o_dtype)
        if ev is not None:
            ev[3].record()
        dp.decode()
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[E() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    stages = (("quantize_qkv", 0, 1), ("traversal", 1, 2), ("prefill", 2, 3), ("decode", 3, 4))
    per_step = {n: [e[a].elapsed_time(e[b]) for e in evs] for n, a, b in stages}
    k_mean = {n: sum(v_) / len(v_) for n, v_ in per_step.items()}
    k_median = {n: sorted(v_)[len(v_) // 2] for n, v_ in per_step.items()}
    k_min = {n: min(v_) for n, v_ in per_step.items()}
    log(f"[bench] ms/step {ms_step:.4f}: " + " ".join(f"{n} {t:.4f}" for n, t in k_mean.items()))

    flops = dense_causal_flops(w)
    value = flops / (ms_step * 1e-3) / 1e12
    roof = prefill_roofline(w, census, k_mean["prefill"],
                            pmc_traffic(f"prefill_{w.name}_pmc.json", prefill_kernel_of(w)[1]))
    log(f"[bench] prefill_kernel {k_mean['prefill']:.3f} ms: {roof['achieved']:.0f} of {roof['peak']:.0f} TFLOP/s "
        f"({roof['frac'] * 100:.1f} % of the precision-weighted peak)")
    out = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "i8+f16" if census["fp16"] == 0 else "i8+f16(+f16 QK)",
           "data": "synthetic (seeded N(0,1), shapes of the pages' Llama-3-8B-class attention layers)",
           "config": {"workload": describe(w), "global_batch": len(w.seqlens), "seq_len": max(w.seqlens),
                      "parallelism": "none (1 GPU)",
                      "decode_in_step": f"1 query/seq over the prompt cache, (b8, b4) = ({b8}, {b4}) blocks, sink, "
                                        f"tail 128"},
           "roofline": roof, "mfma_util": roof["frac"],
           "prefill_kernel_ms": k_mean["prefill"], "prefill_only_tflops": flops / (k_mean["prefill"] * 1e-3) / 1e12,
           "kernels_ms": k_mean, "kernels_ms_median": k_median, "kernels_ms_min": k_min, "census": census}
    if not args.no_fp64_error:
        log("[bench] error against unquantized float64 attention on sampled rows ...")
        out["fp64_error"] = {w.name: prefill_fp64_error(w, pol, pp, q, k, v, 40)}
    del pp, dp
    torch.cuda.empty_cache()
    if not args.no_decode_bench:
        d = decode_bench(max(20, args.steps), fp64_pairs=0 if args.no_fp64_error else 12)
        out["decode"] = d
        out["decode_kv_gbs"] = d["GBps"]
        if "fp64_error" in d and "fp64_error" in out:
            out["fp64_error"]["decode16x32k"] = d.pop("fp64_error")
        log(f"[bench] decode {d['ms_mean']:.4f} ms, {d['GBps']:.1f} GB/s ({d['hbm_frac'] * 100:.1f} % of HBM)")
        ds = decode_bench(max(20, args.steps), select_frac=0.05)
        out["decode_selected"] = ds
        log(f"[bench] decode with 5 % selected tokens {ds['ms_mean']:.4f} ms, {ds['GBps']:.1f} GB/s")
        dq_ = decode_bench(max(20, args.steps), per_q_head=True)
        out["decode_per_query_head"] = dq_
        log(f"[bench] decode with per-query-head maps {dq_['ms_mean']:.4f} ms, {dq_['GBps']:.1f} GB/s")
        out["decode_tag_variants"] = []
        for tg in ((2, 5), (128, 1 << 30)):   # the literal toy bands; no skipped block
            dv = decode_bench(max(20, args.steps), tags=tg)
            out["decode_tag_variants"].append(dv)
            log(f"[bench] decode tags {tg}: {dv['ms_mean']:.4f} ms, {dv['GBps']:.1f} GB/s")
        torch.cuda.empty_cache()
        dl = decode_loop_bench()
        out["decode_loop"] = dl
        log(f"[bench] decode loop {dl['ms_per_step']:.4f} ms/step (decode + cache append), "
            f"{dl['tokens_per_s']:.0f} tokens/s")
    if not args.no_other_configs:
        out["other_configs"] = []
        for name, hyb, fw in (("toy512", None, False), ("gqa8k", None, False), ("varlen32k", None, False),
                              ("gqa8k", (0.05, 128), False), ("gqa8k", None, True)):
            if name == w.name and hyb is None and not fw:
                continue
            r = prefill_line(name, hybrid=hyb, fp64_rows=0 if args.no_fp64_error else 48, fourway=fw)
            out["other_configs"].append(r)
            log(f"[bench] {name}{' hybrid' if hyb else ''}{' four-way' if fw else ''}: prefill {r['prefill_ms']:.4f} ms, "
                f"{r['effective_tflops_dense_causal']:.1f} TFLOP/s dense-causal, "
                f"{r['roofline']['frac'] * 100:.1f} % of the weighted MFMA peak"
                + (f"; selection {r['selection_ms']:.4f} ms + traversal {r['hybrid_traversal_ms']:.4f} ms = "
                   f"{r['selection_plus_traversal_frac_of_prefill'] * 100:.1f} % of the prefill" if hyb else ""))
            if "fp64_error" in r and "fp64_error" in out:
                out["fp64_error"][name + ("_hybrid" if hyb else "") + ("_fourway" if fw else "")] = r["fp64_error"]
    if not args.no_ceiling:
        out["ceilings"] = ceilings()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, pol, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
