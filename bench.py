#!/usr/bin/env python3
"""Benchmark of the tile-routed mixed-precision attention hot path on one GPU.

One step = one pass of the whole path over one batch of synthetic input that
is already resident in HBM:
  tm_quantize_pack(Q), tm_quantize_pack(K), tm_quantize_pack(V, transposed +
  fp16 copy), tm_build_traversal, tm_prefill, and tm_decode of one new query
  per sequence over the compressed cache the prefill just quantized.

Default workload: one 8192-token sequence, 32 query / 8 KV heads, d = 128, bf16,
128x64 tiles, K with 4 outlier channels x10, per-head random diagonal-distance
boundaries (about 40 % of legal tiles skipped).  ``value`` is the effective
dense-causal prefill rate of the whole step: 4*d*hq*S^2/2 FLOPs per step over
the measured step time.  A decode sub-benchmark (16 sequences x 32768 cached
tokens, rotating three caches so the read set exceeds the 256 MB last-level
cache) reports compressed-cache read GB/s.

Prints one JSON line.  --gpus N > 1 is refused: this path runs on one GPU.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective prefill attn TFLOP/s (dense-causal) + MFMA util; decode KV GB/s"
PEAK_F16 = 2.5e15     # MI355X dense MFMA, fp16/bf16 (FLOP/s)
PEAK_I8 = 5.0e15      # MI355X dense MFMA, int8 (OP/s)
PEAK_HBM = 8.0e12     # MI355X HBM3E (B/s)
PMC_SUMMARY = os.path.join(ROOT, "profiles", "prefill_gqa8k_pmc.json")
PREFILL_SRC = os.path.join(ROOT, "tile_routed_mixed_amd", "csrc", "k_prefill.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def describe(w):
    pol = "per-head diagonal-distance boundaries" if w.policy == "boundaries" else \
        f"packed bitmask, {w.group} key tiles per bit, P(FP16)={w.p_fp16}"
    return (f"{w.name}: seqs {w.seqlens if len(w.seqlens) <= 4 else str(len(w.seqlens)) + 'x' + str(w.seqlens[0])}"
            f", {w.hq}/{w.hkv} heads, d={w.d}, {w.dtype}, {w.bq}x{w.bk} tiles, {pol}"
            + (", key tile 0 INT8" if w.sink else "") + (f", K outliers {w.outliers}x{w.outlier_scale:g}"
                                                          if w.outliers else ""))


def dense_causal_flops(w):
    return sum(4.0 * w.d * w.hq * S * S / 2.0 for S in w.seqlens)


def decode_policy_for(S):
    """Cache tags for the decode step after a prefill of S tokens: the toy
    workload's bands (INT8 below 2/8, INT4 below 5/8 of the blocks) scaled to the
    cache, first block INT8, last 128 tokens FP16."""
    nb = -(-S // 64)
    b8 = max(1, nb // 4)
    return b8, max(b8, (nb * 5) // 8)


def prefill_roofline(w, census, t_prefill):
    qk = 2.0 * w.bq * w.bk * w.d
    pv = 2.0 * w.bq * w.bk * w.d
    n_int = census["int8"] + census["int4"]
    n16 = census["fp16"]
    ops = (n_int + n16) * (qk + pv)
    t_peak = n_int * qk / PEAK_I8 + n16 * qk / PEAK_F16 + (n_int + n16) * pv / PEAK_F16
    return ops, t_peak


def pmc_traffic():
    """HBM bytes per prefill launch from the committed rocprofv3 counter
    summary, or None when absent or taken on a different kernel source."""
    try:
        s = json.load(open(PMC_SUMMARY))
    except (OSError, ValueError):
        return None
    h = hashlib.sha256(open(PREFILL_SRC, "rb").read()).hexdigest()
    if s.get("kernel_source_sha256") != h:
        return None
    return s.get("hbm_bytes_per_launch")


def cpu_baseline(w, q, k, v, pol, seconds):
    """The oracle (numpy float64) on a bounded, seeded sample of whole query
    tiles of the same workload, timed on this host's cores."""
    import numpy as np
    from oracle import attention as OA
    from oracle import quant as OQ
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    qq = OQ.quantize(q[1], w.seqlens)
    kq = OQ.quantize(k[1], w.seqlens)
    q64, k64, v64 = (x[1].astype(np.float64) for x in (q, k, v))
    rng = np.random.default_rng(12345)
    items = [(s, h, i) for s, S in enumerate(w.seqlens) for h in range(w.hq) for i in range(-(-S // w.bq))]
    order = rng.permutation(len(items))
    done, flops, t0 = 0, 0.0, time.perf_counter()
    for n in order:
        s, h, i = items[n]
        OA.prefill(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.bk, pol, q64, k64, v64, qq, kq, qtiles=[(s, h, i)])
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
            "sample": f"{done} of {len(items)} (sequence, head, query tile) items drawn with seed 12345, "
                      f"{dt:.1f} s; attention rows only (codes precomputed); dense-causal FLOPs of those rows; "
                      f"{cpu}, os.cpu_count() = {os.cpu_count()}, BLAS threads = {int(threads)}"}


def prefill_config_line(name, steps=10, warmup=2, hybrid=None):
    """Prefill alone on another of the five workloads: time per launch (HIP
    events on the launch stream, back to back), effective dense-causal rate,
    and the fraction of the precision-weighted MFMA peak of its executed tiles.
    hybrid = (fraction selected, window): the workload's shape under the
    token-granular policy instead of its own, with the selected keys picked
    on the GPU by the vertical-line pass (tm_select_vertical, timed apart)."""
    import torch
    import tile_routed_mixed_amd as T
    import workloads as W
    w = W.get(name)
    q, k, v = W.make_qkv(w)
    pol = W.make_policy(w) if hybrid is None else W.make_selection(w, hybrid[0], hybrid[1])
    pp = T.PrefillPipeline(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, pol)
    pp.upload(q[0], k[0], v[0])
    del q, k, v
    pp.quantize()
    t_sel = None
    if hybrid is not None:
        pol = pp.vertical_policy(hybrid[0], hybrid[1])
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(5):
            pp.vertical_policy(hybrid[0], hybrid[1])
        s1.record()
        torch.cuda.synchronize()
        t_sel = s0.elapsed_time(s1) / 5
        pp.set_policy(pol)
    census = pp.traversal(census=True)
    o_dtype = T.TM_BF16 if w.dtype == "bf16" else T.TM_F16
    for _ in range(warmup):
        pp.prefill(o_dtype)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        pp.prefill(o_dtype)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / steps
    ops, t_peak = prefill_roofline(w, census, t * 1e-3)
    desc = describe(w) if hybrid is None else describe(w).replace(
        "per-head diagonal-distance boundaries",
        f"hybrid: {hybrid[0] * 100:.0f} % of keys per head selected by the vertical-line pass (attention mass "
        f"from the last 64 rows), {hybrid[1]}-token window in FP16, the rest INT8")
    res = {"workload": desc, "prefill_ms": t,
           **({} if t_sel is None else {"selection_ms_incl_host": t_sel}),
           "effective_tflops_dense_causal": dense_causal_flops(w) / (t * 1e-3) / 1e12,
           "mfma_frac_precision_weighted": (ops / (t * 1e-3)) / (ops / t_peak),
           "census": census}
    del pp
    torch.cuda.empty_cache()
    return res


def decode_loop_bench(steps=64):
    """Generation loop over the 16 x 32768-token workload: the caches start
    `steps` tokens short of 32768 and every step decodes one query per
    sequence, then appends that step's token (tm_cache_append for K and V,
    the new rows already in device memory).  Returns time per step."""
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
    p.start(L0)
    torch.cuda.synchronize()
    lens = [L0 + i for i in range(steps + 1)]
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        p.decode()
        p.dpol.set_lengths(lens[i + 1])
        B.tm_cache_append(p.shape, lens[i + 1], p.k, p.kq)
        B.tm_cache_append(p.shape, lens[i + 1], p.v, p.vq)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    return {"workload": "decode16x32k generation loop: decode + K/V cache append per step, lengths "
                        f"{int(L0[0])} -> {int(lens[-1][0])}", "steps": steps, "ms_per_step": ms,
            "tokens_per_s": len(w.seqlens) / (ms * 1e-3)}


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


def decode_bench(steps, rotate=3, select_frac=None, tags=None):
    """Decode over a 16 x 32768-token compressed cache; returns timing and bytes.
    select_frac: that fraction of every (sequence, KV head)'s tokens (seeded)
    is kept in FP16 as selected tokens."""
    import numpy as np
    import torch
    import tile_routed_mixed_amd as T
    import workloads as W
    w = W.get("decode16x32k")
    dpol = W.make_decode_policy(w)
    if tags is not None:   # another reading of the cache tags: (b8, b4) in blocks
        dpol = dict(dpol, b8=np.full(w.hkv, tags[0], np.int32), b4=np.full(w.hkv, tags[1], np.int32))
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
    del k, v
    torch.cuda.synchronize()
    # algorithmic bytes: codes + two scales of every INT block (K and V), 16-bit K
    # and V^T of every FP16 block, per (sequence, KV head); q and o are negligible
    per = {"int8": 64 * w.d * 2 + 8, "int4": 64 * w.d + 8, "fp16": 64 * w.d * 2 * 2, "skip": 0}
    counts = {"int8": 0, "int4": 0, "fp16": 0, "skip": 0}
    for L in w.seqlens:
        for g in range(w.hkv):
            for t, n in decode_block_counts(L, int(dpol["b8"][g]), int(dpol["b4"][g]), dpol["sink"],
                                            dpol["tail"]).items():
                counts[t] += n
    nbytes = sum(per[t] * n for t, n in counts.items())
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
    # the launch stream: the mean is whole-job time per step (split + merge
    # kernels and the launch gaps between them); per-step events beside it give
    # the spread
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        caches[i % rotate].decode()
    ev1.record()
    torch.cuda.synchronize()
    mean = ev0.elapsed_time(ev1) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        caches[i % rotate].decode()
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    b8t, b4t = int(dpol["b8"][0]), int(dpol["b4"][0])
    desc = describe(w) + f", cache tags (b8, b4) = ({b8t}, {b4t if b4t < 1 << 20 else 'never'}) blocks, " \
                         f"last 128 tokens FP16"
    if select_frac is not None:
        desc += f", {select_frac * 100:g} % of tokens per (sequence, KV head) selected and read in FP16 ({n_sel} in all)"
    return {"workload": desc,
            "bytes_per_step": nbytes, "ms_mean": mean, "ms_median_single": ms[len(ms) // 2],
            "ms_min_single": ms[0],
            "GBps": nbytes / (mean * 1e-3) / 1e9, "hbm_frac": nbytes / (mean * 1e-3) / PEAK_HBM,
            "blocks": counts, "rotated_caches": rotate}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa8k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-bench", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the prefill-only lines for the toy, varlen and 128K workloads")
    ap.add_argument("--decode-only", action="store_true",
                    help="only run the decode sub-benchmark (16 x 32768-token cache) and print its JSON")
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
    if args.decode_only:
        print(json.dumps(decode_bench(max(5, args.steps))), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this hot path runs on one GPU; --gpus N > 1 is not supported (see DESIGN.md for "
              "how it would shard)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
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
    part = lambda a, b: sum(e[a].elapsed_time(e[b]) for e in evs) / args.steps
    t_quant, t_trav, t_pref, t_dec = part(0, 1), part(1, 2), part(2, 3), part(3, 4)
    stages = (("quantize_qkv", 0, 1), ("traversal", 1, 2), ("prefill", 2, 3), ("decode", 3, 4))
    per_step = {n: sorted(e[a].elapsed_time(e[b]) for e in evs) for n, a, b in stages}
    k_median = {n: v[len(v) // 2] for n, v in per_step.items()}
    k_min = {n: v[0] for n, v in per_step.items()}
    log(f"[bench] ms/step {ms_step:.4f}: quantize {t_quant:.4f} traversal {t_trav:.4f} "
        f"prefill {t_pref:.4f} decode {t_dec:.4f}")

    flops = dense_causal_flops(w)
    value = flops / (ms_step * 1e-3) / 1e12
    ops, t_peak = prefill_roofline(w, census, t_pref * 1e-3)
    achieved = ops / (t_pref * 1e-3) / 1e12
    peak = ops / t_peak / 1e12
    roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
            "traffic": pmc_traffic(), "kernel": "prefill_kernel",
            "peak_note": "precision-weighted: INT8/INT4 QK at 5.0 POP/s, FP16 QK and every PV at 2.5 PFLOP/s, "
                         "over the executed tiles of this workload"}
    out = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "i8+f16" if census["fp16"] == 0 else "i8+f16(+f16 QK)",
           "data": "synthetic (seeded N(0,1), shapes of the pages' Llama-3-8B-class attention layers)",
           "config": {"workload": describe(w), "global_batch": len(w.seqlens), "seq_len": max(w.seqlens),
                      "parallelism": "none (1 GPU)", "decode_in_step": f"1 query/seq over the prompt cache, "
                                                                       f"(b8, b4) = ({b8}, {b4}) blocks, sink, "
                                                                       f"tail 128"},
           "roofline": roof,
           "mfma_util": achieved / peak,
           "prefill_kernel_ms": t_pref, "prefill_only_tflops": flops / (t_pref * 1e-3) / 1e12,
           "kernels_ms": {"quantize_qkv": t_quant, "traversal": t_trav, "prefill": t_pref, "decode": t_dec},
           "kernels_ms_median": k_median, "kernels_ms_min": k_min,
           "census": census}
    if not args.no_decode_bench:
        del pp, dp
        torch.cuda.empty_cache()
        d = decode_bench(max(20, args.steps))
        out["decode"] = d
        out["decode_kv_gbs"] = d["GBps"]
        log(f"[bench] decode {d['ms_mean']:.4f} ms, {d['GBps']:.1f} GB/s ({d['hbm_frac'] * 100:.1f} % of HBM)")
        torch.cuda.empty_cache()
        torch.cuda.empty_cache()
        ds = decode_bench(max(20, args.steps), select_frac=0.05)
        out["decode_selected"] = ds
        log(f"[bench] decode with 5 % selected tokens {ds['ms_mean']:.4f} ms, {ds['GBps']:.1f} GB/s")
        out["decode_tag_variants"] = []
        for tg in ((2, 5), (128, 1 << 30)):   # the literal toy bands; no skipped block
            torch.cuda.empty_cache()
            dv = decode_bench(max(20, args.steps), tags=tg)
            out["decode_tag_variants"].append(dv)
            log(f"[bench] decode tags {tg}: {dv['ms_mean']:.4f} ms, {dv['GBps']:.1f} GB/s")
        torch.cuda.empty_cache()
        dl = decode_loop_bench()
        out["decode_loop"] = dl
        log(f"[bench] decode loop {dl['ms_per_step']:.4f} ms/step (decode + cache append), "
            f"{dl['tokens_per_s']:.0f} tokens/s")
    if not args.no_other_configs and args.workload == "gqa8k":
        out["other_configs"] = []
        for name, hyb in (("toy512", None), ("varlen32k", None), ("long128k", None), ("gqa8k", (0.05, 128))):
            r = prefill_config_line(name, hybrid=hyb)
            out["other_configs"].append(r)
            log(f"[bench] {name}: prefill {r['prefill_ms']:.4f} ms, {r['effective_tflops_dense_causal']:.1f} "
                f"TFLOP/s dense-causal, {r['mfma_frac_precision_weighted'] * 100:.1f} % of the weighted MFMA peak")
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, pol, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
