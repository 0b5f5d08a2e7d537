"""Full-size parity: the four workloads at their real sizes, in the launch
configuration bench.py times, checked on sampled outputs the oracle computes
one row (or one decode query) at a time.

* traversal and census of the full policy against brute-force enumeration;
* integer QK scores of sampled tiles bit-exact (debug capture);
* sampled output rows (first and last rows of sequences, rows on either side
  of query-tile and block boundaries, seeded random rows) within the gate, for
  the fp32 output and the 16-bit output the bench writes (gate + half an ulp).
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import policy as OP
from oracle import quant as OQ

from _gpu_helpers import (TOL_MAX, assert_all_written, check_int_scores, compare, guard_decode, guard_prefill,
                          int_tiles, run_prefill, say)

pytestmark = pytest.mark.gpu


def _sample_rows(w, n_random=24, seed=0):
    rng = np.random.default_rng(seed)
    rows = set()
    heads = sorted(set([0, w.hq - 1, w.hq // 2] + rng.integers(0, w.hq, size=3).tolist()))
    for s, S in enumerate(w.seqlens):
        fixed = [0, 1, 63, 64, min(127, S - 1), min(128, S - 1), S // 2, S - 2, S - 1]
        for h in heads[:3]:
            for r in fixed:
                if 0 <= r < S:
                    rows.add((s, h, r))
    for _ in range(n_random):
        s = int(rng.integers(0, len(w.seqlens)))
        rows.add((s, int(rng.choice(heads)), int(rng.integers(0, w.seqlens[s]))))
    return sorted(rows)


def _sparse_q_codes(q32, seqlens, rows_blocks):
    """Oracle codes of Q for the listed (sequence, block) pairs only; the
    quantizer works per 64-token block, so quantizing a block's 64 tokens on
    their own gives the same codes as quantizing the whole tensor."""
    starts, nblk = OQ.block_starts(seqlens)
    T, H, d = q32.shape
    out = dict(c8=np.zeros((H, nblk, 64, d), np.int8), c4=np.zeros((H, nblk, 64, d), np.int8),
               s8=np.zeros((H, nblk), np.float32), s4=np.zeros((H, nblk), np.float32), blk_start=starts,
               nblk=nblk)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    for s, b in sorted(rows_blocks):
        t0 = int(cu[s]) + 64 * b
        t1 = min(t0 + 64, int(cu[s + 1]))
        blk = OQ.quantize(q32[t0:t1], [t1 - t0])
        g = int(starts[s]) + b
        for key in ("c8", "c4", "s8", "s4"):
            out[key][:, g] = blk[key][:, 0]
    return out


def _full_prefill(name, n_random=24, n_tiles=8, pol=None, label=None):
    import tile_routed_mixed_amd as T
    w = W.get(name)
    pol = W.make_policy(w) if pol is None else pol
    name = label or name
    say(f"[gpu] full-size {name}: generating inputs")
    q, k, v = W.make_qkv(w)
    tiles = int_tiles(w, pol, limit=n_tiles, seed=1)
    p, census, o32, lse, dbg = run_prefill(w, pol, q, k, v, dbg_tiles=[t[:4] for t in tiles])
    c = OP.census(OP.grids(w.seqlens, w.hq, w.bq, w.bk, pol))
    assert {kk: census[kk] for kk in c} == c
    o16_dtype = T.TM_BF16 if w.dtype == "bf16" else T.TM_F16
    import torch
    p.o = p.guards.alloc((w.total_tokens, w.hq, w.d), torch.bfloat16 if w.dtype == "bf16" else torch.float16,
                         float("nan"))
    p.o_dtype = o16_dtype
    p.guards.poison()
    o16, _ = p.prefill(o16_dtype)
    torch.cuda.synchronize()
    p.guards.check()
    assert_all_written(o16, f"{name} 16-bit O")
    o16 = o16.float().cpu().numpy()
    rows = _sample_rows(w, n_random)
    need = set((s, r // 64) for s, h, r in rows)
    for s, h, i, j, prec in tiles:
        need |= set((s, (i * w.bq + x) // 64) for x in range(0, w.bq, 64) if i * w.bq + x < w.seqlens[s])
    qq = _sparse_q_codes(q[1], w.seqlens, need)
    kq = OQ.quantize(k[1], w.seqlens)
    check_int_scores(w, tiles, dbg, qq, kq)
    say(f"[gpu] full-size {name}: oracle on {len(rows)} sampled rows")
    O, L = OA.prefill(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.bk, pol, q[1].astype(np.float64),
                      k[1].astype(np.float64), v[1].astype(np.float64), qq, kq, rows=rows)
    cu = w.cu_seqlens
    idx = [(int(cu[s]) + r, h) for s, h, r in rows]
    ti = np.array([a for a, _ in idx])
    hi = np.array([b for _, b in idx])
    compare(o32[ti, hi], O[ti, hi], lse[hi, ti], L[hi, ti], what=f"{name} fp32")
    ulp = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -11
    err16 = np.abs(o16[ti, hi] - O[ti, hi])
    assert np.all(err16 <= TOL_MAX + ulp * np.abs(O[ti, hi]) + 1e-7), float(err16.max())
    return p


def test_gqa8k_full():
    _full_prefill("gqa8k")


def test_varlen32k_full():
    _full_prefill("varlen32k")


def test_long128k_full():
    _full_prefill("long128k", n_random=40, n_tiles=6)


def test_fourway_gqa8k_full():
    """The four-way policy at the 8K layer's full size: the layer's per-head
    boundaries with the sink tile, plus a seeded 2-bit code per group of 4 key
    tiles (0 = the boundary rule with probability 1/2, else INT4, INT8 or FP16
    uniformly), so every precision and SKIP occur in every long row."""
    w = W.get("gqa8k")
    pol = W.make_fourway_policy(w)
    c = OP.census(OP.grids(w.seqlens, w.hq, w.bq, w.bk, pol))
    assert min(c["int8"], c["int4"], c["fp16"], c["skip"]) > 0, c
    _full_prefill("gqa8k", pol=pol, label="gqa8k four-way")


def test_decode16x32k_full():
    import torch
    import tile_routed_mixed_amd as T
    w = W.get("decode16x32k")
    dpol = W.make_decode_policy(w)
    say("[gpu] full-size decode16x32k: generating inputs")
    _, k, v = W.make_qkv(w)
    dq = W.make_decode_query(w)
    p = T.DecodePipeline(w.seqlens, w.hq, w.hkv, w.d, dpol, dtype=w.dtype)
    p.upload(dq[0], k[0], v[0])
    g = guard_decode(p)
    p.build_cache()
    o = p.decode()
    torch.cuda.synchronize()
    g.check()
    assert_all_written(o, "decode16x32k O")
    o = o.cpu().numpy()
    cu = w.cu_seqlens
    for b in (0, 7, 15):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        L = w.seqlens[b]
        kq = OQ.quantize(k[1][sl], [L])
        vq = OQ.quantize(v[1][sl], [L], layout="cols")
        O = OA.decode([L], w.hq, w.hkv, w.d, dq[1][b:b + 1].astype(np.float64), kq, vq,
                      k[1][sl].astype(np.float64), v[1][sl].astype(np.float64), dpol)
        compare(o[b], O[0], what=f"decode16x32k seq {b}")


def test_gqa8k_hybrid_full():
    """The bench's hybrid line: 8K, 32/8 heads, keys selected on the GPU by the
    vertical-line pass (5 % per head, 64 probe rows), 128-token window; the
    selection checked against the oracle's masses on sampled heads, the
    traversal census against the oracle's window classes, sampled rows
    against the oracle prefill on the same lists."""
    import math
    import torch
    import tile_routed_mixed_amd as T
    w = W.get("gqa8k")
    say("[gpu] full-size hybrid gqa8k: generating inputs")
    q, k, v = W.make_qkv(w)
    p = T.PrefillPipeline(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, W.make_policy(w))
    p.upload(q[0], k[0], v[0])
    g = guard_prefill(p, T.TM_F32)
    p.quantize()
    pol = p.vertical_policy(0.05, 128)
    S = w.seqlens[0]
    grp = w.hq // w.hkv
    for h in (0, 13, w.hq - 1):
        imp = OP.vline_importance(q[1][:, h].astype(np.float64), k[1][:, h // grp].astype(np.float64), 64,
                                  1 / math.sqrt(w.d))
        sel = pol["sel_idx"][pol["sel_off"][h]:pol["sel_off"][h + 1]]
        kk = int(round(0.05 * S))
        assert len(sel) == kk and np.all(np.diff(sel) > 0)
        kth = np.sort(imp)[::-1][kk - 1]
        chosen = np.zeros(S, bool)
        chosen[sel] = True
        tol = 1e-5 + 1e-4 * kth
        assert np.all(imp[chosen] >= kth - tol) and np.all(imp[~chosen] <= kth + tol), h
    p.set_policy(pol)
    census = p.traversal(census=True)
    cls = OP.hybrid_tile_classes(S, w.bq, w.bk, 128)
    n_full, n_edge, n_none = int((cls == OP.WIN_FULL).sum()), int((cls == OP.WIN_EDGE).sum()), \
        int((cls == OP.WIN_NONE).sum())
    assert census["int8"] == w.hq * (n_edge + n_none)
    o32, _ = p.prefill(T.TM_F32)
    torch.cuda.synchronize()
    g.check()
    assert_all_written(o32, "hybrid O")
    o32 = o32.cpu().numpy()
    lse = p.lse.cpu().numpy()
    rows = _sample_rows(w, 24)
    need = set((s, r // 64) for s, h, r in rows)
    qq = _sparse_q_codes(q[1], w.seqlens, need)
    kq = OQ.quantize(k[1], w.seqlens)
    say(f"[gpu] full-size hybrid gqa8k: oracle on {len(rows)} sampled rows")
    O, L = OA.prefill(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.bk, pol, q[1].astype(np.float64),
                      k[1].astype(np.float64), v[1].astype(np.float64), qq, kq, rows=rows)
    ti = np.array([r for s, h, r in rows])
    hi = np.array([h for s, h, r in rows])
    compare(o32[ti, hi], O[ti, hi], lse[hi, ti], L[hi, ti], what="hybrid gqa8k fp32")


def test_decode16x32k_selected_full():
    """The bench's decode with 5 % of every (sequence, KV head)'s tokens
    selected and read in FP16, on three sequences."""
    import torch
    import tile_routed_mixed_amd as T
    w = W.get("decode16x32k")
    dpol = W.make_decode_policy(w)
    say("[gpu] full-size decode16x32k with selected tokens: generating inputs")
    _, k, v = W.make_qkv(w)
    dq = W.make_decode_query(w)
    sel_off, sel_idx = W.make_decode_selection(w, 0.05)
    p = T.DecodePipeline(w.seqlens, w.hq, w.hkv, w.d, dpol, dtype=w.dtype)
    p.upload(dq[0], k[0], v[0])
    g = guard_decode(p)
    p.build_cache()
    p.select(sel_off, sel_idx)
    o = p.decode()
    torch.cuda.synchronize()
    g.check()
    assert_all_written(o, "decode16x32k O with selected tokens")
    o = o.cpu().numpy()
    cu = w.cu_seqlens
    for b in (0, 9, 15):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        L = w.seqlens[b]
        kq = OQ.quantize(k[1][sl], [L])
        vq = OQ.quantize(v[1][sl], [L], layout="cols")
        r0 = b * w.hkv
        off = (sel_off[r0:r0 + w.hkv + 1] - sel_off[r0]).astype(np.int32)
        idx = sel_idx[sel_off[r0]:sel_off[r0 + w.hkv]]
        O = OA.decode([L], w.hq, w.hkv, w.d, dq[1][b:b + 1].astype(np.float64), kq, vq,
                      k[1][sl].astype(np.float64), v[1][sl].astype(np.float64),
                      dict(dpol, sel_off=off, sel_idx=idx))
        compare(o[b], O[0], what=f"decode16x32k with selected tokens, seq {b}")


def _check_codes_chunked(x16, seqlens, qt, layout, what, chunk=16384):
    """Every code, scale (and fp16 copy) of a block-major device QTensor
    against the oracle's binary32 quantizer, a chunk of whole 64-token blocks
    at a time (blocks are independent, so quantizing a chunk on its own gives
    the oracle's codes for those blocks)."""
    starts, _ = OQ.block_starts(seqlens)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    n = 0
    for s, S in enumerate(seqlens):
        for t0 in range(0, S, chunk):
            t1 = min(S, t0 + chunk)
            ref = OQ.quantize(x16[cu[s] + t0:cu[s] + t1], [t1 - t0], layout=layout, with_t16=(layout == "cols"))
            b0 = int(starts[s]) + t0 // 64
            b1 = b0 + -(-(t1 - t0) // 64)

            def hm(t):   # block-major on the GPU, head-major in the oracle
                return np.swapaxes(t[b0:b1].cpu().numpy(), 0, 1)
            assert np.array_equal(hm(qt.s8).view(np.uint32), ref["s8"].view(np.uint32)), (what, s, t0, "s8")
            assert np.array_equal(hm(qt.s4).view(np.uint32), ref["s4"].view(np.uint32)), (what, s, t0, "s4")
            assert np.array_equal(hm(qt.c8), ref["c8p"]), (what, s, t0, "c8")
            assert np.array_equal(hm(qt.c4), ref["c4p"]), (what, s, t0, "c4")
            if getattr(qt, "c4x", None) is not None:
                assert np.array_equal(hm(qt.c4x), ref["c4"]), (what, s, t0, "c4x")
            if layout == "cols":
                assert np.array_equal(hm(qt.t16).view(np.uint16), ref["t16"].view(np.uint16)), (what, s, t0)
            n += t1 - t0
    assert n == sum(seqlens)


@pytest.mark.parametrize("name", ["gqa8k", "varlen32k", "long128k"])
def test_quantize_full_bitexact(name):
    """Every code and scale of Q, K and V at full size (bf16 8K x 32/8 heads;
    fp16 varlen 32K; bf16 128K x 32/8 heads with outlier channels), bit for
    bit against the oracle's binary32 quantizer."""
    import torch
    import tile_routed_mixed_amd as T
    w = W.get(name)
    say(f"[gpu] full-size quantize {name}: generating inputs")
    q, k, v = W.make_qkv(w)
    p = T.PrefillPipeline(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, W.make_policy(w))
    p.upload(q[0], k[0], v[0])
    g = guard_prefill(p, T.TM_F32)
    say(f"[gpu] full-size quantize {name}")
    p.quantize()
    torch.cuda.synchronize()
    g.check()
    for x, qt, layout, what in ((q, p.qq, "rows", "Q"), (k, p.kq, "rows", "K"), (v, p.vq, "cols", "V")):
        say(f"[gpu] full-size quantize {name}: checking {what}")
        _check_codes_chunked(x[1], w.seqlens, qt, layout, f"{name} {what}")


def test_decode_cache_full_bitexact():
    """The 16 x 32768-token decode cache: every K (rows) and V (transposed,
    with its fp16 copy) code and scale bit for bit against the oracle."""
    import torch
    import tile_routed_mixed_amd as T
    w = W.get("decode16x32k")
    say("[gpu] full-size decode cache: generating inputs")
    _, k, v = W.make_qkv(w)
    dq = W.make_decode_query(w)
    p = T.DecodePipeline(w.seqlens, w.hq, w.hkv, w.d, W.make_decode_policy(w), dtype=w.dtype)
    p.upload(dq[0], k[0], v[0])
    g = guard_decode(p)
    p.build_cache()
    torch.cuda.synchronize()
    g.check()
    for x, qt, layout, what in ((k, p.kq, "rows", "K"), (v, p.vq, "cols", "V")):
        say(f"[gpu] full-size decode cache: checking {what}")
        _check_codes_chunked(x[1], w.seqlens, qt, layout, f"decode16x32k {what}")
