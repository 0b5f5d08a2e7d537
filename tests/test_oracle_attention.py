"""Pins for the oracle attention (CPU only).

* all-FP16 routing with nothing skipped is ordinary causal softmax attention:
  checked against torch's scaled_dot_product_attention in float64;
* all-INT8 (or all-INT4) routing is attention on the dequantized Q-hat, K-hat,
  because a * sq * sk = Q-hat . K-hat exactly: checked against the same
  library routine, with and without a skip band (boolean mask);
* skipped tiles contribute nothing: perturbing K or V inside tiles that a
  query tile skips leaves that query tile's rows bit-identical;
* softmax rows sum to one; the first row of a sequence returns v_0 exactly;
* varlen batches equal the sequences run one by one (and permute with them);
* integer tile scores: with Q codes = 127 * unit vectors the tile product is a
  known transposition of the K codes;
* decode: an all-FP16 cache is one-query softmax attention (library routine);
  an all-INT8 cache is attention on dequantized K-hat, V-hat; skipped cache
  blocks do not matter; an FP16-everything decode equals the last row of an
  all-FP16 prefill.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import policy as P
from oracle import quant as Q


def _inputs(seqlens, hq, hkv, d, seed, dtype="f16", scale_k=None):
    rng = np.random.default_rng(seed)
    T = sum(seqlens)
    q = rng.standard_normal((T, hq, d)).astype(np.float32)
    k = rng.standard_normal((T, hkv, d)).astype(np.float32)
    if scale_k is not None:
        k[:, :, :4] *= scale_k
    v = rng.standard_normal((T, hkv, d)).astype(np.float32)
    q = W.round16(q, dtype)[1]
    k = W.round16(k, dtype)[1]
    v = W.round16(v, dtype)[1]
    return q, k, v


def _sdpa(q, k, v, seqlens, hq, hkv, mask_fn=None, tau=None):
    """Library causal attention per sequence, float64, GQA by repeating K/V heads."""
    grp = hq // hkv
    out = []
    tok = 0
    for s, S in enumerate(seqlens):
        qs = torch.from_numpy(np.ascontiguousarray(q[tok:tok + S].transpose(1, 0, 2))).double()
        ks = torch.from_numpy(np.ascontiguousarray(k[tok:tok + S].transpose(1, 0, 2))).double()
        vs = torch.from_numpy(np.ascontiguousarray(v[tok:tok + S].transpose(1, 0, 2))).double()
        ks = ks.repeat_interleave(grp, dim=0)
        vs = vs.repeat_interleave(grp, dim=0)
        if mask_fn is None:
            o = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, is_causal=True, scale=tau)
        else:
            m = torch.from_numpy(mask_fn(s, S))
            o = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, attn_mask=m, scale=tau)
        out.append(o.numpy().transpose(1, 0, 2))
        tok += S
    return np.concatenate(out, axis=0)


SEQ = [200, 77, 300]
HQ, HKV, D = 4, 2, 64


def _quant(q, k):
    return Q.quantize(q, SEQ), Q.quantize(k, SEQ)


def test_all_fp16_equals_causal_attention():
    q, k, v = _inputs(SEQ, HQ, HKV, D, 1)
    qq, kq = _quant(q, k)
    _, tot = P.bitmask_row_base(SEQ, HQ, 128, 64, 4)
    pol = dict(kind=1, group=4, words=np.full(tot, 0xFFFFFFFF, np.uint32))
    O, lse = A.prefill(SEQ, HQ, HKV, D, 128, 64, pol, q.astype(np.float64), k.astype(np.float64),
                       v.astype(np.float64), qq, kq)
    ref = _sdpa(q, k, v, SEQ, HQ, HKV)
    assert np.max(np.abs(O - ref)) < 1e-12


@pytest.mark.parametrize("bits", [8, 4])
def test_int_only_equals_dequantized_attention(bits):
    q, k, v = _inputs(SEQ, HQ, HKV, D, 2, dtype="bf16", scale_k=10.0)
    qq, kq = _quant(q, k)
    big = 10 ** 6
    b8 = big if bits == 8 else 0
    pol = dict(kind=0, b8=[b8] * HQ, b4=[big] * HQ, sink=0)
    O, _ = A.prefill(SEQ, HQ, HKV, D, 128, 64, pol, q.astype(np.float64), k.astype(np.float64),
                     v.astype(np.float64), qq, kq)
    qh = Q.dequantize_rows(qq, bits, SEQ)
    kh = Q.dequantize_rows(kq, bits, SEQ)
    ref = _sdpa(qh, kh, v.astype(np.float64), SEQ, HQ, HKV)
    assert np.max(np.abs(O - ref)) < 1e-12


def test_int8_with_skip_band_equals_masked_attention():
    q, k, v = _inputs(SEQ, HQ, HKV, D, 3)
    qq, kq = _quant(q, k)
    b = [1, 2, 3, 1]
    pol = dict(kind=0, b8=b, b4=b, sink=1)
    O, _ = A.prefill(SEQ, HQ, HKV, D, 128, 64, pol, q.astype(np.float64), k.astype(np.float64),
                     v.astype(np.float64), qq, kq)
    qh = Q.dequantize_rows(qq, 8, SEQ)
    kh = Q.dequantize_rows(kq, 8, SEQ)

    def mask_fn(s, S):
        r = np.arange(S)[:, None]
        c = np.arange(S)[None, :]
        m = np.zeros((HQ, S, S), bool)
        for h in range(HQ):
            dl = np.maximum(0, ((r // 128) * 128 - (c // 64) * 64) // 64)
            keep = (dl < b[h]) | (c // 64 == 0)
            m[h] = keep & (c <= r)
        return m
    ref = _sdpa(qh, kh, v.astype(np.float64), SEQ, HQ, HKV, mask_fn=mask_fn)
    assert np.max(np.abs(O - ref)) < 1e-12


def test_skipped_tiles_contribute_nothing():
    seqlens = [640]
    q, k, v = _inputs(seqlens, 2, 1, D, 4)
    pol = dict(kind=0, b8=[1, 2], b4=[2, 4], sink=0)
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    qq, kq = Q.quantize(q, seqlens), Q.quantize(k, seqlens)
    O0, _ = A.prefill(seqlens, 2, 1, D, 128, 64, pol, q64, k64, v64, qq, kq)
    g = P.grids(seqlens, 2, 128, 64, pol)[0]
    # key tile 0 is skipped by query tile 4 of both heads (delta = 8 >= b4)
    assert g[0, 4, 0] == P.SKIP and g[1, 4, 0] == P.SKIP
    k2, v2 = k.copy(), v.copy()
    k2[0:64] = k2[0:64] * 3 + 1
    v2[0:64] = -v2[0:64] + 5
    kq2 = Q.quantize(k2, seqlens)
    O1, _ = A.prefill(seqlens, 2, 1, D, 128, 64, pol, q64, k2.astype(np.float64),
                      v2.astype(np.float64), qq, kq2)
    rows = slice(4 * 128, 5 * 128)
    assert np.array_equal(O0[rows], O1[rows])
    assert not np.allclose(O0[64:128], O1[64:128])     # rows that do execute tile 0 change


def test_rows_sum_to_one_and_first_row():
    q, k, v = _inputs(SEQ, HQ, HKV, D, 5)
    qq, kq = _quant(q, k)
    pol = dict(kind=0, b8=[1, 2, 0, 3], b4=[2, 3, 2, 3], sink=1)
    O, lse, plist = A.prefill(SEQ, HQ, HKV, D, 128, 64, pol, q.astype(np.float64), k.astype(np.float64),
                              v.astype(np.float64), qq, kq, return_p=True)
    for _, p in plist:
        assert np.allclose(p.sum(axis=1), 1.0, atol=1e-13)
    tok = 0
    for S in SEQ:
        for h in range(HQ):
            assert np.array_equal(O[tok, h], v[tok, h // 2].astype(np.float64))
        tok += S


def test_varlen_equals_separate_and_permutes():
    seqlens = [130, 64, 257]
    q, k, v = _inputs(seqlens, HQ, HKV, D, 6)
    _, tot = P.bitmask_row_base(seqlens, HQ, 128, 64, 1)
    words = np.random.default_rng(9).integers(0, 2 ** 32, size=tot, dtype=np.uint64).astype(np.uint32)
    pol = dict(kind=1, group=1, words=words)
    f64 = lambda x: x.astype(np.float64)
    O, _ = A.prefill(seqlens, HQ, HKV, D, 128, 64, pol, f64(q), f64(k), f64(v),
                     Q.quantize(q, seqlens), Q.quantize(k, seqlens))
    bases, _ = P.bitmask_row_base(seqlens, HQ, 128, 64, 1)
    tok = 0
    outs = []
    for s, S in enumerate(seqlens):
        n = HQ * P.n_tiles(S, 128) * P.bitmask_words_per_row(S, 64, 1)
        ps = dict(kind=1, group=1, words=words[bases[s]:bases[s] + n])
        sl = slice(tok, tok + S)
        Os, _ = A.prefill([S], HQ, HKV, D, 128, 64, ps, f64(q[sl]), f64(k[sl]), f64(v[sl]),
                          Q.quantize(q[sl], [S]), Q.quantize(k[sl], [S]))
        assert np.array_equal(Os, O[sl])
        outs.append((S, sl, ps))
        tok += S
    # permuted batch: sequences in order 2, 0, 1
    order = [2, 0, 1]
    perm_len = [seqlens[i] for i in order]
    qp = np.concatenate([q[outs[i][1]] for i in order])
    kp = np.concatenate([k[outs[i][1]] for i in order])
    vp = np.concatenate([v[outs[i][1]] for i in order])
    wp = np.concatenate([outs[i][2]["words"] for i in order])
    Op, _ = A.prefill(perm_len, HQ, HKV, D, 128, 64, dict(kind=1, group=1, words=wp), f64(qp), f64(kp),
                      f64(vp), Q.quantize(qp, perm_len), Q.quantize(kp, perm_len))
    assert np.array_equal(Op, np.concatenate([O[outs[i][1]] for i in order]))


@pytest.mark.parametrize("prec", [P.INT8, P.INT4])
def test_int_tile_scores_transposition(prec):
    seqlens = [100, 200]
    d, hq, hkv = 64, 2, 1
    qmax = 127 if prec == P.INT8 else 7
    rng = np.random.default_rng(10)
    q = np.zeros((300, hq, d), np.float32)
    for t in range(300):
        r = t - (0 if t < 100 else 100)
        q[t, :, r % d] = qmax                      # unit vector times qmax: scale 1, code qmax
    k = rng.integers(-qmax, qmax + 1, size=(300, hkv, d)).astype(np.float32)
    k[:, :, d - 1] = qmax                           # force amax = qmax in every block: codes = k
    k[:, :, d - 1][::2] = -qmax
    qq, kq = Q.quantize(q, seqlens), Q.quantize(k, seqlens)
    for (seq, qtile, ktile) in [(0, 0, 0), (0, 0, 1), (1, 1, 0), (1, 1, 3)]:
        a = A.int_tile_scores(qq, kq, seq, 1, 0, qtile, ktile, 128, 64, prec, seqlens)
        S = seqlens[seq]
        tok0 = 0 if seq == 0 else 100
        for rr in range(128):
            r = qtile * 128 + rr
            for cc in range(64):
                c = ktile * 64 + cc
                want = 0 if (r >= S or c >= S) else qmax * int(k[tok0 + c, 0, r % d])
                assert a[rr, cc] == want


DQ_SEQ = [100, 1000, 700]


def _decode_inputs(seed=12):
    rng = np.random.default_rng(seed)
    T = sum(DQ_SEQ)
    k = W.round16(rng.standard_normal((T, HKV, D)).astype(np.float32), "f16")[1]
    v = W.round16(rng.standard_normal((T, HKV, D)).astype(np.float32), "f16")[1]
    q = W.round16(rng.standard_normal((len(DQ_SEQ), HQ, D)).astype(np.float32), "f16")[1]
    return q, k, v


def _sdpa_one(q, k, v):
    """One query per (sequence, head) against all cache rows of the sequence."""
    out = np.zeros(q.shape)
    tok = 0
    for b, L in enumerate(DQ_SEQ):
        for h in range(HQ):
            qs = torch.from_numpy(q[b, h][None, None, :]).double()
            ks = torch.from_numpy(np.ascontiguousarray(k[tok:tok + L, h // 2]))[None].double()
            vs = torch.from_numpy(np.ascontiguousarray(v[tok:tok + L, h // 2]))[None].double()
            out[b, h] = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs)[0, 0].numpy()
        tok += L
    return out


def test_decode_all_fp16_is_attention():
    q, k, v = _decode_inputs()
    kq, vq = Q.quantize(k, DQ_SEQ), Q.quantize(v, DQ_SEQ, layout="cols")
    dpol = dict(b8=[0, 0], b4=[0, 0], sink=0, tail=10 ** 6)
    O = A.decode(DQ_SEQ, HQ, HKV, D, q.astype(np.float64), kq, vq, k.astype(np.float64),
                 v.astype(np.float64), dpol)
    assert np.max(np.abs(O - _sdpa_one(q, k, v))) < 1e-12


def test_decode_all_int8_is_dequantized_attention():
    q, k, v = _decode_inputs(13)
    kq, vq = Q.quantize(k, DQ_SEQ), Q.quantize(v, DQ_SEQ, layout="cols")
    dpol = dict(b8=[10 ** 6] * 2, b4=[10 ** 6] * 2, sink=1, tail=0)
    O = A.decode(DQ_SEQ, HQ, HKV, D, q.astype(np.float64), kq, vq, k.astype(np.float64),
                 v.astype(np.float64), dpol)
    kh = Q.dequantize_rows(kq, 8, DQ_SEQ)
    vh = Q.dequantize_rows(vq, 8, DQ_SEQ)
    assert np.max(np.abs(O - _sdpa_one(q, kh, vh))) < 1e-12


def test_decode_skipped_blocks_do_not_matter():
    q, k, v = _decode_inputs(14)
    dpol = dict(b8=[2, 3], b4=[4, 5], sink=1, tail=128)
    kq, vq = Q.quantize(k, DQ_SEQ), Q.quantize(v, DQ_SEQ, layout="cols")
    O0, tags = A.decode(DQ_SEQ, HQ, HKV, D, q.astype(np.float64), kq, vq, k.astype(np.float64),
                        v.astype(np.float64), dpol, return_tags=True)
    t = tags[(1, 0)]
    j = int(np.nonzero(t == P.SKIP)[0][0])
    k2, v2 = k.copy(), v.copy()
    rows = slice(100 + 64 * j, 100 + 64 * j + 64)
    k2[rows] = 7.0
    v2[rows] = -3.0
    kq2, vq2 = Q.quantize(k2, DQ_SEQ), Q.quantize(v2, DQ_SEQ, layout="cols")
    O1 = A.decode(DQ_SEQ, HQ, HKV, D, q.astype(np.float64), kq2, vq2, k2.astype(np.float64),
                  v2.astype(np.float64), dpol)
    assert np.array_equal(O0[1, :2], O1[1, :2])


def test_decode_fp16_equals_last_prefill_row():
    L = 300
    rng = np.random.default_rng(15)
    q = W.round16(rng.standard_normal((L, HQ, D)).astype(np.float32), "f16")[1]
    k = W.round16(rng.standard_normal((L, HKV, D)).astype(np.float32), "f16")[1]
    v = W.round16(rng.standard_normal((L, HKV, D)).astype(np.float32), "f16")[1]
    _, tot = P.bitmask_row_base([L], HQ, 128, 64, 4)
    pol = dict(kind=1, group=4, words=np.full(tot, 0xFFFFFFFF, np.uint32))
    f64 = lambda x: x.astype(np.float64)
    Op, _ = A.prefill([L], HQ, HKV, D, 128, 64, pol, f64(q), f64(k), f64(v),
                      Q.quantize(q, [L]), Q.quantize(k, [L]), rows=[(0, h, L - 1) for h in range(HQ)])
    dpol = dict(b8=[0, 0], b4=[0, 0], sink=0, tail=L)
    Od = A.decode([L], HQ, HKV, D, f64(q[L - 1:L]), Q.quantize(k, [L]), Q.quantize(v, [L], layout="cols"),
                  f64(k), f64(v), dpol)
    assert np.max(np.abs(Od[0] - Op[L - 1])) < 1e-13


def test_decode_per_query_head_maps_reduce_to_per_kv_maps():
    """A per-query-head map tags head h's blocks as a per-KV-head map holding
    head h's (b8, b4) for every KV head would; heads of one KV group may
    differ."""
    q, k, v = _decode_inputs(16)
    kq, vq = Q.quantize(k, DQ_SEQ), Q.quantize(v, DQ_SEQ, layout="cols")
    f64 = lambda x: x.astype(np.float64)
    b8, b4 = [1, 3, 0, 2], [2, 5, 4, 2]
    dq = dict(b8=b8, b4=b4, sink=1, tail=100, per_q_head=1)
    O = A.decode(DQ_SEQ, HQ, HKV, D, f64(q), kq, vq, f64(k), f64(v), dq)
    for h in range(HQ):
        dk = dict(b8=[b8[h]] * HKV, b4=[b4[h]] * HKV, sink=1, tail=100)
        Oh = A.decode(DQ_SEQ, HQ, HKV, D, f64(q), kq, vq, f64(k), f64(v), dk)
        assert np.array_equal(O[:, h], Oh[:, h])
    # heads 0 and 1 share a KV head but not a map: their tags differ
    _, tags = A.decode(DQ_SEQ, HQ, HKV, D, f64(q), kq, vq, f64(k), f64(v), dq, return_tags=True)
    assert not np.array_equal(tags[(1, 0)], tags[(1, 1)])


def _dsel(lists):
    off = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    idx = np.concatenate([np.asarray(x, np.int64) for x in lists]).astype(np.int32)
    return off, idx


def test_decode_selected_tokens():
    """Selected decode tokens: none changes nothing; every key selected is the
    all-FP16 decode; selecting keys of FP16 blocks changes nothing; selecting a
    key of a skipped block adds exactly that key in FP16 (checked against a
    softmax written out for that row)."""
    q, k, v = _decode_inputs(17)
    kq, vq = Q.quantize(k, DQ_SEQ), Q.quantize(v, DQ_SEQ, layout="cols")
    f64 = lambda x: x.astype(np.float64)
    base = dict(b8=[2, 3], b4=[4, 5], sink=1, tail=128)
    O = A.decode(DQ_SEQ, HQ, HKV, D, f64(q), kq, vq, f64(k), f64(v), base)
    nl = len(DQ_SEQ) * HKV
    off, idx = _dsel([[] for _ in range(nl)])
    O0 = A.decode(DQ_SEQ, HQ, HKV, D, f64(q), kq, vq, f64(k), f64(v), dict(base, sel_off=off, sel_idx=idx))
    assert np.array_equal(O, O0)
    every = [list(range(L)) for L in DQ_SEQ for _ in range(HKV)]
    off, idx = _dsel(every)
    Oa = A.decode(DQ_SEQ, HQ, HKV, D, f64(q), kq, vq, f64(k), f64(v), dict(base, sel_off=off, sel_idx=idx))
    O16 = A.decode(DQ_SEQ, HQ, HKV, D, f64(q), kq, vq, f64(k), f64(v), dict(base, tail=10 ** 6))
    assert np.max(np.abs(Oa - O16)) < 1e-12
    # keys inside the FP16 tail of sequence 1 (length L1): selecting them changes nothing
    L1 = DQ_SEQ[1]
    lists = [[] for _ in range(nl)]
    lists[1 * HKV + 0] = [L1 - 3, L1 - 1]
    off, idx = _dsel(lists)
    Ot = A.decode(DQ_SEQ, HQ, HKV, D, f64(q), kq, vq, f64(k), f64(v), dict(base, sel_off=off, sel_idx=idx))
    assert np.max(np.abs(Ot - O)) < 1e-12
    # a key of a skipped block of sequence 1, KV head 0: only heads 0, 1 of sequence 1 change
    _, tags = A.decode(DQ_SEQ, HQ, HKV, D, f64(q), kq, vq, f64(k), f64(v), base, return_tags=True)
    j = int(np.nonzero(tags[(1, 0)] == P.SKIP)[0][0])
    c = 64 * j + 5
    lists[1 * HKV + 0] = [c]
    off, idx = _dsel(lists)
    Os = A.decode(DQ_SEQ, HQ, HKV, D, f64(q), kq, vq, f64(k), f64(v), dict(base, sel_off=off, sel_idx=idx))
    changed = {(b, h) for b in range(len(DQ_SEQ)) for h in range(HQ) if not np.array_equal(Os[b, h], O[b, h])}
    assert changed == {(1, 0), (1, 1)}
    # head 0 of sequence 1 written out: the unselected softmax plus key c at 16-bit precision
    tok0 = DQ_SEQ[0]
    tau = 1 / np.sqrt(D)
    t = tags[(1, 0)]
    sc, vals = [], []
    for jj, tg in enumerate(t):
        n = min(64, L1 - 64 * jj)
        if tg == P.SKIP:
            continue
        if tg == P.FP16:
            sc += list(tau * (f64(k)[tok0 + 64 * jj: tok0 + 64 * jj + n, 0] @ f64(q)[1, 0]))
            vals += list(f64(v)[tok0 + 64 * jj: tok0 + 64 * jj + n, 0])
        else:
            c8 = kq["c8"] if tg == P.INT8 else kq["c4"]
            v8 = vq["c8"] if tg == P.INT8 else vq["c4"]
            s8 = kq["s8"] if tg == P.INT8 else kq["s4"]
            w8 = vq["s8"] if tg == P.INT8 else vq["s4"]
            b0 = int(kq["blk_start"][1])
            sc += list(tau * float(s8[0, b0 + jj]) * (c8[0, b0 + jj, :n].astype(np.float64) @ f64(q)[1, 0]))
            vals += list(float(w8[0, b0 + jj]) * v8[0, b0 + jj, :n].astype(np.float64))
    sc.append(tau * float(f64(k)[tok0 + c, 0] @ f64(q)[1, 0]))
    vals.append(f64(v)[tok0 + c, 0])
    sc = np.array(sc)
    pr = np.exp(sc - sc.max())
    pr /= pr.sum()
    assert np.max(np.abs(Os[1, 0] - pr @ np.array(vals))) < 1e-12


# ---------------------------------------------------------------- error references

def _band_mask(b8, b4, sink, hq):
    """Executed keys of each row under per-head boundaries, written out from the
    diagonal-distance reading for 128-row query tiles and 64-key tiles."""
    def mask_fn(s, S):
        r = np.arange(S)[:, None]
        c = np.arange(S)[None, :]
        m = np.zeros((hq, S, S), bool)
        for h in range(hq):
            dl = np.maximum(0, ((r // 128) * 128 - (c // 64) * 64) // 64)
            keep = dl < b4[h]
            if sink:
                keep = keep | (c // 64 == 0)
            m[h] = keep & (c <= r)
        return m
    return mask_fn


def test_unquantized_dense_is_causal_attention():
    """prefill_unquantized(dense=True) ignores the policy: plain causal softmax
    attention on the 16-bit values (library routine, float64)."""
    q, k, v = _inputs(SEQ, HQ, HKV, D, 21, dtype="bf16", scale_k=10.0)
    pol = dict(kind=0, b8=[1, 0, 2, 1], b4=[2, 1, 3, 2], sink=0)
    f64 = lambda x: x.astype(np.float64)
    O = A.prefill_unquantized(SEQ, HQ, HKV, D, 128, 64, pol, f64(q), f64(k), f64(v), dense=True)
    assert np.max(np.abs(O - _sdpa(q, k, v, SEQ, HQ, HKV))) < 1e-12


@pytest.mark.parametrize("sink", [0, 1])
def test_unquantized_same_skip_is_band_masked_attention(sink):
    """prefill_unquantized(dense=False) keeps exactly the keys whose tiles are
    executed: attention on the 16-bit values under the band mask of the
    boundaries (and the sink tile)."""
    q, k, v = _inputs(SEQ, HQ, HKV, D, 22)
    b8, b4 = [1, 0, 2, 1], [2, 1, 3, 2]
    pol = dict(kind=0, b8=b8, b4=b4, sink=sink)
    f64 = lambda x: x.astype(np.float64)
    O = A.prefill_unquantized(SEQ, HQ, HKV, D, 128, 64, pol, f64(q), f64(k), f64(v))
    ref = _sdpa(q, k, v, SEQ, HQ, HKV, mask_fn=_band_mask(b8, b4, sink, HQ))
    assert np.max(np.abs(O - ref)) < 1e-12
    # and it differs from the dense reference (some tiles are skipped)
    Od = A.prefill_unquantized(SEQ, HQ, HKV, D, 128, 64, pol, f64(q), f64(k), f64(v), dense=True)
    assert np.max(np.abs(O - Od)) > 1e-3


def test_unquantized_equals_quantized_oracle_on_all_fp16():
    """With every tile FP16 and nothing skipped, the quantized oracle, the
    same-skip reference and the dense reference are one computation."""
    q, k, v = _inputs(SEQ, HQ, HKV, D, 23)
    qq, kq = _quant(q, k)
    _, tot = P.bitmask_row_base(SEQ, HQ, 128, 64, 4)
    pol = dict(kind=1, group=4, words=np.full(tot, 0xFFFFFFFF, np.uint32))
    f64 = lambda x: x.astype(np.float64)
    O, _ = A.prefill(SEQ, HQ, HKV, D, 128, 64, pol, f64(q), f64(k), f64(v), qq, kq)
    Ou = A.prefill_unquantized(SEQ, HQ, HKV, D, 128, 64, pol, f64(q), f64(k), f64(v))
    assert np.max(np.abs(O - Ou)) < 1e-12


def test_decode_all_int4_is_dequantized_attention():
    """Every cache block INT4 (b8 = 0, no sink, no FP16 window): one-query
    attention on K-hat = s4 * c4 and V-hat = s4 * c4 (library routine)."""
    q, k, v = _decode_inputs(18)
    kq, vq = Q.quantize(k, DQ_SEQ), Q.quantize(v, DQ_SEQ, layout="cols")
    dpol = dict(b8=[0, 0], b4=[10 ** 6] * 2, sink=0, tail=0)
    O = A.decode(DQ_SEQ, HQ, HKV, D, q.astype(np.float64), kq, vq, k.astype(np.float64),
                 v.astype(np.float64), dpol)
    kh = Q.dequantize_rows(kq, 4, DQ_SEQ)
    vh = Q.dequantize_rows(vq, 4, DQ_SEQ)
    assert np.max(np.abs(O - _sdpa_one(q, kh, vh))) < 1e-12
    # the INT8 reading of the same cache is a different computation
    vh8 = Q.dequantize_rows(vq, 8, DQ_SEQ)
    assert np.max(np.abs(O - _sdpa_one(q, Q.dequantize_rows(kq, 8, DQ_SEQ), vh8))) > 1e-3


def test_decode_unquantized_references():
    """decode_unquantized: dense = one-query attention over the whole cache;
    same-skip = attention over the keys of the blocks the tags read, with the
    block mask written out from the decode reading (last `tail` tokens FP16,
    block 0 under a sink, distance floor((L-1)/64) - j below b4)."""
    q, k, v = _decode_inputs(19)
    f64 = lambda x: x.astype(np.float64)
    dpol = dict(b8=[2, 3], b4=[4, 6], sink=1, tail=100)
    Od = A.decode_unquantized(DQ_SEQ, HQ, HKV, D, f64(q), f64(k), f64(v), dpol, dense=True)
    assert np.max(np.abs(Od - _sdpa_one(q, k, v))) < 1e-12
    Os = A.decode_unquantized(DQ_SEQ, HQ, HKV, D, f64(q), f64(k), f64(v), dpol)
    tok = 0
    for b, L in enumerate(DQ_SEQ):
        for h in range(HQ):
            kv = h // 2
            c = np.arange(L)
            j = c // 64
            blk_end = np.minimum(64 * j + 64, L)
            keep = (blk_end > L - dpol["tail"]) | (j == 0) | ((L - 1) // 64 - j < dpol["b4"][kv])
            qs = torch.from_numpy(q[b, h][None, None, :]).double()
            ks = torch.from_numpy(np.ascontiguousarray(k[tok:tok + L, kv][keep]))[None].double()
            vs = torch.from_numpy(np.ascontiguousarray(v[tok:tok + L, kv][keep]))[None].double()
            ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs)[0, 0].numpy()
            assert np.max(np.abs(Os[b, h] - ref)) < 1e-12, (b, h)
        tok += L
    assert np.max(np.abs(Os - Od)) > 1e-4


def test_unquantized_compact_rows_match_full():
    q, k, v = _inputs(SEQ, HQ, HKV, D, 24)
    pol = dict(kind=0, b8=[1, 0, 2, 1], b4=[2, 1, 3, 2], sink=1)
    rows = [(2, 3, 299), (0, 0, 0), (1, 2, 76), (2, 1, 130)]
    full = A.prefill_unquantized(SEQ, HQ, HKV, D, 128, 64, pol, q, k, v)
    comp = A.prefill_unquantized(SEQ, HQ, HKV, D, 128, 64, pol, q, k, v, rows=rows, compact=True)
    cu = np.concatenate([[0], np.cumsum(SEQ)])
    for n, (s, h, r) in enumerate(rows):
        assert np.array_equal(comp[n], full[cu[s] + r, h])


# ---------------------------------------------------------------- fp16 copies of bf16 values

def _plant_big(x, seed, vals=(1.0e5, -3.0e38, 70000.0)):
    """bf16 values beyond the fp16 range planted at a few seeded places."""
    rng = np.random.default_rng(seed)
    y = x.copy()
    flat = y.reshape(-1)
    for i, val in zip(rng.choice(flat.size, len(vals), replace=False), vals):
        flat[i] = W.round16(np.array([val], np.float32), "bf16")[1][0]
    return y


def test_fp16_copy_saturates_and_keeps_nan():
    x = np.array([65504.0, 65505.0, -1e5, 3e38, -65504.0, 1.0, np.nan])
    y = A.fp16_copy(x)
    assert list(y[:6]) == [65504.0, 65504.0, -65504.0, 65504.0, -65504.0, 1.0] and np.isnan(y[6])


def test_bf16_beyond_fp16_range_prefill_is_attention_with_saturated_v():
    """All-FP16 policy over bf16 inputs whose V holds values beyond the fp16
    range: causal SDPA with V saturated to +-65504 (the fp16 copy PV uses)."""
    q, k, v = _inputs(SEQ, HQ, HKV, D, 21, dtype="bf16")
    v = _plant_big(v, 22)
    assert np.max(np.abs(v)) > 65504
    qq, kq = _quant(q, k)
    _, tot = P.bitmask_row_base(SEQ, HQ, 128, 64, 4)
    pol = dict(kind=1, group=4, words=np.full(tot, 0xFFFFFFFF, np.uint32))
    O, _ = A.prefill(SEQ, HQ, HKV, D, 128, 64, pol, q.astype(np.float64), k.astype(np.float64),
                     v.astype(np.float64), qq, kq)
    ref = _sdpa(q, k, np.clip(v.astype(np.float64), -65504.0, 65504.0), SEQ, HQ, HKV)
    assert np.all(np.isfinite(O))
    assert np.max(np.abs(O - ref)) < 1e-9
    # and the quantizer's fp16 copy holds the same saturated values
    vq = Q.quantize(v, SEQ, layout="cols", with_t16=True)
    t = vq["t16"].astype(np.float64)
    assert np.max(np.abs(t)) == 65504.0 and np.all(np.isfinite(t))


def test_bf16_beyond_fp16_range_decode_is_attention_with_saturated_q_and_window():
    """All-FP16 decode (every block in the window) over bf16 values beyond the
    fp16 range in q, K and V: one-query SDPA on the saturated values."""
    q, k, v = _decode_inputs(23)
    q, k, v = (W.round16(x.astype(np.float32), "bf16")[1] for x in (q, k, v))
    q, k, v = _plant_big(q, 24, (1.0e5,)), _plant_big(k, 25), _plant_big(v, 26)
    kq, vq = Q.quantize(k, DQ_SEQ), Q.quantize(v, DQ_SEQ, layout="cols")
    dpol = dict(b8=[0, 0], b4=[0, 0], sink=0, tail=10 ** 6)
    f64 = lambda x: x.astype(np.float64)
    O = A.decode(DQ_SEQ, HQ, HKV, D, f64(q), kq, vq, f64(k), f64(v), dpol)
    c = lambda x: np.clip(f64(x), -65504.0, 65504.0)
    ref = _sdpa_one(c(q), c(k), c(v))
    assert np.all(np.isfinite(O))
    assert np.max(np.abs(O - ref)) < 1e-9 * max(1.0, float(np.max(np.abs(ref))))
