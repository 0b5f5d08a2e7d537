"""Oracle attention (test infrastructure only; see the package docstring).

Prefill ([TriAttention] abstract: the fused kernel skips omitted tiles and
combines both QK precisions into one normalized attention output; [TileMix]
abstract: FP16 and INT8 tile paths update one shared online-softmax state).
An online softmax over any order of the executed tiles reaches, in exact
arithmetic, the plain softmax over each row's executed key set, so that is what
is computed here, row by row, in float64:

* executed keys of row r (sequence-relative): c <= r whose tile is not SKIP
  (under the hybrid policy every c <= r, each with its own precision);
* INT8 / INT4 tile: a = sum_d cq[r, d] * ck[c, d] (exact integers),
  score = a * sq(block of r) * sk(block of c) * tau;
* FP16 tile: score = tau * sum_d q[r, d] * k[c, d] on the 16-bit values;
* m = max score, p = exp(score - m), l = sum p, O_r = sum_c (p / l) v_c with the
  unquantized 16-bit V; lse_r = m + ln l.

The method multiplies P with an fp16 copy of V ([TriAttention] abstract: one
normalized output from the unquantized values; the precision of that copy is
a reading).  A bf16 value beyond the fp16 range takes the nearest finite fp16
value, +-65504, in every fp16 copy (fp16_copy): V in the prefill's PV; the
query, and the FP16 blocks' and selected tokens' keys and values, in decode.
The INT8/INT4 codes keep the true values through their scales.  For fp16
inputs this changes nothing.

tau = 1/sqrt(d) unless given.  Query head h reads key/value head h // (hq/hkv)
(grouped-query attention, [TileMix] abstract).
"""
from __future__ import annotations

import math

import numpy as np

from . import policy as P
from .quant import BLOCK


def fp16_copy(x):
    """Values as their fp16 copy holds them, for inputs already exact in fp16
    or bf16: magnitudes beyond 65504 saturate to +-65504 (NaN stays NaN).
    Rounding of bf16 values below the fp16 normal range is not modelled (it
    moves an output by at most about 3e-8 per unit of weight)."""
    return np.clip(x, -65504.0, 65504.0)


def _tau(d, tau):
    return 1.0 / math.sqrt(d) if tau is None else float(tau)


def _rows_scores(r0, r1, h, kv, tok0, grid_h, bq, bk, q64, k64, qq, kq, blk0, tau, hybrid=None):
    """Scores [r1-r0][r1] (float64, -inf where not executed) for sequence rows
    r0..r1-1 of query head h; keys 0..r1-1 of the sequence.  The precision of
    (row, key) is its tile's entry of grid_h, or, with hybrid = (selected
    keys, window), the hybrid policy's per-key precision."""
    nrow, nkey = r1 - r0, r1
    rows = np.arange(r0, r1)
    keys = np.arange(nkey)
    if hybrid is None:
        prec = grid_h[(rows // bq)[:, None], (keys // bk)[None, :]]       # [nrow][nkey]
    else:
        prec = P.hybrid_prec(rows, keys, hybrid[0], hybrid[1])
    S = np.full((nrow, nkey), -np.inf)
    causal = keys[None, :] <= rows[:, None]
    qb = blk0 + rows // BLOCK
    kb = blk0 + keys // BLOCK
    for pr, cq, ck, sq, sk in (
        (P.INT8, qq["c8"], kq["c8"], qq["s8"], kq["s8"]),
        (P.INT4, qq["c4"], kq["c4"], qq["s4"], kq["s4"]),
    ):
        sel = (prec == pr) & causal
        if not sel.any():
            continue
        a = cq[h, qb, rows % BLOCK].astype(np.float64) @ ck[kv, kb, keys % BLOCK].astype(np.float64).T
        sc = a * sq[h, qb].astype(np.float64)[:, None] * sk[kv, kb].astype(np.float64)[None, :] * tau
        S = np.where(sel, sc, S)
    sel = (prec == P.FP16) & causal
    if sel.any():
        sc = tau * (q64[tok0 + rows, h] @ k64[tok0 + keys, kv].T)
        S = np.where(sel, sc, S)
    return S


def prefill(seqlens, hq, hkv, d, bq, bk, pol, q64, k64, v64, qq, kq, tau=None,
            rows=None, return_p=False, qtiles=None, compact=False):
    """Oracle prefill output.

    q64 [T][hq][d], k64/v64 [T][hkv][d]: float64 copies of the 16-bit inputs.
    qq, kq: oracle quantizer outputs (rows layout) for Q and K.
    rows: None for every row, else an iterable of (seq, head, row) triples.
    qtiles: alternatively, an iterable of (seq, head, query tile) triples whose
    rows are computed (used to time a bounded sample of a workload).
    Returns (O, lse) with O [T][hq][d] and lse [hq][T] (NaN where not computed),
    plus the list of probability rows when return_p is set.  With ``compact``
    nothing of size T is allocated: the result is a list of
    ((seq, head, r0, r1), O rows [r1 - r0][d], lse rows [r1 - r0]).
    """
    tau = _tau(d, tau)
    T = int(np.sum(seqlens))
    grp = hq // hkv
    O = None if compact else np.full((T, hq, d), np.nan)
    lse = None if compact else np.full((hq, T), np.nan)
    blocks = []
    hyb = int(pol["kind"]) == 3
    gs = None if hyb else P.grids(seqlens, hq, bq, bk, pol)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    plist = []
    if qtiles is not None:
        work = [(s, h, [i]) for s, h, i in qtiles]
    elif rows is None:
        work = [(s, h, None) for s in range(len(seqlens)) for h in range(hq)]
    else:
        by = {}
        for s, h, r in rows:
            by.setdefault((s, h), []).append(int(r))
        work = [(s, h, sorted(set(rs))) for (s, h), rs in sorted(by.items())]
    for s, h, rlist in work:
        S_len = int(seqlens[s])
        tok0 = int(cu[s])
        kv = h // grp
        blk0 = int(qq["blk_start"][s])
        assert int(kq["blk_start"][s]) == blk0
        g = None if hyb else gs[s][h]
        hy = (P.hybrid_selected(pol, s, h, hq), int(pol["window"])) if hyb else None
        if rlist is None:
            chunks = [(i * bq, min((i + 1) * bq, S_len)) for i in range(P.n_tiles(S_len, bq))]
        elif qtiles is not None:
            chunks = [(i * bq, min((i + 1) * bq, S_len)) for i in rlist]
        else:
            chunks = [(r, r + 1) for r in rlist]
        for r0, r1 in chunks:
            Sc = _rows_scores(r0, r1, h, kv, tok0, g, bq, bk, q64, k64, qq, kq, blk0, tau, hy)
            m = np.max(Sc, axis=1)
            assert np.all(np.isfinite(m)), "a row with no executed key"
            p = np.exp(Sc - m[:, None])
            l = np.sum(p, axis=1)
            ob = (p / l[:, None]) @ fp16_copy(v64[tok0:tok0 + r1, kv])
            if compact:
                blocks.append(((s, h, r0, r1), ob, m + np.log(l)))
            else:
                O[tok0 + r0:tok0 + r1, h] = ob
                lse[h, tok0 + r0:tok0 + r1] = m + np.log(l)
            if return_p:
                plist.append(((s, h, r0, r1), p / l[:, None]))
    if compact:
        return blocks
    if return_p:
        return O, lse, plist
    return O, lse


def int_tile_scores(qq, kq, seq, head, kv, qtile, ktile, bq, bk, prec, seqlens):
    """Exact integer QK scores of one INT8 or INT4 tile: int64 [bq][bk].

    Rows/keys past the sequence end read the zero padding codes.  Entries above
    the diagonal are included (the integer product is defined for the whole
    tile; masking happens after scaling)."""
    blk0 = int(qq["blk_start"][seq])
    nb = -(-int(seqlens[seq]) // BLOCK)
    c_q = qq["c8"] if prec == P.INT8 else qq["c4"]
    c_k = kq["c8"] if prec == P.INT8 else kq["c4"]
    d = c_q.shape[-1]

    def rows_of(c, hh, first, n):
        out = np.zeros((n, d), np.int64)
        for t in range(n):
            r = first + t
            b = r // BLOCK
            if b < nb:
                out[t] = c[hh, blk0 + b, r % BLOCK]
        return out

    A = rows_of(c_q, head, qtile * bq, bq)
    B = rows_of(c_k, kv, ktile * bk, bk)
    out = np.zeros((bq, bk), np.int64)
    for r in range(bq):
        for c in range(bk):
            out[r, c] = int(np.dot(A[r], B[c]))
    return out


def prefill_unquantized(seqlens, hq, hkv, d, bq, bk, pol, q64, k64, v64, tau=None,
                        rows=None, dense=False, compact=False):
    """Error reference, reported and never gated: softmax attention computed
    on the unquantized 16-bit values ([TriAttention] abstract: the routed
    attention keeps quality comparable to the original model; these figures
    measure how far the quantized scores move the output on synthetic inputs).

    dense=False: each row attends to the keys its policy executes (every key
    c <= r whose tile is not SKIP), so the difference to ``prefill`` is the
    quantization error alone.  dense=True: every key c <= r (plain causal
    attention), which adds the error of the skipped tiles.  Bitmask and
    hybrid policies skip nothing, so both readings coincide for them.
    rows: iterable of (seq, head, row); None for every row.  q64, k64, v64
    may be float32 copies of the 16-bit values (they are widened exactly, row
    by row).  Returns O [T][hq][d] (NaN where not computed), or with
    ``compact`` the listed rows only, [len(rows)][d] in their order."""
    tau = _tau(d, tau)
    grp = hq // hkv
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    skips = (not dense) and int(pol["kind"]) in (0, 2)
    gs = P.grids(seqlens, hq, bq, bk, pol) if skips else None
    T = int(cu[-1])
    if rows is None:
        rows = [(s, h, r) for s in range(len(seqlens)) for h in range(hq) for r in range(int(seqlens[s]))]
    rows = list(rows)
    O = np.full((len(rows), d) if compact else (T, hq, d), np.nan)
    for n, (s, h, r) in enumerate(rows):
        tok0 = int(cu[s])
        kv = h // grp
        keys = np.arange(r + 1)
        kk = np.asarray(k64[tok0 + keys, kv], np.float64)
        sc = tau * (kk @ np.asarray(q64[tok0 + r, h], np.float64))
        if skips:
            prec = gs[s][h][r // bq, keys // bk]
            sc = np.where(prec == P.SKIP, -np.inf, sc)
        m = np.max(sc)
        p = np.exp(sc - m)
        o = (p / p.sum()) @ np.asarray(v64[tok0 + keys, kv], np.float64)
        if compact:
            O[n] = o
        else:
            O[tok0 + r, h] = o
    return O


def decode_unquantized(seqlens, hq, hkv, d, q64, k64, v64, dpol, tau=None, dense=False, pairs=None):
    """Decode error reference, reported and never gated: one-query softmax
    attention over the unquantized 16-bit cache.  dense=False keeps the keys
    the cache policy reads (keys of blocks not tagged SKIP, plus selected
    tokens), dense=True every key of the cache.  Tags as in ``decode``.
    Returns O [B][hq][d]; with ``pairs`` only those (b, h) are computed."""
    tau = _tau(d, tau)
    grp = hq // hkv
    B = len(seqlens)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    O = np.zeros((B, hq, d))
    for b in range(B):
        L = int(seqlens[b])
        for h in range(hq):
            if pairs is not None and (b, h) not in pairs:
                continue
            kv = h // grp
            keep = np.ones(L, bool)
            if not dense:
                mi = h if dpol.get("per_q_head", 0) else kv
                tags = P.decode_block_tags(L, int(dpol["b8"][mi]), int(dpol["b4"][mi]), int(dpol["sink"]),
                                           int(dpol["tail"]))
                keep = np.repeat(tags != P.SKIP, BLOCK)[:L]
                if "sel_off" in dpol:
                    r = b * hkv + kv
                    lst = dpol["sel_idx"][int(dpol["sel_off"][r]):int(dpol["sel_off"][r + 1])]
                    keep[np.asarray(lst, np.int64)] = True
            keys = np.nonzero(keep)[0]
            sc = tau * (np.asarray(k64[cu[b] + keys, kv], np.float64) @ np.asarray(q64[b, h], np.float64))
            m = np.max(sc)
            p = np.exp(sc - m)
            O[b, h] = (p / p.sum()) @ np.asarray(v64[cu[b] + keys, kv], np.float64)
    return O


def decode(seqlens, hq, hkv, d, q64, kq, vq, k64, v64, dpol, tau=None, return_tags=False, pairs=None):
    """Oracle decode: one new query per sequence over its compressed cache.

    seqlens: cache length L_b per sequence (the cache includes the new token);
    q64 [B][hq][d]; kq: K quantized (rows layout), vq: V quantized (any layout:
    the unpacked rows-layout codes are used); k64/v64 [T][hkv][d] hold the
    16-bit cache values read for FP16 blocks.
    Block tags follow policy.decode_block_tags with (b8, b4) of the query's KV
    head, or of the query head itself when dpol["per_q_head"] is set (b8, b4
    then have hq entries; the reading of a per-query-head decode map).
    Selected tokens ([HyQuant] "How HyQuant works": selected tokens stay FP16
    in the decode cache too): with dpol["sel_off"] ([nseq * hkv + 1], rows
    sequence-major then KV head) and dpol["sel_idx"] (positions < L, strictly
    increasing per list), a selected key is read in FP16 whatever its block's
    tag, SKIP included; the other keys follow their block's tag.
    INT blocks: score = tau * sk * (q . ck), value = sv * cv; FP16 blocks:
    score = tau * (q . k), value = v.  Returns O [B][hq][d]; with ``pairs`` (a
    list of (b, h)) only those outputs are computed (the rest stay zero).
    """
    tau = _tau(d, tau)
    grp = hq // hkv
    B = len(seqlens)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    O = np.zeros((B, hq, d))
    tags_all = {}
    for b in range(B):
        L = int(seqlens[b])
        blk0 = int(kq["blk_start"][b])
        for h in range(hq):
            if pairs is not None and (b, h) not in pairs:
                continue
            kv = h // grp
            mi = h if dpol.get("per_q_head", 0) else kv     # whose map tags the blocks
            tags = P.decode_block_tags(L, int(dpol["b8"][mi]), int(dpol["b4"][mi]),
                                       int(dpol["sink"]), int(dpol["tail"]))
            tags_all[(b, mi)] = tags
            chosen = np.zeros(L, bool)
            if "sel_off" in dpol:
                r = b * hkv + kv
                lst = dpol["sel_idx"][int(dpol["sel_off"][r]):int(dpol["sel_off"][r + 1])]
                chosen[np.asarray(lst, np.int64)] = True
            sc_list, val_list = [], []
            qh = fp16_copy(q64[b, h])
            for j, t in enumerate(tags):
                n = min(BLOCK, L - j * BLOCK)
                keep = ~chosen[j * BLOCK: j * BLOCK + n]      # selected keys are read in FP16 below
                if t == P.SKIP:
                    continue
                if t == P.FP16:
                    kk = fp16_copy(k64[cu[b] + j * BLOCK: cu[b] + j * BLOCK + n, kv])
                    vv = fp16_copy(v64[cu[b] + j * BLOCK: cu[b] + j * BLOCK + n, kv])
                    sc_list.append((tau * (kk @ qh))[keep])
                    val_list.append(vv[keep])
                else:
                    ck = kq["c8"] if t == P.INT8 else kq["c4"]
                    cv = vq["c8"] if t == P.INT8 else vq["c4"]
                    sk = kq["s8"] if t == P.INT8 else kq["s4"]
                    sv = vq["s8"] if t == P.INT8 else vq["s4"]
                    kc = ck[kv, blk0 + j, :n].astype(np.float64)
                    vc = cv[kv, blk0 + j, :n].astype(np.float64)
                    sc_list.append((tau * float(sk[kv, blk0 + j]) * (kc @ qh))[keep])
                    val_list.append((float(sv[kv, blk0 + j]) * vc)[keep])
            sel = np.nonzero(chosen)[0]
            if len(sel):
                sc_list.append(tau * (fp16_copy(k64[cu[b] + sel, kv]) @ qh))
                val_list.append(fp16_copy(v64[cu[b] + sel, kv]))
            sc = np.concatenate(sc_list)
            vals = np.concatenate(val_list, axis=0)
            m = np.max(sc)
            p = np.exp(sc - m)
            O[b, h] = (p / p.sum()) @ vals
    if return_tags:
        return O, tags_all
    return O
