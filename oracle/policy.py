"""Oracle tile-precision policy (test infrastructure only; see the package docstring).

Sources:
* [TriAttention] abstract: each query-key tile goes to skip, 4-bit or 8-bit
  computation; each head's regions are encoded by two diagonal-distance
  boundaries (storage independent of context length); the boundaries expand
  into precision-grouped traversals and omitted tiles are skipped.
* [TileMix] abstract: the score matrix is split into hardware-aligned tiles;
  routing decisions are packed into compact bitmasks; one routing bit governs a
  group of adjacent key tiles; each group runs FP16 or INT8 score computation;
  all legal tile groups are routed (no skip); grouped-query attention and
  variable-length batches are supported.

Readings taken where the pages are silent:
* tiles restart at each sequence start; tile (i, j) covers query rows
  [i*bq, (i+1)*bq) and keys [j*bk, (j+1)*bk) of the sequence; it is legal iff
  its first key is causally visible from its last valid row:
  j*bk <= min((i+1)*bq, S) - 1;
* diagonal distance in key-tile units from the query tile's first row, clipped
  at zero: delta(i, j) = max(0, floor((i*bq - j*bk) / bk));
* boundaries (b8, b4) per query head, 0 <= b8 <= b4: delta < b8 -> INT8,
  b8 <= delta < b4 -> INT4, delta >= b4 -> SKIP; with ``sink`` set, key tile 0
  is INT8 for every query tile;
* bitmask: bit = 1 -> FP16, 0 -> INT8; group g covers key tiles
  [g*G, (g+1)*G); each (sequence, query head, query tile) row holds
  ceil(ceil(nk / G) / 32) uint32 words, LSB-first; rows are laid out
  sequence-major, then head, then query tile; the legal tiles of a partly
  legal group take the group's bit;
* four-way (both encodings in one): the boundaries (b8, b4, sink) of a head
  plus a 2-bit code per group of G key tiles, 16 codes per uint32 word
  (group g in bits 2(g mod 16) .. 2(g mod 16) + 1 of the row's word g div 16),
  ceil(ceil(nk / G) / 16) words per row in the bitmask's row order; code 0
  leaves the tile to the boundary rule (so SKIP comes only from there),
  codes 1, 2, 3 set INT4, INT8, FP16.  All-zero codes give the boundary
  policy; codes drawn from {2, 3} give the bitmask policy with bit = (code
  == 3).
* hybrid ([HyQuant] "How HyQuant works": selected vertical-line tokens and a
  local sliding window stay FP16, the rest of the context is quantized):
  precision is per (row, key) rather than per tile.  Key c of row r (c <= r)
  is FP16 if c is in the selected set of the row's (sequence, query head) or
  r - c < window, else INT8 (the rest is read as INT8, the cache precision the
  other pages name; nothing is skipped).  Selected sets are index lists:
  sel_off [nseq * hq + 1] row offsets (sequence-major, then query head) into
  sel_idx, each list strictly increasing positions within its sequence.
"""
from __future__ import annotations

import numpy as np

SKIP, INT4, INT8, FP16 = 0, 1, 2, 3
ILLEGAL = -1


def n_tiles(S: int, b: int) -> int:
    return -(-int(S) // int(b))


def is_legal(i: int, j: int, S: int, bq: int, bk: int) -> bool:
    return j * bk <= min((i + 1) * bq, S) - 1


def diag_distance(i: int, j: int, bq: int, bk: int) -> int:
    return max(0, (i * bq - j * bk) // bk)


def boundary_prec(i: int, j: int, bq: int, bk: int, b8: int, b4: int, sink: int) -> int:
    if sink and j == 0:
        return INT8
    dl = diag_distance(i, j, bq, bk)
    if dl < b8:
        return INT8
    if dl < b4:
        return INT4
    return SKIP


def bitmask_words_per_row(S: int, bk: int, group: int) -> int:
    ng = n_tiles(n_tiles(S, bk), group)
    return n_tiles(ng, 32)


def bitmask_row_base(seqlens, hq: int, bq: int, bk: int, group: int):
    """Word offset of row (s, h=0, i=0) for each sequence, and the total."""
    bases, acc = [], 0
    for S in seqlens:
        bases.append(acc)
        acc += hq * n_tiles(S, bq) * bitmask_words_per_row(S, bk, group)
    return bases, acc


def bitmask_bit(words: np.ndarray, row_off: int, g: int) -> int:
    return int((int(words[row_off + g // 32]) >> (g % 32)) & 1)


def fourway_words_per_row(S: int, bk: int, group: int) -> int:
    ng = n_tiles(n_tiles(S, bk), group)
    return n_tiles(ng, 16)


def fourway_row_base(seqlens, hq: int, bq: int, bk: int, group: int):
    """Word offset of row (s, h=0, i=0) of a four-way code map, and the total."""
    bases, acc = [], 0
    for S in seqlens:
        bases.append(acc)
        acc += hq * n_tiles(S, bq) * fourway_words_per_row(S, bk, group)
    return bases, acc


def fourway_code(words: np.ndarray, row_off: int, g: int) -> int:
    return int((int(words[row_off + g // 16]) >> (2 * (g % 16))) & 3)


CODE_PREC = {1: INT4, 2: INT8, 3: FP16}


def precision_grid_loop(S, bq, bk, head, pol, seq=0, seqlens=None, hq=None):
    """Brute force over every (i, j) with plain Python loops: [nq][nk] int8."""
    nq, nk = n_tiles(S, bq), n_tiles(S, bk)
    g = np.full((nq, nk), ILLEGAL, np.int8)
    if pol["kind"] == 1:
        bases, _ = bitmask_row_base(seqlens, hq, bq, bk, pol["group"])
        wpr = bitmask_words_per_row(S, bk, pol["group"])
    if pol["kind"] == 2:
        bases, _ = fourway_row_base(seqlens, hq, bq, bk, pol["group"])
        wpr = fourway_words_per_row(S, bk, pol["group"])
    for i in range(nq):
        for j in range(nk):
            if not is_legal(i, j, S, bq, bk):
                continue
            if pol["kind"] in (0, 2):
                g[i, j] = boundary_prec(i, j, bq, bk, int(pol["b8"][head]), int(pol["b4"][head]),
                                        int(pol["sink"]))
                if pol["kind"] == 2:
                    code = fourway_code(pol["words"], bases[seq] + (head * nq + i) * wpr, j // pol["group"])
                    if code:
                        g[i, j] = CODE_PREC[code]
            else:
                row = bases[seq] + (head * nq + i) * wpr
                g[i, j] = FP16 if bitmask_bit(pol["words"], row, j // pol["group"]) else INT8
    return g


def precision_grid(S, bq, bk, head, pol, seq=0, seqlens=None, hq=None):
    """Same map as precision_grid_loop, with the loops vectorized by numpy."""
    nq, nk = n_tiles(S, bq), n_tiles(S, bk)
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    legal = j * bk <= np.minimum((i + 1) * bq, S) - 1
    if pol["kind"] in (0, 2):
        dl = np.maximum(0, (i * bq - j * bk) // bk)
        b8, b4 = int(pol["b8"][head]), int(pol["b4"][head])
        p = np.where(dl < b8, INT8, np.where(dl < b4, INT4, SKIP))
        if int(pol["sink"]) and nk > 0:   # (an empty sequence has no tiles)
            p[:, 0] = INT8
        if pol["kind"] == 2:
            G = pol["group"]
            bases, _ = fourway_row_base(seqlens, hq, bq, bk, G)
            wpr = fourway_words_per_row(S, bk, G)
            row = bases[seq] + (head * nq + np.arange(nq)) * wpr           # [nq]
            gidx = np.arange(nk) // G                                      # [nk]
            words = np.asarray(pol["words"], dtype=np.uint64)
            w = words[row[:, None] + gidx[None, :] // 16]
            code = (w >> (2 * (gidx[None, :] % 16)).astype(np.uint64)) & np.uint64(3)
            p = np.where(code == 1, INT4, np.where(code == 2, INT8, np.where(code == 3, FP16, p)))
    else:
        G = pol["group"]
        bases, _ = bitmask_row_base(seqlens, hq, bq, bk, G)
        wpr = bitmask_words_per_row(S, bk, G)
        row = bases[seq] + (head * nq + np.arange(nq)) * wpr                # [nq]
        gidx = np.arange(nk) // G                                          # [nk]
        words = np.asarray(pol["words"], dtype=np.uint64)
        w = words[row[:, None] + gidx[None, :] // 32]
        bit = (w >> (gidx[None, :] % 32).astype(np.uint64)) & np.uint64(1)
        p = np.where(bit == 1, FP16, INT8)
    return np.where(legal, p, ILLEGAL).astype(np.int8)


def grids(seqlens, hq, bq, bk, pol, loop=False):
    """Precision grids for every (sequence, query head): list over sequences of
    [hq][nq][nk] int8 arrays (ILLEGAL = -1 outside the causal region)."""
    f = precision_grid_loop if loop else precision_grid
    out = []
    for s, S in enumerate(seqlens):
        out.append(np.stack([f(int(S), bq, bk, h, pol, s, seqlens, hq) for h in range(hq)]))
    return out


def census(gs):
    """Tile counts over all grids: legal, INT8, INT4, FP16, SKIP."""
    c = dict(legal=0, int8=0, int4=0, fp16=0, skip=0)
    for g in gs:
        c["legal"] += int(np.sum(g != ILLEGAL))
        c["int8"] += int(np.sum(g == INT8))
        c["int4"] += int(np.sum(g == INT4))
        c["fp16"] += int(np.sum(g == FP16))
        c["skip"] += int(np.sum(g == SKIP))
    return c


def executed_tiles(gs):
    """Set of (seq, head, qtile, ktile, prec) for every non-skipped legal tile."""
    out = set()
    for s, g in enumerate(gs):
        h, i, j = np.nonzero((g != ILLEGAL) & (g != SKIP))
        for a, b, c in zip(h.tolist(), i.tolist(), j.tolist()):
            out.add((s, a, b, c, int(g[a, b, c])))
    return out


def decode_block_tags(L: int, b8: int, b4: int, sink: int, tail: int, block: int = 64):
    """Precision of each 64-token block of a cache of L tokens, for the one new
    query at position L - 1 (the cache includes the current token).

    [HyQuant] section "How HyQuant works": recent tokens stay FP16 and the rest
    is quantized, with dequantization fused into decode attention;
    [TriAttention] abstract: the prefill codes are reused as the decode cache.
    Reading taken: blocks overlapping the last ``tail`` tokens are FP16; every
    other block j has distance delta = floor((L - 1) / 64) - j from the query's
    block and is tagged by the boundary rule (INT8 below b8, INT4 below b4,
    SKIP otherwise), with block 0 kept INT8 when ``sink`` is set.
    """
    nb = n_tiles(L, block)
    tags = np.zeros(nb, np.int8)
    last = (L - 1) // block
    for j in range(nb):
        if min(j * block + block, L) > L - tail:
            tags[j] = FP16
        elif sink and j == 0:
            tags[j] = INT8
        else:
            dl = last - j
            tags[j] = INT8 if dl < b8 else (INT4 if dl < b4 else SKIP)
    return tags


# ---------------------------------------------------------------- hybrid

def hybrid_selected(pol, seq: int, head: int, hq: int) -> np.ndarray:
    """Selected key positions of (sequence, query head), ascending."""
    r = seq * hq + head
    off = pol["sel_off"]
    return np.asarray(pol["sel_idx"][int(off[r]):int(off[r + 1])], dtype=np.int64)


def hybrid_prec(rows: np.ndarray, keys: np.ndarray, sel: np.ndarray, window: int) -> np.ndarray:
    """[len(rows)][len(keys)] int8: FP16 where the key is selected or lies
    within `window` tokens before the row, else INT8 (causality is the
    caller's)."""
    fp = np.isin(keys, sel)[None, :] | ((rows[:, None] - keys[None, :]) < window)
    return np.where(fp, FP16, INT8).astype(np.int8)


def hybrid_prec_loop(S: int, sel, window: int) -> np.ndarray:
    """Brute force over every (r, c) with plain loops: [S][S] int8, ILLEGAL
    above the diagonal."""
    chosen = set(int(x) for x in sel)
    g = np.full((S, S), ILLEGAL, np.int8)
    for r in range(S):
        for c in range(r + 1):
            g[r, c] = FP16 if (c in chosen or r - c < window) else INT8
    return g


WIN_NONE, WIN_EDGE, WIN_FULL = 0, 1, 2


def hybrid_tile_classes(S: int, bq: int, bk: int, window: int) -> np.ndarray:
    """Window class of every legal tile, from the causal (row, key) pairs it
    holds (rows and keys inside the sequence): FULL if all are within the
    window, NONE if none is, else EDGE.  [nq][nk] int8, ILLEGAL outside."""
    nq, nk = n_tiles(S, bq), n_tiles(S, bk)
    out = np.full((nq, nk), ILLEGAL, np.int8)
    for i in range(nq):
        for j in range(nk):
            if not is_legal(i, j, S, bq, bk):
                continue
            r = np.arange(i * bq, min((i + 1) * bq, S))[:, None]
            c = np.arange(j * bk, min((j + 1) * bk, S))[None, :]
            causal = c <= r
            inwin = (r - c < window) & causal
            n_in, n_all = int(inwin.sum()), int(causal.sum())
            out[i, j] = WIN_FULL if n_in == n_all else (WIN_NONE if n_in == 0 else WIN_EDGE)
    return out


# ---------------------------------------------------------------- selection

def vline_importance(q64: np.ndarray, k64: np.ndarray, n_obs: int, tau: float) -> np.ndarray:
    """Vertical-line signal of one (sequence, query head) ([HyQuant] "How
    HyQuant works": tokens are picked from attention-pattern signals; section
    "The observation behind the method": a few key positions are attended by
    many queries).  Reading: the attention mass each key receives from the
    last n_obs query rows of the sequence, with 16-bit scores (float64 here):
    I(c) = sum over probe rows r >= c of softmax_r(tau q_r . k)[c].
    q64 [S][d], k64 [S][d] of one head; returns I [S]."""
    S = q64.shape[0]
    imp = np.zeros(S)
    for r in range(max(0, S - n_obs), S):
        s = tau * (k64[:r + 1] @ q64[r])
        p = np.exp(s - s.max())
        imp[:r + 1] += p / p.sum()
    return imp


def top_k_positions(imp: np.ndarray, k: int) -> np.ndarray:
    """The k positions of largest importance (ties to the lower position),
    ascending."""
    order = np.lexsort((np.arange(len(imp)), -imp))
    return np.sort(order[:k]).astype(np.int64)
