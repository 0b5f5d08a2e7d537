"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds shapes, random draws and 16-bit rounding only: it performs
none of the attention method's arithmetic (no quantization, no tile
classification, no scores).  Every array is drawn with
``numpy.random.default_rng([workload_id, stream])`` so that the HIP path and the
CPU oracle receive identical bits.

Streams: Q = 1, K = 2, V = 3, policy = 4, outlier channels = 5, decode query = 6,
locality = 7, selected keys = 8, selected decode tokens = 9.  Values are N(0, 1) in float32, rounded half-to-even to the
16-bit input type.

Workloads (the shapes are those of the attention layers the pages benchmark:
Llama-3-8B-like heads, 32 query heads over 8 key/value heads, d = 128):

* ``toy512``      1 sequence of 512 tokens, 1 head, d = 64, fp16, 64x64 tiles,
                  boundaries (b8, b4) = (2, 5) key tiles, key tile 0 kept at INT8.
* ``gqa8k``       1 x 8192 tokens, 32/8 heads, d = 128, bf16, 128x64 tiles,
                  K with 4 outlier channels scaled x10, per-head random
                  boundaries (about 40 % of legal tiles skipped), no sink.
* ``varlen32k``   sequences {4096, 8192, 16384, 4096}, 32/8 heads, d = 128,
                  fp16, 128x64 tiles, packed group bitmask with 4 key tiles per
                  bit, bit = 1 (FP16) with probability 0.35, else INT8.
* ``long128k``    1 x 131072 tokens, 32/8 heads, d = 128, bf16, 128x64 tiles,
                  K outliers as gqa8k, per-head boundaries giving about
                  15 % INT8 / 25 % INT4 / 60 % skipped tiles, sink tile INT8.
* ``local8k``     the gqa8k shape without outliers, plus a position signal
                  shared by Q and K that gives every query head its own
                  preference for nearby keys (see ``make_qkv``); the input of
                  the boundary-calibration demonstration.
* ``decode16x32k`` 16 sequences x 32768 cached tokens, 32/8 heads, d = 128,
                  fp16 cache and one fp16 query per sequence; cache blocks
                  tagged by boundaries (128, 320) in 64-token blocks with the
                  first block kept at INT8 and the last 128 tokens in FP16.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

WORKLOAD_IDS = {"toy512": 1, "gqa8k": 2, "varlen32k": 3, "long128k": 4, "decode16x32k": 5, "local8k": 6}
STREAM_Q, STREAM_K, STREAM_V, STREAM_POLICY, STREAM_OUTLIER, STREAM_DQ, STREAM_LOCAL, STREAM_SEL = 1, 2, 3, 4, 5, 6, 7, 8
STREAM_DSEL = 9
STREAM_FOURWAY, STREAM_QMAPS = 10, 11


@dataclasses.dataclass
class Workload:
    name: str
    seqlens: List[int]
    hq: int
    hkv: int
    d: int
    dtype: str            # "f16" or "bf16"
    bq: int = 128
    bk: int = 64
    policy: str = "boundaries"    # "boundaries" | "bitmask"
    sink: int = 0
    outliers: int = 0
    outlier_scale: float = 10.0
    locality: float = 0.0         # largest per-head strength of the position signal
    # boundaries: draw ranges (inclusive) in key-tile units; or fixed lists
    b8_fixed: Optional[List[int]] = None
    b4_fixed: Optional[List[int]] = None
    b4_range: Optional[tuple] = None       # b4 ~ U_int[lo, hi], b8 ~ U_int[1, b4-1]
    b8_range: Optional[tuple] = None       # b8 ~ U_int[lo, hi], b4 = b8 + U_int[gap]
    b4_gap: Optional[tuple] = None
    # bitmask
    group: int = 4
    p_fp16: float = 0.35
    # decode
    decode: bool = False
    dec_b8: int = 0
    dec_b4: int = 0
    dec_tail: int = 128

    @property
    def wid(self) -> int:
        return WORKLOAD_IDS.get(self.name, 99)

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))


def get(name: str) -> Workload:
    if name == "toy512":
        return Workload("toy512", [512], 1, 1, 64, "f16", bq=64, bk=64, sink=1,
                        b8_fixed=[2], b4_fixed=[5])
    if name == "gqa8k":
        # b4 in [36, 57] key tiles: 50 % .. 30 % of the 4160 legal tiles skipped
        return Workload("gqa8k", [8192], 32, 8, 128, "bf16", outliers=4, b4_range=(36, 57))
    if name == "varlen32k":
        return Workload("varlen32k", [4096, 8192, 16384, 4096], 32, 8, 128, "f16",
                        policy="bitmask", group=4, p_fp16=0.35)
    if name == "long128k":
        # b8 in [145, 175], b4 - b8 in [296, 306]: about 15 % INT8, 25 % INT4, 60 % skip
        return Workload("long128k", [131072], 32, 8, 128, "bf16", outliers=4, sink=1,
                        b8_range=(145, 175), b4_gap=(296, 306))
    if name == "local8k":
        return Workload("local8k", [8192], 32, 8, 128, "bf16", locality=0.6, b4_range=(36, 57))
    if name == "decode16x32k":
        return Workload("decode16x32k", [32768] * 16, 32, 8, 128, "f16", decode=True,
                        dec_b8=128, dec_b4=320, sink=1, dec_tail=128)
    raise KeyError(name)


def small(name: str, seqlens: List[int], **kw) -> Workload:
    """A reduced copy of a named workload (same dtype, heads layout and policy kind)."""
    w = get(name)
    w = dataclasses.replace(w, seqlens=list(seqlens), **kw)
    return w


# ----------------------------------------------------------------------------- rounding

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, half to even; returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # uint32 cannot overflow here except for NaN patterns, which are fixed below
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round16(x: np.ndarray, dtype: str):
    """Return (bits uint16, exact float32 value) of x rounded to the 16-bit type."""
    if dtype == "f16":
        h = x.astype(np.float16)
        return h.view(np.uint16), h.astype(np.float32)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return bits, bf16_bits_to_f32(bits)
    raise ValueError(dtype)


def _normal(w: Workload, stream: int, shape) -> np.ndarray:
    rng = np.random.default_rng([w.wid, stream])
    return rng.standard_normal(shape, dtype=np.float32)


def outlier_channels(w: Workload) -> np.ndarray:
    if w.outliers == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng([w.wid, STREAM_OUTLIER])
    return np.sort(rng.choice(w.d, size=w.outliers, replace=False))


def make_qkv(w: Workload):
    """Q [T][hq][d], K [T][hkv][d], V [T][hkv][d] as (bits, float32) pairs."""
    T = w.total_tokens
    q = _normal(w, STREAM_Q, (T, w.hq, w.d))
    k = _normal(w, STREAM_K, (T, w.hkv, w.d))
    ch = outlier_channels(w)
    if len(ch):
        k[:, :, ch] *= np.float32(w.outlier_scale)
    v = _normal(w, STREAM_V, (T, w.hkv, w.d))
    if w.locality > 0:
        # r(t)[c] = sqrt(2) cos(w_c t + phi_c) with w_c log-uniform over periods
        # of 128 .. 8192 tokens, added to every key and, times a per-head
        # strength a_h ~ U[0, locality], to every query: the logit of key s for
        # query t gains a_h * sum_c 2 cos(w_c t + phi_c) cos(w_c s + phi_c),
        # about a_h * d at s = t and fading as |t - s| grows
        rng = np.random.default_rng([w.wid, STREAM_LOCAL])
        om = 2.0 * np.pi / np.exp(rng.uniform(np.log(128.0), np.log(8192.0), w.d))
        ph = rng.uniform(0.0, 2.0 * np.pi, w.d)
        a = rng.uniform(0.0, w.locality, w.hq).astype(np.float32)
        pos = np.concatenate([np.arange(n) for n in w.seqlens]).astype(np.float64)
        r = (np.sqrt(2.0) * np.cos(pos[:, None] * om[None, :] + ph[None, :])).astype(np.float32)
        q += a[None, :, None] * r[:, None, :]
        k += r[:, None, :]
    return round16(q, w.dtype), round16(k, w.dtype), round16(v, w.dtype)


def make_decode_query(w: Workload):
    """One new query per sequence: [B][hq][d] (bits, float32)."""
    q = _normal(w, STREAM_DQ, (len(w.seqlens), w.hq, w.d))
    return round16(q, w.dtype)


def make_policy(w: Workload):
    """Policy inputs.  Boundaries: dict(kind=0, b8, b4, sink).  Bitmask:
    dict(kind=1, group, words) where words is a flat uint32 array holding, per
    sequence s, per query head, per query tile, ceil(ceil(nk_s / group) / 32)
    words; bit g (LSB first) of a row is drawn Bernoulli(p_fp16)."""
    rng = np.random.default_rng([w.wid, STREAM_POLICY])
    if w.policy == "boundaries":
        if w.b8_fixed is not None:
            b8 = np.array(w.b8_fixed * (w.hq // len(w.b8_fixed)), dtype=np.int32)
            b4 = np.array(w.b4_fixed * (w.hq // len(w.b4_fixed)), dtype=np.int32)
        elif w.b4_range is not None:
            b4 = rng.integers(w.b4_range[0], w.b4_range[1] + 1, size=w.hq).astype(np.int32)
            b8 = np.array([rng.integers(1, x) for x in b4], dtype=np.int32)
        else:
            b8 = rng.integers(w.b8_range[0], w.b8_range[1] + 1, size=w.hq).astype(np.int32)
            b4 = (b8 + rng.integers(w.b4_gap[0], w.b4_gap[1] + 1, size=w.hq)).astype(np.int32)
        return dict(kind=0, b8=b8, b4=b4, sink=int(w.sink))
    words = []
    for S in w.seqlens:
        nq = -(-S // w.bq)
        nk = -(-S // w.bk)
        ng = -(-nk // w.group)
        nw = -(-ng // 32)
        bits = rng.random((w.hq, nq, nw * 32)) < w.p_fp16
        bits[:, :, ng:] = False
        packed = np.zeros((w.hq, nq, nw), dtype=np.uint64)
        for b in range(32):
            packed |= bits[:, :, b::32].astype(np.uint64) << np.uint64(b)
        words.append(packed.astype(np.uint32).reshape(-1))
    return dict(kind=1, group=w.group, words=np.concatenate(words).astype(np.uint32))


def make_fourway_policy(w: Workload, p_zero: float = 0.5, group: int = 4):
    """Four-way policy input: the workload's boundary policy (per-head b8, b4)
    with the sink tile, plus per (sequence, query head, query tile) a row of
    2-bit codes, one per group of `group` key tiles, 16 per uint32 word (LSB
    first): 0 with probability p_zero, else 1, 2 or 3 uniformly.
    dict(kind=2, b8, b4, sink, group, words)."""
    b = make_policy(w)
    assert b["kind"] == 0, "the four-way draw starts from a boundary workload"
    rng = np.random.default_rng([w.wid, STREAM_FOURWAY])
    words = []
    for S in w.seqlens:
        nq = -(-S // w.bq)
        nk = -(-S // w.bk)
        ng = -(-nk // group)
        nw = -(-ng // 16)
        codes = np.where(rng.random((w.hq, nq, nw * 16)) < p_zero, 0,
                         rng.integers(1, 4, size=(w.hq, nq, nw * 16))).astype(np.uint64)
        codes[:, :, ng:] = 0
        packed = np.zeros((w.hq, nq, nw), dtype=np.uint64)
        for c in range(16):
            packed |= codes[:, :, c::16] << np.uint64(2 * c)
        words.append(packed.astype(np.uint32).reshape(-1))
    return dict(kind=2, b8=b["b8"], b4=b["b4"], sink=1, group=group,
                words=np.concatenate(words).astype(np.uint32))


def make_decode_policy(w: Workload):
    """Decode cache tags: per KV head (b8, b4) in 64-token blocks, sink, FP16 tail."""
    return dict(b8=np.full(w.hkv, w.dec_b8, np.int32), b4=np.full(w.hkv, w.dec_b4, np.int32),
                sink=int(w.sink), tail=int(w.dec_tail))


def make_decode_policy_per_q_head(w: Workload, d8: int = 32, d4: int = 64):
    """Per-query-head decode cache tags: every query head draws its own
    (b8, b4) around the workload's, b8 + U_int[-d8, d8] and b4 + U_int[-d4, d4]
    (in 64-token blocks), so the query heads of a KV head read different block
    sets.  dict(b8 [hq], b4 [hq], sink, tail, per_q_head=1)."""
    rng = np.random.default_rng([w.wid, STREAM_QMAPS])
    b8 = (w.dec_b8 + rng.integers(-d8, d8 + 1, size=w.hq)).astype(np.int32)
    b4 = (w.dec_b4 + rng.integers(-d4, d4 + 1, size=w.hq)).astype(np.int32)
    b8 = np.maximum(b8, 0)
    b4 = np.maximum(b4, b8)
    return dict(b8=b8, b4=b4, sink=int(w.sink), tail=int(w.dec_tail), per_q_head=1)


def make_selection(w: Workload, frac: float, window: int, stream_offset: int = 0):
    """Hybrid policy input: for every (sequence, query head), round(frac * len)
    key positions drawn without replacement (sorted), as index lists
    dict(kind=3, window, sel_off [nseq*hq + 1], sel_idx)."""
    rng = np.random.default_rng([w.wid, STREAM_SEL, stream_offset])
    lists = []
    for S in w.seqlens:
        for _ in range(w.hq):
            n = int(round(frac * S))
            lists.append(np.sort(rng.choice(S, size=n, replace=False)).astype(np.int32))
    off = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    idx = np.concatenate(lists).astype(np.int32) if lists else np.zeros(0, np.int32)
    return dict(kind=3, window=int(window), sel_off=off, sel_idx=idx)


def make_decode_selection(w: Workload, frac: float, lengths=None):
    """Selected decode tokens: for every (sequence, KV head), round(frac * L)
    positions below the sequence's length L (or lengths[s]) drawn without
    replacement, sorted; returns (sel_off [nseq*hkv + 1], sel_idx)."""
    rng = np.random.default_rng([w.wid, STREAM_DSEL])
    lists = []
    for s, S in enumerate(w.seqlens):
        L = int(S if lengths is None else lengths[s])
        for _ in range(w.hkv):
            lists.append(np.sort(rng.choice(L, size=int(round(frac * L)), replace=False)).astype(np.int32))
    off = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    idx = np.concatenate(lists).astype(np.int32) if lists else np.zeros(0, np.int32)
    return off, idx
