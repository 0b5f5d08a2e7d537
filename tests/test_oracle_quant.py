"""Pins for the oracle quantizer (CPU only).

The oracle's quantizer is checked against things other than itself:
* IEEE binary32 division, against exact rational arithmetic rounded to the
  nearest binary32 (ties to even) by brute force over neighbouring floats;
* hand-worked blocks with exactly representable scales, where the quotient
  and its round-half-to-even code are known (tests/golden/quant_ties.json);
* invariants of a symmetric quantizer: code range, the amax element reaching
  +-qmax, reconstruction error bounded by half a step, zero blocks;
* layout: inputs built so that the codes equal the input values (scale 1), so
  each code's position in the blocked layouts can be read off directly;
* the nibble packing of a hand-worked byte table (tests/golden/nibbles.json).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant as Q

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _nearest_f32(q: Fraction) -> np.float32:
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = None
    for c in cands:
        err = abs(Fraction(float(c)) - q)
        key = (err, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def test_binary32_division_matches_exact_rounding():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(400) * 3).astype(np.float32)
    s = (np.abs(rng.standard_normal(400)) * 0.05 + 1e-3).astype(np.float32)
    x[:20] = np.float32(1.0)
    s[:20] = np.float32(3.0)
    got = np.divide(x, s, dtype=np.float32)
    for a, b, g in zip(x, s, got):
        want = _nearest_f32(Fraction(float(a)) / Fraction(float(b)))
        assert np.float32(g) == want, (a, b, g, want)


def test_hand_worked_ties():
    gold = json.load(open(os.path.join(GOLD, "quant_ties.json")))
    for bits, key in ((8, "int8"), (4, "int4")):
        xs = np.array(gold[key]["x"], np.float32)
        x = np.zeros((64, 1, 16), np.float32)
        x[:len(xs), 0, 0] = xs
        qt = Q.quantize(x, [64])
        s = qt["s8" if bits == 8 else "s4"][0, 0]
        c = qt["c8" if bits == 8 else "c4"][0, 0, :len(xs), 0]
        assert s == np.float32(gold[key]["scale"])
        assert c.tolist() == gold[key]["codes"]


def _check_invariants(x, seqlens):
    qt = Q.quantize(x, seqlens)
    for bits, qmax in ((8, 127), (4, 7)):
        c = qt["c8" if bits == 8 else "c4"].astype(np.int64)
        s = qt["s8" if bits == 8 else "s4"].astype(np.float64)
        assert c.min() >= -qmax and c.max() <= qmax
        xb = np.zeros(c.shape, np.float64)
        tok = 0
        for si, S in enumerate(seqlens):
            b0 = qt["blk_start"][si]
            nb = -(-S // 64)
            pad = np.zeros((nb * 64,) + x.shape[1:], np.float32)
            pad[:S] = x[tok:tok + S]
            xb[:, b0:b0 + nb] = pad.reshape(nb, 64, x.shape[1], x.shape[2]).transpose(2, 0, 1, 3)
            tok += S
        amax = np.abs(xb).max(axis=(2, 3))
        nz = amax > 0
        assert np.all(np.abs(c).max(axis=(2, 3))[nz] == qmax)
        assert np.all(s[~nz] == 0) and np.all(c[~nz] == 0)
        err = np.abs(xb - s[:, :, None, None] * c)
        bound = s[:, :, None, None] * (0.5 + 128 * 2.0 ** -24)
        assert np.all(err <= bound)


def test_invariants_random_varlen():
    rng = np.random.default_rng(5)
    seqlens = [1, 63, 64, 65, 200]
    x = rng.standard_normal((sum(seqlens), 3, 64)).astype(np.float32)
    x[:, :, 7] *= 10
    x[64:64 + 63] = 0.0          # a whole block of zeros (sequence 1 is tokens 1..63)
    _check_invariants(x, seqlens)


def test_invariants_bf16_and_subnormal_range():
    from workloads import round16
    rng = np.random.default_rng(6)
    x = rng.standard_normal((130, 2, 128)).astype(np.float32) * np.float32(1e-30)
    _, xf = round16(x, "bf16")
    _check_invariants(xf, [130])


def test_layout_rows_and_cols():
    seqlens = [70, 64, 3]
    T, H, d = sum(seqlens), 2, 64
    t = np.arange(T)[:, None, None]
    h = np.arange(H)[None, :, None]
    c = np.arange(d)[None, None, :]
    x = (((t * 7 + h * 13 + c * 3) % 255) - 127).astype(np.float32)
    # force amax = 127 in every block so s8 = 1 and codes equal x
    x[:, :, 0] = 127.0
    qt = Q.quantize(x, seqlens, layout="rows")
    assert qt["nblk"] == 2 + 1 + 1
    assert qt["blk_start"].tolist() == [0, 2, 3]
    assert np.all(qt["s8"] == 1.0)
    tok = 0
    for si, S in enumerate(seqlens):
        for r in range(S):
            b = qt["blk_start"][si] + r // 64
            for hh in range(H):
                assert np.array_equal(qt["c8p"][hh, b, r % 64], x[tok + r, hh].astype(np.int8))
        # padding rows after the sequence end are zero codes
        nb = -(-S // 64)
        last = qt["blk_start"][si] + nb - 1
        for r in range(S - (nb - 1) * 64, 64):
            assert not qt["c8p"][:, last, r].any()
        tok += S
    qc = Q.quantize(x, seqlens, layout="cols", with_t16=True)
    assert np.array_equal(qc["c8p"], qt["c8p"].transpose(0, 1, 3, 2))
    assert qc["t16"].shape == (H, 4, d, 64)
    assert qc["t16"][1, 3, 5, 2] == np.float16(x[134 + 2, 1, 5])
    assert qc["t16"][1, 2, 5, 2] == np.float16(x[70 + 2, 1, 5])
    assert not qc["t16"][:, 3, :, 3:].any()
    assert qc["c4p"].shape == (H, 4, d, 32)


def test_nibble_table():
    gold = json.load(open(os.path.join(GOLD, "nibbles.json")))
    codes = np.array(gold["codes"], np.int8)
    packed = Q.pack_nibbles(codes)
    assert packed.tolist() == gold["bytes"]
    assert Q.unpack_nibbles(packed).tolist() == gold["codes"]
    allc = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)], np.int8)
    assert np.array_equal(Q.unpack_nibbles(Q.pack_nibbles(allc)), allc)


def test_dequantize_round_trip():
    rng = np.random.default_rng(8)
    seqlens = [100, 37]
    x = rng.standard_normal((137, 2, 64)).astype(np.float32)
    qt = Q.quantize(x, seqlens)
    for bits in (8, 4):
        xh = Q.dequantize_rows(qt, bits, seqlens)
        assert xh.shape == x.shape
        # reconstruction within half a quantization step of each block's scale
        assert np.max(np.abs(xh - x)) <= np.max(qt["s8" if bits == 8 else "s4"]) * 0.5001
