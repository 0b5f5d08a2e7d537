"""Pins for the oracle tile-precision policy (CPU only).

* the vectorized grid equals a plain double loop over every (i, j);
* the toy 512-token grid equals the hand-worked grid in
  tests/golden/toy512_tiles.txt (21 INT8 / 12 INT4 / 3 skipped of 36);
* per-query-tile counts equal an independent closed form in (b8, b4, i, r);
* hand-set bitmask words give the tile precisions worked out by hand in
  tests/golden/bitmask_small.json (multi-word rows, partial groups, varlen);
* the two encodings agree where they describe the same policy (all INT8);
* decode cache tags match the hand-worked counts in tests/golden/decode_tags.json;
* the four-way code map gives the hand-worked precisions of
  tests/golden/fourway_small.json, reduces to the boundary policy when every
  code is 0 and to the bitmask policy when codes are drawn from {2, 3}.
"""
import json
import os

import numpy as np
import pytest

from oracle import policy as P

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand_pol(rng, hq, kind, seqlens=None, bq=128, bk=64, G=4, sink=0):
    if kind == 2:
        b = _rand_pol(rng, hq, 0, sink=sink)
        _, tot = P.fourway_row_base(seqlens, hq, bq, bk, G)
        return dict(kind=2, b8=b["b8"], b4=b["b4"], sink=sink, group=G,
                    words=rng.integers(0, 2 ** 32, size=tot, dtype=np.uint64).astype(np.uint32))
    if kind == 0:
        b4 = rng.integers(0, 12, size=hq)
        b8 = np.array([rng.integers(0, x + 1) for x in b4])
        return dict(kind=0, b8=b8, b4=b4, sink=sink)
    _, tot = P.bitmask_row_base(seqlens, hq, bq, bk, G)
    return dict(kind=1, group=G, words=rng.integers(0, 2 ** 32, size=tot, dtype=np.uint64).astype(np.uint32))


@pytest.mark.parametrize("kind", [0, 1, 2])
@pytest.mark.parametrize("bq", [64, 128])
def test_vectorized_equals_loop(kind, bq):
    rng = np.random.default_rng(3 + kind + bq)
    seqlens = [1, 63, 129, 700, 2600]
    for sink in (0, 1):
        pol = _rand_pol(rng, 3, kind, seqlens, bq=bq, sink=sink)
        a = P.grids(seqlens, 3, bq, 64, pol, loop=True)
        b = P.grids(seqlens, 3, bq, 64, pol, loop=False)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def test_toy_grid_hand_worked():
    lines = [l.split() for l in open(os.path.join(GOLD, "toy512_tiles.txt")) if not l.startswith("#")]
    sym = {"8": P.INT8, "4": P.INT4, "s": P.SKIP, ".": P.ILLEGAL}
    want = np.array([[sym[c] for c in row] for row in lines], np.int8)
    pol = dict(kind=0, b8=[2], b4=[5], sink=1)
    g = P.grids([512], 1, 64, 64, pol, loop=True)[0][0]
    assert np.array_equal(g, want)
    c = P.census([g[None]])
    assert (c["int8"], c["int4"], c["skip"], c["legal"]) == (21, 12, 3, 36)


def _closed_form_counts(i, r, b8, b4, sink):
    legal = r * (i + 1)

    def below(b):
        return (r if b >= 1 else 0) + min(max(b - 1, 0), r * i)

    n8, n4 = below(b8), below(b4) - below(b8)
    ns = legal - below(b4)
    if sink:
        d0 = r * i           # distance of key tile 0 from query tile i
        if d0 >= b8:
            n8 += 1
            if d0 < b4:
                n4 -= 1
            else:
                ns -= 1
    return legal, n8, n4, ns


@pytest.mark.parametrize("r", [1, 2])
def test_closed_form_census(r):
    bq, bk = 64 * r, 64
    S = bq * 40
    rng = np.random.default_rng(r)
    pairs = [(0, 0), (0, 1), (1, 1), (2, 5), (3, 3), (0, 100), (100, 100)] + [
        tuple(sorted(rng.integers(0, 90, size=2))) for _ in range(12)]
    for sink in (0, 1):
        for b8, b4 in pairs:
            if b4 == 0 and not sink:
                continue
            g = P.precision_grid(S, bq, bk, 0, dict(kind=0, b8=[b8], b4=[b4], sink=sink))
            for i in range(S // bq):
                row = g[i]
                got = (int(np.sum(row != P.ILLEGAL)), int(np.sum(row == P.INT8)),
                       int(np.sum(row == P.INT4)), int(np.sum(row == P.SKIP)))
                assert got == _closed_form_counts(i, r, b8, b4, sink), (b8, b4, sink, i)


def test_bitmask_hand_worked():
    gold = json.load(open(os.path.join(GOLD, "bitmask_small.json")))
    seqlens, hq, bq, bk, G = gold["seqlens"], gold["hq"], gold["bq"], gold["bk"], gold["group"]
    _, tot = P.bitmask_row_base(seqlens, hq, bq, bk, G)
    assert tot == gold["total_words"]
    words = np.zeros(tot, np.uint32)
    for k, v in gold["set_words"].items():
        words[int(k)] = v
    pol = dict(kind=1, group=G, words=words)
    for loop in (True, False):
        gs = P.grids(seqlens, hq, bq, bk, pol, loop=loop)
        for e in gold["expect"]:
            row = gs[e["seq"]][e["head"], e["qtile"]]
            legal = np.nonzero(row != P.ILLEGAL)[0].tolist()
            fp16 = np.nonzero(row == P.FP16)[0].tolist()
            assert fp16 == e["fp16"]
            assert not np.any(row == P.SKIP)
            if "illegal_from" in e:
                assert legal == list(range(e["illegal_from"]))
                assert np.nonzero(row == P.INT8)[0].tolist() == e["int8"]
            else:
                assert len(legal) == e["n_legal"]


def test_encodings_agree_all_int8():
    seqlens = [300, 1000]
    big = 10 ** 6
    a = P.grids(seqlens, 2, 128, 64, dict(kind=0, b8=[big, big], b4=[big, big], sink=0))
    _, tot = P.bitmask_row_base(seqlens, 2, 128, 64, 4)
    b = P.grids(seqlens, 2, 128, 64, dict(kind=1, group=4, words=np.zeros(tot, np.uint32)))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert P.census(a) == P.census(b)


def test_decode_tags_hand_worked():
    gold = json.load(open(os.path.join(GOLD, "decode_tags.json")))
    for c in gold["cases"]:
        t = P.decode_block_tags(c["L"], c["b8"], c["b4"], c["sink"], c["tail"])
        assert int(np.sum(t == P.FP16)) == c["fp16"]
        assert int(np.sum(t == P.INT8)) == c["int8"]
        assert int(np.sum(t == P.INT4)) == c["int4"]
        assert int(np.sum(t == P.SKIP)) == c["skip"]
    assert np.all(P.decode_block_tags(100, 0, 0, 0, 128) == P.FP16)
    assert np.all(P.decode_block_tags(1, 0, 0, 0, 128) == P.FP16)


def test_workload_policies_hit_their_targets():
    """The seeded per-head boundary draws give the stated tile mixes."""
    import workloads as W
    w = W.get("gqa8k")
    pol = W.make_policy(w)
    gs = P.grids(w.seqlens, w.hq, w.bq, w.bk, pol)
    for h in range(w.hq):
        c = P.census([gs[0][h:h + 1]])
        assert 0.29 <= c["skip"] / c["legal"] <= 0.51
    c = P.census(gs)
    assert 0.35 <= c["skip"] / c["legal"] <= 0.45
    w = W.get("toy512")
    c = P.census(P.grids(w.seqlens, w.hq, w.bq, w.bk, W.make_policy(w)))
    assert (c["int8"], c["int4"], c["skip"]) == (21, 12, 3)
    w = W.get("varlen32k")
    pol = W.make_policy(w)
    c = P.census(P.grids(w.seqlens, w.hq, w.bq, w.bk, pol))
    assert c["skip"] == 0 and c["legal"] == 729088
    assert 0.32 <= c["fp16"] / c["legal"] <= 0.38


@pytest.mark.slow
def test_long_policy_mix():
    import workloads as W
    w = W.get("long128k")
    pol = W.make_policy(w)
    c = P.census(P.grids(w.seqlens, w.hq, w.bq, w.bk, pol))
    assert abs(c["int8"] / c["legal"] - 0.15) < 0.02
    assert abs(c["int4"] / c["legal"] - 0.25) < 0.02
    assert abs(c["skip"] / c["legal"] - 0.60) < 0.02


def test_fourway_hand_worked():
    gold = json.load(open(os.path.join(GOLD, "fourway_small.json")))
    _, tot = P.fourway_row_base(gold["seqlens"], gold["hq"], gold["bq"], gold["bk"], gold["group"])
    assert tot == gold["total_words"]
    words = np.zeros(tot, np.uint32)
    for k, v in gold["set_words"].items():
        words[int(k)] = v
    pol = dict(kind=2, b8=gold["b8"], b4=gold["b4"], sink=gold["sink"], group=gold["group"], words=words)
    for loop in (True, False):
        gs = P.grids(gold["seqlens"], gold["hq"], gold["bq"], gold["bk"], pol, loop=loop)
        for e in gold["expect"]:
            row = gs[e["seq"]][0][e["qtile"]]
            legal = np.nonzero(row != P.ILLEGAL)[0].tolist()
            assert sorted(e["fp16"] + e["int8"] + e["int4"] + e["skip"]) == legal, e
            for key, prec in (("fp16", P.FP16), ("int8", P.INT8), ("int4", P.INT4), ("skip", P.SKIP)):
                assert np.nonzero(row == prec)[0].tolist() == e[key], (e, key)


@pytest.mark.parametrize("sink", [0, 1])
def test_fourway_reduces_to_the_two_encodings(sink):
    rng = np.random.default_rng(41 + sink)
    seqlens, hq, G = [1, 200, 1000, 3000], 3, 3
    b = _rand_pol(rng, hq, 0, sink=sink)
    _, tot = P.fourway_row_base(seqlens, hq, 128, 64, G)
    zero = dict(kind=2, b8=b["b8"], b4=b["b4"], sink=sink, group=G, words=np.zeros(tot, np.uint32))
    for x, y in zip(P.grids(seqlens, hq, 128, 64, zero), P.grids(seqlens, hq, 128, 64, b)):
        assert np.array_equal(x, y)
    # codes from {2, 3}: bit (code == 3) of the same group in a bitmask row
    bases4, _ = P.fourway_row_base(seqlens, hq, 128, 64, G)
    bases1, tot1 = P.bitmask_row_base(seqlens, hq, 128, 64, G)
    w4 = np.zeros(tot, np.uint32)
    w1 = np.zeros(tot1, np.uint32)
    for s, S in enumerate(seqlens):
        nq, ng = P.n_tiles(S, 128), P.n_tiles(P.n_tiles(S, 64), G)
        for h in range(hq):
            for i in range(nq):
                r4 = bases4[s] + (h * nq + i) * P.fourway_words_per_row(S, 64, G)
                r1 = bases1[s] + (h * nq + i) * P.bitmask_words_per_row(S, 64, G)
                for g in range(ng):
                    fp = int(rng.integers(0, 2))
                    w4[r4 + g // 16] |= np.uint32((3 if fp else 2) << (2 * (g % 16)))
                    w1[r1 + g // 32] |= np.uint32(fp << (g % 32))
    four = dict(kind=2, b8=b["b8"], b4=b["b4"], sink=sink, group=G, words=w4)
    bm = dict(kind=1, group=G, words=w1)
    for x, y in zip(P.grids(seqlens, hq, 128, 64, four), P.grids(seqlens, hq, 128, 64, bm)):
        assert np.array_equal(x, y)
