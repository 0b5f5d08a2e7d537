"""Pins for the oracle's hybrid (token-granular FP16 retention) policy.

* the per-(row, key) precision map of a small case worked out by hand, and
  the window class of every tile of two sequences, also by hand
  (tests/golden/hybrid_small.json);
* the vectorized precision map equals a plain double loop;
* reductions to policies already pinned: a window covering every row with
  no selected key is the all-FP16 bitmask policy, a zero window with no
  selected key is the all-INT8 boundary policy, and every key selected is
  again all FP16 (outputs compared exactly: same arithmetic);
* selecting a key changes only rows that see it outside their window.
"""
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import policy as P
from oracle import quant as Q

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    return json.load(open(os.path.join(GOLD, "hybrid_small.json")))


def test_element_map_hand_worked():
    e = _gold()["element"]
    sym = {"h": P.FP16, "8": P.INT8}
    g = P.hybrid_prec_loop(e["S"], e["selected"], e["window"])
    rows = np.arange(e["S"])
    v = P.hybrid_prec(rows, rows, np.asarray(e["selected"]), e["window"])
    for r, line in enumerate(e["rows"]):
        want = [sym[c] for c in line]
        assert g[r, :r + 1].tolist() == want
        assert v[r, :r + 1].tolist() == want
        assert np.all(g[r, r + 1:] == P.ILLEGAL)


def test_tile_classes_hand_worked():
    sym = {"F": P.WIN_FULL, "E": P.WIN_EDGE, "N": P.WIN_NONE}
    for t in _gold()["tiles"]:
        c = P.hybrid_tile_classes(t["S"], t["bq"], t["bk"], t["window"])
        for i, line in enumerate(t["rows"]):
            assert c[i, :len(line)].tolist() == [sym[x] for x in line]
            assert np.all(c[i, len(line):] == P.ILLEGAL)


@pytest.mark.parametrize("seed", range(4))
def test_vectorized_map_equals_loop(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 200))
    sel = np.sort(rng.choice(S, size=int(rng.integers(0, S + 1)) // 3, replace=False))
    win = int(rng.integers(0, 80))
    g = P.hybrid_prec_loop(S, sel, win)
    rows = np.arange(S)
    v = P.hybrid_prec(rows, rows, sel, win)
    causal = rows[None, :] <= rows[:, None]
    assert np.array_equal(np.where(causal, v, P.ILLEGAL), g)


def _setup(seed, seqlens=(300, 129, 1), hq=4, hkv=2, d=64):
    w = W.small("gqa8k", list(seqlens), hq=hq, hkv=hkv, d=d)
    q, k, v = W.make_qkv(w)
    f = lambda x: x[1].astype(np.float64)
    return w, f(q), f(k), f(v), Q.quantize(q[1], w.seqlens), Q.quantize(k[1], w.seqlens)


def _hyb(w, window, sel_lists):
    off = np.concatenate([[0], np.cumsum([len(x) for x in sel_lists])]).astype(np.int32)
    idx = np.concatenate([np.asarray(x, np.int32) for x in sel_lists]) if len(sel_lists) else np.zeros(0, np.int32)
    return dict(kind=3, window=window, sel_off=off, sel_idx=idx)


def _run(w, pol, q, k, v, qq, kq):
    return A.prefill(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.bk, pol, q, k, v, qq, kq)


def test_reductions_to_pinned_policies():
    w, q, k, v, qq, kq = _setup(1)
    n = len(w.seqlens) * w.hq
    none = [[] for _ in range(n)]
    _, tot = P.bitmask_row_base(w.seqlens, w.hq, w.bq, w.bk, 4)
    fp16 = dict(kind=1, group=4, words=np.full(tot, 0xFFFFFFFF, np.uint32))
    int8 = dict(kind=0, b8=[10 ** 6] * w.hq, b4=[10 ** 6] * w.hq, sink=0)
    O16, L16 = _run(w, fp16, q, k, v, qq, kq)
    O8, L8 = _run(w, int8, q, k, v, qq, kq)
    Ow, Lw = _run(w, _hyb(w, max(w.seqlens), none), q, k, v, qq, kq)
    assert np.array_equal(Ow, O16) and np.array_equal(Lw, L16)
    O0, L0 = _run(w, _hyb(w, 0, none), q, k, v, qq, kq)
    assert np.array_equal(O0, O8) and np.array_equal(L0, L8)
    every = [list(range(w.seqlens[s])) for s in range(len(w.seqlens)) for _ in range(w.hq)]
    Oa, La = _run(w, _hyb(w, 0, every), q, k, v, qq, kq)
    assert np.array_equal(Oa, O16) and np.array_equal(La, L16)
    assert not np.array_equal(O16, O8)


def test_selecting_a_key_touches_only_rows_that_see_it_outside_the_window():
    w, q, k, v, qq, kq = _setup(2, seqlens=(300,), hq=2, hkv=1)
    win, c = 40, 100
    base = [[] for _ in range(w.hq)]
    sel = [[c], []]                     # head 0 selects key 100
    O0, _ = _run(w, _hyb(w, win, base), q, k, v, qq, kq)
    O1, _ = _run(w, _hyb(w, win, sel), q, k, v, qq, kq)
    changed = np.nonzero(np.any(O0[:, 0] != O1[:, 0], axis=1))[0]
    assert changed.tolist() == list(range(c + win, 300))      # rows with r - c >= window
    assert np.array_equal(O0[:, 1], O1[:, 1])                  # the other head is untouched
