"""Host-side pieces of boundary calibration, checked without a GPU.

* the budgeted allocator (an exact multiple-choice knapsack) against brute
  force over every assignment of small instances, its infeasible and
  degenerate cases, and monotonicity in the budget;
* the candidate ladder and the bitmask word count used for the all-FP16
  reference policy (the latter against the oracle's row layout);
* the bench's decode byte accounting against the oracle's decode block tags.
"""
import itertools

import numpy as np
import pytest

from tile_routed_mixed_amd import calibrate as C
from oracle import policy as OP


def brute(err, cost, budget):
    H, K = err.shape
    best, arg = np.inf, None
    for ch in itertools.product(range(K), repeat=H):
        c = sum(cost[h, ch[h]] for h in range(H))
        e = sum(err[h, ch[h]] for h in range(H))
        if c <= budget and e < best - 1e-12:
            best, arg = e, ch
    return best, arg


@pytest.mark.parametrize("seed", range(40))
def test_allocator_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    H, K = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    err = rng.random((H, K))
    cost = rng.integers(0, 7, size=(H, K))
    for budget in range(0, int(cost.max(axis=1).sum()) + 2):
        want, _ = brute(err, cost, budget)
        got = C.allocate(err, cost, budget)
        if not np.isfinite(want):
            assert got is None
            continue
        assert got is not None and got.shape == (H,)
        rows = np.arange(H)
        assert cost[rows, got].sum() <= budget
        assert abs(err[rows, got].sum() - want) < 1e-12


def test_allocator_monotone_in_budget():
    rng = np.random.default_rng(7)
    err = rng.random((6, 5))
    cost = rng.integers(1, 20, size=(6, 5))
    prev = np.inf
    rows = np.arange(6)
    for budget in range(int(cost.min(axis=1).sum()), int(cost.max(axis=1).sum()) + 1):
        ch = C.allocate(err, cost, budget)
        tot = err[rows, ch].sum()
        assert tot <= prev + 1e-12
        prev = tot
    # with room for everything each head takes its own least-error candidate
    ch = C.allocate(err, cost, int(cost.max(axis=1).sum()))
    assert np.array_equal(ch, err.argmin(axis=1))


def test_allocator_degenerate_cases():
    err = np.array([[0.5, 0.1], [0.4, 0.2]])
    cost = np.array([[1, 3], [1, 3]])
    assert C.allocate(err, cost, 1) is None          # cheapest total is 2
    assert C.allocate(err, cost, -1) is None
    assert list(C.allocate(err, cost, 2)) == [0, 0]
    # one extra unit of budget cannot buy an upgrade (each costs 2 more)
    assert list(C.allocate(err, cost, 3)) == [0, 0]
    # two extra units: the larger improvement (head 0: 0.4 vs head 1: 0.2)
    assert list(C.allocate(err, cost, 4)) == [1, 0]
    assert list(C.allocate(err, cost, 6)) == [1, 1]
    # zero-cost candidates are always affordable
    assert list(C.allocate(np.array([[1.0, 0.0]]), np.array([[0, 0]]), 0)) == [1]
    with pytest.raises(ValueError):
        C.allocate(err, -cost, 10)
    with pytest.raises(ValueError):
        C.allocate(err, cost[:, :1], 10)


def test_default_candidates():
    c = C.default_candidates(8192)               # 128 key tiles
    assert (C.NEVER, C.NEVER) in c                # all INT8
    assert (0, C.NEVER) in c                      # all INT4
    assert all(b8 <= b4 and b4 > 0 for b8, b4 in c)
    assert len(set(c)) == len(c)
    ladder = sorted({b for p in c for b in p})
    assert ladder == [0, 1, 2, 4, 8, 16, 32, 64, C.NEVER]


@pytest.mark.parametrize("seqlens,bq,group", [([512], 128, 4), ([4096, 8192, 100, 1], 128, 4),
                                               ([1000, 64, 65], 64, 1), ([3000], 128, 2)])
def test_bitmask_word_count_matches_oracle_layout(seqlens, bq, group):
    _, tot = OP.bitmask_row_base(seqlens, 3, bq, 64, group)
    assert C._bitmask_words(seqlens, 3, bq, 64, group) == tot


def test_bench_decode_byte_accounting_matches_oracle_tags():
    import bench
    names = {OP.INT8: "int8", OP.INT4: "int4", OP.FP16: "fp16", OP.SKIP: "skip"}
    for L in [1, 2, 63, 64, 65, 127, 128, 129, 1000, 4097, 32768]:
        for b8, b4, sink, tail in itertools.product([0, 1, 2, 128], [0, 3, 320, 1000], [0, 1], [0, 1, 64, 65, 128, 5000]):
            if b4 < b8:
                continue
            ref = {"int8": 0, "int4": 0, "fp16": 0, "skip": 0}
            for t in OP.decode_block_tags(L, b8, b4, sink, tail).tolist():
                ref[names[t]] += 1
            assert bench.decode_block_counts(L, b8, b4, sink, tail) == ref, (L, b8, b4, sink, tail)
