"""GPU property cases: seeded random shapes and policies against the oracle.

Each case draws from one seeded generator: 1 to 4 sequences whose lengths
are 0, 1 or uniform in [2, 1024]; 1 or 2 KV heads with 1, 2 or 4 query heads
each; d in {64, 128}; 64- or 128-row query tiles; fp16 or bf16; and a policy
of any of the four kinds with random parameters (boundaries with or without
the sink tile, random group bitmasks, random four-way codes over random
boundaries, random hybrid lists with a random window).  The gate is the
parity gate of the fixed cases (fp32 O and lse against the float64 oracle)
plus the closed-form census of the oracle's precision grid.  The cases are
fixed by the seed, so a failure names a reproducible case.
"""
import numpy as np
import pytest

import workloads as W
from oracle import policy as OP

from _gpu_helpers import compare, oracle_prefill, run_prefill, say

pytestmark = pytest.mark.gpu

N_CASES = 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import tile_routed_mixed_amd as T
    T.lib()


def draw_case(n):
    """Case n: (workload, policy), from generator seed 7000 + n."""
    rng = np.random.default_rng(7000 + n)
    nseq = int(rng.integers(1, 5))
    seqlens = []
    for _ in range(nseq):
        u = rng.random()
        seqlens.append(0 if u < 0.15 else 1 if u < 0.3 else int(rng.integers(2, 1025)))
    if sum(seqlens) == 0:
        seqlens[-1] = int(rng.integers(2, 1025))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    bq = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    kind = n % 4   # every kind equally often
    w = W.small("gqa8k", seqlens, hq=hq, hkv=hkv, d=d, bq=bq, dtype=dtype,
                outliers=int(rng.choice([0, 4])), policy="boundaries" if kind in (0, 2) else "bitmask")
    nk_max = max(1, -(-max(seqlens) // 64))
    if kind in (0, 2):
        sink = int(rng.integers(0, 2))
        b4 = rng.integers(0 if sink else 1, nk_max + 2, size=hq)
        b8 = np.array([rng.integers(0, x + 1) for x in b4])
        pol = dict(kind=0, b8=b8.astype(np.int32), b4=b4.astype(np.int32), sink=sink)
        if kind == 2:
            G = int(rng.choice([1, 2, 4]))
            _, tot = OP.fourway_row_base(seqlens, hq, bq, 64, G)
            pol = dict(pol, kind=2, group=G,
                       words=rng.integers(0, 2 ** 32, size=tot, dtype=np.uint64).astype(np.uint32))
    elif kind == 1:
        G = int(rng.choice([1, 2, 4]))
        _, tot = OP.bitmask_row_base(seqlens, hq, bq, 64, G)
        pol = dict(kind=1, group=G, words=rng.integers(0, 2 ** 32, size=tot, dtype=np.uint64).astype(np.uint32))
    else:
        frac = float(rng.choice([0.0, 0.05, 0.3]))
        lists = [np.sort(rng.choice(S, size=int(round(frac * S)), replace=False)).astype(np.int32)
                 for S in seqlens for _ in range(hq)]
        off = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
        idx = np.concatenate(lists).astype(np.int32) if lists else np.zeros(0, np.int32)
        pol = dict(kind=3, window=int(rng.choice([0, 1, int(rng.integers(2, 300)), 10 ** 6])), sel_off=off,
                   sel_idx=idx)
    return w, pol


@pytest.mark.parametrize("n", range(N_CASES))
def test_random_case(n):
    w, pol = draw_case(n)
    say(f"[gpu] property case {n}: seqlens={w.seqlens} hq={w.hq} hkv={w.hkv} d={w.d} bq={w.bq} {w.dtype} "
        f"kind={pol['kind']}")
    q, k, v = W.make_qkv(w)
    _, census, o, lse, _ = run_prefill(w, pol, q, k, v)
    if pol["kind"] != 3:
        c = OP.census(OP.grids(w.seqlens, w.hq, w.bq, w.bk, pol))
        assert (census["int8"], census["int4"], census["fp16"], census["skip"]) == \
            (c["int8"], c["int4"], c["fp16"], c["skip"]), (census, c)
    O, L, _, _ = oracle_prefill(w, pol, q, k, v)
    compare(o, O, lse, L, what=f"property case {n}")
