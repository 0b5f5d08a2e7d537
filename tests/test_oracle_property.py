"""Property tests of the oracle over random shapes and policies (CPU only).

The fixed pins elsewhere check the oracle on chosen shapes; these draw the
shapes and policies at random (hypothesis, derandomized so every run draws
the same examples): sequence lengths from 0 up, ragged tails, both query-tile
heights, every policy kind.  What they check holds at any size:

* the vectorized precision grid equals the brute-force double loop;
* every full query tile's counts under boundaries equal the closed form in
  (b8, b4, sink, i, r) (the census of the TriAttention abstract's two
  diagonal-distance boundaries, worked out by hand);
* the quantizer's codes stay in range, reach qmax in every nonzero block and
  reconstruct within half a step;
* all-FP16 routing is the library's causal attention, and the same holds
  batch-wise for varlen batches with empty and one-token sequences.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import attention as A
from oracle import policy as P
from oracle import quant as Q
from test_oracle_attention import _inputs, _sdpa
from test_oracle_policy import _closed_form_counts
from test_oracle_quant import _check_invariants

SETTINGS = dict(deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])

seqlens_st = st.lists(st.one_of(st.just(0), st.just(1), st.integers(2, 700)), min_size=1, max_size=4).filter(
    lambda s: sum(s) > 0)


def _policy(draw, kind, seqlens, hq, bq):
    if kind in (0, 2):
        sink = draw(st.integers(0, 1))
        b4 = [draw(st.integers(0 if sink else 1, 14)) for _ in range(hq)]
        b8 = [draw(st.integers(0, x)) for x in b4]
        pol = dict(kind=0, b8=b8, b4=b4, sink=sink)
        if kind == 0:
            return pol
        G = draw(st.sampled_from([1, 2, 4]))
        _, tot = P.fourway_row_base(seqlens, hq, bq, 64, G)
        seed = draw(st.integers(0, 2 ** 31))
        words = np.random.default_rng(seed).integers(0, 2 ** 32, size=tot, dtype=np.uint64).astype(np.uint32)
        return dict(pol, kind=2, group=G, words=words)
    G = draw(st.sampled_from([1, 2, 4]))
    _, tot = P.bitmask_row_base(seqlens, hq, bq, 64, G)
    seed = draw(st.integers(0, 2 ** 31))
    words = np.random.default_rng(seed).integers(0, 2 ** 32, size=tot, dtype=np.uint64).astype(np.uint32)
    return dict(kind=1, group=G, words=words)


@settings(max_examples=60, **SETTINGS)
@given(st.data())
def test_grid_vectorized_equals_loop(data):
    seqlens = data.draw(seqlens_st)
    hq = data.draw(st.integers(1, 3))
    bq = data.draw(st.sampled_from([64, 128]))
    kind = data.draw(st.integers(0, 2))
    pol = _policy(data.draw, kind, seqlens, hq, bq)
    a = P.grids(seqlens, hq, bq, 64, pol, loop=True)
    b = P.grids(seqlens, hq, bq, 64, pol, loop=False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@settings(max_examples=200, **SETTINGS)
@given(r=st.sampled_from([1, 2]), b4=st.integers(0, 60), b8f=st.floats(0, 1), sink=st.integers(0, 1),
       nq=st.integers(1, 40))
def test_boundary_counts_closed_form(r, b4, b8f, sink, nq):
    if b4 == 0 and not sink:
        return
    b8 = int(round(b8f * b4))
    bq = 64 * r
    g = P.precision_grid(nq * bq, bq, 64, 0, dict(kind=0, b8=[b8], b4=[b4], sink=sink))
    for i in range(nq):
        row = g[i]
        got = (int(np.sum(row != P.ILLEGAL)), int(np.sum(row == P.INT8)), int(np.sum(row == P.INT4)),
               int(np.sum(row == P.SKIP)))
        assert got == _closed_form_counts(i, r, b8, b4, sink), (b8, b4, sink, i)


@settings(max_examples=40, **SETTINGS)
@given(seqlens=seqlens_st, heads=st.integers(1, 3), d=st.sampled_from([64, 128]), seed=st.integers(0, 2 ** 31),
       scale=st.sampled_from([1e-30, 1e-3, 1.0, 30.0]), dtype=st.sampled_from(["f16", "bf16"]))
def test_quantizer_invariants(seqlens, heads, d, seed, scale, dtype):
    import workloads as W
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((sum(seqlens), heads, d)) * scale).astype(np.float32)
    if dtype == "f16" and scale < 1e-20:
        return   # below the fp16 range: all zeros, covered by the zero-block pin
    _, xf = W.round16(x, dtype)
    _check_invariants(xf, seqlens)


@settings(max_examples=25, **SETTINGS)
@given(seqlens=st.lists(st.one_of(st.just(0), st.just(1), st.integers(2, 300)), min_size=1, max_size=4).filter(
    lambda s: sum(s) > 0), hkv=st.integers(1, 2), grp=st.sampled_from([1, 2, 4]), bq=st.sampled_from([64, 128]),
    seed=st.integers(0, 2 ** 31))
def test_all_fp16_is_causal_attention_varlen(seqlens, hkv, grp, bq, seed):
    hq, d = hkv * grp, 64
    q, k, v = _inputs(seqlens, hq, hkv, d, seed)
    qq, kq = Q.quantize(q, seqlens), Q.quantize(k, seqlens)
    _, tot = P.bitmask_row_base(seqlens, hq, bq, 64, 4)
    pol = dict(kind=1, group=4, words=np.full(tot, 0xFFFFFFFF, np.uint32))
    O, lse = A.prefill(seqlens, hq, hkv, d, bq, 64, pol, q.astype(np.float64), k.astype(np.float64),
                       v.astype(np.float64), qq, kq)
    nz = [S for S in seqlens if S > 0]
    ref = _sdpa(q, k, v, nz, hq, hkv)
    assert O.shape[0] == sum(seqlens)
    assert np.max(np.abs(O - ref)) < 1e-12
