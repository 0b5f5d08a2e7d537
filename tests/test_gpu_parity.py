"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Gates: quantized codes, scales, the fp16 V copy, the traversal and the integer
QK tile scores bit-exact; fp32 attention outputs within max-abs 4e-3 and
mean-abs 5e-4 of the float64 oracle computed from the oracle's own codes.
Small cases span several tiles with ragged tails; the full-size workloads are
checked on sampled rows (the oracle computes rows one by one).
"""
import zlib

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import policy as OP
from oracle import quant as OQ

from _gpu_helpers import (TOL_LSE, TOL_MAX, assert_all_written, check_int_scores, compare, guard_decode,
                          guard_prefill, int_tiles, oracle_prefill, run_prefill, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import tile_routed_mixed_amd as T
    T.lib()


def _inputs(w):
    return W.make_qkv(w)


# ---------------------------------------------------------------------------- quantize

@pytest.mark.parametrize("dtype,d,seqlens", [("f16", 64, [512]), ("bf16", 128, [1, 63, 64, 65, 300]),
                                             ("f16", 128, [700, 129])])
def test_quantize_bitexact(dtype, d, seqlens):
    import torch
    import tile_routed_mixed_amd as T
    w = W.small("gqa8k", seqlens, d=d, dtype=dtype, hq=4, hkv=2)
    q, k, v = _inputs(w)
    p = T.PrefillPipeline(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, dict(kind=0, b8=[1] * 4, b4=[2] * 4, sink=0))
    p.upload(q[0], k[0], v[0])
    g = guard_prefill(p, T.TM_F32)
    say(f"[gpu] quantize {dtype} d={d} {seqlens}")
    p.quantize()
    torch.cuda.synchronize()
    g.check()
    for x, qt, layout in ((q, p.qq, "rows"), (k, p.kq, "rows"), (v, p.vq, "cols")):
        ref = OQ.quantize(x[1], w.seqlens, layout=layout, with_t16=(layout == "cols"))
        # the library stores blocks block-major ([nblk][heads]...), the oracle head-major
        def hm(t):
            return np.swapaxes(t.cpu().numpy(), 0, 1)
        assert np.array_equal(hm(qt.s8).view(np.uint32), ref["s8"].view(np.uint32))
        assert np.array_equal(hm(qt.s4).view(np.uint32), ref["s4"].view(np.uint32))
        assert np.array_equal(hm(qt.c8), ref["c8p"])
        assert np.array_equal(hm(qt.c4), ref["c4p"])
        if qt.c4x is not None:   # K's INT4 codes one per byte
            assert np.array_equal(hm(qt.c4x), ref["c4"])
        if layout == "cols":
            assert np.array_equal(hm(qt.t16).view(np.uint16), ref["t16"].view(np.uint16))


# ---------------------------------------------------------------------------- traversal

def _check_traversal(w, pol, p, census):
    import tile_routed_mixed_amd as T
    tr = T.read_traversal(p.trav.cpu().numpy())
    gs = OP.grids(w.seqlens, w.hq, w.bq, w.bk, pol)
    c = OP.census(gs)
    assert census["legal"] == c["legal"] and census["int8"] == c["int8"] and census["int4"] == c["int4"]
    assert census["fp16"] == c["fp16"] and census["skip"] == c["skip"]
    assert tr["census"] == c
    assert tr["magic"] == T._binding.TRAV_MAGIC
    got = set()
    seen = set()
    prev_q = None
    for n in range(tr["n_items"]):
        s, h, qt, nr = (int(x) for x in tr["items"][n, :4])
        assert (s, h, qt) not in seen
        seen.add((s, h, qt))
        if prev_q is not None:
            assert qt <= prev_q            # heavy-first: query tiles in descending order
        prev_q = qt
        precs = []
        for r in range(nr):
            first, cp = (int(x) for x in tr["runs"][n, r])
            cnt, prec = cp & 0xFFFFFF, cp >> 24
            precs.append(prec)
            for j in range(first, first + cnt):
                key = (s, h, qt, j, prec)
                assert key not in got
                got.add(key)
        # runs are grouped by precision: each precision forms one contiguous stretch
        groups = [x for i, x in enumerate(precs) if i == 0 or precs[i - 1] != x]
        assert len(groups) == len(set(groups))
    assert len(seen) == sum(w.hq * OP.n_tiles(S, w.bq) for S in w.seqlens)
    assert got == OP.executed_tiles(gs)


@pytest.mark.parametrize("case", ["toy", "boundaries_varlen", "bitmask_varlen", "sink_edge", "fourway_varlen",
                                  "fourway_d64"])
def test_traversal_bruteforce(case):
    w, pol = _case(case)
    q, k, v = _inputs(w)
    p, census, o, lse, _ = run_prefill(w, pol, q, k, v)
    _check_traversal(w, pol, p, census)


# ---------------------------------------------------------------------------- prefill (small)

def _case(case):
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    if case == "toy":
        w = W.get("toy512")
        return w, W.make_policy(w)
    if case == "boundaries_varlen":
        w = W.small("gqa8k", [1000, 1, 130, 64], hq=8, hkv=2)
        b4 = rng.integers(1, 9, size=8)
        b8 = np.array([rng.integers(0, x + 1) for x in b4])
        return w, dict(kind=0, b8=b8, b4=b4, sink=0)
    if case == "bitmask_varlen":
        w = W.small("varlen32k", [700, 64, 1, 1500, 129], hq=8, hkv=2)
        _, tot = OP.bitmask_row_base(w.seqlens, w.hq, w.bq, w.bk, 2)
        words = (rng.random(tot * 32) < 0.35).reshape(tot, 32)
        packed = (words * (1 << np.arange(32, dtype=np.uint64))).sum(axis=1).astype(np.uint32)
        return w, dict(kind=1, group=2, words=packed)
    if case == "sink_edge":
        w = W.small("long128k", [2200, 333], hq=4, hkv=1, d=64)
        return w, dict(kind=0, b8=[0, 2, 3, 0], b4=[0, 2, 9, 5], sink=1)
    if case == "bq64_d128":
        w = W.small("gqa8k", [900], hq=4, hkv=4, bq=64)
        return w, dict(kind=0, b8=[1, 2, 3, 4], b4=[3, 4, 5, 6], sink=1)
    if case == "bitmask_bf16":
        w = W.small("varlen32k", [1100, 200], hq=4, hkv=1, dtype="bf16")
        _, tot = OP.bitmask_row_base(w.seqlens, w.hq, w.bq, w.bk, 4)
        words = rng.integers(0, 2 ** 32, size=tot, dtype=np.uint64).astype(np.uint32)
        return w, dict(kind=1, group=4, words=words)
    if case == "fourway_varlen":
        w = W.small("gqa8k", [1000, 1, 130, 64, 2200], hq=8, hkv=2)
        b4 = rng.integers(1, 12, size=8)
        b8 = np.array([rng.integers(0, x + 1) for x in b4])
        return w, _fourway(rng, w, b8, b4, sink=1, group=3, p_zero=0.4)
    if case == "fourway_d64":
        w = W.small("long128k", [1500, 333, 64], hq=4, hkv=1, d=64)
        return w, _fourway(rng, w, [0, 1, 2, 5], [1, 3, 6, 40], sink=0, group=1, p_zero=0.6)
    raise KeyError(case)


def _fourway(rng, w, b8, b4, sink, group, p_zero):
    """Four-way policy with random 2-bit codes: 0 with probability p_zero, else
    1, 2 or 3 uniformly."""
    _, tot = OP.fourway_row_base(w.seqlens, w.hq, w.bq, w.bk, group)
    codes = np.where(rng.random((tot, 16)) < p_zero, 0, rng.integers(1, 4, size=(tot, 16))).astype(np.uint64)
    words = (codes << (2 * np.arange(16, dtype=np.uint64))).sum(axis=1).astype(np.uint32)
    return dict(kind=2, b8=np.asarray(b8), b4=np.asarray(b4), sink=sink, group=group, words=words)


CASES = ["toy", "boundaries_varlen", "bitmask_varlen", "sink_edge", "bq64_d128", "bitmask_bf16", "fourway_varlen",
         "fourway_d64"]


@pytest.mark.parametrize("case", CASES)
def test_prefill_small(case):
    w, pol = _case(case)
    q, k, v = _inputs(w)
    tiles = int_tiles(w, pol, limit=24)
    dbg_in = [t[:4] for t in tiles] if tiles else None
    p, census, o, lse, dbg = run_prefill(w, pol, q, k, v, dbg_tiles=dbg_in)
    O, L, qq, kq = oracle_prefill(w, pol, q, k, v)
    compare(o, O, lse, L, what=case)
    if tiles:
        check_int_scores(w, tiles, dbg, qq, kq)
    # the capture build of the kernel computes the same outputs bit for bit
    _, _, o2, lse2, _ = run_prefill(w, pol, q, k, v)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_toy_all_int_tiles_bitexact():
    w = W.get("toy512")
    pol = W.make_policy(w)
    q, k, v = _inputs(w)
    tiles = int_tiles(w, pol)
    assert len(tiles) == 33
    _, census, o, lse, dbg = run_prefill(w, pol, q, k, v, dbg_tiles=[t[:4] for t in tiles])
    assert (census["int8"], census["int4"], census["skip"]) == (21, 12, 3)
    _, _, qq, kq = oracle_prefill(w, pol, q, k, v, rows=[(0, 0, 0)])
    check_int_scores(w, tiles, dbg, qq, kq)


def test_first_row_is_v0_and_rows_normalized():
    w, pol = _case("boundaries_varlen")
    q, k, v = _inputs(w)
    _, _, o, lse, _ = run_prefill(w, pol, q, k, v)
    cu = w.cu_seqlens
    for s in range(len(w.seqlens)):
        for h in range(w.hq):
            ref = v[1][cu[s], h // (w.hq // w.hkv)]
            assert np.max(np.abs(o[cu[s], h] - ref)) <= 1e-3     # fp16 probability 1.0 is exact
    # sum_c exp(s_c - lse) == 1 per row, with the oracle's scores and the GPU's lse
    O, L, qq, kq = oracle_prefill(w, pol, q, k, v, rows=[(0, 3, 999), (2, 5, 129), (3, 0, 63)])
    for (s, h, r) in [(0, 3, 999), (2, 5, 129), (3, 0, 63)]:
        t = cu[s] + r
        assert abs(lse[h, t] - L[h, t]) <= TOL_LSE


def test_skipped_tiles_do_not_matter_on_gpu():
    w = W.small("gqa8k", [1024], hq=2, hkv=1)
    pol = dict(kind=0, b8=[1, 2], b4=[2, 4], sink=0)
    q, k, v = _inputs(w)
    _, _, o0, _, _ = run_prefill(w, pol, q, k, v)
    gs = OP.grids(w.seqlens, w.hq, w.bq, w.bk, pol)[0]
    assert np.all(gs[:, 7, 0:2] == OP.SKIP)         # query tile 7 skips key tiles 0, 1 in both heads
    k2 = (k[0].copy(), k[1].copy())
    v2 = (v[0].copy(), v[1].copy())
    rng = np.random.default_rng(1)
    pert = W.round16(rng.standard_normal((128, 1, 128)).astype(np.float32) * 5, "bf16")
    k2[0][:128], v2[0][:128] = pert[0], pert[0][:, :, ::-1].copy()
    _, _, o1, _, _ = run_prefill(w, pol, q, k2, v2)
    assert np.array_equal(o0[7 * 128:8 * 128], o1[7 * 128:8 * 128])
    assert not np.array_equal(o0[128:256], o1[128:256])


def test_boundaries_all_int8_equals_zero_bitmask():
    """Both policy encodings routing every legal tile to INT8 (boundaries
    b8 = b4 = infinity; a bitmask of zeros) give the same census, and outputs
    equal within the fp32 rounding of their different tile orders."""
    w = W.small("varlen32k", [700, 64, 1, 1300], hq=4, hkv=2, dtype="f16")
    q, k, v = _inputs(w)
    big = 10 ** 6
    pol_b = dict(kind=0, b8=[big] * w.hq, b4=[big] * w.hq, sink=0)
    _, tot = OP.bitmask_row_base(w.seqlens, w.hq, w.bq, w.bk, 4)
    pol_m = dict(kind=1, group=4, words=np.zeros(tot, np.uint32))
    _, cb, ob, lb, _ = run_prefill(w, pol_b, q, k, v)
    _, cm, om, lm, _ = run_prefill(w, pol_m, q, k, v)
    for key in ("legal", "int8", "int4", "fp16", "skip"):
        assert cb[key] == cm[key], key
    assert cb["int8"] == cb["legal"] and cb["skip"] == 0
    compare(ob, om.astype(np.float64), lb, lm.astype(np.float64), what="all-INT8 encodings")


def test_fourway_reduces_to_boundaries_and_bitmask():
    """The four-way kernel on all-zero codes computes the boundary policy
    (the same tiles at the same precisions; the boundary kernel orders the
    tiles and sums the rows its own way, so the two agree within the fp32
    gate, and both with the oracle), and on codes from {2, 3} the bitmask
    policy: same outputs bit for bit as the bitmask kernel."""
    rng = np.random.default_rng(77)
    w = W.small("gqa8k", [900, 300], hq=4, hkv=2)
    q, k, v = _inputs(w)
    b = dict(kind=0, b8=[1, 2, 0, 3], b4=[2, 5, 4, 3], sink=1)
    _, tot = OP.fourway_row_base(w.seqlens, w.hq, w.bq, w.bk, 2)
    zero = dict(b, kind=2, group=2, words=np.zeros(tot, np.uint32))
    _, c0, o0, l0, _ = run_prefill(w, b, q, k, v)
    _, c2, o2, l2, _ = run_prefill(w, zero, q, k, v)
    assert all(c0[key] == c2[key] for key in ("legal", "int8", "int4", "fp16", "skip"))
    compare(o0, o2.astype(np.float64), l0, l2.astype(np.float64), what="four-way zero codes vs boundaries")
    O, L, _, _ = oracle_prefill(w, b, q, k, v)
    compare(o0, O, l0, L, what="boundaries")
    compare(o2, O, l2, L, what="four-way zero codes")
    # codes 2/3 <-> bitmask bits 0/1 of the same groups
    _, tot1 = OP.bitmask_row_base(w.seqlens, w.hq, w.bq, w.bk, 2)
    bases4, _ = OP.fourway_row_base(w.seqlens, w.hq, w.bq, w.bk, 2)
    bases1, _ = OP.bitmask_row_base(w.seqlens, w.hq, w.bq, w.bk, 2)
    w4, w1 = np.zeros(tot, np.uint32), np.zeros(tot1, np.uint32)
    for s_, S in enumerate(w.seqlens):
        nq, ng = OP.n_tiles(S, w.bq), OP.n_tiles(OP.n_tiles(S, w.bk), 2)
        for h in range(w.hq):
            for i in range(nq):
                r4 = bases4[s_] + (h * nq + i) * OP.fourway_words_per_row(S, w.bk, 2)
                r1 = bases1[s_] + (h * nq + i) * OP.bitmask_words_per_row(S, w.bk, 2)
                for g in range(ng):
                    fp = int(rng.integers(0, 2))
                    w4[r4 + g // 16] |= np.uint32((3 if fp else 2) << (2 * (g % 16)))
                    w1[r1 + g // 32] |= np.uint32(fp << (g % 32))
    _, _, o1, l1, _ = run_prefill(w, dict(kind=1, group=2, words=w1), q, k, v)
    _, _, o3, l3, _ = run_prefill(w, dict(b, kind=2, group=2, words=w4), q, k, v)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


# ---------------------------------------------------------------------------- hybrid (token-granular)

HYBRID_CASES = {
    # name: (workload, seqlens, overrides, selected fraction, window)
    "hyb_gqa": ("gqa8k", [700, 1, 300, 64], dict(hq=4, hkv=2), 0.1, 128),
    "hyb_d64_bq64_bf16": ("long128k", [1000, 333], dict(hq=2, hkv=1, d=64, bq=64), 0.05, 100),
    "hyb_nowindow": ("varlen32k", [900, 65], dict(hq=4, hkv=1), 0.2, 0),
    "hyb_allwindow": ("varlen32k", [500, 129], dict(hq=2, hkv=2), 0.1, 10 ** 6),
    "hyb_mask_bits": ("gqa8k", [700], dict(hq=2, hkv=1), None, 40),
}


def _hyb_case(name):
    wl, seqlens, kw, frac, win = HYBRID_CASES[name]
    w = W.small(wl, seqlens, **kw)
    if frac is None:   # keys at the sign bit and the top bit of the 64-bit column masks
        lists = [[14, 31, 39, 63, 64, 95, 127, 300, 351]] * w.hq
        off = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
        return w, dict(kind=3, window=win, sel_off=off, sel_idx=np.concatenate(lists).astype(np.int32))
    return w, W.make_selection(w, frac, win)


def _check_hybrid_traversal(w, pol, p, census):
    import tile_routed_mixed_amd as T
    tr = T.read_traversal(p.trav.cpu().numpy())
    want = {}
    n_full = n_edge = n_none = n_g = 0
    gbase, g = {}, 0
    for s_, S in enumerate(w.seqlens):
        cls = OP.hybrid_tile_classes(S, w.bq, w.bk, pol["window"])
        for h in range(w.hq):
            sel = OP.hybrid_selected(pol, s_, h, w.hq)
            gbase[(s_, h)] = g
            g += -(-len(sel) // 64)
            for i in range(cls.shape[0]):
                rl = min((i + 1) * w.bq, S) - 1
                ng = -(-int(np.sum(sel <= rl)) // 64)
                want[(s_, h, i)] = (set(np.nonzero(cls[i] == OP.WIN_FULL)[0].tolist()),
                                    set(np.nonzero(cls[i] == OP.WIN_EDGE)[0].tolist()),
                                    set(np.nonzero(cls[i] == OP.WIN_NONE)[0].tolist()), ng)
                n_full += len(want[(s_, h, i)][0])
                n_edge += len(want[(s_, h, i)][1])
                n_none += len(want[(s_, h, i)][2])
                n_g += ng
    assert census["fp16"] == n_full + n_edge + n_g and census["int8"] == n_edge + n_none
    assert census["int4"] == 0 and census["skip"] == 0
    assert tr["n_items"] == len(want)
    for n in range(tr["n_items"]):
        s_, h, qt, nr = (int(x) for x in tr["items"][n, :4])
        got = {3: set(), 7: set(), 6: set(), 2: set()}
        ng = 0
        for r in range(nr):
            first, cp = (int(x) for x in tr["runs"][n, r])
            cnt, prec = cp & 0xFFFFFF, cp >> 24
            if prec == 11:
                assert first == gbase[(s_, h)]
                ng += cnt
            else:
                got[prec] |= set(range(first, first + cnt))
        full, edge, none, wng = want[(s_, h, qt)]
        assert got[3] == full and got[7] == edge and got[6] == edge and got[2] == none, (s_, h, qt)
        assert ng == wng


@pytest.mark.parametrize("case", list(HYBRID_CASES))
def test_hybrid_prefill(case):
    w, pol = _hyb_case(case)
    q, k, v = _inputs(w)
    p, census, o, lse, _ = run_prefill(w, pol, q, k, v)
    _check_hybrid_traversal(w, pol, p, census)
    O, L, _, _ = oracle_prefill(w, pol, q, k, v)
    compare(o, O, lse, L, what=case)


def test_hybrid_reduces_to_fp16_and_int8_kernels():
    """No selected key: a window covering every row runs the bitmask kernel's
    all-FP16 work, tile for tile in the same order (same outputs bit for bit),
    and a zero window the all-INT8 work of the boundary policy (computed by
    the boundary kernel in its own tile order: within the fp32 gate)."""
    w = W.small("gqa8k", [900, 300], hq=4, hkv=2)
    q, k, v = _inputs(w)
    none = dict(kind=3, sel_off=np.zeros(len(w.seqlens) * w.hq + 1, np.int32), sel_idx=np.zeros(0, np.int32))
    _, tot = OP.bitmask_row_base(w.seqlens, w.hq, w.bq, w.bk, 4)
    _, _, o1, l1, _ = run_prefill(w, dict(kind=1, group=4, words=np.full(tot, 0xFFFFFFFF, np.uint32)), q, k, v)
    _, _, o2, l2, _ = run_prefill(w, dict(none, window=10 ** 6), q, k, v)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    _, _, o3, l3, _ = run_prefill(w, dict(kind=0, b8=[10 ** 6] * 4, b4=[10 ** 6] * 4, sink=0), q, k, v)
    _, _, o4, l4, _ = run_prefill(w, dict(none, window=0), q, k, v)
    compare(o3, o4.astype(np.float64), l3, l4.astype(np.float64), what="hybrid zero window vs all-INT8 boundaries")


def test_varlen_permutation_equivariance():
    """Permuting the sequences of a varlen batch permutes the outputs: every
    sequence's rows come out bit for bit the same."""
    seqs = [700, 64, 1, 1300, 129]
    perm = [3, 0, 4, 2, 1]
    w = W.small("gqa8k", seqs, hq=8, hkv=2)
    pol = dict(kind=0, b8=[1, 2, 3, 4, 1, 2, 3, 4], b4=[3, 5, 7, 9, 4, 6, 8, 10], sink=1)
    q, k, v = _inputs(w)
    cu = np.concatenate([[0], np.cumsum(seqs)])
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in perm])
    wp = W.small("gqa8k", [seqs[s] for s in perm], hq=8, hkv=2)
    qp, kp, vp = ((x[0][idx], x[1][idx]) for x in (q, k, v))
    _, _, o, lse, _ = run_prefill(w, pol, q, k, v)
    _, _, op, lsep, _ = run_prefill(wp, pol, qp, kp, vp)
    assert np.array_equal(o[idx], op)
    assert np.array_equal(lse[:, idx], lsep)


def test_prefill_16bit_outputs():
    import tile_routed_mixed_amd as T
    w, pol = _case("boundaries_varlen")
    q, k, v = _inputs(w)
    O, _, _, _ = oracle_prefill(w, pol, q, k, v)
    for odt, ulp in ((T.TM_F16, 2.0 ** -11), (T.TM_BF16, 2.0 ** -8)):
        _, _, o, _, _ = run_prefill(w, pol, q, k, v, o_dtype=odt)
        err = np.abs(o - O)
        assert np.all(err <= TOL_MAX + ulp * np.abs(O) + 1e-7), (odt, float(err.max()))


def test_deterministic():
    w, pol = _case("bitmask_varlen")
    q, k, v = _inputs(w)
    _, _, o1, l1, _ = run_prefill(w, pol, q, k, v)
    _, _, o2, l2, _ = run_prefill(w, pol, q, k, v)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------------------- decode (small)

def _with_sel(dp, sel):
    """A copy of a binding DPolicy carrying the lists `sel` (for size queries)."""
    import copy
    d = copy.copy(dp)
    d.c = type(dp.c).from_buffer_copy(dp.c)
    d.set_selection(*sel)
    return d


def _decode_case(seqlens, dpol, hq=8, hkv=2, d=128, dtype="f16", sel=None, plant=None):
    """sel: (sel_off, sel_idx) selected tokens per (sequence, KV head), or None.
    plant: a function of (decode query, K, V) input pairs returning new ones."""
    import torch
    import tile_routed_mixed_amd as T
    w = W.small("decode16x32k", seqlens, hq=hq, hkv=hkv, d=d, dtype=dtype)
    q, k, v = W.make_qkv(w)
    dq = W.make_decode_query(w)
    if plant is not None:
        dq, k, v = plant(dq, k, v)
    say(f"[gpu] decode {seqlens} hq={hq} hkv={hkv} d={d} {dtype} {dpol} "
        f"{'' if sel is None else str(len(sel[1])) + ' selected'}")
    p = T.DecodePipeline(w.seqlens, hq, hkv, d, dpol, dtype=dtype)
    p.upload(dq[0], k[0], v[0])
    g = guard_decode(p)
    p.build_cache()
    if sel is not None:
        p.sel_buf = g.alloc((max(256, T._binding.decode_sel_bytes(p.shape, _with_sel(p.dpol, sel))),), torch.uint8,
                            0xFF, role="sel")
        p.select(*sel)
        dpol = dict(dpol, sel_off=sel[0], sel_idx=sel[1])
    o = p.decode()
    torch.cuda.synchronize()
    g.check()
    assert_all_written(o, "decode O")
    kq = OQ.quantize(k[1], w.seqlens)
    vq = OQ.quantize(v[1], w.seqlens, layout="cols")
    O = OA.decode(w.seqlens, hq, hkv, d, dq[1].astype(np.float64), kq, vq, k[1].astype(np.float64),
                  v[1].astype(np.float64), dpol)
    return o.cpu().numpy(), O


@pytest.mark.parametrize("seqlens,dpol,d,dtype", [
    ([1, 100, 1000, 2000], dict(b8=[2, 3], b4=[5, 9], sink=1, tail=128), 128, "f16"),
    ([64, 65, 4097], dict(b8=[1, 4], b4=[1, 40], sink=0, tail=128), 64, "f16"),
    ([3000, 777], dict(b8=[10 ** 6] * 2, b4=[10 ** 6] * 2, sink=0, tail=0), 128, "f16"),
    ([2500], dict(b8=[0, 0], b4=[30, 30], sink=1, tail=1), 128, "f16"),
    ([1500, 3000], dict(b8=[4, 8], b4=[20, 30], sink=1, tail=128), 128, "bf16"),
])
def test_decode_small(seqlens, dpol, d, dtype):
    o, O = _decode_case(seqlens, dpol, d=d, dtype=dtype)
    compare(o, O, what=f"decode {seqlens} {dtype}")


@pytest.mark.parametrize("hq,hkv,b8,b4", [
    # groups of 4 with maps that differ inside a group, runs of equal maps, and
    # one group whose maps agree
    (8, 2, [1, 1, 3, 0, 2, 2, 2, 2], [4, 9, 9, 2, 6, 6, 6, 6]),
    # groups of 8 (the unpacked softmax) cut into classes of 1, 3 and 4 heads
    (16, 2, [0] + [2] * 3 + [5] * 4 + [1] * 8, [3] + [8] * 3 + [40] * 4 + [2] * 8),
])
def test_decode_per_query_head_maps(hq, hkv, b8, b4):
    dpol = dict(b8=b8, b4=b4, sink=1, tail=100, per_q_head=1)
    o, O = _decode_case([300, 2100, 64, 1000], dpol, hq=hq, hkv=hkv)
    compare(o, O, what=f"decode per-query-head maps hq={hq}")


@pytest.mark.parametrize("seqlens,hq,hkv,d,dtype,dpol", [
    ([1, 100, 1000, 2000], 8, 2, 128, "f16", dict(b8=[2, 3], b4=[5, 9], sink=1, tail=128)),
    ([3000, 777], 16, 2, 128, "f16", dict(b8=[1] * 8 + [3] * 8, b4=[4] * 8 + [12] * 8, sink=0, tail=100,
                                          per_q_head=1)),
    ([1500, 64, 65], 4, 1, 64, "bf16", dict(b8=[4], b4=[10], sink=1, tail=128)),
])
def test_decode_selected_tokens(seqlens, hq, hkv, d, dtype, dpol):
    w = W.small("decode16x32k", seqlens, hq=hq, hkv=hkv, d=d, dtype=dtype)
    sel = W.make_decode_selection(w, 0.05)
    o, O = _decode_case(seqlens, dpol, hq=hq, hkv=hkv, d=d, dtype=dtype, sel=sel)
    compare(o, O, what=f"decode selected tokens {seqlens} hq={hq}")


def test_decode_selected_tokens_growing_cache():
    """Selected tokens in a cache grown one token per step: every step matches
    the oracle at the current lengths."""
    import torch
    import tile_routed_mixed_amd as T
    seqlens, hq, hkv, d = [700, 1300], 8, 2, 128
    w = W.small("decode16x32k", seqlens, hq=hq, hkv=hkv, d=d)
    q, k, v = W.make_qkv(w)
    dq = W.make_decode_query(w)
    dpol = dict(b8=[2, 3], b4=[5, 9], sink=1, tail=128)
    start = np.array([S - 3 for S in seqlens], np.int32)
    sel = W.make_decode_selection(w, 0.05, lengths=start)
    say(f"[gpu] decode growing cache with {len(sel[1])} selected tokens")
    p = T.DecodePipeline(w.seqlens, hq, hkv, d, dpol)
    p.upload(dq[0], k[0], v[0])
    g = guard_decode(p)
    p.start(start)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    L = start.copy()
    for step in range(3):
        p.select(*sel)
        g.poison()
        o = p.decode()
        torch.cuda.synchronize()
        g.check()
        assert_all_written(o, "decode O")
        rows = np.concatenate([np.arange(cu[s_], cu[s_] + L[s_]) for s_ in range(len(seqlens))])
        kq = OQ.quantize(k[1][rows], list(L))
        vq = OQ.quantize(v[1][rows], list(L), layout="cols")
        O = OA.decode(list(L), hq, hkv, d, dq[1].astype(np.float64), kq, vq, k[1][rows].astype(np.float64),
                      v[1][rows].astype(np.float64), dict(dpol, sel_off=sel[0], sel_idx=sel[1]))
        compare(o.cpu().numpy(), O, what=f"growing cache with selection, step {step}")
        nxt = cu[:-1] + L
        p.append(k[0][nxt], v[0][nxt])
        L = L + 1


def test_decode_empty_selection_equals_none():
    """The selection variant of the kernel with empty lists computes the same
    outputs bit for bit as the plain one."""
    seqlens = [1500, 3000]
    dpol = dict(b8=[3, 5], b4=[9, 20], sink=1, tail=128)
    o1, _ = _decode_case(seqlens, dpol)
    n = len(seqlens) * 2
    o2, _ = _decode_case(seqlens, dpol, sel=(np.zeros(n + 1, np.int32), np.zeros(0, np.int32)))
    assert np.array_equal(o1, o2)


def test_decode_uniform_per_query_head_maps_equal_per_kv_maps():
    """Per-query-head maps that agree inside each group take the per-KV-head
    launch: the same outputs bit for bit."""
    seqlens = [1500, 3000]
    o1, _ = _decode_case(seqlens, dict(b8=[3, 5], b4=[9, 20], sink=1, tail=128))
    o2, _ = _decode_case(seqlens, dict(b8=[3] * 4 + [5] * 4, b4=[9] * 4 + [20] * 4, sink=1, tail=128, per_q_head=1))
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("hq,hkv,d", [(2, 2, 128), (6, 2, 128), (16, 2, 128), (16, 1, 64)])
def test_decode_group_sizes(hq, hkv, d):
    """Query groups of 1, 3, 8 and 16 heads per KV head: groups of up to 4
    heads take the compacted softmax, larger ones the full-width one."""
    dpol = dict(b8=[3] * hkv, b4=[11] * hkv, sink=1, tail=128)
    o, O = _decode_case([700, 1900, 65], dpol, hq=hq, hkv=hkv, d=d)
    compare(o, O, what=f"decode group {hq}/{hkv} d={d}")


@pytest.mark.parametrize("d", [128, 64])
def test_decode_deterministic_long_splits(d):
    """Splits that walk dozens of mixed INT4/INT8 blocks in a register
    double buffer (the loads' wait counts decide correctness there): bitwise
    identical over repeated calls, and within the gate against the oracle."""
    import torch
    import tile_routed_mixed_amd as T
    seqlens = [12000, 9000]
    dpol = dict(b8=[40, 60], b4=[150, 140], sink=1, tail=128)
    w = W.small("decode16x32k", seqlens, hq=8, hkv=2, d=d, dtype="f16")
    q, k, v = W.make_qkv(w)
    dq = W.make_decode_query(w)
    say(f"[gpu] decode determinism {seqlens} d={d} {dpol}")
    p = T.DecodePipeline(w.seqlens, 8, 2, d, dpol, dtype="f16")
    p.upload(dq[0], k[0], v[0])
    g = guard_decode(p)
    p.build_cache()
    outs = []
    for _ in range(3):
        g.poison()
        g.poison("ws")
        o = p.decode()
        torch.cuda.synchronize()
        g.check()
        assert_all_written(o, "decode O")
        outs.append(o.cpu().numpy().copy())
    assert all(np.array_equal(outs[0], x) for x in outs[1:])
    kq = OQ.quantize(k[1], w.seqlens)
    vq = OQ.quantize(v[1], w.seqlens, layout="cols")
    O = OA.decode(w.seqlens, 8, 2, d, dq[1].astype(np.float64), kq, vq, k[1].astype(np.float64),
                  v[1].astype(np.float64), dpol)
    compare(outs[0], O, what=f"decode determinism d={d}")


def test_decode_growing_cache_matches_rebuilt_oracle():
    """Generation loop: caches of 1000- and 950-token prompts grow by one token
    per step for 140 steps (crossing two 64-token block boundaries, so blocks
    leave the 128-token FP16 window and become INT8/INT4), each step through
    tm_cache_append; at every 20th step the decode equals the oracle over the
    cache quantized from scratch at the current lengths."""
    import torch
    import tile_routed_mixed_amd as T
    caps, L0, steps = [1200, 1100], np.array([1000, 950]), 140
    hq, hkv, d = 8, 2, 128
    dpol = dict(b8=[4, 6], b4=[10, 12], sink=1, tail=128)
    w = W.small("decode16x32k", caps, hq=hq, hkv=hkv, d=d, dtype="f16")
    _, k, v = W.make_qkv(w)                        # rows past the prompts are the generated tokens
    rng = np.random.default_rng(77)
    queries = [W.round16(rng.standard_normal((2, hq, d)).astype(np.float32), "f16") for _ in range(steps + 1)]
    cu = w.cu_seqlens
    say(f"[gpu] growing cache {caps} from {L0.tolist()}, {steps} steps")
    p = T.DecodePipeline(w.seqlens, hq, hkv, d, dpol, dtype="f16")
    p.upload(queries[0][0], k[0], v[0])
    g = guard_decode(p)
    p.start(L0)
    for step in range(steps + 1):
        L = L0 + step
        if step % 20 == 0:
            g.poison()
            o = p.decode()
            torch.cuda.synchronize()
            g.check()
            assert_all_written(o, "decode O")
            o = o.cpu().numpy()
            for b in range(2):
                sl = slice(int(cu[b]), int(cu[b]) + int(L[b]))
                kq = OQ.quantize(k[1][sl], [int(L[b])])
                vq = OQ.quantize(v[1][sl], [int(L[b])], layout="cols")
                O = OA.decode([int(L[b])], hq, hkv, d, queries[step][1][b:b + 1].astype(np.float64), kq, vq,
                              k[1][sl].astype(np.float64), v[1][sl].astype(np.float64), dpol)
                compare(o[b], O[0], what=f"growing cache step {step} seq {b} L={int(L[b])}")
        if step < steps:
            rows = cu[:-1] + L
            p.append(k[0][rows], v[0][rows], q_bits=queries[step + 1][0])


# ------------------------------------------------- bf16 values beyond the fp16 range

def _plant16(pair, seed, vals, dtype="bf16"):
    """The (bits, values) input pair with bf16 values beyond the fp16 range
    planted at a few seeded places."""
    y = np.array(pair[1], np.float32)
    flat = y.reshape(-1)
    rng = np.random.default_rng(seed)
    for i, val in zip(rng.choice(flat.size, len(vals), replace=False), vals):
        flat[i] = val
    return W.round16(y, dtype)


def _near(o, ref, big, what):
    """Gate plus 2^-11 of the largest |value| the output mixes (big, broadcast
    to o's shape): fp16 probabilities carry a relative error of 2^-12, which a
    channel holding values near 65504 turns into absolute error."""
    m = ~np.isnan(ref)
    assert np.all(np.isfinite(o[m])), what
    err = np.abs(o - ref)[m]
    tol = (TOL_MAX + 2.0 ** -11 * big)[m]
    say(f"[cmp] {what}: max err/tol {float(np.max(err / tol)):.3f}")
    assert np.all(err <= tol), what


@pytest.mark.parametrize("kind", [0, 1])
def test_bf16_beyond_fp16_range_prefill(kind):
    """bf16 V values beyond the fp16 range (1e5, -3e38, ...): the fp16 V^T
    copy saturates them to +-65504 (bit-exact with the oracle quantizer, which
    takes the same reading), and both prefill kernels give finite outputs that
    match the oracle."""
    w = W.small("gqa8k", [700, 129], hq=4, hkv=2)
    q, k, v = _inputs(w)
    v = _plant16(v, 31, [1.0e5, -3.0e38, 7.0e4, -9.0e4, 6.6e4])
    assert np.max(np.abs(v[1])) > 65504
    if kind == 0:
        pol = dict(kind=0, b8=[1, 2, 0, 3], b4=[2, 5, 4, 3], sink=1)
    else:
        _, tot = OP.bitmask_row_base(w.seqlens, w.hq, w.bq, w.bk, 4)
        pol = dict(kind=1, group=4, words=np.full(tot, 0xFFFFFFFF, np.uint32))
    p, _, o, lse, _ = run_prefill(w, pol, q, k, v)
    ref = OQ.quantize(v[1], w.seqlens, layout="cols", with_t16=True)
    t16 = np.swapaxes(p.vq.t16.cpu().numpy(), 0, 1)
    assert np.array_equal(t16.view(np.uint16), ref["t16"].view(np.uint16))
    O, L, _, _ = oracle_prefill(w, pol, q, k, v)
    big = np.max(np.abs(np.clip(v[1], -65504, 65504)), axis=0)          # [hkv][d]
    grp = w.hq // w.hkv
    _near(o, O, np.broadcast_to(np.repeat(big, grp, axis=0)[None], o.shape), f"prefill kind {kind}")
    assert np.all(np.isfinite(lse[~np.isnan(L)]))


def test_bf16_beyond_fp16_range_decode():
    """bf16 values beyond the fp16 range in the decode query and in the cache
    (FP16 window and quantized blocks): finite outputs matching the oracle,
    whose fp16 copies saturate as the kernel's do."""
    dpol = dict(b8=[4, 8], b4=[20, 30], sink=1, tail=128)
    seqlens, hq, hkv = [1500, 3000], 8, 2
    held = {}

    def plant(dq, k, v):
        held["v"] = _plant16(v, 43, [1.0e5, -3.0e38, 7.0e4], "bf16")
        return _plant16(dq, 41, [1.0e5], "bf16"), _plant16(k, 42, [2.0e5, -7.0e4], "bf16"), held["v"]
    o, O = _decode_case(seqlens, dpol, hq=hq, hkv=hkv, dtype="bf16", plant=plant)
    vv = np.abs(np.clip(held["v"][1], -65504, 65504))
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    big = np.stack([np.repeat(np.max(vv[cu[b]:cu[b + 1]], axis=0), hq // hkv, axis=0) for b in range(len(seqlens))])
    assert np.max(big) == 65504.0
    _near(o, O, big, "decode")
