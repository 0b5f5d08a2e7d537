"""C-ABI checks that need no GPU: the library loads, exports every function
include/tm.h declares, answers size queries, and rejects every invalid
argument with the documented status before touching the device.

Device pointers in these tests are fake non-NULL addresses: each call here
fails host validation (or is a size query), so nothing is dereferenced or
launched.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def B():
    from tile_routed_mixed_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from tile_routed_mixed_amd import build
        build.build()
    _binding.lib()
    return _binding


FAKE = 0x10000


def declared_functions():
    text = open(os.path.join(ROOT, "include", "tm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tm_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(B):
    names = declared_functions()
    assert {"tm_quantize_pack", "tm_build_traversal", "tm_prefill", "tm_decode"} <= set(names)
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (tm_\w+)", out))
    assert set(names) <= exported


def test_version_and_status_strings(B):
    L = B.lib()
    assert L.tm_version() >> 16 == 1
    for s in range(7):
        assert L.tm_status_string(s).decode().startswith("TM_")


def _shape(B, seqlens, hq=4, hkv=2, d=64, bq=128, bk=64, dtype=0, dev=True):
    s = B.Shape(seqlens, hq, hkv, d, bq, bk, dtype)
    s.c.cu_seqlens_dev = FAKE if dev else None
    return s


def test_num_blocks(B):
    assert _shape(B, [1, 63, 64, 65, 200]).nblk() == 1 + 1 + 1 + 2 + 4
    assert _shape(B, [0, 64]).nblk() == 1


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), 2), (dict(hq=3, hkv=2), 2), (dict(bq=96), 2), (dict(bk=32), 2), (dict(dtype=2), 2),
])
def test_bad_shapes(B, kw, status):
    s = _shape(B, [100], **kw)
    pol = B.Policy(dict(kind=0, b8=[1] * s.hq, b4=[2] * s.hq, sink=0))
    n = ctypes.c_size_t(0)
    assert B.lib().tm_build_traversal(ctypes.byref(s.c), ctypes.byref(pol.c), None, ctypes.byref(n), None,
                                      None) == status


def test_bad_cu_seqlens(B):
    s = _shape(B, [100, 20])
    s.cu_host[1] = 130          # non-monotone: 0, 130, 120
    pol = B.Policy(dict(kind=0, b8=[1] * 4, b4=[2] * 4, sink=0))
    n = ctypes.c_size_t(0)
    assert B.lib().tm_build_traversal(ctypes.byref(s.c), ctypes.byref(pol.c), None, ctypes.byref(n), None,
                                      None) == B.TM_E_SHAPE
    s.cu_host[:] = [5, 105, 125]
    assert B.lib().tm_num_blocks(ctypes.byref(s.c)) == -1


@pytest.mark.parametrize("pol,status", [
    (dict(kind=0, b8=[3, 1, 1, 1], b4=[2, 2, 2, 2], sink=0), 3),      # b8 > b4
    (dict(kind=0, b8=[0, 1, 1, 1], b4=[0, 2, 2, 2], sink=0), 3),      # a row with no key
    (dict(kind=0, b8=[-1, 1, 1, 1], b4=[2, 2, 2, 2], sink=0), 3),
    (dict(kind=0, b8=[1] * 4, b4=[2] * 4, sink=2), 3),
    (dict(kind=7, b8=[1] * 4, b4=[2] * 4, sink=0), 1),
])
def test_bad_boundary_policies(B, pol, status):
    s = _shape(B, [300, 50])
    p = B.Policy(pol) if pol["kind"] in (0,) else None
    if p is None:
        p = B.Policy(dict(kind=0, b8=pol["b8"], b4=pol["b4"], sink=0))
        p.c.kind = pol["kind"]
    n = ctypes.c_size_t(0)
    assert B.lib().tm_build_traversal(ctypes.byref(s.c), ctypes.byref(p.c), None, ctypes.byref(n), None,
                                      None) == status


def test_zero_b4_with_sink_is_valid(B):
    s = _shape(B, [300])
    p = B.Policy(dict(kind=0, b8=[0] * 4, b4=[0] * 4, sink=1))
    n = ctypes.c_size_t(0)
    assert B.lib().tm_build_traversal(ctypes.byref(s.c), ctypes.byref(p.c), None, ctypes.byref(n), None,
                                      None) == B.TM_OK


def test_bitmask_validation_and_size(B):
    from oracle import policy as P   # the word count the pages' layout implies
    s = _shape(B, [1000, 10240], hq=2, hkv=1)
    _, tot = P.bitmask_row_base([1000, 10240], 2, 128, 64, 4)
    p = B.Policy(dict(kind=1, group=4, words=np.zeros(tot, np.uint32)))
    p.c.bits = FAKE
    n = ctypes.c_size_t(0)
    L = B.lib()
    assert L.tm_build_traversal(ctypes.byref(s.c), ctypes.byref(p.c), None, ctypes.byref(n), None, None) == 0
    n_items = 2 * (8 + 80)
    max_runs = (160 + 3) // 4
    align = lambda x: (x + 255) // 256 * 256
    want = align(align(align(256 + 2 * 16) + 32 * n_items) + 8 * n_items * max_runs)
    assert n.value == want
    p.c.n_words = tot - 1
    assert L.tm_build_traversal(ctypes.byref(s.c), ctypes.byref(p.c), None, ctypes.byref(n), None, None) == 3
    p.c.n_words = tot
    p.c.group = 0
    assert L.tm_build_traversal(ctypes.byref(s.c), ctypes.byref(p.c), None, ctypes.byref(n), None, None) == 3


def test_fourway_validation_and_size(B):
    from oracle import policy as P   # the word count the four-way layout implies
    s = _shape(B, [1000, 10240], hq=2, hkv=1)
    _, tot = P.fourway_row_base([1000, 10240], 2, 128, 64, 4)
    p = B.Policy(dict(kind=2, b8=[1, 2], b4=[3, 4], sink=0, group=4, words=np.zeros(tot, np.uint32)))
    p.c.bits = FAKE
    n = ctypes.c_size_t(0)
    L = B.lib()

    def st():
        return L.tm_build_traversal(ctypes.byref(s.c), ctypes.byref(p.c), None, ctypes.byref(n), None, None)

    assert st() == 0
    n_items = 2 * (8 + 80)
    max_runs = (160 + 3) // 4 + 3          # one run per group plus the three boundary edges
    align = lambda x: (x + 255) // 256 * 256
    assert n.value == align(align(align(256 + 2 * 16) + 32 * n_items) + 8 * n_items * max_runs)
    p.c.n_words = tot - 1                  # 16 codes per word: a bitmask-sized map is too small
    assert st() == B.TM_E_POLICY
    p.c.n_words = tot
    p.c.group = 0
    assert st() == B.TM_E_POLICY
    p.c.group = 4
    p.b8[0] = 5                            # b8 > b4
    assert st() == B.TM_E_POLICY
    p.b8[0] = 1
    p.b8[1] = p.b4[1] = 0                  # b4 == 0 without a sink
    assert st() == B.TM_E_POLICY
    p.c.sink = 1
    assert st() == B.TM_OK
    p.c.sink = 2
    assert st() == B.TM_E_POLICY
    p.c.sink = 0
    p.b8[1], p.b4[1] = 2, 4
    p.c.bits = None                        # no code map
    assert st() == B.TM_E_ARG
    p.c.bits = FAKE
    p.c.b8 = None
    assert st() == B.TM_E_ARG


def _hybrid(B, window, lists):
    off = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    idx = np.concatenate([np.asarray(x, np.int32) for x in lists]).astype(np.int32)
    return B.Policy(dict(kind=3, window=window, sel_off=off, sel_idx=idx))


def test_hybrid_validation_and_size(B):
    L = B.lib()
    s = _shape(B, [1000, 130], hq=2, hkv=1, d=128)
    lists = [[0, 5, 999], list(range(70)), [], [129]]     # rows (seq 0, h 0), (0, 1), (1, 0), (1, 1)
    p = _hybrid(B, 128, lists)
    n = ctypes.c_size_t(0)

    def st(pp):
        return L.tm_build_traversal(ctypes.byref(s.c), ctypes.byref(pp.c), None, ctypes.byref(n), None, None)

    assert st(p) == B.TM_OK
    align = lambda x: (x + 255) // 256 * 256
    n_items = 2 * (8 + 2)
    end = align(align(align(256 + 2 * 16) + 32 * n_items) + 8 * n_items * 5)   # 5 runs per item
    n_gt = 1 + 2 + 0 + 1                                   # ceil(len / 64) per list
    end = align(end + 16 * 4)                              # list table
    end = align(end + 4 * (4 + 1))                         # staged list offsets
    end = align(end + 4 * (3 + 70 + 0 + 1))                # positions
    end = align(end + 8 * (2 * 16 + 2 * 3))                # column masks: hq * nk per sequence
    end = align(end + 512 * n_gt)                          # gathered tile headers
    end = align(end + n_gt * 64 * 128 * 2)                 # K rows
    end = align(end + n_gt * 128 * 64 * 2)                 # V^T
    assert n.value == end
    assert st(_hybrid(B, -1, lists)) == B.TM_E_POLICY                       # negative window
    assert st(_hybrid(B, 0, [[0, 5, 5], [], [], []])) == B.TM_E_POLICY      # not strictly increasing
    assert st(_hybrid(B, 0, [[], [], [130], []])) == B.TM_E_POLICY          # past the sequence end
    assert st(_hybrid(B, 0, [[-1], [], [], []])) == B.TM_E_POLICY           # negative position
    bad = _hybrid(B, 0, lists)
    bad.sel_off[0] = 1
    assert st(bad) == B.TM_E_POLICY                                        # offsets not from 0
    bad = _hybrid(B, 0, lists)
    bad.c.sel_off = None
    assert st(bad) == B.TM_E_ARG
    # lists in device memory (sel_idx NULL, device arrays set): the positions
    # are not read on the host, so the same size comes out and only the
    # offsets are checked
    dv = _hybrid(B, 128, lists)
    dv.c.sel_idx = None
    dv.c.sel_idx_dev = FAKE
    dv.c.sel_off_dev = FAKE
    n.value = 0
    assert st(dv) == B.TM_OK and n.value == end
    dv.c.sel_idx_dev = None                                                  # neither host nor device lists
    assert st(dv) == B.TM_E_ARG
    dv = _hybrid(B, 0, [[], [], list(range(131)), []])                      # longer than its sequence
    dv.c.sel_idx, dv.c.sel_idx_dev, dv.c.sel_off_dev = None, FAKE, FAKE
    assert st(dv) == B.TM_E_POLICY
    # gather: hybrid policies only, device pointers required
    assert L.tm_gather_selected(ctypes.byref(s.c), ctypes.byref(p.c), FAKE, None, FAKE, None) == B.TM_E_ARG
    assert L.tm_gather_selected(ctypes.byref(s.c), ctypes.byref(p.c), FAKE, FAKE, None, None) == B.TM_E_ARG
    b = B.Policy(dict(kind=0, b8=[1, 1], b4=[2, 2], sink=0))
    assert L.tm_gather_selected(ctypes.byref(s.c), ctypes.byref(b.c), FAKE, FAKE, FAKE, None) == B.TM_E_ARG
    # build and gather in one launch: the same size query and checks, hybrid
    # policies only, K and V required when a traversal is given
    fused = lambda pp, k, v, t=None: L.tm_build_traversal_gather(ctypes.byref(s.c), ctypes.byref(pp.c), t,
                                                                 ctypes.byref(n), None, k, v, None)
    n.value = 0
    assert fused(p, None, None) == B.TM_OK and n.value == end
    assert fused(_hybrid(B, -1, lists), FAKE, FAKE) == B.TM_E_POLICY
    assert fused(p, None, FAKE, FAKE) == B.TM_E_ARG
    assert fused(p, FAKE, None, FAKE) == B.TM_E_ARG
    assert fused(b, FAKE, FAKE) == B.TM_E_ARG


def test_traversal_capacity(B):
    s = _shape(B, [512], hq=1, hkv=1, bq=64)
    p = B.Policy(dict(kind=0, b8=[2], b4=[5], sink=1))
    n = ctypes.c_size_t(0)
    L = B.lib()
    assert L.tm_build_traversal(ctypes.byref(s.c), ctypes.byref(p.c), None, ctypes.byref(n), None, None) == 0
    need = n.value
    assert need == 256 + 256 + 256 + 256        # header, seq table, 8 items, 8 x 3 runs (aligned)
    small = ctypes.c_size_t(need - 1)
    assert L.tm_build_traversal(ctypes.byref(s.c), ctypes.byref(p.c), FAKE, ctypes.byref(small), None,
                                None) == B.TM_E_SPACE


def _qt(B, heads, layout, nblk, t16=True, c4x=False):
    return B.tm_qtensor(FAKE, FAKE, FAKE, FAKE, FAKE if t16 else None, heads, layout, nblk, FAKE if c4x else None)


def test_quantize_validation(B):
    s = _shape(B, [100, 30])
    L = B.lib()
    nb = s.nblk()
    q = _qt(B, 4, B.TM_ROWS, nb, t16=True)           # rows layout with t16 set
    assert L.tm_quantize_pack(ctypes.byref(s.c), FAKE, 4, ctypes.byref(q), None) == B.TM_E_ARG
    q = _qt(B, 4, B.TM_ROWS, nb + 1, t16=False)
    assert L.tm_quantize_pack(ctypes.byref(s.c), FAKE, 4, ctypes.byref(q), None) == B.TM_E_SHAPE
    q = _qt(B, 4, 5, nb, t16=False)
    assert L.tm_quantize_pack(ctypes.byref(s.c), FAKE, 4, ctypes.byref(q), None) == B.TM_E_ARG
    q = _qt(B, 3, B.TM_ROWS, nb, t16=False)
    assert L.tm_quantize_pack(ctypes.byref(s.c), FAKE, 4, ctypes.byref(q), None) == B.TM_E_SHAPE
    assert L.tm_quantize_pack(ctypes.byref(s.c), None, 4, ctypes.byref(q), None) == B.TM_E_ARG
    s2 = _shape(B, [100, 30], dev=False)
    q = _qt(B, 4, B.TM_ROWS, nb, t16=False)
    assert L.tm_quantize_pack(ctypes.byref(s2.c), FAKE, 4, ctypes.byref(q), None) == B.TM_E_ARG
    q = _qt(B, 4, B.TM_COLS, nb, t16=True, c4x=True)    # the one-byte INT4 copy exists in the rows layout only
    assert L.tm_quantize_pack(ctypes.byref(s.c), FAKE, 4, ctypes.byref(q), None) == B.TM_E_ARG


def test_prefill_validation(B):
    s = _shape(B, [100, 30])
    L = B.lib()
    nb = s.nblk()
    qq, kq, vq = _qt(B, 4, 0, nb, False), _qt(B, 2, 0, nb, False), _qt(B, 2, 1, nb, True)
    args = lambda **kw: dict(dict(trav=FAKE, kind=0, q=FAKE, k=FAKE, qq=qq, kq=kq, vq=vq, o=FAKE, odt=0, ndbg=0),
                             **kw)

    def call(a):
        return L.tm_prefill(ctypes.byref(s.c), a["trav"], a["kind"], a["q"], a["k"], ctypes.byref(a["qq"]),
                            ctypes.byref(a["kq"]), ctypes.byref(a["vq"]), a["o"], a["odt"], None, None, None,
                            a["ndbg"], None)
    assert call(args(q=None)) == B.TM_E_ARG
    assert call(args(kind=7)) == B.TM_E_ARG
    assert call(args(trav=None)) == B.TM_E_ARG
    assert call(args(odt=9)) == B.TM_E_ARG
    assert call(args(ndbg=2)) == B.TM_E_ARG
    assert call(args(vq=_qt(B, 2, 1, nb, False))) == B.TM_E_ARG
    assert call(args(vq=_qt(B, 2, 0, nb, True))) == B.TM_E_SHAPE
    assert call(args(kq=_qt(B, 4, 0, nb, False))) == B.TM_E_SHAPE
    assert call(args(qq=_qt(B, 4, 0, nb - 1, False))) == B.TM_E_SHAPE
    # boundary policies read K's one-byte INT4 copy: refused without it
    assert call(args(kq=_qt(B, 2, 0, nb, False, c4x=False))) == B.TM_E_ARG


def test_decode_validation_and_workspace(B):
    L = B.lib()
    s = _shape(B, [32768] * 16, hq=32, hkv=8, d=128)
    dp = B.DPolicy(dict(b8=[128] * 8, b4=[320] * 8, sink=1, tail=128))
    n = ctypes.c_size_t(0)
    assert L.tm_decode(ctypes.byref(s.c), None, None, None, None, ctypes.byref(dp.c), None, 2, None,
                       ctypes.byref(n), None) == B.TM_OK
    # 16 x 8 (sequence, KV head) pairs -> 16 splits (2048 waves); ws = B * hq * splits * (d + 2) floats
    assert n.value == 16 * 32 * 16 * 130 * 4
    small = ctypes.c_size_t(n.value - 4)
    nb = s.nblk()
    kq, vq = _qt(B, 8, 0, nb, False), _qt(B, 8, 1, nb, True)
    assert L.tm_decode(ctypes.byref(s.c), FAKE, ctypes.byref(kq), ctypes.byref(vq), FAKE, ctypes.byref(dp.c),
                       FAKE, 2, FAKE, ctypes.byref(small), None) == B.TM_E_SPACE
    bad = B.DPolicy(dict(b8=[300] * 8, b4=[200] * 8, sink=1, tail=128))
    assert L.tm_decode(ctypes.byref(s.c), None, None, None, None, ctypes.byref(bad.c), None, 2, None,
                       ctypes.byref(n), None) == B.TM_E_POLICY
    empty = B.DPolicy(dict(b8=[0] * 8, b4=[0] * 8, sink=0, tail=0))
    assert L.tm_decode(ctypes.byref(s.c), None, None, None, None, ctypes.byref(empty.c), None, 2, None,
                       ctypes.byref(n), None) == B.TM_E_POLICY
    sb = _shape(B, [64], hq=32, hkv=8, d=128, dtype=1)     # bf16 caches are supported
    assert L.tm_decode(ctypes.byref(sb.c), None, None, None, None, ctypes.byref(dp.c), None, 2, None,
                       ctypes.byref(n), None) == B.TM_OK
    sk = _shape(B, [64], hq=65 * 2, hkv=65, d=128)
    dp65 = B.DPolicy(dict(b8=[1] * 65, b4=[2] * 65, sink=1, tail=128))
    assert L.tm_decode(ctypes.byref(sk.c), None, None, None, None, ctypes.byref(dp65.c), None, 2, None,
                       ctypes.byref(n), None) == B.TM_E_UNSUPPORTED
    sg = _shape(B, [64], hq=34, hkv=2, d=128)
    dp2 = B.DPolicy(dict(b8=[1] * 2, b4=[2] * 2, sink=1, tail=128))
    assert L.tm_decode(ctypes.byref(sg.c), None, None, None, None, ctypes.byref(dp2.c), None, 2, None,
                       ctypes.byref(n), None) == B.TM_E_UNSUPPORTED
    sz = _shape(B, [64, 0], hq=4, hkv=2, d=128)
    assert L.tm_decode(ctypes.byref(sz.c), None, None, None, None, ctypes.byref(dp2.c), None, 2, None,
                       ctypes.byref(n), None) == B.TM_E_SHAPE


def test_decode_per_query_head_maps_validation_and_workspace(B):
    L = B.lib()
    s = _shape(B, [32768] * 16, hq=32, hkv=8, d=128)
    n = ctypes.c_size_t(0)

    def size(dp):
        return L.tm_decode(ctypes.byref(s.c), None, None, None, None, ctypes.byref(dp.c), None, 2, None,
                           ctypes.byref(n), None)

    # maps that agree inside every group: one class per KV head, the per-KV workspace
    same = B.DPolicy(dict(b8=[128] * 32, b4=[320] * 32, sink=1, tail=128, per_q_head=1))
    assert size(same) == B.TM_OK and n.value == 16 * 32 * 16 * 130 * 4
    # all maps distinct: one class per KV head over the union of its heads'
    # bands, so the per-KV split count and workspace
    mixed = B.DPolicy(dict(b8=list(range(100, 132)), b4=[400] * 32, sink=1, tail=128, per_q_head=1))
    assert size(mixed) == B.TM_OK and n.value == 16 * 32 * 16 * 130 * 4
    # more query heads than the kernel arguments hold maps for: the groups are
    # cut into runs of equal maps (128 classes -> 16 x 128 pairs -> 1 split)
    s128 = _shape(B, [32768] * 16, hq=128, hkv=8, d=128)
    many = B.DPolicy(dict(b8=[100 + h % 7 for h in range(128)], b4=[400] * 128, sink=1, tail=128, per_q_head=1))
    assert L.tm_decode(ctypes.byref(s128.c), None, None, None, None, ctypes.byref(many.c), None, 2, None,
                       ctypes.byref(n), None) == B.TM_OK and n.value == 16 * 128 * 1 * 130 * 4
    # the query-head maps are all checked (head 20 is past the 8 KV heads)
    bad = B.DPolicy(dict(b8=[1] * 20 + [9] + [1] * 11, b4=[4] * 32, sink=1, tail=128, per_q_head=1))
    assert size(bad) == B.TM_E_POLICY
    flag = B.DPolicy(dict(b8=[1] * 32, b4=[4] * 32, sink=1, tail=128, per_q_head=1))
    flag.c.per_q_head = 2
    assert size(flag) == B.TM_E_POLICY


def test_decode_selection_validation_and_size(B):
    L = B.lib()
    s = _shape(B, [1000, 130], hq=4, hkv=2, d=128)
    n = ctypes.c_size_t(0)
    dp = B.DPolicy(dict(b8=[2, 2], b4=[5, 5], sink=1, tail=128))
    lists = [[0, 31, 999], list(range(70)), [], [129]]      # (seq 0, kv 0), (0, 1), (1, 0), (1, 1)
    off = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    idx = np.concatenate([np.asarray(x, np.int32) for x in lists]).astype(np.int32)

    def size(o, x):
        dp.set_selection(o, x)
        return L.tm_decode_select(ctypes.byref(s.c), ctypes.byref(dp.c), None, None, None, ctypes.byref(n), None)

    assert size(off, idx) == B.TM_OK
    align = lambda v: (v + 255) // 256 * 256
    n_gt = 1 + 2 + 0 + 1
    nblk = 16 + 3
    end = align(4 * 2 * 4)                    # {first tile, keys} per list
    end = align(end + 8 * nblk * 2)           # column masks [nblk][hkv]
    end = align(end + 512 * n_gt)             # tile headers
    end = align(end + n_gt * 64 * 128 * 2)    # K rows
    end = align(end + n_gt * 128 * 64 * 2)    # V^T
    assert n.value == end
    bad = idx.copy()
    bad[1] = 0                                # not strictly increasing
    assert size(off, bad) == B.TM_E_POLICY
    bad = idx.copy()
    bad[-1] = 130                             # past sequence 1's length
    assert size(off, bad) == B.TM_E_POLICY
    lens = np.array([500, 130], np.int32)     # a growing cache: the lists follow the current lengths
    dp.set_lengths(lens)
    assert size(off, idx) == B.TM_E_POLICY    # 999 >= 500
    dp.set_lengths(None)
    dp.set_selection(None, None)
    assert L.tm_decode_select(ctypes.byref(s.c), ctypes.byref(dp.c), None, None, None, ctypes.byref(n),
                              None) == B.TM_E_ARG
    # a decode step with lists but no buffer
    dp.set_selection(off, idx)
    ws = ctypes.c_size_t(1 << 30)
    nb = s.nblk()
    kq, vq = _qt(B, 2, 0, nb, False), _qt(B, 2, 1, nb, True)
    assert L.tm_decode(ctypes.byref(s.c), FAKE, ctypes.byref(kq), ctypes.byref(vq), FAKE, ctypes.byref(dp.c),
                       FAKE, 2, FAKE, ctypes.byref(ws), None) == B.TM_E_ARG


def test_select_vertical_validation_and_size(B):
    L = B.lib()
    s = _shape(B, [1000, 130], hq=4, hkv=2, d=128)
    n = ctypes.c_size_t(0)

    def size(counts, n_obs=64, per_kv=0):
        c = np.asarray(counts, np.int32)
        return L.tm_select_vertical(ctypes.byref(s.c), None, None, n_obs,
                                    c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), per_kv, None, None, None,
                                    ctypes.byref(n), None)

    assert size([50, 7]) == B.TM_OK
    align = lambda v: (v + 255) // 256 * 256
    tiles = 16 + 3
    assert n.value == align(align(tiles * 4 * 128 * 4 + 2 * 4 * 128 * 4) + 4 * 3 * 2)
    assert size([1001, 7]) == B.TM_E_POLICY        # more keys than the sequence has
    assert size([-1, 7]) == B.TM_E_POLICY
    assert size([5, 5], n_obs=0) == B.TM_E_POLICY
    assert size([5, 5], n_obs=65) == B.TM_E_POLICY
    assert size([5, 5], per_kv=2) == B.TM_E_POLICY
    assert L.tm_select_vertical(ctypes.byref(s.c), None, None, 64, None, 0, None, None, None, ctypes.byref(n),
                                None) == B.TM_E_ARG


def test_growing_cache_validation(B):
    """Lengths of a growing cache are checked against the capacities before any
    GPU work: tm_decode through tm_dpolicy.lengths, tm_cache_append directly."""
    L = B.lib()
    s = _shape(B, [256, 100], hq=8, hkv=2, d=128)
    n = ctypes.c_size_t(0)
    dp = B.DPolicy(dict(b8=[1] * 2, b4=[2] * 2, sink=1, tail=128), lengths=[200, 100])
    assert L.tm_decode(ctypes.byref(s.c), None, None, None, None, ctypes.byref(dp.c), None, 2, None,
                       ctypes.byref(n), None) == B.TM_OK
    full = ctypes.c_size_t(0)
    dp_full = B.DPolicy(dict(b8=[1] * 2, b4=[2] * 2, sink=1, tail=128))
    assert L.tm_decode(ctypes.byref(s.c), None, None, None, None, ctypes.byref(dp_full.c), None, 2, None,
                       ctypes.byref(full), None) == B.TM_OK
    assert n.value == full.value            # the workspace follows the capacities
    for bad in ([257, 100], [200, 0]):
        dp.set_lengths(bad)
        assert L.tm_decode(ctypes.byref(s.c), None, None, None, None, ctypes.byref(dp.c), None, 2, None,
                           ctypes.byref(n), None) == B.TM_E_SHAPE
    nb = s.nblk()
    kq = _qt(B, 2, 0, nb, False)
    ln = np.array([200, 100], np.int32)
    ptr = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert L.tm_cache_append(ctypes.byref(s.c), None, FAKE, 2, ctypes.byref(kq), None) == B.TM_E_ARG
    assert L.tm_cache_append(ctypes.byref(s.c), ptr(ln), None, 2, ctypes.byref(kq), None) == B.TM_E_ARG
    for bad in ([0, 100], [200, 101]):
        b = np.array(bad, np.int32)
        assert L.tm_cache_append(ctypes.byref(s.c), ptr(b), FAKE, 2, ctypes.byref(kq), None) == B.TM_E_SHAPE
    wrong = _qt(B, 2, 0, nb - 1, False)
    assert L.tm_cache_append(ctypes.byref(s.c), ptr(ln), FAKE, 2, ctypes.byref(wrong), None) == B.TM_E_SHAPE
    vrows_t16 = _qt(B, 2, 0, nb, True)       # rows layout with an fp16 copy is not a valid target
    assert L.tm_cache_append(ctypes.byref(s.c), ptr(ln), FAKE, 2, ctypes.byref(vrows_t16), None) == B.TM_E_ARG


def test_decode_noalloc_rejects_workspace_beyond_its_array(B):
    """A decode whose split-K workspace exceeds the library's 8 MiB scratch
    array is refused with TM_E_SPACE before any HIP call (so this runs
    without a GPU): 4096 sequences x 32 query heads need 4096 * 32 * 130 * 4
    bytes of partials even with one split each."""
    L = B.lib()
    assert L.tm_decode_noalloc_max_workspace() == 8 << 20
    s = _shape(B, [2] * 4096, hq=32, hkv=8, d=128)
    dp = B.DPolicy(dict(b8=[1] * 8, b4=[2] * 8, sink=1, tail=128))
    need = ctypes.c_size_t(0)
    assert L.tm_decode(ctypes.byref(s.c), None, None, None, None, ctypes.byref(dp.c), None, B.TM_F32, None,
                       ctypes.byref(need), None) == B.TM_OK
    assert need.value > 8 << 20
    qt = B.tm_qtensor(FAKE, FAKE, FAKE, FAKE, FAKE, 8, B.TM_COLS, 4096)
    kt = B.tm_qtensor(FAKE, FAKE, FAKE, FAKE, None, 8, B.TM_ROWS, 4096)
    st = L.tm_decode_noalloc(ctypes.byref(s.c), FAKE, ctypes.byref(kt), ctypes.byref(qt), FAKE, ctypes.byref(dp.c),
                             FAKE, B.TM_F32, None)
    assert st == B.TM_E_SPACE
