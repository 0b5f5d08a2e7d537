"""GPU: hybrid and decode selection lists held in device memory.

tm_build_traversal (hybrid) and tm_decode_select accept the selected-key lists
in device memory (sel_idx_dev / sel_off_dev) and then build their tables with
a kernel instead of staging them from the host.  Both routes must give the
same tables, the same gathered tiles and bit-identical outputs; the host
route is the one the oracle parity tests cover.
"""
import numpy as np
import pytest

import workloads as W
from oracle import policy as OP

from _gpu_helpers import assert_all_written, compare, guard_decode, guard_prefill, oracle_prefill, say
from test_gpu_parity import HYBRID_CASES, _hyb_case, _with_sel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import tile_routed_mixed_amd as T
    T.lib()


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).to("cuda:0")


def _regions(w, trav):
    """The hybrid parts of a traversal buffer (host copy): items, runs, list
    table, positions, column masks, gathered-tile headers (entry and
    positions) and the gathered K rows and V^T."""
    import tile_routed_mixed_amd as T
    b = trav.view(np.uint8)
    tr = T.read_traversal(b)
    h = b[:256].view(np.uint32)
    n_gt, tab, idx, cm, gh, gk, gv = (int(x) for x in h[17:24])
    nr = len(w.seqlens) * w.hq
    te = b[tab:tab + 16 * nr].view(np.uint32).reshape(nr, 4)
    n_sel = int(te[:, 1].astype(np.int64).sum())
    n_cm = sum(w.hq * -(-S // 64) for S in w.seqlens)
    return dict(items=tr["items"], runs=tr["runs"], census=np.array(list(tr["census"].values())), tab=te,
                idx=b[idx:idx + 4 * n_sel], cm=b[cm:cm + 8 * n_cm],
                gh=b[gh:gh + 512 * n_gt].reshape(n_gt, 512)[:, :16 + 4 * 64],
                gk=b[gk:gk + n_gt * 64 * w.d * 2], gv=b[gv:gv + n_gt * 64 * w.d * 2])


def _run(w, pol, q, k, v):
    import torch
    import tile_routed_mixed_amd as T
    p = T.PrefillPipeline(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, pol)
    p.upload(q[0], k[0], v[0])
    g = guard_prefill(p, T.TM_F32)
    p.trav.fill_(0xA5)   # every byte the tables leave alone reads the same in both runs
    p.quantize()
    census = p.traversal(census=True)
    o, _ = p.prefill(T.TM_F32)
    torch.cuda.synchronize()
    g.check()
    assert_all_written(o, "O")
    return census, p.trav.cpu().numpy(), o.cpu().numpy(), p.lse.cpu().numpy()


@pytest.mark.parametrize("case", list(HYBRID_CASES))
def test_hybrid_device_lists_match_host_lists(case):
    """The same lists from the host and from device memory: equal census,
    items, runs, tables and gathered tiles, bit-identical O and lse."""
    w, pol = _hyb_case(case)
    q, k, v = W.make_qkv(w)
    say(f"[gpu] hybrid {case}: host lists vs device lists")
    c1, t1, o1, l1 = _run(w, pol, q, k, v)
    dpol = dict(kind=3, window=pol["window"], sel_off=pol["sel_off"], sel_idx_dev=_dev(pol["sel_idx"]))
    c2, t2, o2, l2 = _run(w, dpol, q, k, v)
    assert c1 == c2
    r1, r2 = _regions(w, t1), _regions(w, t2)
    for key in r1:
        assert np.array_equal(np.asarray(r1[key]), np.asarray(r2[key])), (case, key)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_hybrid_device_lists_out_of_range_tail():
    """Device lists are not checked on the host: positions at or past the
    sequence end become empty slots.  Lists whose valid prefix is followed by
    such positions give the outputs of the valid prefix alone, bit for bit,
    and the oracle's on those lists."""
    w = W.small("gqa8k", [700, 300], hq=4, hkv=2)
    q, k, v = W.make_qkv(w)
    rng = np.random.default_rng(5)
    lists, bad = [], []
    for s, S in enumerate(w.seqlens):
        for h in range(w.hq):
            good = np.sort(rng.choice(S, size=40 + 10 * h, replace=False)).astype(np.int32)
            tail = np.array([S, S + 3, 1 << 30][: 1 + (h % 3)], np.int32)
            lists.append(good)
            bad.append(np.concatenate([good, tail]))
    off = lambda ls: np.concatenate([[0], np.cumsum([len(x) for x in ls])]).astype(np.int32)
    pol = dict(kind=3, window=64, sel_off=off(lists), sel_idx=np.concatenate(lists))
    say("[gpu] hybrid device lists with out-of-range tails")
    _, _, o1, l1 = _run(w, pol, q, k, v)
    dpol = dict(kind=3, window=64, sel_off=off(bad), sel_idx_dev=_dev(np.concatenate(bad)))
    _, _, o2, l2 = _run(w, dpol, q, k, v)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    O, L, _, _ = oracle_prefill(w, pol, q, k, v)
    compare(o2, O, l2, L, what="device lists, valid prefix")


def test_pipeline_selection_on_device_equals_host_route():
    """vertical_policy(on_device=True) keeps the selection pass's output in
    device memory; the prefill on it equals the one on the host copy."""
    import torch
    import tile_routed_mixed_amd as T
    w = W.small("local8k", [900, 333], hq=4, hkv=2)
    q, k, v = W.make_qkv(w)
    pp = T.PrefillPipeline(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, W.make_policy(w))
    pp.upload(q[0], k[0], v[0])
    pp.quantize()
    say("[gpu] vertical selection on device vs host")
    outs = []
    for dev in (False, True):
        pol = pp.vertical_policy(0.1, 64, on_device=dev)
        pp.set_policy(pol)
        pp.traversal()
        o, _ = pp.prefill(T.TM_F32)
        torch.cuda.synchronize()
        outs.append((o.cpu().numpy().copy(), pp.lse.cpu().numpy().copy()))
        if dev:
            n = int(pol["sel_off"][-1])
            assert np.array_equal(pol["sel_idx_dev"][:n].cpu().numpy(), host_idx)
        else:
            host_idx = pol["sel_idx"]
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("seqlens,dpol,frac", [
    ([1, 100, 1000, 2000], dict(b8=[2, 3], b4=[5, 9], sink=1, tail=128), 0.1),
    ([3000, 777], dict(b8=[4, 4], b4=[8, 8], sink=0, tail=64), 0.05),
])
def test_decode_device_lists_match_host_lists(seqlens, dpol, frac):
    """tm_decode_select with the lists in device memory: same tables and
    gathered tiles as with host lists, bit-identical decode outputs."""
    import torch
    import tile_routed_mixed_amd as T
    hq, hkv, d = 8, 2, 128
    w = W.small("decode16x32k", seqlens, hq=hq, hkv=hkv, d=d)
    _, k, v = W.make_qkv(w)
    dq = W.make_decode_query(w)
    sel = W.make_decode_selection(w, frac)
    say(f"[gpu] decode {seqlens}: selection lists on host vs device")
    res = []
    for dev in (False, True):
        p = T.DecodePipeline(w.seqlens, hq, hkv, d, dpol, dtype=w.dtype)
        p.upload(dq[0], k[0], v[0])
        g = guard_decode(p)
        p.build_cache()
        n = T._binding.decode_sel_bytes(p.shape, _with_sel(p.dpol, sel))
        p.sel_buf = g.alloc((max(256, n),), torch.uint8, 0xA5, role="sel")
        p.select(sel[0], _dev(sel[1]) if dev else sel[1])
        o = p.decode()
        torch.cuda.synchronize()
        g.check()
        assert_all_written(o, "decode O")
        res.append((o.cpu().numpy(), p.sel_buf.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0])
    # list table, column masks, headers and gathered tiles (the host route
    # zero-fills the alignment gaps and header padding the kernel leaves alone)
    nl = len(seqlens) * hkv
    a, b = res[0][1], res[1][1]
    up = lambda x: (x + 255) // 256 * 256
    nblk = sum(-(-S // 64) for S in seqlens)
    counts = np.diff(sel[0])
    n_gt = int(sum(-(-int(c) // 64) for c in counts))
    cm0 = up(8 * nl)
    gh0 = up(cm0 + 8 * nblk * hkv)
    gk0 = up(gh0 + 512 * n_gt)
    gv0 = up(gk0 + n_gt * 64 * d * 2)
    for lo, hi in ((0, 8 * nl), (cm0, cm0 + 8 * nblk * hkv), (gk0, gk0 + n_gt * 64 * d * 2),
                   (gv0, gv0 + n_gt * 64 * d * 2)):
        assert np.array_equal(a[lo:hi], b[lo:hi]), (lo, hi)
    ha = a[gh0:gh0 + 512 * n_gt].reshape(max(n_gt, 0), 512)[:, :16 + 4 * 64]
    hb = b[gh0:gh0 + 512 * n_gt].reshape(max(n_gt, 0), 512)[:, :16 + 4 * 64]
    assert np.array_equal(ha, hb)


@pytest.mark.parametrize("case", list(HYBRID_CASES))
@pytest.mark.parametrize("device", [False, True])
def test_build_and_gather_in_one_launch_equals_two_calls(case, device):
    """tm_build_traversal_gather leaves the traversal buffer byte for byte as
    tm_build_traversal followed by tm_gather_selected does."""
    import torch
    import tile_routed_mixed_amd as T
    w, pol = _hyb_case(case)
    if device:
        pol = dict(kind=3, window=pol["window"], sel_off=pol["sel_off"], sel_idx_dev=_dev(pol["sel_idx"]))
    q, k, v = W.make_qkv(w)
    say(f"[gpu] hybrid {case}: build + gather in one launch vs two calls (device lists: {device})")
    p = T.PrefillPipeline(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, pol)
    p.upload(q[0], k[0], v[0])
    bufs = []
    for fused in (False, True):
        p.trav.fill_(0xA5)
        c = p.traversal(census=True, fused=fused)
        torch.cuda.synchronize()
        bufs.append((c, p.trav.cpu().numpy().copy()))
    assert bufs[0][0] == bufs[1][0]
    assert np.array_equal(bufs[0][1], bufs[1][1])
