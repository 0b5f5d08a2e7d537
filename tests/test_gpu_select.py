"""GPU: vertical-line token selection (tm_select_vertical) against the oracle.

The attention mass of every key (fp32 on the GPU, float64 in the oracle) must
agree within 1e-5 + 1e-4 x mass; the selected lists must be valid top-k sets
of the oracle's masses (where masses sit within that tolerance of the k-th
largest, either choice is correct): ascending, unique, no unselected key
clearly above the k-th largest and no selected key clearly below it.  The
lists then drive a hybrid prefill, checked against the oracle on the same
lists.
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import policy as OP

from _gpu_helpers import Guards, assert_all_written, compare, oracle_prefill, run_prefill, say

pytestmark = pytest.mark.gpu


def _run(w, n_obs, counts, per_kv):
    import torch
    import tile_routed_mixed_amd as T
    q, k, v = W.make_qkv(w)
    shape = T.Shape(w.seqlens, w.hq, w.hkv, w.d, w.bq, 64, T.TM_BF16 if w.dtype == "bf16" else T.TM_F16,
                    device="cuda:0")
    dq = torch.from_numpy(q[0].view(np.int16).copy()).to("cuda:0")
    dk = torch.from_numpy(k[0].view(np.int16).copy()).to("cuda:0")
    say(f"[gpu] select seqlens={w.seqlens} hq={w.hq} hkv={w.hkv} d={w.d} n_obs={n_obs} counts={counts} per_kv={per_kv}")
    g = Guards()
    nl = w.hkv if per_kv else w.hq
    total = nl * int(np.sum(counts))
    mass_out = g.alloc((w.hq, shape.T), torch.float32, float("nan"))
    sel_out = g.alloc((max(total, 1),), torch.int32, -1)
    mass, off, idx = T.tm_select_vertical(shape, dq, dk, n_obs, counts, per_kv, mass_out=mass_out, sel_out=sel_out)
    torch.cuda.synchronize()
    g.check()
    assert_all_written(mass, "key masses")
    return (q, k, v), mass.cpu().numpy(), off, idx


def _check(w, qkv, mass, off, idx, n_obs, counts, per_kv):
    q, k, _ = qkv
    tau = 1 / math.sqrt(w.d)
    cu = w.cu_seqlens
    grp = w.hq // w.hkv
    nl = w.hkv if per_kv else w.hq
    for s, S in enumerate(w.seqlens):
        imps = []
        for h in range(w.hq):
            ref = OP.vline_importance(q[1][cu[s]:cu[s + 1], h].astype(np.float64),
                                      k[1][cu[s]:cu[s + 1], h // grp].astype(np.float64), n_obs, tau)
            got = mass[h, cu[s]:cu[s + 1]]
            assert np.all(np.abs(got - ref) <= 1e-5 + 1e-4 * ref), (s, h, float(np.abs(got - ref).max()))
            imps.append(ref)
        for g in range(nl):
            ref = sum(imps[g * grp:(g + 1) * grp]) if per_kv else imps[g]
            r = s * nl + g
            sel = idx[off[r]:off[r + 1]]
            kk = counts[s]
            assert len(sel) == kk
            if kk == 0:
                continue
            assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] < S
            kth = np.sort(ref)[::-1][kk - 1]
            tol = 1e-5 * (grp if per_kv else 1) + 1e-4 * kth
            chosen = np.zeros(S, bool)
            chosen[sel] = True
            assert np.all(ref[chosen] >= kth - tol), (s, g)
            assert np.all(ref[~chosen] <= kth + tol), (s, g)


@pytest.mark.parametrize("name,seqlens,kw,n_obs,frac,per_kv", [
    ("gqa8k", [1000, 30, 2100], dict(hq=4, hkv=2), 64, 0.05, False),
    ("gqa8k", [1000, 30, 2100], dict(hq=4, hkv=2), 64, 0.05, True),
    ("long128k", [700, 64], dict(hq=2, hkv=1, d=64), 17, 0.2, False),
    ("varlen32k", [129, 1], dict(hq=2, hkv=2), 64, 1.0, False),
    # more sequences than the kernel arguments carry: the table is staged
    ("varlen32k", [1 + (37 * i) % 150 for i in range(70)], dict(hq=2, hkv=1), 16, 0.1, True),
    # 8 query heads per KV head: two workgroups of 4 heads share its keys
    ("gqa8k", [300, 2000, 77], dict(hq=8, hkv=1), 64, 0.05, False),
    # 3 query heads per KV head: one head per workgroup, lists summed over 3
    ("gqa8k", [500, 1300], dict(hq=3, hkv=1), 33, 0.1, True),
    # a sequence long enough for several key tiles per workgroup, and a list
    # longer than the top-k holds in registers
    ("long128k", [70000], dict(hq=4, hkv=1, d=64), 64, 0.02, False),
])
def test_vertical_selection(name, seqlens, kw, n_obs, frac, per_kv):
    w = W.small(name, seqlens, **kw)
    counts = [int(round(frac * S)) for S in seqlens]
    qkv, mass, off, idx = _run(w, n_obs, counts, per_kv)
    _check(w, qkv, mass, off, idx, n_obs, counts, per_kv)


def test_selection_on_locality_inputs_drives_hybrid_prefill():
    """On inputs with a position signal the selected keys differ by head;
    the lists feed the hybrid prefill, which matches the oracle on them."""
    w = W.small("local8k", [1500, 600], hq=4, hkv=2)
    counts = [int(round(0.05 * S)) for S in w.seqlens]
    qkv, mass, off, idx = _run(w, 64, counts, False)
    _check(w, qkv, mass, off, idx, 64, counts, False)
    pol = dict(kind=3, window=128, sel_off=off, sel_idx=idx)
    q, k, v = qkv
    _, _, o, lse, _ = run_prefill(w, pol, q, k, v)
    O, L, _, _ = oracle_prefill(w, pol, q, k, v)
    compare(o, O, lse, L, what="hybrid prefill on selected keys")


def test_vertical_selection_full_size():
    """The 8K x 32-head workload in the configuration the bench's hybrid line
    times (64 probe rows, 5 % of the keys per query head): every key's mass
    and every list against the oracle."""
    w = W.get("gqa8k")
    counts = [int(round(0.05 * S)) for S in w.seqlens]
    qkv, mass, off, idx = _run(w, 64, counts, False)
    _check(w, qkv, mass, off, idx, 64, counts, False)


def test_pipeline_selection_buffers_follow_the_sizes():
    """The pipeline keeps the selection buffers between calls: calls with
    other counts (other buffer sizes) and back give the same lists as calls
    on fresh buffers."""
    import tile_routed_mixed_amd as T
    w = W.small("local8k", [700, 300], hq=4, hkv=2)
    q, k, v = W.make_qkv(w)
    pp = T.PrefillPipeline(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, W.make_policy(w))
    pp.upload(q[0], k[0], v[0])
    say("[gpu] pipeline selection buffer reuse")
    got = [pp.vertical_policy(f, 64) for f in (0.05, 0.2, 0.05)]
    for f, pol in zip((0.05, 0.2, 0.05), got):
        counts = [int(round(f * S)) for S in w.seqlens]
        _, off, idx = T.tm_select_vertical(pp.shape, pp.q, pp.k, 64, counts, False)
        assert np.array_equal(pol["sel_off"], off) and np.array_equal(pol["sel_idx"], idx), f


def test_selection_ties_go_to_lower_positions():
    """Zero keys: every probe row spreads its attention evenly, so all keys up
    to the first probe row receive exactly the same mass (each the same sum
    of the same terms) and the later ones less; the lists must be the first
    counts[s] positions."""
    import torch
    import tile_routed_mixed_amd as T
    w = W.small("gqa8k", [900, 200], hq=4, hkv=1)
    q, _, _ = W.make_qkv(w)
    shape = T.Shape(w.seqlens, w.hq, w.hkv, w.d, w.bq, 64, T.TM_BF16 if w.dtype == "bf16" else T.TM_F16,
                    device="cuda:0")
    dq = torch.from_numpy(q[0].view(np.int16).copy()).to("cuda:0")
    dk = torch.zeros((shape.T, w.hkv, w.d), dtype=torch.int16, device="cuda:0")
    counts = [100, 20]
    say("[gpu] selection ties on zero keys")
    for per_kv in (False, True):
        _, off, idx = T.tm_select_vertical(shape, dq, dk, 64, counts, per_kv)
        nl = w.hkv if per_kv else w.hq
        for s, c in enumerate(counts):
            for g in range(nl):
                r = s * nl + g
                assert np.array_equal(idx[off[r]:off[r + 1]], np.arange(c)), (per_kv, s, g)
