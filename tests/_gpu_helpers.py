"""Shared plumbing for the GPU parity tests (not a test module).

Inputs come from the seeded generators in ``workloads``; expected values come
from ``oracle`` only.  The HIP path is reached through the C ABI via the
ctypes binding.
"""
import sys

import numpy as np

import workloads as W
from oracle import attention as OA
from oracle import policy as OP
from oracle import quant as OQ

TOL_MAX = 4e-3     # max-abs gate on fp32 outputs against the float64 oracle
TOL_MEAN = 5e-4    # mean-abs gate
# log-sum-exp: the kernel's row sum adds the same fp16-rounded probabilities
# the PV product uses (round to nearest: relative error <= 2^-11 per term), so
# ln(sum) may be off by up to ~2^-11 = 4.9e-4, plus fp32 score/exp2 rounding.
TOL_LSE = 6e-4


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_prefill(w, pol, q, k, v, o_dtype=None, dbg_tiles=None):
    """Run quantize x3 + traversal + prefill on the GPU.  Returns the pipeline,
    the census, O (numpy) and lse (numpy) and the debug capture (or None)."""
    import torch
    import tile_routed_mixed_amd as T
    say(f"[gpu] prefill {w.name} seqlens={w.seqlens[:6]}{'...' if len(w.seqlens) > 6 else ''} "
        f"hq={w.hq} hkv={w.hkv} d={w.d} bq={w.bq} {w.dtype} policy={pol['kind']}")
    p = T.PrefillPipeline(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, pol)
    p.upload(q[0], k[0], v[0])
    p.quantize()
    census = p.traversal(census=True)
    dt = None
    if dbg_tiles is not None:
        dt = torch.from_numpy(np.ascontiguousarray(np.asarray(dbg_tiles, np.int32))).to("cuda:0")
    o, dbg = p.prefill(o_dtype if o_dtype is not None else T.TM_F32, dbg_tiles=dt)
    torch.cuda.synchronize()
    return p, census, o.float().cpu().numpy(), p.lse.cpu().numpy(), (None if dbg is None else dbg.cpu().numpy())


def oracle_prefill(w, pol, q, k, v, rows=None):
    qq = OQ.quantize(q[1], w.seqlens)
    kq = OQ.quantize(k[1], w.seqlens)
    O, lse = OA.prefill(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.bk, pol, q[1].astype(np.float64),
                        k[1].astype(np.float64), v[1].astype(np.float64), qq, kq, rows=rows)
    return O, lse, qq, kq


def compare(o_gpu, o_ref, lse_gpu=None, lse_ref=None, what=""):
    m = ~np.isnan(o_ref)
    err = np.abs(o_gpu[m] - o_ref[m])
    mx, mean = float(err.max()), float(err.mean())
    say(f"[cmp] {what}: max-abs {mx:.3e} mean-abs {mean:.3e} over {err.size} values")
    assert np.all(np.isfinite(o_gpu[m]))
    assert mx <= TOL_MAX, (what, mx)
    assert mean <= TOL_MEAN, (what, mean)
    if lse_gpu is not None:
        ml = ~np.isnan(lse_ref)
        le = float(np.abs(lse_gpu[ml] - lse_ref[ml]).max())
        say(f"[cmp] {what}: lse max-abs {le:.3e}")
        assert le <= TOL_LSE, (what, le)
    return mx, mean


def int_tiles(w, pol, limit=None, seed=0):
    """Executed integer tiles (seq, head, qtile, ktile, prec) of a policy, a
    deterministic sample of at most `limit` (always with the first/last)."""
    gs = OP.grids(w.seqlens, w.hq, w.bq, w.bk, pol)
    parts = []
    for s, g in enumerate(gs):
        h, i, j = np.nonzero((g == OP.INT8) | (g == OP.INT4))
        parts.append(np.stack([np.full_like(h, s), h, i, j, g[h, i, j].astype(h.dtype)], axis=1))
    ex = np.concatenate(parts, axis=0) if parts else np.zeros((0, 5), np.int64)
    n = len(ex)
    if limit is None or n <= limit:
        pick = range(n)
    else:
        rng = np.random.default_rng(seed)
        pick = sorted(set([0, n - 1]) | set(rng.choice(n, size=limit - 2, replace=False).tolist()))
    return [tuple(int(x) for x in ex[p]) for p in pick]


def check_int_scores(w, tiles, dbg, qq, kq):
    grp = w.hq // w.hkv
    for n, (s, h, i, j, prec) in enumerate(tiles):
        ref = OA.int_tile_scores(qq, kq, s, h, h // grp, i, j, w.bq, w.bk, prec, w.seqlens)
        got = dbg[n]
        assert np.array_equal(got.astype(np.int64), ref), ((s, h, i, j, prec),
                                                           int(np.abs(got - ref).max()))
