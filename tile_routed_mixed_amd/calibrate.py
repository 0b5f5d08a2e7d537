"""Per-head boundary calibration and the budgeted allocator.

[TriAttention] "TriAttention: Unified Sparse Mixed-Precision Attention for
Long-Context LLM Inference", abstract: each head's two diagonal-distance
boundaries are picked offline from the normalized output error of candidate
boundary pairs and the measured execution cost of complete tiles, with a
model-wide allocator that spends a shared compute budget where it lowers the
error most.

This module is that mechanism on the library's own kernels:
  * ``tile_costs``: time of one executed tile per precision on this GPU
    (prefill launches under all-INT8 and all-INT4 boundary policies and an
    all-FP16 bitmask policy, divided by their executed tiles);
  * ``head_errors``: for every candidate (b8, b4), the normalized error of
    each head's output against the all-FP16, nothing-skipped prefill (the
    pages project through the layer's output matrix; without model weights
    the projection is the identity);
  * ``head_costs``: each candidate's executed tiles per head (from the
    traversal census) priced with the tile costs;
  * ``allocate``: exact multiple-choice knapsack over integer cost units:
    one candidate per head, least total error within the budget.
Everything that computes attention runs in libtm.so; this file only drives
it and does host bookkeeping.
"""
from __future__ import annotations

import numpy as np

from . import _binding as B
from .pipeline import PrefillPipeline


def _ceil(a, b):
    return -(-int(a) // int(b))


def _bitmask_words(seqlens, hq, bq, bk, group):
    """Words of a bitmask policy for this shape: one row of
    ceil(ceil(nk / group) / 32) words per (sequence, query head, query tile)."""
    return sum(hq * _ceil(S, bq) * _ceil(_ceil(S, bk), group * 32) for S in seqlens)


class _Runner:
    """One set of uploaded, quantized inputs, run under successive policies."""

    def __init__(self, seqlens, hq, hkv, d, bq, dtype, bits, policy):
        self.pp = PrefillPipeline(seqlens, hq, hkv, d, bq, dtype, policy)
        self.pp.upload(*bits)
        self.pp.quantize()

    def run(self, policy, steps=0):
        """Prefill under `policy`; returns (output copy [T][hq][d] f32, census,
        mean ms of `steps` further launches or None)."""
        import torch
        pp = self.pp
        pp.set_policy(policy)
        census = pp.traversal(census=True)
        o = pp.prefill(B.TM_F32)[0].clone()
        ms = None
        if steps:
            pp.prefill(B.TM_F32)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                pp.prefill(B.TM_F32)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
        return o, census, ms


def all_fp16_policy(seqlens, hq, bq=128, bk=64, group=4):
    words = _bitmask_words(seqlens, hq, bq, bk, group)
    return dict(kind=B.TM_POLICY_BITMASK, group=group, words=np.full(words, 0xFFFFFFFF, np.uint32))


def _boundaries(hq, b8, b4, sink=0):
    return dict(kind=B.TM_POLICY_BOUNDARIES, b8=[b8] * hq, b4=[b4] * hq, sink=sink)


NEVER = 1 << 30   # a boundary no diagonal distance reaches


def tile_costs(seqlens, hq, hkv, d, bq, dtype, bits, steps=10, runner=None):
    """Nanoseconds of prefill per executed complete tile (bq x 64), for INT8,
    INT4 and FP16 tiles: each is the mean time of one prefill launch whose
    every legal tile has that precision, divided by the tiles it executed.
    `bits`: (q, k, v) 16-bit patterns [T][heads][d]."""
    r = runner or _Runner(seqlens, hq, hkv, d, bq, dtype, bits, _boundaries(hq, NEVER, NEVER))
    out = {}
    for prec, key, pol in ((B.TM_INT8, "int8", _boundaries(hq, NEVER, NEVER)),
                           (B.TM_INT4, "int4", _boundaries(hq, 0, NEVER)),
                           (B.TM_FP16, "fp16", all_fp16_policy(seqlens, hq, bq))):
        _, census, ms = r.run(pol, steps=steps)
        if census[key] != census["legal"]:
            raise RuntimeError(f"cost run for {key} executed {census[key]} of {census['legal']} legal tiles")
        out[prec] = ms * 1e6 / max(census[key], 1)
    return out


def head_errors(seqlens, hq, hkv, d, bq, dtype, bits, candidates, sink=0, runner=None):
    """err[h][c] = ||O_h(c) - O_h(ref)||_F / ||O_h(ref)||_F over all tokens of
    head h, where ref routes every legal tile to FP16 and c = (b8, b4) is
    applied to every head at once (heads do not interact).  Also returns the
    tile census of each candidate, per head."""
    r = runner or _Runner(seqlens, hq, hkv, d, bq, dtype, bits, _boundaries(hq, NEVER, NEVER))
    # outputs come back to the host; the norms are host arithmetic (float64)
    ref = r.run(all_fp16_policy(seqlens, hq, bq))[0].cpu().numpy().astype(np.float64)
    norm = np.sqrt(np.einsum("thd,thd->h", ref, ref))
    err = np.zeros((hq, len(candidates)))
    census = []
    for c, (b8, b4) in enumerate(candidates):
        o, cen, _ = r.run(_boundaries(hq, b8, b4, sink))
        diff = o.cpu().numpy().astype(np.float64) - ref
        err[:, c] = np.sqrt(np.einsum("thd,thd->h", diff, diff)) / norm
        census.append(dict(int8=cen["int8"] // hq, int4=cen["int4"] // hq, skip=cen["skip"] // hq))
        del o, diff
    return err, census


def default_candidates(max_len, bk=64):
    """Boundary pairs (b8, b4) in key-tile units: b8 from a doubling ladder,
    b4 >= b8 from the same ladder, plus "never" (2**30) for either; the pair
    (never, never) is the all-INT8 policy."""
    never = NEVER
    nk = _ceil(max_len, bk)
    ladder = [0]
    v = 1
    while v < nk:
        ladder.append(v)
        v *= 2
    ladder.append(never)
    return [(b8, b4) for b8 in ladder for b4 in ladder if b4 >= b8 and b4 > 0]


def head_costs(census, costs, hq):
    """cost[h][c] in nanoseconds: candidate c's INT8 and INT4 tiles priced
    with the measured tile costs (skipped tiles cost nothing)."""
    per = np.array([c["int8"] * costs[B.TM_INT8] + c["int4"] * costs[B.TM_INT4] for c in census], dtype=np.float64)
    return np.tile(per, (hq, 1))


def allocate(err, cost, budget):
    """Exact multiple-choice knapsack: one candidate per head, minimizing
    sum_h err[h][c_h] subject to sum_h cost[h][c_h] <= budget, with integer
    costs >= 0 (dynamic program over the budget spent so far, O(H C budget)).
    Ties go to the first candidate reached.  Returns the choice per head
    [H] (int64), or None when the cheapest candidates already exceed the
    budget."""
    err = np.asarray(err, dtype=np.float64)
    cost = np.asarray(cost, dtype=np.int64)
    if err.ndim != 2 or err.shape != cost.shape or err.shape[1] == 0:
        raise ValueError("err and cost must be [heads][candidates] of the same shape")
    if (cost < 0).any():
        raise ValueError("costs must be non-negative integers")
    H, C = err.shape
    budget = int(budget)
    if budget < 0 or int(cost.min(axis=1).sum()) > budget:
        return None
    best = np.full(budget + 1, np.inf)    # best[b]: least error of the heads so far spending exactly b
    best[0] = 0.0
    pick = np.zeros((H, budget + 1), dtype=np.int64)
    for h in range(H):
        new = np.full(budget + 1, np.inf)
        for c in range(C):
            k = int(cost[h, c])
            if k > budget:
                continue
            cand = np.full(budget + 1, np.inf)
            cand[k:] = best[:budget + 1 - k] + err[h, c]
            better = cand < new
            new[better] = cand[better]
            pick[h, better] = c
        best = new
    b = int(np.argmin(best))
    choice = np.zeros(H, dtype=np.int64)
    for h in range(H - 1, -1, -1):
        choice[h] = pick[h, b]
        b -= int(cost[h, choice[h]])
    return choice


def calibrate(seqlens, hq, hkv, d, bq, dtype, bits, candidates, budget_frac, sink=0, resolution=20000,
              costs=None):
    """Per-head (b8, b4) minimizing the summed normalized error while the
    priced tiles stay within `budget_frac` of the all-INT8 prefill (every
    legal tile at INT8).  Costs are quantized to `resolution` units of that
    full cost before the allocator runs.  Returns (boundary policy dict,
    report dict)."""
    r = _Runner(seqlens, hq, hkv, d, bq, dtype, bits, _boundaries(hq, NEVER, NEVER))
    if costs is None:
        costs = tile_costs(seqlens, hq, hkv, d, bq, dtype, bits, runner=r)
    err, cen = head_errors(seqlens, hq, hkv, d, bq, dtype, bits, candidates, sink, runner=r)
    cost_ns = head_costs(cen, costs, hq)
    legal = cen[0]["int8"] + cen[0]["int4"] + cen[0]["skip"]
    full_ns = hq * legal * costs[B.TM_INT8]
    unit = full_ns / resolution
    units = np.ceil(cost_ns / unit - 1e-9).astype(np.int64)
    budget = int(np.floor(budget_frac * resolution + 1e-9))
    choice = allocate(err, units, budget)
    if choice is None:
        raise ValueError(f"budget {budget_frac} of the all-INT8 cost is below the cheapest candidates")
    rows = np.arange(hq)
    report = dict(costs_ns_per_tile={"int8": costs[B.TM_INT8], "int4": costs[B.TM_INT4], "fp16": costs[B.TM_FP16]},
                  candidates=list(candidates), errors=err, census=cen, cost_ns=cost_ns, choice=choice,
                  full_int8_ns=full_ns, budget_ns=budget_frac * full_ns,
                  spent_ns=float(cost_ns[rows, choice].sum()), total_error=float(err[rows, choice].sum()))
    pol = dict(kind=B.TM_POLICY_BOUNDARIES, b8=[int(candidates[c][0]) for c in choice],
               b4=[int(candidates[c][1]) for c in choice], sink=sink)
    return pol, report


def _main():
    import argparse
    import json
    import sys
    import os
    ap = argparse.ArgumentParser(description="Measure tile costs and calibrate per-head boundaries on a "
                                             "seeded synthetic workload.")
    ap.add_argument("--workload", default="gqa8k")
    ap.add_argument("--budget", type=float, default=0.5, help="fraction of the all-INT8 prefill cost")
    ap.add_argument("--costs-only", action="store_true")
    args = ap.parse_args()
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import workloads as W
    w = W.get(args.workload)
    q, k, v = W.make_qkv(w)
    bits = (q[0], k[0], v[0])   # 16-bit patterns
    costs = tile_costs(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, bits)
    line = {"workload": args.workload, "ns_per_tile": {"int8": costs[B.TM_INT8], "int4": costs[B.TM_INT4],
                                                        "fp16": costs[B.TM_FP16]}}
    if not args.costs_only:
        cands = default_candidates(max(w.seqlens))
        pol, rep = calibrate(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, bits, cands, args.budget,
                             sink=int(w.sink), costs=costs)
        line.update(budget=args.budget, b8=pol["b8"], b4=pol["b4"], spent_frac=rep["spent_ns"] / rep["full_int8_ns"],
                    mean_error=rep["total_error"] / w.hq)
    print(json.dumps(line))


if __name__ == "__main__":
    _main()
