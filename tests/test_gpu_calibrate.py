"""GPU: boundary calibration on a small seeded workload.

The tile costs come from timed prefill launches, the per-head errors from
prefill outputs under each candidate; both run in the HIP library.  Checks:
the costs are sane, the allocator's choice stays within the budget, the
calibrated policy reproduces the error table when it is run, the error table
agrees with the same errors computed from oracle outputs, and the budget
extremes behave as the allocator's definition says.
"""
import numpy as np
import pytest

import workloads as W
from tile_routed_mixed_amd import calibrate as C

from _gpu_helpers import oracle_prefill, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def calib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    w = W.small("gqa8k", [700, 300], hq=4, hkv=2)
    q, k, v = W.make_qkv(w)
    bits = (q[0], k[0], v[0])
    cands = C.default_candidates(max(w.seqlens))
    say(f"[gpu] calibrate seqlens={w.seqlens} hq={w.hq} hkv={w.hkv} candidates={len(cands)}")
    pol, rep = C.calibrate(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, bits, cands, 0.5)
    return w, (q, k, v), cands, pol, rep


def test_tile_costs_are_sane(calib):
    _, _, _, _, rep = calib
    c = rep["costs_ns_per_tile"]
    say(f"[calib] ns per tile {c}")
    for key in ("int8", "int4", "fp16"):
        assert np.isfinite(c[key]) and 0.0 < c[key] < 1e6


def test_choice_within_budget(calib):
    w, _, cands, pol, rep = calib
    assert rep["spent_ns"] <= rep["budget_ns"]
    assert len(pol["b8"]) == w.hq and all(0 <= a <= b for a, b in zip(pol["b8"], pol["b4"]))
    rows = np.arange(w.hq)
    assert abs(rep["total_error"] - rep["errors"][rows, rep["choice"]].sum()) < 1e-12
    say(f"[calib] b8={pol['b8']} b4={pol['b4']} spent {rep['spent_ns'] / rep['full_int8_ns']:.3f} "
        f"of all-INT8, mean error {rep['total_error'] / w.hq:.4f}")


def test_calibrated_policy_reproduces_error_table(calib):
    w, (q, k, v), _, pol, rep = calib
    r = C._Runner(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, (q[0], k[0], v[0]), pol)
    ref = r.run(C.all_fp16_policy(w.seqlens, w.hq, w.bq))[0].double()
    o = r.run(pol)[0].double()
    e = ((o - ref).pow(2).sum(dim=(0, 2)).sqrt() / ref.pow(2).sum(dim=(0, 2)).sqrt()).cpu().numpy()
    want = rep["errors"][np.arange(w.hq), rep["choice"]]
    assert np.allclose(e, want, rtol=1e-10, atol=1e-12), (e, want)


def test_error_table_matches_oracle(calib):
    """Each head's error from oracle outputs and from GPU outputs may differ by
    no more than the GPU-vs-oracle output differences allow (triangle
    inequality), and those outputs pass the usual parity gates."""
    from _gpu_helpers import compare
    w, (q, k, v), cands, _, rep = calib
    fp16 = C.all_fp16_policy(w.seqlens, w.hq, w.bq)
    r = C._Runner(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, (q[0], k[0], v[0]), fp16)
    G_ref = r.run(fp16)[0].double().cpu().numpy()
    O_ref, _, _, _ = oracle_prefill(w, fp16, q, k, v)
    compare(G_ref, O_ref, what="calibration reference (all FP16)")
    n_or = np.sqrt((O_ref ** 2).sum(axis=(0, 2)))
    n_gpu = np.sqrt((G_ref ** 2).sum(axis=(0, 2)))
    d_ref = np.sqrt(((G_ref - O_ref) ** 2).sum(axis=(0, 2)))
    for c in (cands.index((C.NEVER, C.NEVER)), cands.index((0, C.NEVER)), cands.index((1, 2)),
              cands.index((0, 1))):
        b8, b4 = cands[c]
        pol = dict(kind=0, b8=[b8] * w.hq, b4=[b4] * w.hq, sink=0)
        O, _, _, _ = oracle_prefill(w, pol, q, k, v)
        G = r.run(pol)[0].double().cpu().numpy()
        compare(G, O, what=f"candidate ({b8}, {b4})")
        e_or = np.sqrt(((O - O_ref) ** 2).sum(axis=(0, 2))) / n_or
        d_c = np.sqrt(((G - O) ** 2).sum(axis=(0, 2)))
        bound = (d_c + d_ref) / n_gpu + e_or * np.abs(n_or / n_gpu - 1.0) + 1e-6
        gap = np.abs(rep["errors"][:, c] - e_or)
        say(f"[calib] ({b8}, {b4}) oracle {np.round(e_or, 5)} gpu {np.round(rep['errors'][:, c], 5)} "
            f"gap {gap.max():.2e} bound {bound.min():.2e}")
        assert np.all(gap <= bound), (gap, bound)


def test_error_and_cost_order(calib):
    w, _, cands, _, rep = calib
    full, narrow = cands.index((C.NEVER, C.NEVER)), cands.index((0, 1))
    assert np.all(rep["errors"][:, full] < rep["errors"][:, narrow])
    assert np.all(rep["cost_ns"][:, full] > rep["cost_ns"][:, narrow])
    # the census of the all-INT8 candidate covers every legal tile
    cen = rep["census"][full]
    assert cen["int4"] == 0 and cen["skip"] == 0 and cen["int8"] > 0


def test_budget_extremes(calib):
    w, _, _, _, rep = calib
    err, cost = rep["errors"], np.ceil(rep["cost_ns"]).astype(np.int64)
    roomy = C.allocate(err, cost, int(cost.max(axis=1).sum()))
    assert np.array_equal(roomy, err.argmin(axis=1))
    assert C.allocate(err, cost, int(cost.min(axis=1).sum()) - 1) is None
