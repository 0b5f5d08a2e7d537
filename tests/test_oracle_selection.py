"""Pins for the oracle's vertical-line selection signal.

* every probe row's probabilities sum to one, so the importances sum to the
  number of probe rows, and a key no probe row sees has importance zero;
* a hand-made case: two keys whose vectors align with every query take
  nearly all of the mass and are the top 2;
* the vectorized importance equals a plain loop over (row, key);
* top-k breaks ties toward the lower position and returns ascending
  positions.
"""
import math

import numpy as np

from oracle import policy as P


def test_mass_and_visibility():
    rng = np.random.default_rng(0)
    S, d, n = 300, 16, 40
    q, k = rng.standard_normal((S, d)), rng.standard_normal((S, d))
    imp = P.vline_importance(q, k, n, 1 / math.sqrt(d))
    assert abs(imp.sum() - n) < 1e-9
    assert np.all(imp >= 0)
    # the short sequence: fewer rows than the probe
    imp2 = P.vline_importance(q[:10], k[:10], n, 0.25)
    assert abs(imp2.sum() - 10) < 1e-9


def test_two_vertical_lines():
    S, d = 200, 8
    q = np.zeros((S, d))
    q[:, 0] = 1.0
    k = np.zeros((S, d))
    k[[17, 90], 0] = 30.0                 # keys 17 and 90 dominate every row that sees them
    imp = P.vline_importance(q, k, 32, 1.0)
    assert P.top_k_positions(imp, 2).tolist() == [17, 90]
    assert imp[17] > 15 and imp[90] > 15   # about half of each of the 32 rows


def test_loop_equals_vectorized():
    rng = np.random.default_rng(3)
    S, d, n, tau = 70, 8, 20, 0.3
    q, k = rng.standard_normal((S, d)), rng.standard_normal((S, d))
    want = np.zeros(S)
    for r in range(S - n, S):
        row = [math.exp(tau * float(np.dot(q[r], k[c]))) for c in range(r + 1)]
        tot = sum(row)
        for c in range(r + 1):
            want[c] += row[c] / tot
    assert np.max(np.abs(P.vline_importance(q, k, n, tau) - want)) < 1e-12


def test_top_k_ties():
    imp = np.array([0.5, 2.0, 1.0, 2.0, 1.0, 0.0])
    assert P.top_k_positions(imp, 3).tolist() == [1, 2, 3]
    assert P.top_k_positions(imp, 4).tolist() == [1, 2, 3, 4]
    assert P.top_k_positions(imp, 0).tolist() == []
