"""Host check of the quantizer's reciprocal path (quantize_kernel): a code
taken from q0 = RN(x * RN(1/s)) when q0 lies more than |q0| 2^-20 + 2^-22
inside the half-integer edges around rint(q0), and from the IEEE quotient
RN(x / s) otherwise, equals rint(RN(x / s)) for every input.

The kernel's steps are emulated in binary32 with numpy (products and
quotients round to nearest even; the threshold's fused multiply-add is exact
in float64 before its one rounding to float32), over every finite bf16 value
or fp16 value of x and a spread of scales: the scales a block of amax values produces
(amax / 127 and amax / 7 in binary32), scales down to 2^-100, and random
24-bit significands.  Where the fast path is taken its code must equal the
one from IEEE division; the fallback must stay rare.
"""
import numpy as np


def _all_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    return x[np.isfinite(x)]


def _all_inputs():
    """Every finite bf16 and fp16 value, widened exactly to binary32."""
    h = np.arange(1 << 16, dtype=np.uint16).view(np.float16).astype(np.float32)
    return np.unique(np.concatenate([_all_bf16(), h[np.isfinite(h)]]))


def _scales(rng):
    amax = np.concatenate([
        _all_bf16()[rng.integers(0, 60000, 150)],
        (rng.uniform(1, 2, 100) * 2.0 ** rng.integers(-60, 60, 100)).astype(np.float32),
    ])
    amax = np.abs(amax)
    amax = amax[amax > 0]
    s = np.concatenate([amax / np.float32(127), amax / np.float32(7),
                        np.float32(2.0 ** -100) * np.float32([1.0, 1.5, 1.9999999]),
                        (rng.uniform(1, 2, 60) * 2.0 ** rng.integers(-100, 100, 60)).astype(np.float32)])
    s = s.astype(np.float32)
    return s[(s >= np.float32(2.0 ** -100)) & np.isfinite(s)]


def _codes(x, s, qmax):
    """(fast code, exact code, fast path taken) for all x at scale s."""
    y = np.float32(1.0) / s                      # RN(1/s)
    q0 = (x * y).astype(np.float32)              # RN(x y)
    c = np.rint(q0)
    t = (-np.abs(q0).astype(np.float64) * 2.0 ** -20 + (0.5 - 2.0 ** -22)).astype(np.float32)
    take = np.abs(q0 - c) <= t
    exact = np.rint((x / s).astype(np.float32))
    return np.clip(c, -qmax, qmax), np.clip(exact, -qmax, qmax), take


def test_reciprocal_codes_equal_ieee_codes():
    rng = np.random.default_rng(20)
    xs = _all_inputs()
    n = taken = 0
    for s in _scales(rng):
        for qmax in (127.0, 7.0):
            # the inputs a block with this scale can hold: |x| <= amax ~ qmax s
            x = xs[np.abs(xs).astype(np.float64) <= qmax * float(s) * 1.0001]
            if x.size == 0:
                continue
            fast, exact, take = _codes(x, s, qmax)
            bad = take & (fast != exact)
            assert not bad.any(), (float(s), qmax, x[bad][:4])
            n += x.size
            taken += int(take.sum())
    assert n > 1_000_000
    assert taken >= n * (1 - 1e-3), (taken, n)


def test_edge_cases_take_the_division():
    """x exactly on a half-integer edge (x = (k + 1/2) s, representable) and
    its float neighbours fall back to the division, whose tie goes to even."""
    s = np.float32(0.25)
    x = np.float32([0.125, 0.375, 0.625, -0.375, 31.875])   # 0.5, 1.5, 2.5, -1.5, 127.5 times s
    fast, exact, take = _codes(x, s, 127.0)
    assert not take.any()
    assert list(exact) == [0.0, 2.0, 2.0, -2.0, 127.0]
    nxt = np.nextafter(x, np.float32(np.inf))
    _, _, take2 = _codes(nxt, s, 127.0)
    assert not take2.any()
