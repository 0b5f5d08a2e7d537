"""tm_decode_noalloc (the decode entry point that allocates nothing) against
tm_decode on the same inputs, through the C ABI: two calls in a row, the
second on a smaller cache, each output bit-identical to tm_decode's and within
the parity gate of the oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import quant as OQ

from _gpu_helpers import Guards, compare, say

pytestmark = pytest.mark.gpu


def _case(seqlens, hq, hkv, d, dpol):
    import torch
    import tile_routed_mixed_amd as T
    from tile_routed_mixed_amd import _binding as B
    w = W.small("decode16x32k", seqlens, hq=hq, hkv=hkv, d=d, dtype="f16")
    _, k, v = W.make_qkv(w)
    dq = W.make_decode_query(w)
    say(f"[gpu] decode_noalloc {seqlens} hq={hq} hkv={hkv} d={d} {dpol}")
    p = T.DecodePipeline(w.seqlens, hq, hkv, d, dpol, dtype="f16")
    p.upload(dq[0], k[0], v[0])
    p.build_cache()
    g = Guards()
    o_ref = g.alloc((len(seqlens), hq, d), torch.float32, float("nan"))
    o_new = g.alloc((len(seqlens), hq, d), torch.float32, float("nan"))
    B.tm_decode(p.shape, p.q, p.kq, p.vq, p.k, p.dpol, o=o_ref, ws=p.ws)
    B.tm_decode_noalloc(p.shape, p.q, p.kq, p.vq, p.k, p.dpol, o_new)
    torch.cuda.synchronize()
    g.check()
    a, b = o_ref.cpu().numpy(), o_new.cpu().numpy()
    assert np.all(np.isfinite(b))
    assert np.array_equal(a, b)
    kq = OQ.quantize(k[1], w.seqlens)
    vq = OQ.quantize(v[1], w.seqlens, layout="cols")
    O = OA.decode(w.seqlens, hq, hkv, d, dq[1].astype(np.float64), kq, vq, k[1].astype(np.float64),
                  v[1].astype(np.float64), dpol)
    compare(b, O, what=f"decode_noalloc {seqlens}")


def test_decode_noalloc_matches_decode_twice_shrinking():
    _case([3000, 1500, 700, 2100], 8, 2, 128, dict(b8=[3, 5], b4=[9, 20], sink=1, tail=128))
    # a second call on a smaller cache: the scratch array keeps the first
    # call's partials, none of which the second may read
    _case([900, 65], 4, 1, 64, dict(b8=[2], b4=[6], sink=0, tail=64))
