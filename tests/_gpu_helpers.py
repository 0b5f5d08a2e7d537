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
DBG_POISON = 0x7EADBEEF   # above every integer tile score (|a| <= 127^2 * 128)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------- poison and guard bands
# Every buffer a GPU call writes is allocated here with a guard band after it
# and filled with a poison value before the call (a value the kernel never
# writes: NaN for floats, -128 for INT8 codes, 0x88 for packed INT4 codes, a
# sentinel for integer captures), so a kernel that leaves part of its output
# unwritten fails the comparison instead of passing on stale memory, and a
# write past the end shows up in the guard band.

GUARD_BYTES = 64 * 1024


class Guards:
    """Buffers with guard bands; `poison(role)` refills the buffers of a role
    with their poison value, `check()` asserts every guard band is intact."""

    _SENT = {1: 0xA5, 2: 0x7E5A, 4: 0x7FA5A5A5}

    def __init__(self, device="cuda:0"):
        self.device = device
        self.bufs = []   # (full buffer, number of elements in use, poison value, role)

    def alloc(self, shape, dtype, poison, role="out"):
        import torch
        n = 1
        for x in shape:
            n *= int(x)
        es = torch.empty((), dtype=dtype).element_size()
        g = GUARD_BYTES // es
        buf = torch.empty(n + g, dtype=dtype, device=self.device)
        ityp = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[es]
        buf[n:].view(ityp).fill_(self._SENT[es])
        self.bufs.append((buf, n, poison, role))
        view = buf[:n].view(*shape) if len(shape) else buf[:n]
        self._fill(buf, n, poison)
        return view

    @staticmethod
    def _fill(buf, n, poison):
        buf[:n].fill_(poison)

    def poison(self, role="out"):
        for buf, n, p, r in self.bufs:
            if r == role:
                self._fill(buf, n, p)

    def check(self):
        import torch
        for buf, n, _, r in self.bufs:
            es = buf.element_size()
            ityp = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[es]
            tail = buf[n:].view(ityp)
            bad = int((tail != self._SENT[es]).sum())
            assert bad == 0, f"guard band of a {r} buffer of {n} elements overwritten ({bad} elements)"


def guarded_qtensor(g, shape, heads, layout, with_t16, role="codes", with_c4x=False):
    """A QTensor (see the binding) whose buffers carry guard bands and
    poison: codes that the quantizer never writes, NaN scales and copies."""
    import torch
    from tile_routed_mixed_amd import _binding as B
    qt = B.QTensor.__new__(B.QTensor)
    nblk, d = shape.nblk(), shape.d
    qt.heads, qt.layout, qt.nblk = heads, layout, nblk
    if layout == B.TM_ROWS:
        qt.c8 = g.alloc((nblk, heads, 64, d), torch.int8, -128, role)
        qt.c4 = g.alloc((nblk, heads, 64, d // 2), torch.uint8, 0x88, role)
    else:
        qt.c8 = g.alloc((nblk, heads, d, 64), torch.int8, -128, role)
        qt.c4 = g.alloc((nblk, heads, d, 32), torch.uint8, 0x88, role)
    qt.s8 = g.alloc((nblk, heads), torch.float32, float("nan"), role)
    qt.s4 = g.alloc((nblk, heads), torch.float32, float("nan"), role)
    qt.t16 = g.alloc((nblk, heads, d, 64), torch.float16, float("nan"), role) if with_t16 else None
    qt.c4x = g.alloc((nblk, heads, 64, d), torch.int8, -128, role) if with_c4x else None
    ptr = lambda t: None if t is None else int(t.data_ptr())
    qt.c = B.tm_qtensor(ptr(qt.c8), ptr(qt.c4), ptr(qt.s8), ptr(qt.s4), ptr(qt.t16), heads, layout, nblk,
                        ptr(qt.c4x))
    return qt


def guard_prefill(p, o_dtype):
    """Give a PrefillPipeline guarded, poisoned quantized tensors and outputs
    (O of o_dtype, lse).  Returns the Guards."""
    import torch
    from tile_routed_mixed_amd import _binding as B
    g = Guards(p.device)
    sh = p.shape
    p.qq = guarded_qtensor(g, sh, sh.hq, B.TM_ROWS, False)
    p.kq = guarded_qtensor(g, sh, sh.hkv, B.TM_ROWS, False, with_c4x=True)
    p.vq = guarded_qtensor(g, sh, sh.hkv, B.TM_COLS, True)
    tdt = {B.TM_F32: torch.float32, B.TM_F16: torch.float16, B.TM_BF16: torch.bfloat16}[o_dtype]
    p.o = g.alloc((sh.T, sh.hq, sh.d), tdt, float("nan"))
    p.o_dtype = o_dtype
    p.lse = g.alloc((sh.hq, sh.T), torch.float32, float("nan"))
    return g


def guard_decode(p):
    """Give a DecodePipeline guarded, poisoned cache tensors, workspace and
    output.  Returns the Guards."""
    import torch
    from tile_routed_mixed_amd import _binding as B
    g = Guards(p.device)
    sh = p.shape
    p.kq = guarded_qtensor(g, sh, sh.hkv, B.TM_ROWS, False)
    p.vq = guarded_qtensor(g, sh, sh.hkv, B.TM_COLS, True)
    p.ws = g.alloc((max(4, p.ws.numel()),), torch.uint8, 0xFF, role="ws")
    p.o = g.alloc((len(sh.seqlens), sh.hq, sh.d), torch.float32, float("nan"))
    return g


def assert_all_written(t, what):
    """No poison left: every element of an output was written."""
    import torch
    bad = int(torch.isnan(t.float()).sum()) if t.is_floating_point() else 0
    assert bad == 0, f"{what}: {bad} elements never written"


def run_prefill(w, pol, q, k, v, o_dtype=None, dbg_tiles=None):
    """Run quantize x3 + traversal + prefill on the GPU.  Returns the pipeline,
    the census, O (numpy) and lse (numpy) and the debug capture (or None)."""
    import torch
    import tile_routed_mixed_amd as T
    say(f"[gpu] prefill {w.name} seqlens={w.seqlens[:6]}{'...' if len(w.seqlens) > 6 else ''} "
        f"hq={w.hq} hkv={w.hkv} d={w.d} bq={w.bq} {w.dtype} policy={pol['kind']}")
    odt = o_dtype if o_dtype is not None else T.TM_F32
    p = T.PrefillPipeline(w.seqlens, w.hq, w.hkv, w.d, w.bq, w.dtype, pol)
    p.upload(q[0], k[0], v[0])
    g = guard_prefill(p, odt)
    p.quantize()
    census = p.traversal(census=True)
    dt = dbg = None
    if dbg_tiles is not None:
        dt = torch.from_numpy(np.ascontiguousarray(np.asarray(dbg_tiles, np.int32))).to("cuda:0")
        dbg = g.alloc((len(dbg_tiles), w.bq, 64), torch.int32, DBG_POISON)
    o, dbg = p.prefill(odt, dbg_tiles=dt, dbg=dbg)
    torch.cuda.synchronize()
    g.check()
    for t, what in ((p.qq.s8, "Q scales"), (p.kq.s8, "K scales"), (p.vq.t16, "V fp16 copy"), (o, "O"),
                    (p.lse, "lse")):
        assert_all_written(t, what)
    p.guards = g
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
