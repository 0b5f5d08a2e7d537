"""ctypes binding of libtm.so (include/tm.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the stream.
The library must have been built (``__graft_entry__.build()`` or
``python tile_routed_mixed_amd/build.py``); importing this module fails loudly
otherwise -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtm.so")

TM_OK, TM_E_ARG, TM_E_SHAPE, TM_E_POLICY, TM_E_SPACE, TM_E_UNSUPPORTED, TM_E_HIP = range(7)
TM_F16, TM_BF16, TM_F32 = 0, 1, 2
TM_SKIP, TM_INT4, TM_INT8, TM_FP16 = 0, 1, 2, 3
TM_ROWS, TM_COLS = 0, 1
TM_POLICY_BOUNDARIES, TM_POLICY_BITMASK, TM_POLICY_FOURWAY, TM_POLICY_HYBRID = 0, 1, 2, 3
TRAV_HEADER_BYTES = 256
TRAV_MAGIC = 0x564D5454


class tm_shape(ctypes.Structure):
    _fields_ = [("nseq", ctypes.c_int32), ("cu_seqlens", ctypes.POINTER(ctypes.c_int32)),
                ("cu_seqlens_dev", ctypes.c_void_p), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("bq", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class tm_qtensor(ctypes.Structure):
    _fields_ = [("c8", ctypes.c_void_p), ("c4", ctypes.c_void_p), ("s8", ctypes.c_void_p),
                ("s4", ctypes.c_void_p), ("t16", ctypes.c_void_p), ("heads", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("nblk", ctypes.c_int64), ("c4x", ctypes.c_void_p)]


class tm_policy(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("b8", ctypes.POINTER(ctypes.c_int32)),
                ("b4", ctypes.POINTER(ctypes.c_int32)), ("sink", ctypes.c_int32),
                ("bits", ctypes.c_void_p), ("n_words", ctypes.c_int64), ("group", ctypes.c_int32),
                ("sel_off", ctypes.POINTER(ctypes.c_int32)), ("sel_idx", ctypes.POINTER(ctypes.c_int32)),
                ("window", ctypes.c_int32), ("sel_off_dev", ctypes.c_void_p), ("sel_idx_dev", ctypes.c_void_p)]


class tm_census(ctypes.Structure):
    _fields_ = [("legal", ctypes.c_int64), ("n_int8", ctypes.c_int64), ("n_int4", ctypes.c_int64),
                ("n_fp16", ctypes.c_int64), ("n_skip", ctypes.c_int64), ("n_items", ctypes.c_int64),
                ("max_runs", ctypes.c_int64)]


class tm_dpolicy(ctypes.Structure):
    _fields_ = [("b8", ctypes.POINTER(ctypes.c_int32)), ("b4", ctypes.POINTER(ctypes.c_int32)),
                ("sink", ctypes.c_int32), ("tail_tokens", ctypes.c_int32),
                ("lengths", ctypes.POINTER(ctypes.c_int32)), ("per_q_head", ctypes.c_int32),
                ("sel_off", ctypes.POINTER(ctypes.c_int32)), ("sel_idx", ctypes.POINTER(ctypes.c_int32)),
                ("sel_buf", ctypes.c_void_p), ("sel_off_dev", ctypes.c_void_p), ("sel_idx_dev", ctypes.c_void_p)]


class TMError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {lib().tm_status_string(status).decode()}")
        self.status = status


_LIB = None


def lib():
    """Load libtm.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.tm_status_string.restype = ctypes.c_char_p
        L.tm_status_string.argtypes = [i32]
        L.tm_version.restype = i32
        L.tm_version.argtypes = []
        L.tm_num_blocks.restype = i64
        L.tm_num_blocks.argtypes = [ctypes.POINTER(tm_shape)]
        L.tm_quantize_pack.restype = i32
        L.tm_quantize_pack.argtypes = [ctypes.POINTER(tm_shape), vp, i32, ctypes.POINTER(tm_qtensor), vp]
        L.tm_build_traversal.restype = i32
        L.tm_build_traversal.argtypes = [ctypes.POINTER(tm_shape), ctypes.POINTER(tm_policy), vp,
                                         ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(tm_census), vp]
        L.tm_build_traversal_gather.restype = i32
        L.tm_build_traversal_gather.argtypes = [ctypes.POINTER(tm_shape), ctypes.POINTER(tm_policy), vp,
                                                ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(tm_census), vp, vp,
                                                vp]
        L.tm_gather_selected.restype = i32
        L.tm_gather_selected.argtypes = [ctypes.POINTER(tm_shape), ctypes.POINTER(tm_policy), vp, vp, vp, vp]
        L.tm_select_vertical.restype = i32
        L.tm_select_vertical.argtypes = [ctypes.POINTER(tm_shape), vp, vp, i32, ctypes.POINTER(ctypes.c_int32), i32,
                                         vp, vp, vp, ctypes.POINTER(ctypes.c_size_t), vp]
        L.tm_prefill.restype = i32
        L.tm_prefill.argtypes = [ctypes.POINTER(tm_shape), vp, i32, vp, vp, ctypes.POINTER(tm_qtensor),
                                 ctypes.POINTER(tm_qtensor), ctypes.POINTER(tm_qtensor), vp, i32, vp, vp, vp,
                                 i32, vp]
        L.tm_cache_append.restype = i32
        L.tm_cache_append.argtypes = [ctypes.POINTER(tm_shape), ctypes.POINTER(ctypes.c_int32), vp, i32,
                                      ctypes.POINTER(tm_qtensor), vp]
        L.tm_decode_select.restype = i32
        L.tm_decode_select.argtypes = [ctypes.POINTER(tm_shape), ctypes.POINTER(tm_dpolicy), vp,
                                       ctypes.POINTER(tm_qtensor), vp, ctypes.POINTER(ctypes.c_size_t), vp]
        L.tm_decode_noalloc.restype = i32
        L.tm_decode_noalloc.argtypes = [ctypes.POINTER(tm_shape), vp, ctypes.POINTER(tm_qtensor),
                                        ctypes.POINTER(tm_qtensor), vp, ctypes.POINTER(tm_dpolicy), vp, i32, vp]
        L.tm_decode_noalloc_max_workspace.restype = ctypes.c_size_t
        L.tm_decode_noalloc_max_workspace.argtypes = []
        L.tm_decode.restype = i32
        L.tm_decode.argtypes = [ctypes.POINTER(tm_shape), vp, ctypes.POINTER(tm_qtensor),
                                ctypes.POINTER(tm_qtensor), vp, ctypes.POINTER(tm_dpolicy), vp, i32, vp,
                                ctypes.POINTER(ctypes.c_size_t), vp]
        _LIB = L
    return _LIB


def _check(st: int, where: str):
    if st != TM_OK:
        raise TMError(st, where)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


# ----------------------------------------------------------------------------- shapes

class Shape:
    """A tm_shape plus the host and device copies of cu_seqlens it points to."""

    def __init__(self, seqlens, hq, hkv, d, bq=128, bk=64, dtype=TM_F16, softmax_scale=0.0, device=None):
        self.seqlens = [int(s) for s in seqlens]
        self.cu_host = np.ascontiguousarray(np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32))
        self.cu_dev = None
        if device is not None:
            import torch
            self.cu_dev = torch.from_numpy(self.cu_host.copy()).to(device)
        self.c = tm_shape(len(self.seqlens), self.cu_host.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                          _ptr(self.cu_dev), hq, hkv, d, bq, bk, dtype, softmax_scale)
        self.hq, self.hkv, self.d, self.bq, self.bk, self.dtype = hq, hkv, d, bq, bk, dtype

    @property
    def T(self) -> int:
        return int(self.cu_host[-1])

    def nblk(self) -> int:
        n = lib().tm_num_blocks(ctypes.byref(self.c))
        if n < 0:
            raise TMError(TM_E_SHAPE, "tm_num_blocks")
        return int(n)


class QTensor:
    """Device buffers of one quantized tensor (see tm_qtensor in include/tm.h)."""

    def __init__(self, shape: Shape, heads: int, layout: int, with_t16: bool, device, with_c4x: bool = False):
        import torch
        nblk, d = shape.nblk(), shape.d
        self.heads, self.layout, self.nblk = heads, layout, nblk
        # block-major: [nblk][heads][...]
        if layout == TM_ROWS:
            self.c8 = torch.empty((nblk, heads, 64, d), dtype=torch.int8, device=device)
            self.c4 = torch.empty((nblk, heads, 64, d // 2), dtype=torch.uint8, device=device)
        else:
            self.c8 = torch.empty((nblk, heads, d, 64), dtype=torch.int8, device=device)
            self.c4 = torch.empty((nblk, heads, d, 32), dtype=torch.uint8, device=device)
        self.s8 = torch.empty((nblk, heads), dtype=torch.float32, device=device)
        self.s4 = torch.empty((nblk, heads), dtype=torch.float32, device=device)
        self.t16 = (torch.empty((nblk, heads, d, 64), dtype=torch.float16, device=device)
                    if with_t16 else None)
        self.c4x = (torch.empty((nblk, heads, 64, d), dtype=torch.int8, device=device)
                    if with_c4x else None)
        self.c = tm_qtensor(_ptr(self.c8), _ptr(self.c4), _ptr(self.s8), _ptr(self.s4), _ptr(self.t16),
                            heads, layout, nblk, _ptr(self.c4x))


# ----------------------------------------------------------------------------- entry points

def tm_quantize_pack(shape: Shape, x, out: QTensor, stream=None) -> QTensor:
    """x: [T][heads][d] 16-bit device tensor (fp16/bf16 or its uint16 bits)."""
    assert x.is_contiguous() and x.element_size() == 2
    _check(lib().tm_quantize_pack(ctypes.byref(shape.c), _ptr(x), out.heads, ctypes.byref(out.c),
                                  _stream(stream)), "tm_quantize_pack")
    return out


def _dev_offsets(off: np.ndarray, device, given=None):
    """Device copy of list offsets (int32 tensor), or `given` when it is one."""
    import torch
    if given is not None:
        assert given.dtype == torch.int32 and given.numel() == off.size
        return given
    return torch.from_numpy(off.copy()).to(device)


class Policy:
    """Host/device copies of a tile policy: dict(kind=0, b8, b4, sink),
    dict(kind=1, group, words), dict(kind=2, b8, b4, sink, group, words) or
    dict(kind=3, window, sel_off, sel_idx).  A hybrid policy may hold its
    lists in device memory instead: dict(kind=3, window, sel_off, sel_idx_dev
    [, sel_off_dev]) with int32 device tensors (sel_off stays on the host)."""

    def __init__(self, pol: dict, device=None):
        self.kind = int(pol["kind"])
        self.b8 = self.b4 = None
        self.bits = None
        self.sel_off = self.sel_idx = None
        b8p = b4p = None
        sink = 0
        if self.kind in (TM_POLICY_BOUNDARIES, TM_POLICY_FOURWAY):
            self.b8 = np.ascontiguousarray(np.asarray(pol["b8"], dtype=np.int32))
            self.b4 = np.ascontiguousarray(np.asarray(pol["b4"], dtype=np.int32))
            b8p = self.b8.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
            b4p = self.b4.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
            sink = int(pol.get("sink", 0))
        n_words, group = 0, 1
        if self.kind in (TM_POLICY_BITMASK, TM_POLICY_FOURWAY):
            import torch
            words = np.ascontiguousarray(np.asarray(pol["words"], dtype=np.uint32))
            self.bits = torch.from_numpy(words.view(np.int32).copy()).to(device) if device is not None else None
            n_words, group = int(words.size), int(pol["group"])
        self.c = tm_policy(self.kind, b8p, b4p, sink, _ptr(self.bits), n_words, group)
        self.sel_idx_dev = self.sel_off_dev = None
        if self.kind == TM_POLICY_HYBRID:
            self.sel_off = np.ascontiguousarray(np.asarray(pol["sel_off"], dtype=np.int32))
            self.c.sel_off = self.sel_off.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
            self.c.window = int(pol["window"])
            if pol.get("sel_idx_dev") is not None:
                self.sel_idx_dev = pol["sel_idx_dev"]
                assert self.sel_idx_dev.dtype.itemsize == 4 and self.sel_idx_dev.is_contiguous()
                self.sel_off_dev = _dev_offsets(self.sel_off, self.sel_idx_dev.device, pol.get("sel_off_dev"))
                self.c.sel_idx_dev = _ptr(self.sel_idx_dev)
                self.c.sel_off_dev = _ptr(self.sel_off_dev)
            else:
                self.sel_idx = np.ascontiguousarray(np.asarray(pol["sel_idx"], dtype=np.int32))
                self.c.sel_idx = self.sel_idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def tm_gather_selected(shape: "Shape", policy: Policy, trav, k, v, stream=None):
    """Hybrid policies: copy the selected keys' K rows and V columns (k, v:
    [T][hkv][d] 16-bit device tensors) into the traversal's gathered tiles."""
    _check(lib().tm_gather_selected(ctypes.byref(shape.c), ctypes.byref(policy.c), _ptr(trav), _ptr(k), _ptr(v),
                                    _stream(stream)), "tm_gather_selected")


def tm_select_vertical(shape: "Shape", q, k, n_obs: int, counts, per_kv_head: bool = False, stream=None,
                       cache: Optional[dict] = None, mass_out=None, sel_out=None, on_device: bool = False):
    """Attention mass of each key from the last n_obs query rows, and the
    counts[s] keys of largest mass per list.  Returns (mass [hq][T] float32
    device tensor, sel_off (host int32), sel_idx (host int32)): the index
    lists of a hybrid prefill policy (per query head) or of a decode selection
    (per KV head).  on_device: sel_idx is the int32 device tensor the kernel
    wrote (its first sel_off[-1] entries), with no copy to the host and no
    wait.  `cache` (a dict the caller keeps) holds the workspace and
    output buffers between calls of the same sizes; a returned mass tensor (or
    device list) is then overwritten by the next call.  mass_out ([hq][T]
    float32) and sel_out (int32, at least the lists' total length) are caller
    buffers to write instead of the cached or new ones."""
    import torch
    cnt = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
    cp = cnt.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    nl = shape.hkv if per_kv_head else shape.hq
    total = int(nl * cnt.astype(np.int64).sum())
    key = (int(n_obs), cnt.tobytes(), bool(per_kv_head), tuple(shape.seqlens), shape.hq, shape.hkv, shape.d)
    if cache is not None and cache.get("key") == key:
        ws, mass, sel, n = cache["ws"], cache["mass"], cache["sel"], ctypes.c_size_t(cache["ws_bytes"])
    else:
        n = ctypes.c_size_t(0)
        _check(lib().tm_select_vertical(ctypes.byref(shape.c), None, None, int(n_obs), cp, int(per_kv_head), None,
                                        None, None, ctypes.byref(n), None), "tm_select_vertical(size)")
        dev = q.device
        ws = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=dev)
        mass = torch.empty((shape.hq, shape.T), dtype=torch.float32, device=dev)
        sel = torch.empty(max(total, 1), dtype=torch.int32, device=dev)
        if cache is not None:
            cache.clear()
            cache.update(key=key, ws=ws, mass=mass, sel=sel, ws_bytes=int(n.value))
    if mass_out is not None:
        assert mass_out.dtype == torch.float32 and mass_out.numel() == shape.T * shape.hq
        mass = mass_out
    if sel_out is not None:
        assert sel_out.dtype == torch.int32 and sel_out.numel() >= total
        sel = sel_out
    _check(lib().tm_select_vertical(ctypes.byref(shape.c), _ptr(q), _ptr(k), int(n_obs), cp, int(per_kv_head),
                                    _ptr(mass), _ptr(sel), _ptr(ws), ctypes.byref(n), _stream(stream)),
           "tm_select_vertical")
    per_list = np.repeat(cnt, nl)
    sel_off = np.concatenate([[0], np.cumsum(per_list)]).astype(np.int32)
    if on_device:
        return mass, sel_off, sel
    if stream is not None:   # the copy below runs on the current stream: order it after the kernels
        torch.cuda.current_stream().wait_stream(stream)
    return mass, sel_off, sel[:total].cpu().numpy().astype(np.int32)


def traversal_bytes(shape: Shape, policy: Policy) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().tm_build_traversal(ctypes.byref(shape.c), ctypes.byref(policy.c), None, ctypes.byref(n),
                                    None, None), "tm_build_traversal(size)")
    return int(n.value)


def tm_build_traversal(shape: Shape, policy: Policy, trav=None, census: bool = True, stream=None, k=None, v=None):
    """Returns (trav uint8 device tensor, census dict or None).  k, v (hybrid
    policies): also gather the selected keys' rows in the same launch
    (tm_build_traversal_gather)."""
    import torch
    need = traversal_bytes(shape, policy)
    if trav is None:
        trav = torch.empty(need, dtype=torch.uint8, device=shape.cu_dev.device)
    n = ctypes.c_size_t(trav.numel())
    cen = tm_census()
    cp = ctypes.byref(cen) if census else None
    if k is not None:
        _check(lib().tm_build_traversal_gather(ctypes.byref(shape.c), ctypes.byref(policy.c), _ptr(trav),
                                               ctypes.byref(n), cp, _ptr(k), _ptr(v), _stream(stream)),
               "tm_build_traversal_gather")
    else:
        _check(lib().tm_build_traversal(ctypes.byref(shape.c), ctypes.byref(policy.c), _ptr(trav), ctypes.byref(n),
                                        cp, _stream(stream)), "tm_build_traversal")
    out = None
    if census:
        out = dict(legal=cen.legal, int8=cen.n_int8, int4=cen.n_int4, fp16=cen.n_fp16, skip=cen.n_skip,
                   n_items=cen.n_items, max_runs=cen.max_runs)
    return trav, out


def tm_prefill(shape: Shape, trav, policy_kind: int, q, k, qq: QTensor, kq: QTensor, vq: QTensor, o=None,
               o_dtype=TM_F32, lse=None, dbg_tiles=None, stream=None, dbg=None):
    """Returns (o, lse, dbg_qk).  dbg_tiles: int32 device tensor [n][4] or None;
    dbg: int32 device tensor [n][bq][64] to capture into (else a new one)."""
    import torch
    dev = q.device
    if o is None:
        tdt = {TM_F32: torch.float32, TM_F16: torch.float16, TM_BF16: torch.bfloat16}[o_dtype]
        o = torch.empty((shape.T, shape.hq, shape.d), dtype=tdt, device=dev)
    n_dbg = 0
    if dbg_tiles is not None:
        n_dbg = int(dbg_tiles.shape[0])
        if dbg is None:
            dbg = torch.zeros((n_dbg, shape.bq, 64), dtype=torch.int32, device=dev)
        assert dbg.dtype == torch.int32 and dbg.numel() == n_dbg * shape.bq * 64
    else:
        dbg = None
    _check(lib().tm_prefill(ctypes.byref(shape.c), _ptr(trav), int(policy_kind), _ptr(q), _ptr(k), ctypes.byref(qq.c),
                            ctypes.byref(kq.c), ctypes.byref(vq.c), _ptr(o), o_dtype, _ptr(lse), _ptr(dbg),
                            _ptr(dbg_tiles), n_dbg, _stream(stream)), "tm_prefill")
    return o, lse, dbg


class DPolicy:
    def __init__(self, dpol: dict, lengths=None):
        self.b8 = np.ascontiguousarray(np.asarray(dpol["b8"], dtype=np.int32))
        self.b4 = np.ascontiguousarray(np.asarray(dpol["b4"], dtype=np.int32))
        self.c = tm_dpolicy(self.b8.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                            self.b4.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(dpol["sink"]),
                            int(dpol["tail"]), None, int(dpol.get("per_q_head", 0)))
        self.lengths = None
        if lengths is not None:
            self.set_lengths(lengths)

    def set_lengths(self, lengths):
        """Current lengths of a growing cache (host int32 [nseq]), or None."""
        if lengths is None:
            self.lengths = None
            self.c.lengths = None
        else:
            self.lengths = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
            self.c.lengths = self.lengths.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))

    def set_selection(self, sel_off, sel_idx, sel_off_dev=None):
        """Selected tokens kept in FP16: lists per (sequence, KV head), or
        sel_off None for none.  sel_idx: host positions, or an int32 device
        tensor (lists in device memory; sel_off_dev, a device copy of sel_off,
        is made when not given).  The device buffer comes from
        tm_decode_select."""
        self.sel_idx_dev = self.sel_off_dev = None
        self.c.sel_idx_dev = self.c.sel_off_dev = None
        if sel_off is None:
            self.sel_off = self.sel_idx = None
            self.c.sel_off = self.c.sel_idx = None
            self.c.sel_buf = None
            return
        self.sel_off = np.ascontiguousarray(np.asarray(sel_off, dtype=np.int32))
        self.c.sel_off = self.sel_off.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        if hasattr(sel_idx, "data_ptr"):
            assert sel_idx.dtype.itemsize == 4 and sel_idx.is_contiguous()
            self.sel_idx = None
            self.c.sel_idx = None
            self.sel_idx_dev = sel_idx
            self.sel_off_dev = _dev_offsets(self.sel_off, sel_idx.device, sel_off_dev)
            self.c.sel_idx_dev = _ptr(self.sel_idx_dev)
            self.c.sel_off_dev = _ptr(self.sel_off_dev)
        else:
            self.sel_idx = np.ascontiguousarray(np.asarray(sel_idx, dtype=np.int32))
            self.c.sel_idx = self.sel_idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        # the device buffer was built for other lists: tm_decode refuses to run
        # (TM_E_ARG) until tm_decode_select has filled one for these
        self.sel_buf = None
        self.c.sel_buf = None


def decode_sel_bytes(shape: "Shape", dpol: "DPolicy") -> int:
    n = ctypes.c_size_t(0)
    _check(lib().tm_decode_select(ctypes.byref(shape.c), ctypes.byref(dpol.c), None, None, None, ctypes.byref(n),
                                  None), "tm_decode_select(size)")
    return int(n.value)


def tm_decode_select(shape: "Shape", dpol: "DPolicy", k16, vq: "QTensor", buf, stream=None):
    """Fill `buf` (uint8 device tensor) with the selected-token tables and
    gathered tiles of dpol's lists; the policy then points at it."""
    n = ctypes.c_size_t(buf.numel())
    _check(lib().tm_decode_select(ctypes.byref(shape.c), ctypes.byref(dpol.c), _ptr(k16), ctypes.byref(vq.c),
                                  _ptr(buf), ctypes.byref(n), _stream(stream)), "tm_decode_select")
    dpol.sel_buf = buf
    dpol.c.sel_buf = _ptr(buf)


def tm_cache_append(shape: Shape, lengths: np.ndarray, x, out: QTensor, stream=None):
    """Re-quantize the block holding each sequence's newest token (lengths:
    host int32 [nseq], current lengths; x: [T][heads][d] in the capacity
    layout of `shape`)."""
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    assert x.is_contiguous() and x.element_size() == 2
    _check(lib().tm_cache_append(ctypes.byref(shape.c), ln.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _ptr(x),
                                 out.heads, ctypes.byref(out.c), _stream(stream)), "tm_cache_append")


def decode_ws_bytes(shape: Shape, dpol: DPolicy) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().tm_decode(ctypes.byref(shape.c), None, None, None, None, ctypes.byref(dpol.c), None, TM_F32,
                           None, ctypes.byref(n), None), "tm_decode(size)")
    return int(n.value)


def tm_decode(shape: Shape, q, kq: QTensor, vq: QTensor, k16, dpol: DPolicy, o=None, o_dtype=TM_F32, ws=None,
              stream=None):
    import torch
    dev = q.device
    if o is None:
        o = torch.empty((len(shape.seqlens), shape.hq, shape.d),
                        dtype=torch.float32 if o_dtype == TM_F32 else torch.float16, device=dev)
    need = decode_ws_bytes(shape, dpol)
    if ws is None:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    n = ctypes.c_size_t(ws.numel())
    _check(lib().tm_decode(ctypes.byref(shape.c), _ptr(q), ctypes.byref(kq.c), ctypes.byref(vq.c), _ptr(k16),
                           ctypes.byref(dpol.c), _ptr(o), o_dtype, _ptr(ws), ctypes.byref(n), _stream(stream)),
           "tm_decode")
    return o


def tm_decode_noalloc(shape: Shape, q, kq: QTensor, vq: QTensor, k16, dpol: DPolicy, o, o_dtype=TM_F32,
                      stream=None):
    """tm_decode with the library's own scratch array as workspace (o must be
    given: the call allocates nothing)."""
    _check(lib().tm_decode_noalloc(ctypes.byref(shape.c), _ptr(q), ctypes.byref(kq.c), ctypes.byref(vq.c),
                                   _ptr(k16), ctypes.byref(dpol.c), _ptr(o), o_dtype, _stream(stream)),
           "tm_decode_noalloc")
    return o


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
