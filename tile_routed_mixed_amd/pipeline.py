"""Device-buffer plumbing around the entry points.

PrefillPipeline holds the device copies of Q, K, V and every buffer the
prefill path writes, and runs one pass of the path:
  tm_quantize_pack(Q, rows)  tm_quantize_pack(K, rows)
  tm_quantize_pack(V, cols + fp16 copy)   tm_build_traversal
  (tm_gather_selected under a hybrid policy)   tm_prefill.
DecodePipeline does the same for decode steps over a quantized cache, and
for a growing one (start / append: tm_cache_append per step).
Nothing here computes: buffers are allocated once and the C ABI is called.
"""
from __future__ import annotations

import numpy as np

from . import _binding as B


def _dev_bits(bits: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).to(device)


class PrefillPipeline:
    def __init__(self, seqlens, hq, hkv, d, bq, dtype: str, policy: dict, device="cuda:0", softmax_scale=0.0):
        self.dt = B.TM_BF16 if dtype == "bf16" else B.TM_F16
        self.shape = B.Shape(seqlens, hq, hkv, d, bq, 64, self.dt, softmax_scale, device=device)
        self.device = device
        self.policy = B.Policy(policy, device=device)
        self.qq = B.QTensor(self.shape, hq, B.TM_ROWS, False, device)
        self.kq = B.QTensor(self.shape, hkv, B.TM_ROWS, False, device, with_c4x=True)
        self.vq = B.QTensor(self.shape, hkv, B.TM_COLS, True, device)
        import torch
        self.trav = torch.empty(B.traversal_bytes(self.shape, self.policy), dtype=torch.uint8, device=device)
        self.q = self.k = self.v = None
        self.o = None
        self._sel_cache = {}
        self.lse = torch.empty((hq, self.shape.T), dtype=torch.float32, device=device)

    def set_policy(self, policy: dict):
        """Route the same quantized inputs under another policy (the next
        traversal() builds its traversal)."""
        import torch
        self.policy = B.Policy(policy, device=self.device)
        need = B.traversal_bytes(self.shape, self.policy)
        if self.trav.numel() < need:
            self.trav = torch.empty(need, dtype=torch.uint8, device=self.device)

    def vertical_policy(self, frac: float, window: int, n_obs: int = 64, stream=None, on_device: bool = False):
        """Hybrid policy whose selected keys are, per (sequence, query head),
        the round(frac * len) keys of largest attention mass from the last
        n_obs query rows (tm_select_vertical over the uploaded Q and K).
        on_device: the lists stay where the selection wrote them (sel_idx_dev,
        overwritten by the next selection of this pipeline) and nothing waits
        for the GPU; otherwise they are copied to the host (sel_idx)."""
        counts = [int(round(frac * S)) for S in self.shape.seqlens]
        _, off, idx = B.tm_select_vertical(self.shape, self.q, self.k, n_obs, counts, False, stream,
                                           cache=self._sel_cache, on_device=on_device)
        if not on_device:
            return dict(kind=B.TM_POLICY_HYBRID, window=int(window), sel_off=off, sel_idx=idx)
        key = off.tobytes()
        if self._sel_cache.get("off_key") != key:   # device offsets: uploaded once per list sizes
            self._sel_cache["off_key"] = key
            self._sel_cache["off_dev"] = B._dev_offsets(off, self.device)
        return dict(kind=B.TM_POLICY_HYBRID, window=int(window), sel_off=off, sel_idx_dev=idx,
                    sel_off_dev=self._sel_cache["off_dev"])

    def upload(self, q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray):
        self.q = _dev_bits(q_bits, self.device)
        self.k = _dev_bits(k_bits, self.device)
        self.v = _dev_bits(v_bits, self.device)

    def quantize(self, stream=None):
        B.tm_quantize_pack(self.shape, self.q, self.qq, stream)
        B.tm_quantize_pack(self.shape, self.k, self.kq, stream)
        B.tm_quantize_pack(self.shape, self.v, self.vq, stream)

    def traversal(self, census=False, stream=None, fused=True):
        """Build the traversal; under a hybrid policy also gather the selected
        keys' K rows and V columns, in the same launch (fused) or by
        tm_gather_selected after the build."""
        hyb = self.policy.kind == B.TM_POLICY_HYBRID
        if hyb and fused:
            _, c = B.tm_build_traversal(self.shape, self.policy, self.trav, census=census, stream=stream, k=self.k,
                                        v=self.v)
            return c
        _, c = B.tm_build_traversal(self.shape, self.policy, self.trav, census=census, stream=stream)
        if hyb:
            B.tm_gather_selected(self.shape, self.policy, self.trav, self.k, self.v, stream)
        return c

    def prefill(self, o_dtype=B.TM_F32, dbg_tiles=None, stream=None, with_lse=True, dbg=None):
        if self.o is None or self.o_dtype != o_dtype:
            import torch
            tdt = {B.TM_F32: torch.float32, B.TM_F16: torch.float16, B.TM_BF16: torch.bfloat16}[o_dtype]
            self.o = torch.empty((self.shape.T, self.shape.hq, self.shape.d), dtype=tdt, device=self.device)
            self.o_dtype = o_dtype
        _, _, dbg = B.tm_prefill(self.shape, self.trav, self.policy.kind, self.q, self.k, self.qq, self.kq, self.vq, o=self.o,
                                 o_dtype=o_dtype, lse=self.lse if with_lse else None, dbg_tiles=dbg_tiles,
                                 stream=stream, dbg=dbg)
        return self.o, dbg

    def step(self, o_dtype=B.TM_F32, stream=None):
        self.quantize(stream)
        self.traversal(False, stream)
        return self.prefill(o_dtype, stream=stream)[0]


class DecodePipeline:
    """One decode step: the cache is K (rows) and V (cols + fp16 copy) quantized
    over the cached tokens, plus the 16-bit keys for FP16 blocks."""

    def __init__(self, seqlens, hq, hkv, d, dpolicy: dict, device="cuda:0", softmax_scale=0.0, dtype="f16"):
        dt = B.TM_BF16 if dtype == "bf16" else B.TM_F16
        self.shape = B.Shape(seqlens, hq, hkv, d, 128, 64, dt, softmax_scale, device=device)
        self.device = device
        self.dpol = B.DPolicy(dpolicy)
        self.kq = B.QTensor(self.shape, hkv, B.TM_ROWS, False, device)
        self.vq = B.QTensor(self.shape, hkv, B.TM_COLS, True, device)
        import torch
        self.ws = torch.empty(max(4, B.decode_ws_bytes(self.shape, self.dpol)), dtype=torch.uint8, device=device)
        self.o = torch.empty((len(seqlens), hq, d), dtype=torch.float32, device=device)
        self.q = self.k = self.v = None

    def upload(self, q_bits, k_bits, v_bits):
        self.q = _dev_bits(q_bits, self.device)
        self.k = _dev_bits(k_bits, self.device)
        self.v = _dev_bits(v_bits, self.device)

    def build_cache(self, stream=None):
        B.tm_quantize_pack(self.shape, self.k, self.kq, stream)
        B.tm_quantize_pack(self.shape, self.v, self.vq, stream)

    def select(self, sel_off, sel_idx, stream=None, sel_off_dev=None):
        """Keep the listed tokens in FP16 (lists per (sequence, KV head), after
        build_cache / start); call again when the lists or lengths change.
        sel_idx may be an int32 device tensor (lists in device memory)."""
        import torch
        self.dpol.set_selection(sel_off, sel_idx, sel_off_dev)
        if sel_off is None:
            return
        n = B.decode_sel_bytes(self.shape, self.dpol)
        buf = getattr(self, "sel_buf", None)
        if buf is None or buf.numel() < n:
            buf = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        self.sel_buf = buf
        B.tm_decode_select(self.shape, self.dpol, self.k, self.vq, buf, stream)

    def decode(self, stream=None):
        return B.tm_decode(self.shape, self.q, self.kq, self.vq, self.k, self.dpol, o=self.o, ws=self.ws,
                           stream=stream)

    # ---- generation: the shape's lengths are capacities; the cache holds
    # the first `lengths[s]` tokens of sequence s
    def start(self, lengths, stream=None):
        """Cache the first lengths[s] tokens of every sequence (the uploaded K/V
        rows past them are ignored) and decode at those lengths from now on."""
        self.dpol.set_lengths(lengths)
        B.tm_quantize_pack(self.shape, self.k, self.kq, stream)
        B.tm_quantize_pack(self.shape, self.v, self.vq, stream)
        # the block holding each sequence's last cached token, over the cached rows only
        L = self.dpol.lengths
        B.tm_cache_append(self.shape, L, self.k, self.kq, stream)
        B.tm_cache_append(self.shape, L, self.v, self.vq, stream)

    def append(self, k_bits, v_bits, q_bits=None, stream=None):
        """Append one token per sequence: k_bits, v_bits [nseq][hkv][d] (16-bit
        patterns) go to row lengths[s] of each sequence, the cache blocks are
        brought up to date, and q_bits [nseq][hq][d] (if given) becomes the
        next query."""
        import torch
        L = self.dpol.lengths.copy()
        cu = self.shape.cu_host
        cap = cu[1:] - cu[:-1]
        full = np.nonzero(L >= cap)[0]
        if full.size:
            raise ValueError(f"append: sequences {full.tolist()} are at their capacity {cap[full].tolist()}")
        rows = torch.as_tensor((cu[:-1] + L).astype(np.int64), device=self.device)
        # the row writes run on `stream` too, so tm_cache_append sees them
        with torch.cuda.stream(stream):   # (None: the current stream)
            self.k[rows] = _dev_bits(k_bits, self.device)
            self.v[rows] = _dev_bits(v_bits, self.device)
        L += 1
        B.tm_cache_append(self.shape, L, self.k, self.kq, stream)
        B.tm_cache_append(self.shape, L, self.v, self.vq, stream)
        self.dpol.set_lengths(L)   # only once both appends were accepted
        if q_bits is not None:
            self.q = _dev_bits(q_bits, self.device)

    @classmethod
    def from_prefill(cls, pp: "PrefillPipeline", dpolicy: dict, q_bits):
        """Decode over the cache a PrefillPipeline just quantized (its K rows and
        V cols + fp16 copy are the compressed cache); q_bits [nseq][hq][d]."""
        self = cls.__new__(cls)
        self.shape = pp.shape
        self.device = pp.device
        self.dpol = B.DPolicy(dpolicy)
        self.kq, self.vq = pp.kq, pp.vq
        import torch
        self.ws = torch.empty(max(4, B.decode_ws_bytes(self.shape, self.dpol)), dtype=torch.uint8,
                              device=self.device)
        self.o = torch.empty((len(self.shape.seqlens), self.shape.hq, self.shape.d), dtype=torch.float32,
                             device=self.device)
        self.q = _dev_bits(q_bits, self.device)
        self.k, self.v = pp.k, pp.v
        return self


def read_traversal(trav_host: np.ndarray):
    """Decode a traversal buffer copied to the host (layout in include/tm.h)."""
    b = np.ascontiguousarray(trav_host).view(np.uint8)
    h = b[:B.TRAV_HEADER_BYTES].view(np.uint32)
    magic, version, kind, n_items, max_runs, nseq = (int(x) for x in h[:6])
    seq_off, item_off, run_off = int(h[12]), int(h[13]), int(h[14])
    census = b[128:128 + 40].view(np.int64)
    seqs = b[seq_off:seq_off + 16 * nseq].view(np.uint32).reshape(nseq, 4)
    items = b[item_off:item_off + 32 * n_items].view(np.uint32).reshape(n_items, 8)
    runs = b[run_off:run_off + 8 * n_items * max_runs].view(np.uint32).reshape(n_items, max_runs, 2)
    return dict(magic=magic, version=version, kind=kind, n_items=n_items, max_runs=max_runs, seqs=seqs,
                items=items, runs=runs, census=dict(legal=int(census[0]), int8=int(census[1]),
                                                    int4=int(census[2]), fp16=int(census[3]),
                                                    skip=int(census[4])))
