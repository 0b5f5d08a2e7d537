"""Oracle quantizer (test infrastructure only; see the package docstring).

[TriAttention] abstract: keys and values are quantized during prefill and the
same codes form the compressed KV cache reused by decode; query-key tiles are
computed at 4 or 8 bits.  The pages give no formula, so this module takes the
plainest symmetric reading:

* one scale per (sequence, head, 64-token block), over every channel of the
  block's valid rows; blocks restart at each sequence start;
* amax = max |x|;  s8 = amax / 127 and s4 = amax / 7, each an IEEE binary32
  division of binary32 operands (the 16-bit inputs widen exactly to binary32);
* code = clip(round_half_even(x / s), -qmax, qmax) with the division again in
  binary32; codes -128 and -8 are never produced;
* amax == 0 gives scale 0 and all-zero codes;
* rows past the end of a sequence in its last block are zero codes.

Layouts (``heads`` = H, ``nblk`` = sum over sequences of ceil(len / 64)):

* rows:  c8 [H][nblk][64][d] int8; c4 packed [H][nblk][64][d/2] uint8 with
         element 2t in the low nibble and 2t+1 in the high nibble of byte t
         (two's complement nibbles);
* cols (transposed, for V): c8 [H][nblk][d][64]; c4 packed [H][nblk][d][32]
         with token 2t low / 2t+1 high; f16 copy of the block, transposed,
         ``t16`` [H][nblk][d][64] (bf16 inputs converted to fp16, round to
         nearest even, magnitudes beyond 65504 saturated to +-65504; padding
         rows zero);
* s8, s4 [H][nblk] float32 in both layouts.
"""
from __future__ import annotations

import numpy as np

BLOCK = 64
QMAX8 = np.float32(127.0)
QMAX4 = np.float32(7.0)


def block_starts(seqlens):
    """Index of each sequence's first 64-token block in the blocked layout."""
    starts, acc = [], 0
    for S in seqlens:
        starts.append(acc)
        acc += -(-int(S) // BLOCK)
    return np.array(starts, dtype=np.int64), acc


def _codes(xb: np.ndarray, scale: np.ndarray, qmax: np.float32) -> np.ndarray:
    """xb float32 [..., H, ...], scale float32 broadcastable; binary32 division then
    round-half-even then clip."""
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.divide(xb, safe, dtype=np.float32)            # IEEE binary32 division
    c = np.clip(np.rint(q), -qmax, qmax)                  # rint: half to even
    c = np.where(scale > 0, c, np.float32(0.0))
    return c.astype(np.int8)


def quantize(x: np.ndarray, seqlens, layout: str = "rows", with_t16: bool = False):
    """Quantize x float32 [T][H][d] (exact widening of 16-bit inputs).

    Returns a dict with unpacked codes ``c8``/``c4`` in the rows layout
    [H][nblk][64][d] (int8), the packed tensors of the requested layout
    (``c8p``, ``c4p``), scales ``s8``/``s4`` [H][nblk] float32, ``blk_start``
    per sequence and ``nblk``.
    """
    x = np.asarray(x, dtype=np.float32)
    T, H, d = x.shape
    assert T == int(np.sum(seqlens))
    starts, nblk = block_starts(seqlens)
    c8 = np.zeros((H, nblk, BLOCK, d), np.int8)
    c4 = np.zeros((H, nblk, BLOCK, d), np.int8)
    s8 = np.zeros((H, nblk), np.float32)
    s4 = np.zeros((H, nblk), np.float32)
    xpad_all = np.zeros((H, nblk, BLOCK, d), np.float32)
    tok = 0
    for s, S in enumerate(seqlens):
        S = int(S)
        nb = -(-S // BLOCK)
        xs = np.zeros((nb * BLOCK, H, d), np.float32)
        xs[:S] = x[tok:tok + S]
        xb = xs.reshape(nb, BLOCK, H, d).transpose(2, 0, 1, 3)       # [H][nb][64][d]
        amax = np.max(np.abs(xb), axis=(2, 3)) if nb else np.zeros((H, 0), np.float32)
        sc8 = np.divide(amax, QMAX8, dtype=np.float32)
        sc4 = np.divide(amax, QMAX4, dtype=np.float32)
        b0 = starts[s]
        s8[:, b0:b0 + nb] = sc8
        s4[:, b0:b0 + nb] = sc4
        c8[:, b0:b0 + nb] = _codes(xb, sc8[:, :, None, None], QMAX8)
        c4[:, b0:b0 + nb] = _codes(xb, sc4[:, :, None, None], QMAX4)
        xpad_all[:, b0:b0 + nb] = xb
        tok += S
    out = dict(c8=c8, c4=c4, s8=s8, s4=s4, blk_start=starts, nblk=nblk, layout=layout)
    if layout == "rows":
        out["c8p"] = c8
        out["c4p"] = pack_nibbles(c4)
    elif layout == "cols":
        out["c8p"] = np.ascontiguousarray(c8.transpose(0, 1, 3, 2))
        out["c4p"] = pack_nibbles(np.ascontiguousarray(c4.transpose(0, 1, 3, 2)))
    else:
        raise ValueError(layout)
    if with_t16:
        # round to nearest even; beyond the fp16 range the nearest finite value
        t16 = np.clip(xpad_all, -65504.0, 65504.0).astype(np.float16)
        out["t16"] = np.ascontiguousarray(t16.transpose(0, 1, 3, 2))
    return out


def pack_nibbles(c: np.ndarray) -> np.ndarray:
    """Pack int8 codes in [-8, 7] along the last axis: element 2t -> low nibble,
    2t+1 -> high nibble of byte t (two's complement)."""
    c = np.asarray(c, dtype=np.int8)
    assert c.shape[-1] % 2 == 0
    u = c.view(np.uint8) & np.uint8(0x0F)
    return (u[..., 0::2] | (u[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(p: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles."""
    p = np.asarray(p, dtype=np.uint8)
    lo = (p & 0x0F).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequantize_rows(qt: dict, bits: int, seqlens) -> np.ndarray:
    """Q-hat = s * c back in token order [T][H][d] (float64), for checks that
    reduce integer-tile attention to attention on dequantized operands."""
    c = qt["c8"] if bits == 8 else qt["c4"]
    s = qt["s8"] if bits == 8 else qt["s4"]
    H, nblk, _, d = c.shape
    outs = []
    for si, S in enumerate(seqlens):
        b0 = int(qt["blk_start"][si])
        nb = -(-int(S) // BLOCK)
        blk = c[:, b0:b0 + nb].astype(np.float64) * s[:, b0:b0 + nb, None, None].astype(np.float64)
        outs.append(blk.transpose(1, 2, 0, 3).reshape(nb * BLOCK, H, d)[:int(S)])
    return np.concatenate(outs, axis=0)


def quantize_blocks(x: np.ndarray, seqlens, blocks):
    """Rows-layout codes for the listed (sequence, block) pairs only, zero
    elsewhere: each 64-token block is quantized on its own (blocks are
    independent, so this equals the listed blocks of ``quantize``)."""
    starts, nblk = block_starts(seqlens)
    T, H, d = x.shape
    out = dict(c8=np.zeros((H, nblk, BLOCK, d), np.int8), c4=np.zeros((H, nblk, BLOCK, d), np.int8),
               s8=np.zeros((H, nblk), np.float32), s4=np.zeros((H, nblk), np.float32), blk_start=starts, nblk=nblk)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    for s, b in sorted(blocks):
        t0 = int(cu[s]) + BLOCK * b
        t1 = min(t0 + BLOCK, int(cu[s + 1]))
        blk = quantize(x[t0:t1], [t1 - t0])
        g = int(starts[s]) + b
        for key in ("c8", "c4", "s8", "s4"):
            out[key][:, g] = blk[key][:, 0]
    return out
