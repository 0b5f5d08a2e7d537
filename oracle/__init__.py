"""CPU oracle for tile-routed mixed-precision causal attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls, links or
runs this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it, as the reference the HIP library is
checked against.  It shares no code, tables or constants with the HIP sources.

It computes, slowly and plainly, in float64 (integers in int64/float64-exact):

* ``quant``     -- the symmetric per-64-token-block quantizer (INT8 and INT4
                   codes, binary32 scales, nibble packing), emulated in IEEE
                   binary32 so codes are bit-identical to any correct binary32
                   implementation;
* ``policy``    -- the per-tile precision of every query-key score tile under
                   the two policy encodings (two diagonal-distance boundaries,
                   or a packed group bitmask), by brute-force enumeration;
* ``attention`` -- prefill attention as a plain softmax over each row's
                   executed keys (the fixed point that any online-softmax
                   traversal reaches up to rounding), the integer tile scores,
                   and decode attention over the compressed cache.

Sources (the method pages):
  [TriAttention] "TriAttention: Unified Sparse Mixed-Precision Attention for
      Long-Context LLM Inference", abstract (aitop.news item page).
  [TileMix] "TileMix: Tile-Centric Mixed-Precision Attention for LLM Inference
      Acceleration", abstract (chatpaper.ai page; restated on the lapresse
      commentary page).
  [HyQuant] "HyQuant Uses Hybrid Precision to Compress LLM Attention",
      section "How HyQuant works" (cctest.ai article).

Where the pages are silent, the readings taken are listed in each function's
docstring (policy semantics, quantizer rounding, decode tags).

Parity status: every function is pinned by tests under ``tests/`` that check it
against closed forms, library routines on special cases, hand-worked fixtures
in ``tests/golden/`` and exact-arithmetic brute force; see the test module
docstrings.
"""
from . import quant, policy, attention  # noqa: F401

SKIP, INT4, INT8, FP16 = 0, 1, 2, 3
