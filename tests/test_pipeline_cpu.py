"""Host-side checks of the device-buffer plumbing that need no GPU: buffers on
the CPU device, only size queries and validation reach the library."""
import numpy as np
import pytest


@pytest.fixture(scope="module")
def T():
    import os
    from tile_routed_mixed_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from tile_routed_mixed_amd import build
        build.build()
    import tile_routed_mixed_amd as T
    return T


def test_append_rejects_full_sequences_before_touching_buffers(T):
    """A sequence at its capacity cannot take another token: append raises
    before it writes a row or changes the lengths (the row it would write
    belongs to the next sequence, or lies past the buffer for the last one)."""
    dpol = dict(b8=[2], b4=[5], sink=1, tail=128)
    p = T.DecodePipeline([100, 70], 2, 1, 64, dpol, device="cpu")
    p.dpol.set_lengths(np.array([99, 70], np.int32))
    k_rows = np.zeros((2, 1, 64), np.uint16)
    with pytest.raises(ValueError, match=r"\[1\]"):
        p.append(k_rows, k_rows)
    assert p.dpol.lengths.tolist() == [99, 70]


def test_set_selection_drops_the_old_device_buffer(T):
    """New selection lists invalidate the gathered-tile buffer built for the
    old ones: the policy no longer points at it, so tm_decode refuses to run
    until tm_decode_select has built a buffer for the new lists."""
    d = T._binding.DPolicy(dict(b8=[2], b4=[5], sink=1, tail=128))
    d.sel_buf = object()
    d.c.sel_buf = 0x10000
    d.set_selection(np.array([0, 1, 2], np.int32), np.array([3, 4], np.int32))
    assert d.sel_buf is None and not d.c.sel_buf
