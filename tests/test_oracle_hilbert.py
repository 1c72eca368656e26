"""Pins for the oracle's Hilbert keys (oracle/hilbert.py).

What fixes a Hilbert curve: it visits every cell of the 2^b grid exactly once
(bijection), consecutive cells share a face (unit step along one axis), it
starts at the origin, the first 1/8 of the curve fills one octant that
contains the origin (self-similarity), and it ends at a corner one box edge
away from the start.  A Morton (Z) order, a dropped Gray step or a wrong bit
order breaks at least the adjacency test.
"""
import numpy as np
import pytest

from oracle import hilbert


def _all_cells(b):
    g = np.arange(1 << b, dtype=np.uint32)
    gx, gy, gz = np.meshgrid(g, g, g, indexing="ij")
    return gx.ravel(), gy.ravel(), gz.ravel()


@pytest.mark.parametrize("b", [1, 2, 3, 4, 5])
def test_bijection_and_adjacency(b):
    gx, gy, gz = _all_cells(b)
    key = hilbert.hilbert_index(gx, gy, gz, b)
    n = 1 << (3 * b)
    assert key.max() == n - 1
    assert np.unique(key).size == n
    order = np.argsort(key)
    pts = np.stack([gx, gy, gz], 1)[order].astype(np.int64)
    step = np.abs(np.diff(pts, axis=0))
    assert np.all(step.sum(1) == 1), "consecutive keys must be face-adjacent cells"
    assert np.all(pts[0] == 0)
    # ends at a corner one box edge away from the origin
    last = pts[-1]
    assert sorted(last.tolist()) == [0, 0, (1 << b) - 1]
    if b > 1:
        first_oct = pts[: n // 8]
        assert np.all(first_oct < (1 << (b - 1))), "first eighth must fill the origin octant"


def test_default_bits_range():
    key = hilbert.hilbert_index(np.array([1023], np.uint32), np.array([1023], np.uint32),
                                np.array([1023], np.uint32))
    assert key.dtype == np.uint32 and int(key[0]) < (1 << 30)


def test_quantize_edges():
    L = np.float32(10.0)
    x = np.array([[0.0, 9.99999, 5.0]], np.float32)
    g = hilbert.quantize(x, L)
    assert g.tolist() == [[0, 1023, 512]]
