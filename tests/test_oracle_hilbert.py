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


def _spread(v, bits):
    # bit i of v moved to bit 3 i (integer arithmetic, independent of the oracle's loop)
    return sum(((int(v) >> i) & 1) << (3 * i) for i in range(bits))


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_morton_closed_form_and_bijection(b):
    """Z-order key = spread(x) << 2 | spread(y) << 1 | spread(z); a bijection on the cells;
    each aligned 2x2x2 block occupies 8 consecutive keys."""
    from oracle import hilbert
    g = np.arange(1 << b)
    gx, gy, gz = [a.ravel() for a in np.meshgrid(g, g, g, indexing="ij")]
    k = hilbert.morton_index(gx, gy, gz, bits=b)
    ref = np.array([(_spread(x, b) << 2) | (_spread(y, b) << 1) | _spread(z, b) for x, y, z in zip(gx, gy, gz)])
    assert (k.astype(np.int64) == ref).all()
    assert np.array_equal(np.sort(k), np.arange(1 << (3 * b)))
    half = np.array([(_spread(x >> 1, b) << 2) | (_spread(y >> 1, b) << 1) | _spread(z >> 1, b)
                     for x, y, z in zip(gx, gy, gz)])
    assert (k.astype(np.int64) >> 3 == half).all()


@pytest.mark.parametrize("order", ["morton", "input"])
def test_other_orders_give_the_same_graph(order):
    """Any atom order lists the same pairs: mapped back to input indices, the edge set
    equals the Hilbert-ordered one; input order keeps perm = identity."""
    from oracle import neighbors as NB
    rng = np.random.default_rng(3)
    L = 14.0
    x = (rng.random((300, 3)) * L).astype(np.float32)
    a = NB.build_neighbors(x, L, 3.0, 0.5)
    b = NB.build_neighbors(x, L, 3.0, 0.5, order=order)
    if order == "input":
        assert np.array_equal(b["perm"], np.arange(300))

    def pairs(nb):
        src = np.repeat(np.arange(300), np.diff(nb["row_ptr"]))
        return set(zip(nb["perm"][src].tolist(), nb["perm"][nb["col"]].tolist()))
    assert pairs(a) == pairs(b)
    # rows ascending, rev an involution pairing (s -> t) with (t -> s)
    rp, col, rev = b["row_ptr"], b["col"], b["rev"]
    src = np.repeat(np.arange(300), np.diff(rp))
    assert all((np.diff(col[rp[s]:rp[s + 1]]) > 0).all() for s in range(300))
    assert np.array_equal(rev[rev], np.arange(len(col)))
    assert np.array_equal(src[rev], col)
