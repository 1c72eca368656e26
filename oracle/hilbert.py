"""Hilbert space-filling-curve keys (oracle).

The Tessera abstract ("Ab Initio Accuracy Beyond the Cutoff", Abstract) sorts
atoms along a space-filling curve and contrasts it with Morton order.  The
curve used here is the Hilbert curve in J. Skilling's transpose formulation
("Programming the Hilbert curve", AIP Conf. Proc. 707, 2004): the axes are
turned into the "transposed" Hilbert index by an inverse-undo sweep followed by
a Gray encode, then the index bits are read out level by level from the most
significant, axis 0 (x) first within each 3-bit group.
"""
import numpy as np

BITS = 10


def axes_to_transpose(gx, gy, gz, bits=BITS):
    """Skilling's AxesToTranspose for three axes, vectorised over atoms."""
    X = [np.asarray(gx, np.uint32).copy(), np.asarray(gy, np.uint32).copy(),
         np.asarray(gz, np.uint32).copy()]
    n = 3
    top = np.uint32(1 << (bits - 1))
    # inverse undo: walk the levels from the top; at each level either invert
    # the lower bits of axis 0 or exchange the lower bits of axis 0 and axis i
    q = top
    while q > 1:
        low = np.uint32(q - 1)
        for i in range(n):
            set_ = (X[i] & q) != 0
            if i == 0:
                X[0] = np.where(set_, X[0] ^ low, X[0])
            else:
                t = (X[0] ^ X[i]) & low
                X[0] = np.where(set_, X[0] ^ low, X[0] ^ t)
                X[i] = np.where(set_, X[i], X[i] ^ t)
        q = np.uint32(q >> 1)
    # Gray encode
    for i in range(1, n):
        X[i] = X[i] ^ X[i - 1]
    t = np.zeros_like(X[0])
    q = top
    while q > 1:
        t = np.where((X[n - 1] & q) != 0, t ^ np.uint32(q - 1), t)
        q = np.uint32(q >> 1)
    for i in range(n):
        X[i] = X[i] ^ t
    return X


def hilbert_index(gx, gy, gz, bits=BITS):
    """3*bits-bit key: transposed bits interleaved MSB first, x most significant per group."""
    X = axes_to_transpose(gx, gy, gz, bits)
    key = np.zeros(np.asarray(gx).shape, np.uint64)
    for lev in range(bits - 1, -1, -1):
        for a in range(3):
            key = (key << np.uint64(1)) | ((X[a] >> np.uint32(lev)) & np.uint32(1)).astype(np.uint64)
    return key.astype(np.uint32)


def morton_index(gx, gy, gz, bits=BITS):
    """Z-order key (for the curve comparison of the Tessera abstract): the coordinate bits
    interleaved level by level from the most significant, x first within each 3-bit group."""
    key = np.zeros(np.asarray(gx).shape, np.uint64)
    for lev in range(bits - 1, -1, -1):
        for g in (gx, gy, gz):
            key = (key << np.uint64(1)) | ((np.asarray(g, np.uint32) >> np.uint32(lev)) & np.uint32(1)).astype(
                np.uint64)
    return key.astype(np.uint32)


def quantize(xf, L, bits=BITS):
    """Cell coordinates g_a = min(2^b - 1, floor(x_a * 2^b / L)), evaluated in float64."""
    S = float(1 << bits) / float(np.float32(L))
    g = np.floor(np.asarray(xf, np.float32).astype(np.float64) * S)
    g = np.minimum(g, float((1 << bits) - 1))
    return g.astype(np.uint32)
