"""CPU oracle for token reordering along a 3-D Hilbert curve (test infrastructure only).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module.  The product path never calls it.

The pages note that reordering the tokens along a Hilbert curve (or a similar
order) makes the tokens that share a 64-token block more alike, which raises the
sparsity the block prediction finds ("2025稀疏注意力架构综述", section 11
SpargeAttn, the token-reordering remark).  The pages fix no curve variant, so the
reading here is the plainest one with a published definition: Skilling's
transform from axes to the transposed Hilbert index (J. Skilling, "Programming
the Hilbert curve", AIP Conf. Proc. 707, 2004), on the cube of side 2^b that
holds the latent grid, with the coordinates taken in the order (t, h, w).

The order of a T x H x W grid (tokens stored row-major, index (t H + h) W + w):
the valid cells sorted by their Hilbert index; order[n] = the row-major index of
the token placed at position n.  Reordering a tensor: X_r[n] = X[order[n]];
restoring: X[order[n]] = X_r[n].
"""
from __future__ import annotations

from typing import List

import numpy as np


def axes_to_transpose(x: List[int], bits: int) -> List[int]:
    """Skilling's transform of n coordinates (each < 2^bits) to the transposed Hilbert index.

    Two passes: undo the excess work of the recursive construction level by level
    (for each bit Q from the top down, coordinate i either inverts the low bits of
    coordinate 0 or exchanges low bits with it), then Gray-encode across coordinates.
    """
    x = list(x)
    n = len(x)
    q = 1 << (bits - 1)
    while q > 1:
        p = q - 1
        for i in range(n):
            if x[i] & q:
                x[0] ^= p
            else:
                t = (x[0] ^ x[i]) & p
                x[0] ^= t
                x[i] ^= t
        q >>= 1
    for i in range(1, n):
        x[i] ^= x[i - 1]
    t = 0
    q = 1 << (bits - 1)
    while q > 1:
        if x[n - 1] & q:
            t ^= q - 1
        q >>= 1
    for i in range(n):
        x[i] ^= t
    return x


def hilbert_index(coords: List[int], bits: int) -> int:
    """The Hilbert index: the bits of the transposed form read level by level from the top,
    coordinate 0 first within a level."""
    xt = axes_to_transpose(coords, bits)
    h = 0
    for level in range(bits - 1, -1, -1):
        for v in xt:
            h = (h << 1) | ((v >> level) & 1)
    return h


def cube_bits(*dims: int) -> int:
    """Smallest b >= 1 with 2^b >= every dimension."""
    b = 1
    while (1 << b) < max(dims):
        b += 1
    return b


def hilbert_order(T: int, H: int, W: int) -> np.ndarray:
    """order[n] = row-major index of the n-th token along the curve (int64, length T H W)."""
    bits = cube_bits(T, H, W)
    keys = []
    for t in range(T):
        for h in range(H):
            for w in range(W):
                keys.append((hilbert_index([t, h, w], bits), (t * H + h) * W + w))
    keys.sort()
    return np.array([idx for _, idx in keys], dtype=np.int64)


def reorder(X: np.ndarray, order: np.ndarray) -> np.ndarray:
    """X_r[..., n, :] = X[..., order[n], :] for n < len(order); later rows unchanged."""
    out = X.copy()
    out[..., :len(order), :] = X[..., order, :]
    return out


def restore(Xr: np.ndarray, order: np.ndarray) -> np.ndarray:
    """The inverse: X[..., order[n], :] = Xr[..., n, :] for n < len(order); later rows unchanged."""
    out = Xr.copy()
    out[..., order, :] = Xr[..., :len(order), :]
    return out
