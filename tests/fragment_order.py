"""Fragment order of weight matrices, written from its definition (the byte layout that
BEAM_MOE_LAYOUT_FRAGMENTS names): a matrix of R rows x B bytes is cut into blocks of 16 rows and
each block into column slices of W bytes (64 for weights, 16 for MXFP4 scales); slice f of block b
is stored as 16*W bytes at 16*B*b + 16*W*f, whose byte 16*(r + 16*c) + j is byte W*f + 16*c + j of
the block's row r.

A storage order only: nothing of the layer's arithmetic.  Two independent forms, pinned against each
other and against hand positions in test_layout.py: an index formula applied element by element, and
a reshape/transpose of the array."""
from __future__ import annotations

import numpy as np


def _as_rows(w: np.ndarray) -> np.ndarray:
    """w [..., cols] of any fixed-size dtype -> [rows, row_bytes] uint8."""
    w = np.ascontiguousarray(w)
    return w.view(np.uint8).reshape(-1, w.shape[-1] * w.itemsize)


def positions(R: int, B: int, W: int = 64) -> np.ndarray:
    """dst byte offset of each source byte (r, k) of an R x B matrix, from the definition."""
    r = np.arange(R)[:, None]
    k = np.arange(B)[None, :]
    b, rr = r // 16, r % 16
    f, rem = k // W, k % W
    c, j = rem // 16, rem % 16
    return 16 * B * b + 16 * W * f + 16 * (rr + 16 * c) + j


def pack_by_positions(w: np.ndarray, W: int = 64) -> np.ndarray:
    """Fragment order by scattering each byte to its position: same shape and dtype as w."""
    src = _as_rows(w)
    R, B = src.shape
    assert R % 16 == 0 and B % W == 0
    out = np.empty(R * B, np.uint8)
    out[positions(R, B, W).ravel()] = src.ravel()
    return out.view(w.dtype).reshape(w.shape)


def pack_by_reshape(w: np.ndarray, W: int = 64) -> np.ndarray:
    """Fragment order as an array transpose: [R/16, 16 rows, B/W slices, W/16 quarters, 16 bytes] ->
    [R/16, slices, quarters, rows, bytes]."""
    src = _as_rows(w)
    R, B = src.shape
    assert R % 16 == 0 and B % W == 0
    out = src.reshape(R // 16, 16, B // W, W // 16, 16).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(out).reshape(-1).view(w.dtype).reshape(w.shape)


def unpack(packed: np.ndarray, W: int = 64) -> np.ndarray:
    """Row order back from fragment order (the inverse gather)."""
    src = np.ascontiguousarray(packed).view(np.uint8).reshape(-1)
    R = packed.size // packed.shape[-1]
    B = packed.shape[-1] * packed.itemsize
    return src[positions(R, B, W).ravel()].view(packed.dtype).reshape(packed.shape)
