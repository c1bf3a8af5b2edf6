"""Where a (token row, channel) of one KV tile lives in a cache page.

The pages fix only that the cache is written by the prologue and read in
64-token tiles (page A, "Why does dynamic scheduling matter in attention?");
they say nothing about its layout (reading R6).  The library defines its own
page layout, and this module restates that definition independently:

* A page holds 64 consecutive tokens of one sequence (one tile).  Within a
  pool, element (page p, KV head g, row r, channel d) is at
  ``p*page_stride + g*head_stride + tile_offset(kind, dtype, r, d)``.
* A tile is 64 x 128 elements (8192), stored as contiguous 1 KiB fragments.
  Inside a fragment, 64 "lanes" of 16 bytes follow each other.

K tile, BF16 (16 fragments of 64 lanes x 8 elements)::

    tb = r // 16, s = d // 32, kc = (d % 32) // 8, e = d % 8
    offset = 512*(4*tb + s) + 8*(16*kc + r % 16) + e

V tile, BF16 (16 fragments)::

    tb = r // 16, db = d // 16, kc = (r % 16) // 4
    e  = 4*(tb % 2) + r % 4
    offset = 512*(2*db + tb // 2) + 8*(16*kc + d % 16) + e

K tile, FP8 (8 fragments of 64 lanes x 16 bytes)::

    tb, s, kc as for BF16 K
    offset = 1024*(2*tb + s // 2) + 16*(16*kc + r % 16) + 8*(s % 2) + d % 8

V tile, FP8 (8 fragments)::

    db, kc, e as for BF16 V
    offset = 1024*db + 16*(16*kc + d % 16) + 8*(tb // 2) + e

(Why this order is the kernel's business, not the oracle's: the oracle only
needs to find an element.)
"""

import numpy as np

PAGE_SIZE = 64
HEAD_DIM = 128
TILE_ELEMS = PAGE_SIZE * HEAD_DIM


def tile_offset(kind, dtype, r, d):
    """Element offset of (row r, channel d) inside one tile.

    kind: "k" or "v"; dtype: "bf16" or "fp8".  r and d may be numpy arrays
    (broadcast together).  Offsets count elements of the cache dtype.
    """
    r = np.asarray(r, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    if np.any((r < 0) | (r >= PAGE_SIZE)) or np.any((d < 0) | (d >= HEAD_DIM)):
        raise ValueError("row or channel outside the tile")
    tb = r // 16
    if kind == "k":
        s = d // 32
        kc = (d % 32) // 8
        if dtype == "bf16":
            return 512 * (4 * tb + s) + 8 * (16 * kc + r % 16) + d % 8
        if dtype == "fp8":
            return 1024 * (2 * tb + s // 2) + 16 * (16 * kc + r % 16) + 8 * (s % 2) + d % 8
    elif kind == "v":
        db = d // 16
        kc = (r % 16) // 4
        e = 4 * (tb % 2) + r % 4
        if dtype == "bf16":
            return 512 * (2 * db + tb // 2) + 8 * (16 * kc + d % 16) + e
        if dtype == "fp8":
            return 1024 * db + 16 * (16 * kc + d % 16) + 8 * (tb // 2) + e
    raise ValueError(f"unknown tile kind/dtype {kind!r}/{dtype!r}")


def tile_to_rows(kind, dtype, tile):
    """Reorder one flat tile (8192 elements) into logical [64 rows][128 channels]."""
    r, d = np.meshgrid(np.arange(PAGE_SIZE), np.arange(HEAD_DIM), indexing="ij")
    return np.asarray(tile)[tile_offset(kind, dtype, r, d)]
