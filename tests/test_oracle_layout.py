"""Pins for the oracle's page-layout function: hand-derived offsets and bijection."""

import os

import numpy as np
import pytest

from oracle import tile_offset, TILE_ELEMS
from oracle.layout import tile_to_rows


def test_hand_derived_offsets(golden_dir):
    n = 0
    with open(os.path.join(golden_dir, "tile_layout_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, dtype, r, d, off = line.split()
            assert int(tile_offset(kind, dtype, int(r), int(d))) == int(off), line
            n += 1
    assert n >= 30


@pytest.mark.parametrize("kind", ["k", "v"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_layout_is_a_bijection(kind, dtype):
    r, d = np.meshgrid(np.arange(64), np.arange(128), indexing="ij")
    off = tile_offset(kind, dtype, r, d).reshape(-1)
    assert off.min() == 0 and off.max() == TILE_ELEMS - 1
    assert np.unique(off).size == TILE_ELEMS


@pytest.mark.parametrize("dtype,lane_bytes", [("bf16", 16), ("fp8", 16)])
def test_k_lane_holds_consecutive_channels_of_one_row(dtype, lane_bytes):
    """Each 16-byte lane of a K fragment is 8 consecutive channels of one row
    (BF16) or two runs of 8 (FP8), i.e. the unit one MFMA operand needs."""
    esz = 2 if dtype == "bf16" else 1
    per_lane = lane_bytes // esz
    r, d = np.meshgrid(np.arange(64), np.arange(128), indexing="ij")
    off = tile_offset("k", dtype, r, d)
    inv_r = np.empty(TILE_ELEMS, dtype=np.int64)
    inv_d = np.empty(TILE_ELEMS, dtype=np.int64)
    inv_r[off.reshape(-1)] = r.reshape(-1)
    inv_d[off.reshape(-1)] = d.reshape(-1)
    lanes_r = inv_r.reshape(-1, per_lane)
    lanes_d = inv_d.reshape(-1, 8)
    assert np.all(lanes_r == lanes_r[:, :1])
    assert np.all(np.diff(lanes_d, axis=1) == 1)


def test_tile_to_rows_round_trip():
    rng = np.random.default_rng(0)
    rows = rng.standard_normal((64, 128))
    for kind in ("k", "v"):
        for dtype in ("bf16", "fp8"):
            flat = np.empty(TILE_ELEMS)
            r, d = np.meshgrid(np.arange(64), np.arange(128), indexing="ij")
            flat[tile_offset(kind, dtype, r, d)] = rows
            assert np.array_equal(tile_to_rows(kind, dtype, flat), rows)


def test_out_of_tile_raises():
    with pytest.raises(ValueError):
        tile_offset("k", "bf16", 64, 0)
    with pytest.raises(ValueError):
        tile_offset("v", "fp8", 0, 128)
