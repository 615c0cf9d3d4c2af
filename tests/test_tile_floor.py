"""Integer pins for the KV-tile floor and ceiling (the visited-tile set).

The oracle's tile_range() is the formula from the pages (hip-ep #622 "window
in v5"; sglang #34468 "bound the stage-1 prefix loop"): the first row's
lowest kept key fixes the floor, the last row's diagonal key the ceiling.
These tests pin it against a brute-force scan of the mask, the worked
example sglang #34468 prints, the ceil/floor identity that page relies on,
and the "flat in KV depth" property hip-ep #622 measures.
"""
import json
import os

import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sglang_34468_tile_counts.json")

# windows of sglang #34468's sweep (in its W convention, ours is W + 1 keys)
# plus hip-ep #622's window 100 and 128, and "no window"
WINDOWS = [-1, 1, 2, 15, 16, 17, 63, 64, 65, 100, 127, 128, 129, 130, 191, 192, 193, 255,
           256, 257, 1023, 1024, 4096]
PREFIXES = [0, 1, 31, 63, 64, 65, 127, 128, 129, 200, 513]
EXTENDS = [1, 5, 64, 100, 129]
TILINGS = [(16, 64), (32, 32), (32, 64), (64, 64), (64, 128), (128, 64), (128, 128), (8, 16)]


@pytest.mark.parametrize("bm,bkv", TILINGS)
def test_floor_is_conservative_and_tight(bm, bkv):
    """Every tile in [t_lo, t_hi] holds a kept key and no tile outside does."""
    mismatches = 0
    checked = 0
    for window in WINDOWS:
        for past in PREFIXES:
            for sq in EXTENDS:
                skv = past + sq
                n_tiles = (skv + bkv - 1) // bkv
                for q0 in range(0, sq, bm):
                    q1 = min(q0 + bm, sq) - 1
                    lo, hi = oracle.tile_range(past, q0, q1, window, bkv)
                    for t in range(n_tiles):
                        has = oracle.tile_has_kept(past, sq, q0, q1, window, bkv, t)
                        mismatches += has != (lo <= t <= hi)
                        checked += 1
    assert checked > 0
    assert mismatches == 0


def test_ceil_floor_identity_every_residue():
    # sglang #34468: ceil((A - BN + 1) / BN) == A // BN for every residue
    for bn in (16, 32, 64, 128):
        for a in range(-3 * bn, 5 * bn):
            num = a - bn + 1
            ceil = -((-num) // bn)
            assert ceil == a // bn


def _count(past, sq, bm, window, bkv):
    total = 0
    for q0 in range(0, sq, bm):
        lo, hi = oracle.tile_range(past, q0, min(q0 + bm, sq) - 1, window, bkv)
        total += hi - lo + 1
    return total


def test_worked_example_382_to_256():
    g = json.load(open(GOLDEN))
    prefix, extend, bm, bkv, window = g["prefix"], g["extend"], g["block_m"], g["block_n"], \
        g["window"]
    # one loop over prefix + extend keys, floored: the count after the change
    assert _count(prefix, extend, bm, window, bkv) == g["tiles_with_floor"]
    # before: every prefix tile walked by every m-block, extend tiles floored
    # on their own (keys re-indexed from the extend start)
    n_mblocks = (extend + bm - 1) // bm
    prefix_tiles = n_mblocks * ((prefix + bkv - 1) // bkv)
    extend_tiles = _count(0, extend, bm, window, bkv)
    assert prefix_tiles + extend_tiles == g["tiles_without_prefix_floor"]


def test_flat_in_kv_depth():
    # hip-ep #622: with window 128 the tiles a block walks stop growing with
    # the KV length once the window is filled (chunk 512 at past 512 vs 8192)
    a = _count(512, 512, 128, 128, 64)
    b = _count(8192, 512, 128, 128, 64)
    assert a == b == 16
    full_a = _count(512, 512, 128, -1, 64)
    full_b = _count(8192, 512, 128, -1, 64)
    assert full_b > full_a


def test_floor_empties_prefix_once_block_passes_window():
    # sglang #34468: once the m-block start reaches the window, no row of the
    # block sees any prefix key (floor >= prefix)
    prefix, bkv, window = 4096, 64, 129
    for q0 in range(0, 2048, 128):
        lo, _ = oracle.tile_range(prefix, q0, q0 + 127, window, bkv)
        if q0 >= window - 1:
            assert lo * bkv >= prefix - bkv + 1
