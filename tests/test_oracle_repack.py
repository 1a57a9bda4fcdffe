"""Pins of the oracle's planar weight layout (CPU only).

The layout ("#3455 [Engine] GP100 (sm_60): 4-bit slots ...", "Approach": a load-time rewrite of
resident blocks, rebuilt and compared byte for byte): per row, every block's code bytes in block
order, then every block's scale bytes (fp16 scale, then CB2 / CB3 sub-scales). Pinned to closed
forms on rows whose bytes are their own offsets, and to the round trip on random rows.
"""
import numpy as np
import pytest

import oracle
from moe_routed_expert_route_amd import synth

Q8_0, NL4, CB2, CB3, Q5_1, NL4X = 1, 2, 3, 4, 5, 6


def _r(a, b):
    return list(range(a, b))


@pytest.mark.parametrize("fmt,ncols,expect", [
    # two Q8_0 blocks of 34 bytes: codes 2..33 and 36..67, then scales 0,1 and 34,35
    (Q8_0, 64, _r(2, 34) + _r(36, 68) + [0, 1, 34, 35]),
    # two NL4 blocks of 18 bytes
    (NL4, 64, _r(2, 18) + _r(20, 36) + [0, 1, 18, 19]),
    # two Q5_1 blocks of 24 bytes: high bits and nibbles 4..23, 28..47, then d, m of each
    (Q5_1, 64, _r(4, 24) + _r(28, 48) + [0, 1, 2, 3, 24, 25, 26, 27]),
    # one NL4X super-block: its 128 nibble bytes 8..135, then its 8 header bytes
    (NL4X, 256, _r(8, 136) + _r(0, 8)),
    # one CB2 super-block: index and sign bytes 2..65, then D 0,1 and sub-scales 66..69
    (CB2, 256, _r(2, 66) + [0, 1] + _r(66, 70)),
    # one CB3 super-block: low-index, high-bit and sign bytes 2..105, then D and sub-scales
    (CB3, 256, _r(2, 106) + [0, 1] + _r(106, 110)),
])
def test_planar_closed_form(fmt, ncols, expect):
    rb = oracle.row_bytes(fmt, ncols)
    row = np.arange(rb, dtype=np.uint8)
    got = oracle.repack(fmt, row, 1, ncols, True)
    assert got.tolist() == expect
    assert oracle.repack(fmt, got, 1, ncols, False).tolist() == row.tolist()


def test_planar_two_cb3_blocks():
    # codes of both super-blocks first, then (D, sub-scales) of each
    row = np.arange(220, dtype=np.uint8)
    got = oracle.repack(CB3, row, 1, 512, True).tolist()
    assert got == _r(2, 106) + _r(112, 216) + [0, 1] + _r(106, 110) + [110, 111] + _r(216, 220)


@pytest.mark.parametrize("fmt,ncols", [(Q8_0, 256), (NL4, 192), (CB2, 768), (CB3, 512), (Q5_1, 128), (NL4X, 512)])
def test_planar_round_trip_and_permutation(fmt, ncols):
    rows = 5
    m = synth.rng(61, fmt).integers(0, 256, size=rows * oracle.row_bytes(fmt, ncols), dtype=np.uint8)
    p = oracle.repack(fmt, m, rows, ncols, True)
    assert p.shape == m.shape and not np.array_equal(p, m)
    rb = oracle.row_bytes(fmt, ncols)
    for r in range(rows):   # each row is a permutation of its own bytes
        assert np.array_equal(np.sort(p[r * rb:(r + 1) * rb]), np.sort(m[r * rb:(r + 1) * rb]))
    assert np.array_equal(oracle.repack(fmt, p, rows, ncols, False), m)
