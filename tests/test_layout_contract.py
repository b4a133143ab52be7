"""The spread anchor-row layout contract (tests/layout_contract.py), checked
by hand: which buffer rows and which dense query tiles the spread layout
uses.  CPU only."""
import numpy as np
import pytest

from layout_contract import anchor_buffer_rows, dense_rows_mask, spread_dense_rows_mask


def _dense_rows(N, tile, ta, bt):
    m = spread_dense_rows_mask(1, N, tile, ta, bt)[0]
    assert all(r.all() or not r.any() for r in m)     # whole rows on or off
    return m.any(axis=1).nonzero()[0].tolist()


def test_spread_dense_rows_by_hand():
    # 9 tiles, 3 dense in blocks of 2: Rg = 2 over Pg = 5 slots -> slots 0, 2
    assert _dense_rows(9 * 64, 64, 3, 2) == [0, 1, 4]
    # 6 tiles, 2 dense, blocks of 1: Rg = 2 over Pg = 6 -> slots 0, 3
    assert _dense_rows(6 * 64, 64, 2, 1) == [0, 3]
    # 8 tiles, 4 dense in blocks of 2: slots 0, 2
    assert _dense_rows(8 * 64, 64, 4, 2) == [0, 1, 4, 5]
    # 1000 tokens, tile 128: 8 tiles (the last partial), Pg = 4, Rg = 2
    assert _dense_rows(1000, 128, 3, 2) == [0, 1, 4]
    # 5 tiles, all dense in blocks of 2: Rg = Pg = 3, packed
    assert _dense_rows(5 * 64, 64, 5, 2) == [0, 1, 2, 3, 4]
    assert _dense_rows(8 * 64, 64, 0, 2) == []
    with pytest.raises(ValueError):       # 4 blocks, 3 slots
        spread_dense_rows_mask(1, 5 * 64, 64, 7, 2)
    with pytest.raises(ValueError):
        spread_dense_rows_mask(1, 5 * 64, 64, 1, 0)


def test_dense_rows_by_hand():
    got = dense_rows_mask(1, 300, 64, 2)[0]
    want = np.zeros((5, 5), dtype=np.uint8)
    want[:2] = 1
    np.testing.assert_array_equal(got, want)
    assert (dense_rows_mask(1, 300, 64, 0) == 0).all()
    assert (dense_rows_mask(1, 300, 64, 9) == 1).all()
    with pytest.raises(ValueError):
        dense_rows_mask(1, 300, 64, -1)


def test_spread_with_as_many_blocks_as_slots_is_the_packed_mask():
    np.testing.assert_array_equal(spread_dense_rows_mask(1, 5 * 64, 64, 4, 2),
                                  dense_rows_mask(1, 5 * 64, 64, 4))


def test_anchor_buffer_rows_by_hand():
    np.testing.assert_array_equal(anchor_buffer_rows(5, 12, 0), np.arange(5))
    # 5 rows in blocks of 2 over ceil(12 / 2) = 6 slots: Rg = 3 -> slots 0, 2, 4
    np.testing.assert_array_equal(anchor_buffer_rows(5, 12, 2), [0, 1, 4, 5, 8])
    # 4 rows in blocks of 2 over ceil(11 / 2) = 6 slots: slots 0, 3 (the
    # partial last slot, rows 10 .. 11, stays unused)
    np.testing.assert_array_equal(anchor_buffer_rows(4, 11, 2), [0, 1, 6, 7])
    # as many blocks as slots: packed at the front
    np.testing.assert_array_equal(anchor_buffer_rows(7, 7, 2), np.arange(7))
    with pytest.raises(ValueError):
        anchor_buffer_rows(8, 7, 2)   # more anchor rows than rows
    # rows are distinct, increasing and inside the buffer
    for na, n, b in [(300, 768, 128), (16380, 32760, 256), (1, 256, 256), (17, 40, 4)]:
        r = anchor_buffer_rows(na, n, b)
        assert len(r) == na and (np.diff(r) > 0).all() and r[-1] < n


def test_anchor_rows_occupy_the_spread_masks_dense_tiles():
    # 300 rows, tile 64, blocks of 2 tiles (128 rows), 768 tokens
    rows = anchor_buffer_rows(300, 768, 128)
    tiles = sorted(set((rows // 64).tolist()))
    m = spread_dense_rows_mask(1, 768, 64, -(-300 // 64), 2)[0]
    assert tiles == m.any(axis=1).nonzero()[0].tolist() == [0, 1, 4, 5, 8]
