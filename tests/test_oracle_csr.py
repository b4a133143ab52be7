"""Pins for the oracle's per-query-tile active lists (CPU only)."""
import numpy as np

import oracle


def _check_csr(mask, row_ptr, col_idx):
    R = mask.shape[0] * mask.shape[1]
    Tk = mask.shape[2]
    flat = mask.reshape(R, Tk)
    assert row_ptr.dtype == np.int32 and col_idx.dtype == np.int32
    assert row_ptr[0] == 0 and len(row_ptr) == R + 1
    assert (np.diff(row_ptr) >= 0).all()
    assert row_ptr[-1] == int(flat.astype(np.int64).sum()) == len(col_idx)
    for r in range(R):
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        assert (np.diff(cols) > 0).all()              # strictly ascending
        assert all(flat[r, j] == 1 for j in cols)     # only active tiles
        assert len(cols) == int(flat[r].sum())        # and all of them


def test_csr_hand_example():
    mask = np.array([[[1, 0, 1], [0, 0, 0], [1, 1, 1]],
                     [[0, 1, 0], [1, 0, 0], [0, 0, 1]]], dtype=np.uint8)
    rp, ci = oracle.tile_csr(mask)
    assert rp.tolist() == [0, 2, 2, 5, 6, 7, 8]
    assert ci.tolist() == [0, 2, 0, 1, 2, 1, 0, 2]


def test_csr_invariants_on_configs():
    masks = [
        oracle.tile_mask_window_anchor(21, 30, 52, 128, 1, 2, 7)[None],
        oracle.tile_mask_static(3, 40, 33, 5, 1 << 22, True),
        oracle.tile_mask_static(2, 17, 17, 11, 0, False),  # all rows empty
        oracle.tile_mask_dense(1, 9, 9),
    ]
    for m in masks:
        rp, ci = oracle.tile_csr(m)
        _check_csr(m, rp, ci)


def test_csr_round_trip():
    m = oracle.tile_mask_static(2, 31, 29, 123, 1 << 23, False)
    rp, ci = oracle.tile_csr(m)
    back = np.zeros((2 * 31, 29), dtype=np.uint8)
    for r in range(2 * 31):
        back[r, ci[rp[r]:rp[r + 1]]] = 1
    np.testing.assert_array_equal(back.reshape(m.shape), m)
