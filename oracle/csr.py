"""Per-query-tile lists of active key tiles (oracle; test infrastructure).

CalibAtt page, B. Fase di Inferenza: the kernel is handed precomputed lists of
the blocks each query block may skip and computes only the rest.  The library
stores the complement, the active list, in compressed-sparse-row form over the
[Hm*Tq, Tk] tile mask viewed as a matrix with rows r = h*Tq + i:

  row_ptr[0] = 0,  row_ptr[r+1] = row_ptr[r] + (number of active j in row r)
  col_idx[row_ptr[r] : row_ptr[r+1]] = the active j of row r, ascending.
"""
from __future__ import annotations

import numpy as np


def tile_csr(mask: np.ndarray):
    """(row_ptr int32 [R+1], col_idx int32 [nnz]) of a [Hm, Tq, Tk] mask."""
    Hm, Tq, Tk = mask.shape
    rows = mask.reshape(Hm * Tq, Tk) != 0
    row_ptr = np.zeros(Hm * Tq + 1, dtype=np.int64)
    cols = []
    for r in range(Hm * Tq):
        active = [j for j in range(Tk) if rows[r, j]]
        cols.extend(active)
        row_ptr[r + 1] = row_ptr[r] + len(active)
    return row_ptr.astype(np.int32), np.asarray(cols, dtype=np.int32)
