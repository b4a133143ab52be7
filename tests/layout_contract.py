"""Expected buffer layouts of the library's spread anchor-row path.

Not the method: the CalibAtt page ("B. Fase di Inferenza") has a repetitive
head compute attention for its anchor rows and copy the result to the rows
they stand for; where those rows sit in the working buffer is the library's
own choice, made for speed only.  The library packs the anchor rows' tokens
(frame by frame, row by row) and either keeps them at the front of the
buffer or cuts them into blocks of `block_rows` rows spread evenly over it.
These helpers state that contract for the tests of `bsattn_anchor_rows`
(spread gather/broadcast) and of the spread dense-rows mask kind; the oracle
never uses them, and the output of the repeated attention is layout-free.
"""
from __future__ import annotations

import numpy as np


def block_slots(count: int, slots: int) -> list[int]:
    """Slot of block g = 0 .. count-1 when `count` blocks are spread evenly
    over `slots` slots: floor(g * slots / count)."""
    if count > slots:
        raise ValueError("the blocks do not fit the block slots")
    return [g * slots // count for g in range(count)]


def anchor_buffer_rows(na: int, n: int, block_rows: int) -> np.ndarray:
    """Buffer row of each packed anchor index a = 0 .. na-1 in a buffer of n
    rows: a itself when block_rows is 0 (packed at the front); otherwise the
    packed rows are cut into blocks of block_rows (the last one shorter if
    need be) and block g starts at row slot(g) * block_rows, with
    ceil(na / block_rows) blocks over ceil(n / block_rows) slots."""
    if na > n:
        raise ValueError("more anchor rows than rows")
    if block_rows == 0:
        return np.arange(na, dtype=np.int64)
    rg = -(-na // block_rows)
    pg = -(-n // block_rows)
    rows = []
    for g, slot in enumerate(block_slots(rg, pg)):
        size = min(block_rows, na - g * block_rows)
        rows.extend(range(slot * block_rows, slot * block_rows + size))
    return np.asarray(rows, dtype=np.int64)


def dense_rows_mask(Hm: int, N: int, tile: int, query_tiles: int) -> np.ndarray:
    """uint8 [Hm, Tq, Tq]: query tiles 0 .. query_tiles-1 (the anchor rows
    packed at the front) are all ones, every other row all zeros."""
    if query_tiles < 0:
        raise ValueError("query_tiles must be >= 0")
    Tq = -(-N // tile)
    M = np.zeros((Hm, Tq, Tq), dtype=np.uint8)
    M[:, :query_tiles, :] = 1
    return M


def spread_dense_rows_mask(Hm: int, N: int, tile: int, query_tiles: int,
                           block_tiles: int) -> np.ndarray:
    """uint8 [Hm, Tq, Tq]: the query tiles that hold the spread anchor rows
    are all ones, every other row all zeros.  The query_tiles dense tiles
    form blocks of block_tiles tiles spread over ceil(Tq / block_tiles)
    slots as above."""
    if query_tiles < 0 or block_tiles < 1:
        raise ValueError("query_tiles >= 0 and block_tiles >= 1 required")
    Tq = -(-N // tile)
    rg = -(-query_tiles // block_tiles)
    pg = -(-Tq // block_tiles)
    M = np.zeros((Hm, Tq, Tq), dtype=np.uint8)
    for g, slot in enumerate(block_slots(rg, pg)):
        size = min(block_tiles, query_tiles - g * block_tiles)
        M[:, slot * block_tiles:slot * block_tiles + size, :] = 1
    return M
