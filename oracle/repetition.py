"""Spatial repetition: detection by row similarity and attention computed on
anchor rows only (oracle; test infrastructure).

CalibAtt page, "A. Fase di Calibrazione", step 3, and "B. Fase di
Inferenza": in some heads the spatial rows of a frame attend in nearly the
same way.  Calibration measures the cosine similarity between spatial rows
within a frame and marks a head "repetitive" when it exceeds a threshold
gamma; at inference such a head computes attention only for a subset of
rows (the anchor rows) and copies their output to the other rows.

Readings taken where the page leaves a step open:
  * a spatial row is the grid_w tokens (f, y, x), x = 0 .. grid_w-1, of one
    latent row y of frame f (token n = f*P + y*grid_w + x);
  * anchor rows are every stride-th row of a frame, y = 0, s, 2s, ...; row y
    copies from its anchor a(y) = s * floor(y / s);
  * the attention pattern of a row is the grid_w x N matrix of its queries'
    softmax probabilities over all N keys (full attention); the similarity
    of row y is the cosine between its pattern and its anchor's, both
    flattened with the queries matched by x:
        cos(y) = sum_x <p_(y,x), p_(a,x)> / sqrt(sum_x |p_(y,x)|^2 *
                                                  sum_x |p_(a,x)|^2),
    1 for the anchor rows themselves;
  * a head is repetitive when the mean of cos(y) over the prompts (batch
    entries), frames and non-anchor rows, summed in float64 in that order,
    is >= gamma; a head whose frames have no non-anchor row is repetitive;
  * a repetitive head computes full softmax attention (all keys) for the
    anchor-row queries, the repetition taking the place of block skipping
    for that head, and o(f, y, x) = o(f, a(y), x);
  * in one layer (the inference of "B. Fase di Inferenza") the repetitive
    heads do that and every other head computes attention over its static
    block list.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _as_f64, block_sparse_attention_rows


def anchor_row(y: int, stride: int) -> int:
    return stride * (y // stride)


def _probabilities(q_rows, k, scale):
    s = (q_rows @ k.T) * scale
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


def _row_cosine(qbh, kbh, f: int, y: int, grid_h: int, grid_w: int, stride: int,
                scale: float) -> float:
    """cos(y) of frame f for one (prompt, head) slice ([N, d] float64)."""
    a = anchor_row(y, stride)
    if a == y:
        return 1.0
    P = grid_h * grid_w
    r0 = f * P + y * grid_w
    a0 = f * P + a * grid_w
    p1 = _probabilities(qbh[r0:r0 + grid_w], kbh, scale)
    p2 = _probabilities(qbh[a0:a0 + grid_w], kbh, scale)
    return float((p1 * p2).sum() / math.sqrt((p1 * p1).sum() * (p2 * p2).sum()))


def _check_grid(q, frames, grid_h, grid_w, stride, scale):
    B, H, N, d = q.shape
    if N != frames * grid_h * grid_w:
        raise ValueError("N must equal frames * grid_h * grid_w")
    if stride < 1:
        raise ValueError("stride must be >= 1")
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    return scale


def row_cosines(q, k, frames: int, grid_h: int, grid_w: int, stride: int,
                scale: float | None = None) -> np.ndarray:
    """cos[b, h, f, y] as defined above (float64)."""
    q, k = _as_f64(q), _as_f64(k)
    B, H = q.shape[:2]
    scale = _check_grid(q, frames, grid_h, grid_w, stride, scale)
    out = np.ones((B, H, frames, grid_h))
    for b in range(B):
        for h in range(H):
            for f in range(frames):
                for y in range(grid_h):
                    out[b, h, f, y] = _row_cosine(q[b, h], k[b, h], f, y, grid_h, grid_w,
                                                  stride, scale)
    return out


def row_cosines_at(q, k, frames: int, grid_h: int, grid_w: int, stride: int, cells,
                   scale: float | None = None) -> np.ndarray:
    """cos at the listed cells (b, h, f, y) only, in their order (float64):
    the same per-row arithmetic as row_cosines, for shapes whose every row
    would take too long."""
    scale = _check_grid(q, frames, grid_h, grid_w, stride, scale)
    out = np.empty(len(cells))
    cache = {}
    for i, (b, h, f, y) in enumerate(cells):
        if (b, h) not in cache:  # one float64 copy per slice
            cache = {(b, h): (_as_f64(q[b, h]), _as_f64(k[b, h]))}
        qbh, kbh = cache[(b, h)]
        out[i] = _row_cosine(qbh, kbh, f, y, grid_h, grid_w, stride, scale)
    return out


def repetitive_heads(cos, stride: int, gamma: float) -> np.ndarray:
    """uint8 [H]: 1 when the head's mean non-anchor row cosine is >= gamma
    (float64 sum over prompts, frames and rows in ascending order)."""
    c = np.asarray(cos, dtype=np.float32)
    B, H, T, gh = c.shape
    flags = np.zeros(H, dtype=np.uint8)
    for h in range(H):
        total = 0.0
        n = 0
        for b in range(B):
            for f in range(T):
                for y in range(gh):
                    if anchor_row(y, stride) != y:
                        total += float(c[b, h, f, y])
                        n += 1
        flags[h] = 1 if n == 0 or total / n >= float(gamma) else 0
    return flags


def anchor_count(grid_h: int, stride: int) -> int:
    """Anchor rows per frame."""
    return -(-grid_h // stride)


def gather_anchor_rows(x, frames: int, grid_h: int, grid_w: int,
                       stride: int) -> np.ndarray:
    """The anchor rows' tokens, frame by frame, row by row: [..., Na, d]."""
    x = np.asarray(x)
    P = grid_h * grid_w
    idx = [f * P + y * grid_w + xx for f in range(frames)
           for y in range(0, grid_h, stride) for xx in range(grid_w)]
    return x[..., idx, :]


def broadcast_anchor_rows(xa, frames: int, grid_h: int, grid_w: int,
                          stride: int) -> np.ndarray:
    """Every token takes its anchor row's value: [..., N, d] from the
    gathered [..., Na, d]."""
    xa = np.asarray(xa)
    na = anchor_count(grid_h, stride)
    idx = [f * na * grid_w + (y // stride) * grid_w + xx for f in range(frames)
           for y in range(grid_h) for xx in range(grid_w)]
    return xa[..., idx, :]


def repeated_attention(q, k, v, frames: int, grid_h: int, grid_w: int,
                       stride: int, scale: float | None = None) -> np.ndarray:
    """Full attention for the anchor-row queries, copied to their rows."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    qa = gather_anchor_rows(q, frames, grid_h, grid_w, stride)
    oa = np.zeros(qa.shape)
    for b in range(B):
        for h in range(H):
            oa[b, h] = _probabilities(qa[b, h], k[b, h], scale) @ v[b, h]
    return broadcast_anchor_rows(oa, frames, grid_h, grid_w, stride)


def mixed_heads_attention_rows(q, k, v, flags, mask, tile: int, frames: int,
                               grid_h: int, grid_w: int, stride: int, rows,
                               scale: float | None = None, workers: int = 1):
    """One inference layer, for the query rows `rows` of every head: a head
    with flags[h] set takes, for token (f, y, x), the full-attention output
    of its anchor token (f, a(y), x); every other head takes attention over
    its block list (mask [Hm, Tq, Tk], Hm in {1, H}).  Returns o
    [B, H, len(rows), d] (float64)."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q.shape
    P = grid_h * grid_w
    if N != frames * P:
        raise ValueError("N must equal frames * grid_h * grid_w")
    flags = np.asarray(flags)
    mask = np.asarray(mask)
    if flags.shape != (H,) or mask.shape[0] not in (1, H):
        raise ValueError("flags must be [H] and mask [1 or H, Tq, Tk]")
    rows = np.asarray(rows, dtype=np.int64)
    f, rem = rows // P, rows % P
    y, x = rem // grid_w, rem % grid_w
    anchors = f * P + stride * (y // stride) * grid_w + x
    dense = np.ones((1,) + mask.shape[1:], dtype=np.uint8)
    o = np.zeros((B, H, len(rows), v.shape[3]))
    for h in range(H):
        sl = slice(h, h + 1)
        if flags[h]:
            o[:, sl], _ = block_sparse_attention_rows(q[:, sl], k[:, sl], v[:, sl], dense, tile,
                                                      anchors, scale=scale, workers=workers)
        else:
            mh = mask[h if mask.shape[0] == H else 0][None]
            o[:, sl], _ = block_sparse_attention_rows(q[:, sl], k[:, sl], v[:, sl], mh, tile,
                                                      rows, scale=scale, workers=workers)
    return o


def mixed_heads_attention(q, k, v, flags, mask, tile: int, frames: int, grid_h: int,
                          grid_w: int, stride: int, scale: float | None = None,
                          workers: int = 1):
    """mixed_heads_attention_rows for every row."""
    N = np.asarray(q.shape)[2]
    return mixed_heads_attention_rows(q, k, v, flags, mask, tile, frames, grid_h, grid_w,
                                      stride, np.arange(N), scale=scale, workers=workers)
