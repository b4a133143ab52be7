"""Tile masks, written out from their definitions (oracle; test infrastructure).

Geometry.  A video latent of T frames on a grid_h x grid_w grid is flattened
frame-major, so frame f holds tokens [f*P, (f+1)*P) with P = grid_h*grid_w and
N = T*P.  Tokens are cut into square tiles of BT rows/columns; tile i holds
tokens [i*BT, min((i+1)*BT, N)) and there are ceil(N/BT) of them.

LVSA rule (LVSA page, Meccanismo Core): a query frame t attends to the frame
set A(t) = G u W(t) instead of all frames {0..T-1}.  W(t) is the local window
around t; G is the set of global anchor frames, which rotates with the
denoising step so that, over T_per consecutive steps, every frame is an anchor
exactly once.

Readings taken where the page leaves a step open:
  * W(t) = {f in [0, T) : |f - t| <= w}, a symmetric window of half-width w,
    clipped to the video (the plain window mode).
  * n_a anchors evenly spaced from the rotation r:
    G_r = {(r + floor(k*T/n_a)) mod T : 0 <= k < n_a}; the caller chooses r
    (e.g. step mod T_per, or (layer + step) mod T).
  * Anchors are key frames only: every query frame attends to them.
  * A frame pair lifts to tiles by "any overlap": tile pair (i, j) is active
    when some frame covered by tile i may attend to some frame covered by
    tile j.  Inside an active tile pair every token pair is computed.

Expanded adaptive windows (LVSA page, Meccanismo Core, the expanded window
bounds that keep |A(t)| close to a frame budget C, e.g. the model's training
horizon).  The page says the window grows to make up for frames it shares with
G, but not on which side or in which order.  Reading taken:
  * the target is min(C, T) distinct frames in A(t);
  * the window starts as the plain W(t) above and only ever grows;
  * it grows one frame at a time, taking the frame nearest to t that is not
    yet in it, the earlier frame first when two are equally near; frames
    outside [0, T) do not exist, so at either end of the video it grows on
    the other side only;
  * an anchor frame reached this way joins the window but adds nothing to
    |A(t)|, so growth continues past it;
  * growth stops as soon as |G u W(t)| >= min(C, T).
So W(t) stays a contiguous run of frames around t, |A(t)| equals
max(min(C, T), |G u W_plain(t)|), and C = n_a + 2w + 1 makes up exactly for
anchor overlap and for the clipped window at the ends of the video.

Static mode (CalibAtt page, B. Fase di Inferenza: a precomputed, deterministic
per-(timestep, layer, head) block list).  Real calibrated masks need the model
and calibration prompts, so a seeded stand-in is used: tile (h, i, j) is the
c-th cell, c = (h*Tq + i)*Tk + j, and it is active when the top 24 bits of the
(c+1)-th SplitMix64 output for `seed` fall below `thresh24`, or when i == j and
the diagonal is forced.  SplitMix64 is the generator of Steele, Lea and Flood
(OOPSLA 2014): state += 0x9E3779B97F4A7C15, then two xor-shift-multiply rounds
and a final xor-shift.

Dense mode: every tile active (the full-attention baseline).

Block-diagonal mode (SQuad page, 1. Operatore di Attenzione SQuad: each of
its two passes attends inside disjoint groups of consecutive tokens): tile
pair (i, j) is active when i and j lie in the same run of b tiles.

Dense-rows mode (CalibAtt page, B. Fase di Inferenza: a repetitive head
computes its anchor rows only, packed at the front): query tiles below
query_tiles read every key tile, the others none.

Spread dense-rows mode (same passage, with the anchor rows laid out in
blocks spread over the sequence): the query_tiles dense tiles are cut into
blocks of block_tiles tiles (the last one shorter if need be); block g is
placed at block slot floor(g * Pg / Rg), Rg blocks over Pg = ceil(Tq /
block_tiles) slots.
"""
from __future__ import annotations

import numpy as np

_U64 = np.uint64
_GOLDEN = _U64(0x9E3779B97F4A7C15)
_MIX1 = _U64(0xBF58476D1CE4E5B9)
_MIX2 = _U64(0x94D049BB133111EB)


# ----------------------------------------------------------------- frame rule
def window_frames(t: int, T: int, w: int) -> set:
    """W(t): frames within w of t, clipped to [0, T)."""
    return {f for f in range(T) if abs(f - t) <= w}


def anchor_frames(T: int, n_a: int, r: int) -> set:
    """G_r: n_a evenly spaced anchor frames shifted by the rotation r."""
    r = r % T
    return {(r + (k * T) // n_a) % T for k in range(n_a)}


def frame_set(t: int, T: int, w: int, n_a: int, r: int) -> set:
    """A(t) = G_r u W(t)."""
    return anchor_frames(T, n_a, r) | window_frames(t, T, w)


def frame_mask(T: int, w: int, n_a: int, r: int) -> np.ndarray:
    """F[t, f] = 1 when query frame t attends to key frame f."""
    F = np.zeros((T, T), dtype=np.uint8)
    for t in range(T):
        for f in frame_set(t, T, w, n_a, r):
            F[t, f] = 1
    return F


def expanded_window_frames(t: int, T: int, w: int, n_a: int, r: int,
                           budget: int) -> set:
    """W(t) grown from the plain window until |G u W(t)| reaches min(C, T)
    (LVSA page, Meccanismo Core, expanded adaptive windows)."""
    G = anchor_frames(T, n_a, r)
    W = window_frames(t, T, w)
    target = min(budget, T)
    nearest_first = sorted(range(T), key=lambda f: (abs(f - t), f))
    for f in nearest_first:
        if len(G | W) >= target:
            break
        W.add(f)
    return W


def frame_set_expanded(t: int, T: int, w: int, n_a: int, r: int,
                       budget: int) -> set:
    """A(t) = G_r u W(t) with the expanded window."""
    return anchor_frames(T, n_a, r) | expanded_window_frames(t, T, w, n_a, r,
                                                             budget)


def frame_mask_expanded(T: int, w: int, n_a: int, r: int,
                        budget: int) -> np.ndarray:
    """F[t, f] = 1 when query frame t attends to key frame f (expanded)."""
    F = np.zeros((T, T), dtype=np.uint8)
    for t in range(T):
        for f in frame_set_expanded(t, T, w, n_a, r, budget):
            F[t, f] = 1
    return F


# --------------------------------------------------------------- tile lift
def tile_frame_range(i: int, N: int, P: int, BT: int):
    """First and last frame covered by tile i."""
    first_tok = i * BT
    last_tok = min((i + 1) * BT, N) - 1
    return first_tok // P, last_tok // P


def _tile_frame_incidence(T: int, P: int, BT: int) -> np.ndarray:
    """I[i, f] = 1 when tile i covers at least one token of frame f."""
    N = T * P
    nt = -(-N // BT)
    inc = np.zeros((nt, T), dtype=np.int64)
    for i in range(nt):
        a, b = tile_frame_range(i, N, P, BT)
        inc[i, a:b + 1] = 1
    return inc


def _lift(F: np.ndarray, T: int, grid_h: int, grid_w: int,
          BT: int) -> np.ndarray:
    """M[i, j] = OR over frames t of tile i and f of tile j of F[t, f].

    With tile-frame incidence matrix I this is [I F I^T > 0]."""
    inc = _tile_frame_incidence(T, grid_h * grid_w, BT)
    return ((inc @ F.astype(np.int64) @ inc.T) > 0).astype(np.uint8)


def _check_frame_args(T: int, w: int, n_a: int):
    if T <= 0:
        raise ValueError("need at least one frame")
    if not (0 <= n_a <= T):
        raise ValueError("anchor count must lie in [0, T]")
    if w < 0:
        raise ValueError("window half-width must be >= 0")


def tile_mask_window_anchor(T: int, grid_h: int, grid_w: int, BT: int,
                            w: int, n_a: int, r: int) -> np.ndarray:
    """Tile mask of the plain window + anchor rule."""
    _check_frame_args(T, w, n_a)
    return _lift(frame_mask(T, w, n_a, r), T, grid_h, grid_w, BT)


def tile_mask_expanded(T: int, grid_h: int, grid_w: int, BT: int, w: int,
                       n_a: int, r: int, budget: int) -> np.ndarray:
    """Tile mask of the expanded-window + anchor rule."""
    _check_frame_args(T, w, n_a)
    if budget < 0:
        raise ValueError("frame budget must be >= 0")
    return _lift(frame_mask_expanded(T, w, n_a, r, budget), T, grid_h, grid_w,
                 BT)


# ------------------------------------------------------------- static mode
def splitmix64_stream(seed: int, count: int) -> np.ndarray:
    """The first `count` SplitMix64 outputs for `seed` (uint64 array)."""
    c = np.arange(1, count + 1, dtype=_U64)
    with np.errstate(over="ignore"):
        z = _U64(seed & 0xFFFFFFFFFFFFFFFF) + c * _GOLDEN
        z = (z ^ (z >> _U64(30))) * _MIX1
        z = (z ^ (z >> _U64(27))) * _MIX2
        z = z ^ (z >> _U64(31))
    return z


def static_hash24(seed: int, count: int) -> np.ndarray:
    """Top 24 bits of the first `count` SplitMix64 outputs."""
    return (splitmix64_stream(seed, count) >> _U64(40)).astype(np.int64)


def tile_mask_static(Hm: int, Tq: int, Tk: int, seed: int, thresh24: int,
                     force_diagonal: bool) -> np.ndarray:
    """Seeded random block mask, one independent draw per (h, i, j) cell."""
    h24 = static_hash24(seed, Hm * Tq * Tk).reshape(Hm, Tq, Tk)
    M = (h24 < int(thresh24)).astype(np.uint8)
    if force_diagonal:
        for h in range(Hm):
            for i in range(min(Tq, Tk)):
                M[h, i, i] = 1
    return M


def tile_mask_block_diagonal(Hm: int, Tq: int, Tk: int, b: int) -> np.ndarray:
    """M[i, j] = 1 when tiles i and j fall in the same run of b tiles (the
    groups SQuad's passes attend within)."""
    if b < 1:
        raise ValueError("block size must be >= 1 tile")
    M = np.zeros((Hm, Tq, Tk), dtype=np.uint8)
    for i in range(Tq):
        for j in range(Tk):
            if i // b == j // b:
                M[:, i, j] = 1
    return M


def tile_mask_dense(Hm: int, Tq: int, Tk: int) -> np.ndarray:
    return np.ones((Hm, Tq, Tk), dtype=np.uint8)


# ------------------------------------------------------------ entry point
def tile_mask(kind: int, frames: int, grid_h: int, grid_w: int, tile: int,
              window: int = 0, num_anchors: int = 0, rotation: int = 0,
              seed: int = 0, thresh24: int = 0, force_diagonal: int = 0,
              mask_heads: int = 1, budget: int = 0,
              block_tiles: int = 1, query_tiles: int = 0) -> np.ndarray:
    """uint8 [Hm, Tq, Tk] tile mask for kind 0 (window + anchors),
    1 (static random), 2 (dense), 3 (expanded window + anchors) or
    4 (block diagonal)."""
    N = frames * grid_h * grid_w
    nt = -(-N // tile)
    if kind == 0:
        M = tile_mask_window_anchor(frames, grid_h, grid_w, tile, window,
                                    num_anchors, rotation)
        return np.repeat(M[None], mask_heads, axis=0)
    if kind == 1:
        return tile_mask_static(mask_heads, nt, nt, seed, thresh24,
                                bool(force_diagonal))
    if kind == 2:
        return tile_mask_dense(mask_heads, nt, nt)
    if kind == 4:
        return tile_mask_block_diagonal(mask_heads, nt, nt, block_tiles)
    if kind == 3:
        M = tile_mask_expanded(frames, grid_h, grid_w, tile, window,
                               num_anchors, rotation, budget)
        return np.repeat(M[None], mask_heads, axis=0)
    raise ValueError(f"unknown mask kind {kind}")
