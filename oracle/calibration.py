"""Energy-based block selection and cross-prompt aggregation (oracle; test
infrastructure).

CalibAtt page, "A. Fase di Calibrazione":
  step 1  the attention matrix is cut into blocks (128x128 there); for each
          query block the "energy" towards every key block is the sum of the
          attention scores inside that block; the fewest key blocks whose
          cumulative energy reaches the threshold eps(t) are kept, giving one
          binary mask per calibration prompt;
  step 2  the masks of the prompts are averaged and a block is kept when the
          fraction of prompts that selected it reaches the agreement
          threshold rho (0.5 in the page's example).

Readings taken where the page leaves a step open:
  * the attention scores are the softmax probabilities of full (dense)
    attention, p[n, m] = softmax_m(scale * q_n . k_m), scale = 1/sqrt(d) by
    default; block energy E[i, j] = sum over query rows n of tile i and key
    columns m of tile j of p[n, m].  Every query row contributes 1 in total,
    so row i of E sums to the number of query rows in tile i;
  * eps is a fraction of the query block's total energy (its row sum of E);
  * "the fewest blocks" are taken greedily by energy: key blocks sorted by
    decreasing energy, the lower block index first on equal energy, and the
    shortest prefix of that order whose cumulative energy is >= eps * total.
    With eps <= 0 that prefix is empty;
  * the selection decides integers from floating point, so it is defined on
    float32 energies (what the library's energy kernel produces) with the
    cumulative sums taken in float64, one addition at a time in the sorted
    order, total included; the GPU selection does the same arithmetic;
  * prompts are the batch entries of one energy tensor [P, H, Tq, Tk]; a
    block is kept when count >= rho * P (float64), count = number of prompts
    whose mask selected it.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _as_f64


def block_energy(q, k, tile: int, scale: float | None = None) -> np.ndarray:
    """E[b, h, i, j]: dense softmax probabilities summed over query tile i
    and key tile j (float64).  q, k: [B, H, N, d]."""
    q = _as_f64(q)
    k = _as_f64(k)
    B, H, N, d = q.shape
    if k.shape != q.shape:
        raise ValueError("q and k must share the shape [B, H, N, d]")
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    nt = -(-N // tile)
    tile_of = np.arange(N) // tile
    E = np.zeros((B, H, nt, nt), dtype=np.float64)
    onehot = np.zeros((N, nt), dtype=np.float64)
    onehot[np.arange(N), tile_of] = 1.0
    for b in range(B):
        for h in range(H):
            s = (q[b, h] @ k[b, h].T) * scale               # [N, N]
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)               # softmax rows
            E[b, h] = onehot.T @ p @ onehot                 # block sums
    return E


def block_energy_rows(q, k, tile: int, query_tiles,
                      scale: float | None = None) -> np.ndarray:
    """The rows E[b, h, i, :] for the query tiles i in `query_tiles` only
    (same definition as block_energy), [B, H, len(query_tiles), T]."""
    q = _as_f64(q)
    k = _as_f64(k)
    B, H, N, d = q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    nt = -(-N // tile)
    onehot = np.zeros((N, nt), dtype=np.float64)
    onehot[np.arange(N), np.arange(N) // tile] = 1.0
    qts = list(query_tiles)
    E = np.zeros((B, H, len(qts), nt), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r, i in enumerate(qts):
                rows = slice(i * tile, min((i + 1) * tile, N))
                s = (q[b, h, rows] @ k[b, h].T) * scale
                s -= s.max(axis=1, keepdims=True)
                p = np.exp(s)
                p /= p.sum(axis=1, keepdims=True)
                E[b, h, r] = p.sum(axis=0) @ onehot
    return E


def select_row(energy_row, eps: float) -> np.ndarray:
    """uint8 [Tk]: the fewest key blocks reaching eps of the row's energy
    (float32 energies, float64 sequential sums in the sorted order)."""
    e = np.asarray(energy_row, dtype=np.float32)
    order = sorted(range(len(e)), key=lambda j: (-float(e[j]), j))
    total = 0.0
    for j in order:
        total += float(e[j])
    target = float(eps) * total
    keep = np.zeros(len(e), dtype=np.uint8)
    cum = 0.0
    for j in order:
        if cum >= target:
            break
        keep[j] = 1
        cum += float(e[j])
    return keep


def select_mask(energy, eps: float) -> np.ndarray:
    """select_row over every row of an energy tensor [..., Tk]."""
    e = np.asarray(energy, dtype=np.float32)
    flat = e.reshape(-1, e.shape[-1])
    out = np.stack([select_row(r, eps) for r in flat]) if len(flat) else \
        np.zeros((0, e.shape[-1]), dtype=np.uint8)
    return out.reshape(e.shape)


def aggregate(masks, rho: float) -> np.ndarray:
    """uint8 [...]: 1 where at least rho of the P prompt masks [P, ...] are 1."""
    m = np.asarray(masks)
    P = m.shape[0]
    count = (m != 0).sum(axis=0)
    out = np.zeros(m.shape[1:], dtype=np.uint8)
    it = np.nditer(count, flags=["multi_index"])
    for c in it:
        out[it.multi_index] = 1 if float(int(c)) >= float(rho) * float(P) else 0
    return out
