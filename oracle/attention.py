"""Block-masked softmax attention in float64 (oracle; test infrastructure).

The definition (softmax self-attention restricted to the selected blocks, as
the LVSA and CalibAtt pages use it): for batch b, head h and query token n,

    s[n, m] = scale * sum_c q[n, c] * k[m, c]            (float64)
    s[n, m] = -inf  where tile mask M[h', n // BT, m // BT] == 0
    p[n, :] = softmax(s[n, :])
    o[n, :] = sum_m p[n, m] * v[m, :]
    lse[n]  = log(sum_m exp(s[n, m]))                     (natural log)

with h' = h when the mask has one slice per head and h' = 0 when it has one
slice shared by all heads; the mask is shared by all batch entries.  scale
defaults to 1/sqrt(d).  A query row with no active key gets o = 0 and
lse = -inf.  Inputs are read as their exact values (bf16 and fp32 upcast to
float64 exactly).  Rows are processed in chunks only to bound memory; each
row's arithmetic is the definition above.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def _as_f64(x) -> np.ndarray:
    """float64 copy of a numpy array or a CPU torch tensor (bf16 included)."""
    if hasattr(x, "detach"):  # torch tensor; bf16 has no numpy dtype
        x = x.detach().to("cpu")
        import torch
        return x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _rows_attention(q_rows, row_ids, k, v, mask_h, BT, scale):
    """Attention for the query rows `row_ids` of one (b, h) slice."""
    s = (q_rows @ k.T) * scale                       # [R, N]
    N = k.shape[0]
    key_tile = np.arange(N) // BT
    allowed = mask_h[(row_ids // BT)[:, None], key_tile[None, :]] != 0
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)                 # -inf on empty rows
    has_key = np.isfinite(m[:, 0])
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)                           # exp(-inf) = 0
    denom = e.sum(axis=1, keepdims=True)
    o = np.zeros((len(row_ids), v.shape[1]), dtype=np.float64)
    o[has_key] = (e[has_key] / denom[has_key]) @ v
    lse = np.full(len(row_ids), -np.inf)
    lse[has_key] = m[has_key, 0] + np.log(denom[has_key, 0])
    return o, lse


def block_sparse_attention_rows(q, k, v, mask, tile: int, rows,
                                scale: float | None = None, workers: int = 1,
                                chunk: int = 128):
    """Oracle outputs for the query rows `rows` (same for every (b, h)).

    q, k: [B, H, N, d]; v: [B, H, N, dv] (dv = d for attention itself; any
    dv gives the same weights applied to other values); mask: uint8
    [Hm, Tq, Tk] with Hm in {1, H}.
    Returns (o [B, H, len(rows), dv], lse [B, H, len(rows)]), float64.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    mask = np.asarray(mask)
    B, H, N, d = q.shape
    if k.shape != (B, H, N, d) or v.ndim != 4 or v.shape[:3] != (B, H, N):
        raise ValueError("q and k must share the shape [B, H, N, d], v [B, H, N, dv]")
    Hm = mask.shape[0]
    if Hm not in (1, H):
        raise ValueError("mask must have 1 or H head slices")
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((B, H, len(rows), v.shape[3]), dtype=np.float64)
    lse = np.full((B, H, len(rows)), -np.inf)

    jobs = []
    for b in range(B):
        for h in range(H):
            for c0 in range(0, len(rows), chunk):
                jobs.append((b, h, c0))

    def run(job):
        b, h, c0 = job
        ids = rows[c0:c0 + chunk]
        mh = mask[h if Hm == H else 0]
        oc, lc = _rows_attention(q[b, h, ids], ids, k[b, h], v[b, h], mh,
                                 tile, scale)
        o[b, h, c0:c0 + len(ids)] = oc
        lse[b, h, c0:c0 + len(ids)] = lc

    if workers > 1:
        # one BLAS thread per worker thread: the workers already fill the
        # cores, and nested BLAS threads would oversubscribe them
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:  # pragma: no cover
            threadpool_limits = None
        if threadpool_limits is not None:
            with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
                list(ex.map(run, jobs))
        else:  # pragma: no cover
            with ThreadPoolExecutor(workers) as ex:
                list(ex.map(run, jobs))
    else:
        for job in jobs:
            run(job)
    return o, lse


def block_sparse_attention(q, k, v, mask, tile: int, scale: float | None = None,
                           workers: int = 1, chunk: int = 128):
    """Oracle outputs for every query row: (o [B,H,N,d], lse [B,H,N])."""
    N = q.shape[2]
    return block_sparse_attention_rows(q, k, v, mask, tile, np.arange(N),
                                       scale=scale, workers=workers,
                                       chunk=chunk)
