"""SQuad's two-pass local/global attention (oracle; test infrastructure).

SQuad page, "1. Operatore di Attenzione SQuad": full softmax attention is
factored into two softmax passes,
  local pass   tokens attend within fixed windows of w tokens;
  global pass  the tokens at the same position inside every window attend to
               one another across all windows;
and the local pass's output enters the global pass as its values, so the
global pass mixes tokens that are already mixed locally.  With w = sqrt(n)
both passes cost O(n sqrt(n)).

Readings taken where the page leaves a step open:
  * the windows are runs of w consecutive tokens of the flattened latent
    (token order frame-major, as everywhere here), and N is a multiple of w,
    so there are G = N / w windows and w position groups of G tokens each;
  * both passes use the layer's Q and K (the group of position r takes the
    rows a*w + r of Q and K, a = 0 .. G-1) with the softmax scale 1/sqrt(d);
  * the operator's output is the global pass's output, scattered back to the
    original token order.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _as_f64


def _softmax_attention(q, k, v, scale):
    """Dense softmax attention over the last two axes (batched)."""
    s = (q @ np.swapaxes(k, -1, -2)) * scale
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return p @ v


def window_major_to_position_major(x, w: int) -> np.ndarray:
    """[..., N, d] -> [..., N, d] with token a*w + r moved to r*G + a."""
    x = np.asarray(x)
    N = x.shape[-2]
    G = N // w
    y = x.reshape(x.shape[:-2] + (G, w, x.shape[-1]))
    return np.swapaxes(y, -3, -2).reshape(x.shape)


def position_major_to_window_major(x, w: int) -> np.ndarray:
    """The inverse of window_major_to_position_major."""
    x = np.asarray(x)
    N = x.shape[-2]
    G = N // w
    y = x.reshape(x.shape[:-2] + (w, G, x.shape[-1]))
    return np.swapaxes(y, -3, -2).reshape(x.shape)


def squad_local(q, k, v, w: int, scale: float | None = None) -> np.ndarray:
    """The local pass: softmax attention inside each window of w tokens."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q.shape
    if N % w:
        raise ValueError("N must be a multiple of the window size")
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    G = N // w
    sh = (B, H, G, w, d)
    o = _softmax_attention(q.reshape(sh), k.reshape(sh), v.reshape(sh), scale)
    return o.reshape(B, H, N, d)


def squad_attention(q, k, v, w: int, scale: float | None = None) -> np.ndarray:
    """The SQuad operator: the global pass over position groups, with the
    local pass's output as its values.  [B, H, N, d] float64."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q.shape
    if N % w:
        raise ValueError("N must be a multiple of the window size")
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    G = N // w
    o_local = squad_local(q, k, v, w, scale)
    # position group r = tokens a*w + r: [B, H, w, G, d]
    qg = np.swapaxes(q.reshape(B, H, G, w, d), 2, 3)
    kg = np.swapaxes(k.reshape(B, H, G, w, d), 2, 3)
    vg = np.swapaxes(o_local.reshape(B, H, G, w, d), 2, 3)
    og = _softmax_attention(qg, kg, vg, scale)
    return np.swapaxes(og, 2, 3).reshape(B, H, N, d)


def squad_attention_rows(q, k, v, w: int, rows, scale: float | None = None):
    """squad_attention for the output rows `rows` only, [B, H, len(rows), d]:
    the local pass is evaluated for the position groups those rows need."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q.shape
    if N % w:
        raise ValueError("N must be a multiple of the window size")
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    G = N // w
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, H, len(rows), d))
    for r in sorted(set((rows % w).tolist())):
        members = np.arange(G) * w + r                    # the position group
        # local outputs of the group's tokens, window by window
        ol = np.zeros((B, H, G, d))
        for a in range(G):
            win = slice(a * w, (a + 1) * w)
            s = (q[:, :, members[a]][:, :, None, :] @ np.swapaxes(k[:, :, win], -1, -2)) * scale
            s = s - s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=-1, keepdims=True)
            ol[:, :, a] = (p @ v[:, :, win])[:, :, 0]
        og = _softmax_attention(q[:, :, members], k[:, :, members], ol, scale)
        for i, n in enumerate(rows):
            if n % w == r:
                out[:, :, i] = og[:, :, n // w]
    return out
