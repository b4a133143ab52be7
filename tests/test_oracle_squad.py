"""Pins for the oracle's SQuad two-pass attention (CPU only; SQuad page,
"1. Operatore di Attenzione SQuad")."""
import math

import numpy as np
import pytest
import torch

import oracle


def _qkv(B, H, N, d, seed):
    g = torch.Generator().manual_seed(seed)
    return tuple(torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
                 for _ in range(3))


def _full_attention(q, k, v):
    return torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()


def test_one_window_is_full_attention():
    """w = N: the local pass is full attention and every position group holds
    one token, whose softmax over itself is 1, so the output is the local
    pass's: full attention."""
    q, k, v = _qkv(2, 2, 24, 8, 1)
    np.testing.assert_allclose(oracle.squad_attention(q, k, v, 24),
                               _full_attention(q, k, v), rtol=1e-12, atol=1e-13)


def test_unit_windows_are_full_attention():
    """w = 1: every token attends only to itself locally (output = V), and
    the single position group is the whole sequence: full attention."""
    q, k, v = _qkv(1, 3, 20, 8, 2)
    np.testing.assert_allclose(oracle.squad_attention(q, k, v, 1),
                               _full_attention(q, k, v), rtol=1e-12, atol=1e-13)


def test_brute_force_tiny():
    """Explicit loops with math.exp: N = 6, w = 3, d = 2."""
    q, k, v = _qkv(1, 1, 6, 2, 3)
    Q, K, V = q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist()
    N, w, d = 6, 3, 2
    sc = 1.0 / math.sqrt(d)

    def attend(qi, keys, vals):
        s = [sc * sum(qi[c] * kk[c] for c in range(d)) for kk in keys]
        mx = max(s)
        z = sum(math.exp(x - mx) for x in s)
        return [sum(math.exp(s[j] - mx) / z * vals[j][c] for j in range(len(keys)))
                for c in range(d)]

    local = [attend(Q[n], K[(n // w) * w:(n // w + 1) * w], V[(n // w) * w:(n // w + 1) * w])
             for n in range(N)]
    want = []
    for n in range(N):
        grp = [m for m in range(N) if m % w == n % w]
        want.append(attend(Q[n], [K[m] for m in grp], [local[m] for m in grp]))
    got = oracle.squad_attention(q, k, v, w)[0, 0]
    np.testing.assert_allclose(got, np.array(want), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(oracle.squad_local(q, k, v, w)[0, 0], np.array(local),
                               rtol=1e-12, atol=1e-14)


def test_output_is_a_convex_combination_of_values():
    q, k, v = _qkv(1, 2, 64, 16, 4)
    o = oracle.squad_attention(q, k, v, 8)
    lo = v.numpy().min(axis=2, keepdims=True)
    hi = v.numpy().max(axis=2, keepdims=True)
    assert (o >= lo - 1e-12).all() and (o <= hi + 1e-12).all()


def test_window_reorder_by_hand():
    x = np.arange(6).reshape(1, 6, 1)
    y = oracle.window_major_to_position_major(x, 3)
    assert y[0, :, 0].tolist() == [0, 3, 1, 4, 2, 5]
    z = oracle.position_major_to_window_major(y, 3)
    assert z[0, :, 0].tolist() == [0, 1, 2, 3, 4, 5]
    x = np.random.default_rng(0).random((2, 3, 40, 5))
    for w in (1, 4, 8, 40):
        np.testing.assert_array_equal(
            oracle.position_major_to_window_major(oracle.window_major_to_position_major(x, w), w), x)


def test_rows_version_matches():
    q, k, v = _qkv(1, 2, 48, 8, 5)
    rows = [0, 7, 13, 47, 24]
    np.testing.assert_allclose(oracle.squad_attention_rows(q, k, v, 6, rows),
                               oracle.squad_attention(q, k, v, 6)[:, :, rows],
                               rtol=1e-12, atol=1e-14)


def test_rejects_ragged_windows():
    q, k, v = _qkv(1, 1, 10, 4, 6)
    with pytest.raises(ValueError):
        oracle.squad_attention(q, k, v, 4)
