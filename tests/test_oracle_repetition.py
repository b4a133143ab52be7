"""Pins for the oracle's spatial repetition (CPU only; CalibAtt page,
"A. Fase di Calibrazione" step 3 and "B. Fase di Inferenza")."""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle


def _qkv(B, H, N, d, seed):
    g = torch.Generator().manual_seed(seed)
    return tuple(torch.randn(B, H, N, d, generator=g, dtype=torch.float64) for _ in range(3))


def test_cosines_match_the_log_sum_exp_identity():
    """<p1, p2> = Z(q1 + q2) / (Z(q1) Z(q2)) with Z(q) = sum_k exp(scale q.k):
    an independent formula for the same cosine, through logsumexp."""
    T, gh, gw, d, s = 2, 5, 3, 8, 2
    q, k, _ = _qkv(1, 2, T * gh * gw, d, 1)
    sc = 1.0 / math.sqrt(d)
    got = oracle.row_cosines(q, k, T, gh, gw, s)
    qn, kn = q.numpy(), k.numpy()
    P = gh * gw
    for h in range(2):
        lse = lambda x: logsumexp(sc * (kn[0, h] @ x))
        for f in range(T):
            for y in range(gh):
                a = s * (y // s)
                if a == y:
                    assert got[0, h, f, y] == 1.0
                    continue
                d12 = d11 = d22 = 0.0
                for x in range(gw):
                    q1 = qn[0, h, f * P + y * gw + x]
                    q2 = qn[0, h, f * P + a * gw + x]
                    l1, l2 = lse(q1), lse(q2)
                    d12 += math.exp(lse(q1 + q2) - l1 - l2)
                    d11 += math.exp(lse(2 * q1) - 2 * l1)
                    d22 += math.exp(lse(2 * q2) - 2 * l2)
                assert abs(got[0, h, f, y] - d12 / math.sqrt(d11 * d22)) < 1e-12


def test_identical_rows_have_cosine_one():
    T, gh, gw, d = 3, 4, 5, 8
    q, k, _ = _qkv(2, 1, T * gh * gw, d, 2)
    q = q.reshape(2, 1, T, gh, gw, d)
    q[:, :, :, 1:] = q[:, :, :, :1]          # every row repeats row 0
    q = q.reshape(2, 1, T * gh * gw, d)
    cos = oracle.row_cosines(q, k, T, gh, gw, 3)
    np.testing.assert_allclose(cos, 1.0, rtol=0, atol=1e-14)
    assert oracle.repetitive_heads(cos, 3, 0.999).tolist() == [1]
    qr, _, _ = _qkv(2, 1, T * gh * gw, d, 3)
    cr = oracle.row_cosines(qr, k, T, gh, gw, 3)
    assert (cr[:, :, :, [1, 2]] < 0.999).all()


def test_cosine_brute_force():
    T, gh, gw, d, s = 1, 2, 2, 2, 2
    q, k, _ = _qkv(1, 1, 4, d, 4)
    Q, K = q[0, 0].tolist(), k[0, 0].tolist()
    sc = 1.0 / math.sqrt(d)

    def probs(qq):
        e = [math.exp(sc * sum(qq[c] * kk[c] for c in range(d))) for kk in K]
        z = sum(e)
        return [x / z for x in e]

    p = [probs(Q[n]) for n in range(4)]          # rows: y=0 -> 0,1; y=1 -> 2,3
    d12 = sum(p[2 + x][m] * p[x][m] for x in range(2) for m in range(4))
    d11 = sum(p[2 + x][m] ** 2 for x in range(2) for m in range(4))
    d22 = sum(p[x][m] ** 2 for x in range(2) for m in range(4))
    got = oracle.row_cosines(q, k, T, gh, gw, s)
    assert abs(got[0, 0, 0, 1] - d12 / math.sqrt(d11 * d22)) < 1e-13


def test_sampled_cosines_are_the_full_ones():
    """row_cosines_at (the sampled form the full-size GPU checks use) gives,
    cell for cell, what the pinned row_cosines gives, anchors included."""
    B, H, T, gh, gw, d, s = 2, 2, 2, 5, 3, 8, 2
    q, k, _ = _qkv(B, H, T * gh * gw, d, 5)
    full = oracle.row_cosines(q, k, T, gh, gw, s, scale=0.3)
    cells = [(1, 0, 1, 3), (0, 1, 0, 1), (0, 1, 0, 2), (1, 1, 1, 4), (0, 0, 1, 1)]
    got = oracle.row_cosines_at(q, k, T, gh, gw, s, cells, scale=0.3)
    assert np.array_equal(got, np.array([full[c] for c in cells]))


def test_repetitive_heads_by_hand():
    cos = np.ones((2, 3, 1, 4), dtype=np.float32)    # stride 2: rows 1, 3 count
    cos[:, 0, 0, 1] = 0.8
    cos[:, 0, 0, 3] = 1.0                             # head 0 mean 0.9
    cos[:, 1, 0, 1] = 0.5
    cos[:, 1, 0, 3] = 0.5                             # head 1 mean 0.5
    cos[0, 2, 0, 1], cos[1, 2, 0, 1] = 0.25, 1.0      # head 2 mean (0.25 + 1 + 1 + 1) / 4
    assert oracle.repetitive_heads(cos, 2, 0.9).tolist() == [1, 0, 0]
    assert oracle.repetitive_heads(cos, 2, 0.8125).tolist() == [1, 0, 1]
    assert oracle.repetitive_heads(cos, 2, 0.5).tolist() == [1, 1, 1]
    assert oracle.repetitive_heads(cos, 4, 2.0).tolist() == [0, 0, 0]
    assert oracle.repetitive_heads(np.ones((1, 2, 3, 2), np.float32), 2, 2.0).tolist() == [0, 0]
    # stride 1: every row is an anchor, no non-anchor row at all: repetitive
    assert oracle.repetitive_heads(np.ones((1, 2, 3, 2), np.float32), 1, 2.0).tolist() == [1, 1]


def test_gather_and_broadcast_by_hand():
    x = np.arange(12).reshape(1, 12, 1)               # 2 frames of 3 x 2
    g = oracle.gather_anchor_rows(x, 2, 3, 2, 2)
    assert g[0, :, 0].tolist() == [0, 1, 4, 5, 6, 7, 10, 11]
    b = oracle.broadcast_anchor_rows(g, 2, 3, 2, 2)
    assert b[0, :, 0].tolist() == [0, 1, 0, 1, 4, 5, 6, 7, 6, 7, 10, 11]
    assert oracle.anchor_count(3, 2) == 2 and oracle.anchor_count(4, 2) == 2


def test_repeated_attention():
    T, gh, gw, d = 2, 5, 4, 8
    q, k, v = _qkv(1, 2, T * gh * gw, d, 5)
    full = torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()
    np.testing.assert_allclose(oracle.repeated_attention(q, k, v, T, gh, gw, 1), full,
                               rtol=1e-12, atol=1e-13)
    o = oracle.repeated_attention(q, k, v, T, gh, gw, 2).reshape(1, 2, T, gh, gw, d)
    f = full.reshape(1, 2, T, gh, gw, d)
    for y in range(gh):
        np.testing.assert_allclose(o[:, :, :, y], f[:, :, :, 2 * (y // 2)], rtol=1e-12,
                                   atol=1e-13)


def test_mixed_heads_reduce_to_each_kind():
    """The mixed inference layer: no head flagged = block-sparse attention on
    the lists; every head flagged = attention on anchor rows copied; a mix
    gives each head its own kind; a flagged head's rows repeat their
    anchor's and a dense list equals textbook attention."""
    T, gh, gw, d, s, tile = 2, 6, 8, 8, 2, 16
    N = T * gh * gw
    q, k, v = _qkv(1, 3, N, d, 12)
    Tq = -(-N // tile)
    g = np.random.default_rng(3)
    mask = (g.random((3, Tq, Tq)) < 0.5).astype(np.uint8)
    mask[:, np.arange(Tq), np.arange(Tq)] = 1
    sparse, _ = oracle.block_sparse_attention(q, k, v, mask, tile)
    rep = oracle.repeated_attention(q, k, v, T, gh, gw, s)
    none = oracle.mixed_heads_attention(q, k, v, [0, 0, 0], mask, tile, T, gh, gw, s)
    np.testing.assert_allclose(none, sparse, rtol=0, atol=1e-14)
    allf = oracle.mixed_heads_attention(q, k, v, [1, 1, 1], mask, tile, T, gh, gw, s)
    np.testing.assert_allclose(allf, rep, rtol=0, atol=1e-14)
    mix = oracle.mixed_heads_attention(q, k, v, [1, 0, 1], mask, tile, T, gh, gw, s)
    np.testing.assert_allclose(mix[:, [0, 2]], rep[:, [0, 2]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(mix[:, 1], sparse[:, 1], rtol=0, atol=1e-14)
    m4 = mix.reshape(1, 3, T, gh, gw, d)
    for y in range(gh):
        assert np.array_equal(m4[:, 0, :, y], m4[:, 0, :, s * (y // s)])
    dense = np.ones((1, Tq, Tq), dtype=np.uint8)
    full = torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()
    d0 = oracle.mixed_heads_attention(q, k, v, [0, 0, 0], dense, tile, T, gh, gw, s)
    np.testing.assert_allclose(d0, full, rtol=1e-12, atol=1e-13)
    # the rows variant on a sample equals the full one
    rows = np.array([0, 5, 47, 48, 95])
    r = oracle.mixed_heads_attention_rows(q, k, v, [1, 0, 1], mask, tile, T, gh, gw, s, rows)
    np.testing.assert_allclose(r, mix[:, :, rows], rtol=0, atol=1e-14)
