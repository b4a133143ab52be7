"""Pins for the oracle's block-masked softmax attention (CPU only).

None of the pages prints a worked attention output, so these pins come from
the definition and from mathematics: full attention at density 1 (a library
routine), single-block brute force in plain Python floats, block-diagonal
masks against per-tile full attention, convex-combination bounds, permutation
invariance and the empty-row convention.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape)


def _sdpa64(q, k, v, attn_mask=None, scale=None):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.float64)
    with torch.no_grad():
        o = torch.nn.functional.scaled_dot_product_attention(
            t(q), t(k), t(v), attn_mask=None if attn_mask is None else
            torch.from_numpy(attn_mask), scale=scale)
    return o.numpy()


@pytest.mark.parametrize("B,H,N,d,BT", [(1, 2, 64, 16, 16), (2, 3, 50, 8, 16),
                                        (1, 1, 129, 32, 64)])
def test_density_one_equals_full_attention(B, H, N, d, BT):
    q, k, v = (_rand((B, H, N, d), s) for s in (1, 2, 3))
    Tn = -(-N // BT)
    mask = np.ones((1, Tn, Tn), dtype=np.uint8)
    o, lse = oracle.block_sparse_attention(q, k, v, mask, BT)
    np.testing.assert_allclose(o, _sdpa64(q, k, v), rtol=1e-12, atol=1e-12)
    s = np.einsum("bhnc,bhmc->bhnm", q, k) / math.sqrt(d)
    ref_lse = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_explicit_scale():
    q, k, v = (_rand((1, 1, 40, 8), s) for s in (4, 5, 6))
    mask = np.ones((1, 3, 3), dtype=np.uint8)
    o, _ = oracle.block_sparse_attention(q, k, v, mask, 16, scale=0.37)
    np.testing.assert_allclose(o, _sdpa64(q, k, v, scale=0.37), rtol=1e-12,
                               atol=1e-12)


def _brute_force_row(q, k, v, n, keys, scale):
    """o[n] = sum_m e^{s_m} v_m / sum_m e^{s_m} over the listed keys, in plain
    Python floats."""
    d = len(q[0])
    s = [scale * sum(q[n][c] * k[m][c] for c in range(d)) for m in keys]
    mx = max(s)
    e = [math.exp(x - mx) for x in s]
    z = sum(e)
    o = [sum(e[t] * v[m][c] for t, m in enumerate(keys)) / z for c in range(d)]
    return o, mx + math.log(z)


def test_single_active_block_brute_force():
    BT, N, d = 8, 29, 4          # 4 tiles, the last one ragged (5 tokens)
    Tn = 4
    q, k, v = (_rand((1, 1, N, d), s) for s in (7, 8, 9))
    # each query tile reads exactly one key tile, a permutation-like pattern
    pick = [2, 0, 3, 3]
    mask = np.zeros((1, Tn, Tn), dtype=np.uint8)
    for i, j in enumerate(pick):
        mask[0, i, j] = 1
    o, lse = oracle.block_sparse_attention(q, k, v, mask, BT)
    ql, kl, vl = (x[0, 0].tolist() for x in (q, k, v))
    for n in range(N):
        j = pick[n // BT]
        keys = list(range(j * BT, min((j + 1) * BT, N)))
        want, want_lse = _brute_force_row(ql, kl, vl, n, keys, 1 / math.sqrt(d))
        np.testing.assert_allclose(o[0, 0, n], want, rtol=1e-12, atol=1e-13)
        assert abs(lse[0, 0, n] - want_lse) < 1e-12


def test_two_block_row_brute_force_per_head_mask():
    BT, N, d, H = 8, 24, 3, 2
    q, k, v = (_rand((1, H, N, d), s) for s in (10, 11, 12))
    mask = np.zeros((H, 3, 3), dtype=np.uint8)
    mask[0, 0, [0, 2]] = 1
    mask[0, 1, [1]] = 1
    mask[0, 2, [0, 1]] = 1
    mask[1, 0, [1]] = 1
    mask[1, 1, [0, 2]] = 1
    mask[1, 2, [2]] = 1
    o, _ = oracle.block_sparse_attention(q, k, v, mask, BT)
    for h in range(H):
        ql, kl, vl = (x[0, h].tolist() for x in (q, k, v))
        for n in range(N):
            keys = [m for m in range(N) if mask[h, n // BT, m // BT]]
            want, _ = _brute_force_row(ql, kl, vl, n, keys, 1 / math.sqrt(d))
            np.testing.assert_allclose(o[0, h, n], want, rtol=1e-12, atol=1e-13)


def test_block_diagonal_equals_per_tile_attention():
    BT, N, d = 16, 70, 8
    q, k, v = (_rand((2, 2, N, d), s) for s in (13, 14, 15))
    Tn = -(-N // BT)
    mask = np.eye(Tn, dtype=np.uint8)[None]
    o, _ = oracle.block_sparse_attention(q, k, v, mask, BT)
    for i in range(Tn):
        sl = slice(i * BT, min((i + 1) * BT, N))
        want = _sdpa64(q[:, :, sl], k[:, :, sl], v[:, :, sl])
        np.testing.assert_allclose(o[:, :, sl], want, rtol=1e-12, atol=1e-12)


def test_ragged_sparse_equals_library_with_token_mask():
    BT, N, d, H = 16, 75, 8, 3
    q, k, v = (_rand((1, H, N, d), s) for s in (16, 17, 18))
    Tn = -(-N // BT)
    mask = oracle.tile_mask_static(H, Tn, Tn, 99, 1 << 23, True)
    o, _ = oracle.block_sparse_attention(q, k, v, mask, BT)
    tok = np.zeros((1, H, N, N), dtype=bool)
    for h in range(H):
        for n in range(N):
            for m in range(N):
                tok[0, h, n, m] = bool(mask[h, n // BT, m // BT])
    np.testing.assert_allclose(o, _sdpa64(q, k, v, attn_mask=tok), rtol=1e-12,
                               atol=1e-12)


def test_convex_combination_bounds():
    BT, N, d = 16, 90, 6
    q, k, v = (_rand((1, 2, N, d), s) for s in (19, 20, 21))
    q *= 4.0  # sharper softmax, still inside the hull
    Tn = -(-N // BT)
    mask = oracle.tile_mask_static(1, Tn, Tn, 3, 1 << 23, True)
    o, _ = oracle.block_sparse_attention(q, k, v, mask, BT)
    for h in range(2):
        for n in range(N):
            keys = [m for m in range(N) if mask[0, n // BT, m // BT]]
            lo = v[0, h, keys].min(axis=0)
            hi = v[0, h, keys].max(axis=0)
            assert (o[0, h, n] >= lo - 1e-12).all()
            assert (o[0, h, n] <= hi + 1e-12).all()


def test_constant_and_tile_id_values():
    BT, N, d = 16, 77, 4
    q, k = (_rand((1, 1, N, d), s) for s in (22, 23))
    Tn = -(-N // BT)
    mask = oracle.tile_mask_window_anchor(7, 1, 11, BT, 1, 1, 5)[None]
    ones = np.ones((1, 1, N, d))
    o, _ = oracle.block_sparse_attention(q, k, ones, mask, BT)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)
    tid = np.repeat((np.arange(N) // BT).astype(float)[:, None], d, axis=1)
    o, _ = oracle.block_sparse_attention(q, k, tid[None, None], mask, BT)
    for n in range(N):
        act = np.nonzero(mask[0, n // BT])[0]
        assert act.min() - 1e-12 <= o[0, 0, n, 0] <= act.max() + 1e-12


def test_key_tile_permutation_invariance():
    BT, Tn, d = 8, 5, 4
    N = BT * Tn
    q, k, v = (_rand((1, 1, N, d), s) for s in (24, 25, 26))
    mask = oracle.tile_mask_static(1, Tn, Tn, 8, 1 << 23, True)
    o, lse = oracle.block_sparse_attention(q, k, v, mask, BT)
    perm = np.array([3, 0, 4, 2, 1])
    tok = np.concatenate([np.arange(p * BT, (p + 1) * BT) for p in perm])
    o2, lse2 = oracle.block_sparse_attention(q, k[:, :, tok], v[:, :, tok],
                                             mask[:, :, perm], BT)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-12)


def test_empty_rows_give_zero_and_minus_inf():
    BT, N, d = 8, 20, 4
    q, k, v = (_rand((1, 1, N, d), s) for s in (27, 28, 29))
    mask = np.zeros((1, 3, 3), dtype=np.uint8)
    mask[0, 1, 2] = 1
    o, lse = oracle.block_sparse_attention(q, k, v, mask, BT)
    assert (o[0, 0, :8] == 0).all() and (o[0, 0, 16:] == 0).all()
    assert np.isneginf(lse[0, 0, :8]).all() and np.isneginf(lse[0, 0, 16:]).all()
    assert np.isfinite(o).all() and np.isfinite(lse[0, 0, 8:16]).all()


def test_row_sample_matches_full_and_threads():
    BT, N, d = 16, 100, 8
    q, k, v = (_rand((2, 3, N, d), s) for s in (30, 31, 32))
    Tn = -(-N // BT)
    mask = oracle.tile_mask_static(3, Tn, Tn, 4, 1 << 23, True)
    o, lse = oracle.block_sparse_attention(q, k, v, mask, BT, chunk=7)
    rows = [0, 15, 16, 50, 99]
    os_, ls_ = oracle.block_sparse_attention_rows(q, k, v, mask, BT, rows,
                                                  workers=3, chunk=2)
    # chunking changes only the BLAS blocking, hence rounding order
    np.testing.assert_allclose(os_, o[:, :, rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ls_, lse[:, :, rows], rtol=1e-13, atol=1e-14)


def test_bf16_inputs_read_exactly():
    q, k, v = (torch.from_numpy(_rand((1, 1, 32, 8), s)).to(torch.bfloat16)
               for s in (33, 34, 35))
    mask = np.ones((1, 2, 2), dtype=np.uint8)
    o, _ = oracle.block_sparse_attention(q, k, v, mask, 16)
    f = lambda x: x.to(torch.float64).numpy()
    np.testing.assert_allclose(o, _sdpa64(f(q), f(k), f(v)), rtol=1e-12,
                               atol=1e-12)


def test_values_of_another_width_share_the_weights():
    """The weights do not depend on the values: attending over [V | K] gives
    the attention output with V in the first d columns and with V := K in
    the rest (the parity tests' LSE bound uses the second)."""
    g = torch.Generator().manual_seed(11)
    q, k, v = (torch.randn(1, 2, 200, 16, generator=g, dtype=torch.float64) for _ in range(3))
    m = (torch.rand(2, 4, 4, generator=g) < 0.6).to(torch.uint8).numpy()
    m[:, 0, :] = 0                                   # an empty row too
    o1, l1 = oracle.block_sparse_attention(q, k, v, m, 64)
    o2, l2 = oracle.block_sparse_attention(q, k, k, m, 64)
    o3, l3 = oracle.block_sparse_attention(q, k, torch.cat([v, k], -1), m, 64)
    np.testing.assert_array_equal(l1, l3)
    np.testing.assert_array_equal(l2, l3)
    np.testing.assert_allclose(o3[..., :16], o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(o3[..., 16:], o2, rtol=0, atol=1e-13)
