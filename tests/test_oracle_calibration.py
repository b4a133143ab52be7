"""Pins for the oracle's energy calibration (CPU only): block energies,
energy-based selection and cross-prompt aggregation (CalibAtt page,
"A. Fase di Calibrazione", steps 1 and 2)."""
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden


def _qk(B, H, N, d, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    return q, k


# --------------------------------------------------------------- energies
@pytest.mark.parametrize("N,tile", [(37, 8), (64, 16), (5, 8)])
def test_energy_rows_sum_to_query_rows(N, tile):
    """Each softmax row sums to 1, so row i of E sums to the number of query
    rows in tile i (the ragged last tile included)."""
    q, k = _qk(2, 3, N, 16, 11)
    E = oracle.block_energy(q, k, tile)
    nt = -(-N // tile)
    rows = np.minimum(tile, N - np.arange(nt) * tile)
    np.testing.assert_allclose(E.sum(axis=-1), np.broadcast_to(rows, E.shape[:-1]),
                               rtol=0, atol=1e-12)
    assert (E >= 0).all()


def test_energy_zero_queries_is_uniform():
    """q = 0: every key gets probability 1/N, so E[i, j] = r_i * c_j / N."""
    N, tile = 45, 16
    _, k = _qk(1, 2, N, 8, 3)
    q = torch.zeros_like(k)
    E = oracle.block_energy(q, k, tile)
    nt = -(-N // tile)
    sz = np.minimum(tile, N - np.arange(nt) * tile).astype(np.float64)
    np.testing.assert_allclose(E[0, 0], np.outer(sz, sz) / N, rtol=1e-13)
    np.testing.assert_allclose(E[0, 1], np.outer(sz, sz) / N, rtol=1e-13)


def test_energy_matches_brute_force():
    """Plain Python loops with math.exp on a tiny case."""
    N, d, tile, scale = 11, 4, 4, 0.7
    q, k = _qk(1, 1, N, d, 5)
    qa, ka = q[0, 0].double().tolist(), k[0, 0].double().tolist()
    nt = -(-N // tile)
    want = [[0.0] * nt for _ in range(nt)]
    for n in range(N):
        s = [scale * sum(qa[n][c] * ka[m][c] for c in range(d)) for m in range(N)]
        mx = max(s)
        z = sum(math.exp(x - mx) for x in s)
        for m in range(N):
            want[n // tile][m // tile] += math.exp(s[m] - mx) / z
    got = oracle.block_energy(q, k, tile, scale=scale)[0, 0]
    np.testing.assert_allclose(got, np.array(want), rtol=1e-12, atol=1e-15)


def test_energy_one_hot_attention():
    """Keys far apart and each query equal to a large multiple of one key:
    all of a row's probability sits on that key, so E counts, per block
    pair, the query rows whose key falls in the key tile."""
    N, d, tile = 12, 12, 4
    k = torch.eye(N, d).reshape(1, 1, N, d)
    target = [(3 * n + 5) % N for n in range(N)]
    q = torch.stack([60.0 * k[0, 0, t] for t in target]).reshape(1, 1, N, d)
    E = oracle.block_energy(q, k, tile, scale=1.0)[0, 0]
    want = np.zeros((3, 3))
    for n, t in enumerate(target):
        want[n // tile, t // tile] += 1
    np.testing.assert_allclose(E, want, atol=1e-20)


def test_energy_rows_are_rows_of_the_full_tensor():
    q, k = _qk(1, 2, 50, 8, 21)
    full = oracle.block_energy(q, k, 16)
    part = oracle.block_energy_rows(q, k, 16, [3, 0])
    np.testing.assert_allclose(part, full[:, :, [3, 0]], rtol=1e-13, atol=1e-15)


# -------------------------------------------------------------- selection
def test_selection_matches_hand_enumeration():
    lines = read_golden("calib_select_rows.txt")
    assert len(lines) == 9
    for ln in lines:
        eps, energies, sel = (x.strip() for x in ln.split("|"))
        e = np.array([float(x) for x in energies.split()], dtype=np.float32)
        want = np.zeros(len(e), dtype=np.uint8)
        if sel != "-":
            want[[int(x) for x in sel.split()]] = 1
        np.testing.assert_array_equal(oracle.select_row(e, float(eps)), want, ln)


def test_selection_is_the_shortest_greedy_prefix():
    """Random rows: the kept set reaches eps of the total, dropping its
    smallest member falls short, and no dropped block outweighs a kept one."""
    g = np.random.default_rng(9)
    for trial in range(300):
        Tk = int(g.integers(1, 40))
        e = (g.random(Tk) ** 3).astype(np.float32)
        if trial % 7 == 0:
            e[g.integers(0, Tk, size=Tk // 3)] = 0.0
        eps = float(g.choice([0.0, 0.3, 0.5, 0.8, 0.95, 0.99, 1.0]))
        keep = oracle.select_row(e, eps).astype(bool)
        e64 = e.astype(np.float64)
        total = e64.sum()
        if eps == 0.0:
            assert not keep.any()
            continue
        assert e64[keep].sum() >= eps * total * (1 - 1e-12)
        if keep.any():
            smallest = e64[keep].min()
            assert e64[keep].sum() - smallest < eps * total * (1 + 1e-12)
            if (~keep).any():
                assert e64[~keep].max() <= smallest


def test_select_mask_applies_per_row():
    g = np.random.default_rng(4)
    E = g.random((2, 3, 5, 7)).astype(np.float32)
    M = oracle.select_mask(E, 0.6)
    assert M.shape == E.shape and M.dtype == np.uint8
    for idx in np.ndindex(E.shape[:-1]):
        np.testing.assert_array_equal(M[idx], oracle.select_row(E[idx], 0.6))


# ------------------------------------------------------------ aggregation
def test_aggregation_thresholds():
    """Four prompts; cells selected by 0, 1, 2, 3 and 4 of them."""
    m = np.zeros((4, 5), dtype=np.uint8)
    for c in range(5):
        m[:c, c] = 1
    np.testing.assert_array_equal(oracle.aggregate(m, 0.5), [0, 0, 1, 1, 1])
    np.testing.assert_array_equal(oracle.aggregate(m, 0.0), [1, 1, 1, 1, 1])
    np.testing.assert_array_equal(oracle.aggregate(m, 1.0), [0, 0, 0, 0, 1])
    np.testing.assert_array_equal(oracle.aggregate(m, 0.75), [0, 0, 0, 1, 1])
    np.testing.assert_array_equal(oracle.aggregate(m, 0.76), [0, 0, 0, 0, 1])
    one = m[3:4]  # a single prompt: its own mask for any rho in (0, 1]
    np.testing.assert_array_equal(oracle.aggregate(one, 0.5), one[0])
