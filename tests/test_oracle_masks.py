"""Pins for the oracle's tile masks (CPU only)."""
import numpy as np
import pytest

import oracle
import workloads as W
from conftest import read_golden


def _parse_rows(lines):
    return np.array([[int(ch) for ch in ln] for ln in lines], dtype=np.uint8)


# ------------------------------------------------------------- frame rule
def test_tiny_masks_match_hand_enumeration():
    lines = read_golden("tiny_window_anchor_masks.txt")
    blocks = {}
    cur = None
    for ln in lines:
        if ln.startswith("rotation"):
            cur = int(ln.split()[1])
            blocks[cur] = []
        else:
            blocks[cur].append(ln)
    assert sorted(blocks) == [0, 1, 2, 3]
    counts = []
    w = W.WORKLOADS[1]
    for r, rows in blocks.items():
        want = _parse_rows(rows)
        got = oracle.tile_mask(w.mask.kind, w.frames, w.grid_h, w.grid_w,
                               w.tile, window=w.mask.window,
                               num_anchors=w.mask.num_anchors, rotation=r)
        assert got.shape == (1, 4, 4)
        np.testing.assert_array_equal(got[0], want)
        counts.append(int(want.sum()))
    assert counts == [12, 11, 11, 12]


def test_misaligned_mask_matches_hand_enumeration():
    lines = read_golden("misaligned_window_anchor_mask.txt")
    hdr = lines[0].split()
    kv = dict(zip(hdr[0::2], map(int, hdr[1::2])))
    want = _parse_rows(lines[1:])
    got = oracle.tile_mask_window_anchor(kv["frames"], kv["grid_h"], kv["grid_w"],
                                         kv["tile"], kv["window"], kv["anchors"],
                                         kv["rotation"])
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("T,n_a", [(4, 1), (21, 1), (21, 3), (21, 7), (84, 4),
                                   (12, 4), (10, 3)])
def test_every_frame_anchors_equally_often(T, n_a):
    """Over r = 0..T-1 every frame is in G_r exactly n_a times; with n_a | T,
    every frame is an anchor exactly once over T/n_a consecutive rotations
    (LVSA page, Meccanismo Core: each frame serves as a global anchor exactly
    once over T_per consecutive steps)."""
    counts = np.zeros(T, dtype=int)
    for r in range(T):
        G = oracle.anchor_frames(T, n_a, r)
        assert len(G) == n_a
        for f in G:
            counts[f] += 1
    assert (counts == n_a).all()
    if T % n_a == 0:
        per = T // n_a
        for start in range(T):
            seen = np.zeros(T, dtype=int)
            for r in range(start, start + per):
                for f in oracle.anchor_frames(T, n_a, r):
                    seen[f] += 1
            assert (seen == 1).all()


def test_anchor_placement_examples():
    assert oracle.anchor_frames(4, 1, 3) == {3}
    assert oracle.anchor_frames(21, 2, 0) == {0, 10}
    assert oracle.anchor_frames(21, 2, 15) == {15, 4}
    assert oracle.anchor_frames(84, 4, 5) == {5, 26, 47, 68}
    assert oracle.anchor_frames(84, 4, 84 + 5) == {5, 26, 47, 68}
    assert oracle.anchor_frames(7, 0, 2) == set()


def test_window_clipped_and_symmetric():
    assert oracle.window_frames(0, 5, 1) == {0, 1}
    assert oracle.window_frames(4, 5, 2) == {2, 3, 4}
    assert oracle.window_frames(2, 5, 0) == {2}
    F = oracle.frame_mask(9, 2, 0, 0)
    np.testing.assert_array_equal(F, F.T)


def _token_level_tile_mask(T, P, BT, w, n_a, r):
    """Brute force: token-level frame mask, OR-reduced over each tile pair."""
    N = T * P
    nt = -(-N // BT)
    G = {(r % T + (k * T) // n_a) % T for k in range(n_a)}
    M = np.zeros((nt, nt), dtype=np.uint8)
    for n in range(N):
        t = n // P
        for m in range(N):
            f = m // P
            if abs(f - t) <= w or f in G:
                M[n // BT, m // BT] = 1
    return M


@pytest.mark.parametrize("T,gh,gw,BT,w,n_a,r", [
    (5, 1, 3, 2, 0, 1, 4), (5, 1, 3, 2, 1, 2, 3), (7, 1, 5, 4, 1, 1, 2),
    (7, 1, 5, 4, 0, 2, 6), (6, 2, 3, 4, 1, 2, 1), (4, 2, 2, 8, 0, 1, 0),
    (9, 3, 3, 5, 2, 3, 7), (3, 1, 7, 3, 0, 0, 0), (8, 1, 3, 16, 1, 2, 5),
])
def test_tile_lift_equals_token_level_brute_force(T, gh, gw, BT, w, n_a, r):
    got = oracle.tile_mask_window_anchor(T, gh, gw, BT, w, n_a, r)
    want = _token_level_tile_mask(T, gh * gw, BT, w, n_a, r)
    np.testing.assert_array_equal(got, want)


def test_video_shape_counts_and_linear_scaling():
    """Active-tile counts of the two window+anchor video shapes at rotation 0
    (15 509 of 256^2 and 115 559 of 1024^2, an independent cross-check), and
    the LVSA complexity claim (LVSA page, Complessita): at a fixed frame
    budget the mean row length is about (2w+1+n_a)*P/BT, independent of T."""
    m2 = oracle.tile_mask_window_anchor(21, 30, 52, 128, 1, 2, 0)
    m4 = oracle.tile_mask_window_anchor(84, 30, 52, 128, 2, 4, 0)
    assert m2.shape == (256, 256) and int(m2.sum()) == 15509
    assert m4.shape == (1024, 1024) and int(m4.sum()) == 115559
    per_frame = 1560 / 128
    for m, budget in ((m2, 3 + 2), (m4, 5 + 4)):
        mean_row = m.sum() / m.shape[0]
        # clipped windows at the two ends pull the mean down, tiles that
        # straddle a frame boundary push it up; both effects are bounded
        assert (budget - 1) * per_frame <= mean_row <= (budget + 2) * per_frame
    # same budget, 4x the frames -> about 4x the active tiles
    m2b = oracle.tile_mask_window_anchor(84, 30, 52, 128, 1, 2, 0)
    ratio = m2b.sum() / m2.sum()
    assert 3.5 < ratio < 4.5


def test_mask_symmetry_without_anchors():
    m = oracle.tile_mask_window_anchor(21, 30, 52, 128, 1, 0, 0)
    np.testing.assert_array_equal(m, m.T)


def test_diagonal_always_active_window_mode():
    for r in range(21):
        m = oracle.tile_mask_window_anchor(21, 30, 52, 128, 1, 2, r)
        assert (np.diag(m) == 1).all()


# ------------------------------------------------------------ static mode
def test_splitmix64_published_vector():
    want = [int(x) for x in read_golden("splitmix64_seed1234567.txt")]
    got = [int(x) for x in oracle.splitmix64_stream(1234567, 5)]
    assert got == want


def test_static_hash_is_top_24_bits():
    z = [int(x) for x in read_golden("splitmix64_seed1234567.txt")]
    got = oracle.static_hash24(1234567, 5)
    assert [int(x) for x in got] == [x >> 40 for x in z]


def test_static_mask_cell_order_and_threshold():
    """Cell c = (h*Tq + i)*Tk + j takes the (c+1)-th output of the stream."""
    z = [int(x) for x in read_golden("splitmix64_seed1234567.txt")]
    # a 1x1x5 mask with threshold just above/below each hash value
    for c, zc in enumerate(z):
        h24 = zc >> 40
        m_hi = oracle.tile_mask_static(1, 1, 5, 1234567, h24 + 1, False)
        m_lo = oracle.tile_mask_static(1, 1, 5, 1234567, h24, False)
        assert m_hi[0, 0, c] == 1 and m_lo[0, 0, c] == 0


def test_static_mask_density_and_diagonal():
    w = W.WORKLOADS[3]
    Tn = w.num_tiles
    m = oracle.tile_mask(w.mask.kind, w.frames, w.grid_h, w.grid_w, w.tile,
                         seed=w.mask.seed, thresh24=w.mask.thresh24,
                         force_diagonal=w.mask.force_diagonal,
                         mask_heads=w.mask.mask_heads)
    assert m.shape == (12, Tn, Tn)
    for h in range(12):
        assert (np.diag(m[h]) == 1).all()
    p = w.mask.thresh24 / 2 ** 24
    expect = p + (1 - p) / Tn
    n = m.size
    sigma = np.sqrt(p * (1 - p) / n)
    assert abs(m.mean() - expect) < 4 * sigma
    # heads differ (independent draws), repeatable across calls
    assert (m[0] != m[1]).any()
    m2 = oracle.tile_mask_static(12, Tn, Tn, w.mask.seed, w.mask.thresh24, True)
    np.testing.assert_array_equal(m, m2)


def test_static_mask_extremes():
    assert oracle.tile_mask_static(2, 5, 7, 9, 0, False).sum() == 0
    assert oracle.tile_mask_static(2, 5, 7, 9, 1 << 24, False).all()
    d = oracle.tile_mask_static(1, 6, 6, 9, 0, True)[0]
    np.testing.assert_array_equal(d, np.eye(6, dtype=np.uint8))


def test_dense_mask():
    m = oracle.tile_mask(2, 21, 30, 52, 128, mask_heads=1)
    assert m.shape == (1, 256, 256) and m.all()


def test_thresh24_encoding():
    assert W.thresh24_for_density(0.3) == 5033164
    assert W.thresh24_for_density(1.0) == 1 << 24
    assert W.thresh24_for_density(0.0) == 0


# -------------------------------------------------- expanded adaptive windows
def _golden_cases(name):
    cases, cur = [], None
    for ln in read_golden(name):
        if ln.startswith("case"):
            kv = ln.split()[1:]
            cur = (dict(zip(kv[0::2], map(int, kv[1::2]))), {})
            cases.append(cur)
        else:
            t, frames = ln.split(":")
            cur[1][int(t)] = {int(f) for f in frames.split()}
    return cases


def test_expanded_frame_sets_match_hand_enumeration():
    cases = _golden_cases("expanded_window_frame_sets.txt")
    assert len(cases) == 2
    for kv, want in cases:
        T = kv["T"]
        assert sorted(want) == list(range(T))
        for t in range(T):
            got = oracle.frame_set_expanded(t, T, kv["window"], kv["anchors"],
                                            kv["rotation"], kv["budget"])
            assert got == want[t], (kv, t)
            assert len(got) == kv["budget"]


def test_expanded_tile_mask_matches_hand_enumeration():
    lines = read_golden("expanded_window_tile_mask.txt")
    hdr = lines[0].split()
    kv = dict(zip(hdr[0::2], map(int, hdr[1::2])))
    want = _parse_rows(lines[1:])
    got = oracle.tile_mask(3, kv["frames"], kv["grid_h"], kv["grid_w"],
                           kv["tile"], window=kv["window"],
                           num_anchors=kv["anchors"], rotation=kv["rotation"],
                           budget=kv["budget"], mask_heads=2)
    assert got.shape == (2,) + want.shape
    np.testing.assert_array_equal(got[0], want)
    np.testing.assert_array_equal(got[1], want)


@pytest.mark.parametrize("T,w,n_a,r", [(10, 1, 2, 3), (21, 1, 2, 5),
                                       (7, 0, 0, 0), (13, 3, 13, 4)])
def test_expanded_small_budget_is_the_plain_window(T, w, n_a, r):
    """A budget no larger than |G u W_plain(t)| leaves the window alone, so
    the mask equals the plain window + anchor mask."""
    for C in (0, 1, n_a + 1):
        np.testing.assert_array_equal(
            oracle.frame_mask_expanded(T, w, n_a, r, C),
            oracle.frame_mask(T, w, n_a, r))


@pytest.mark.parametrize("T,w,n_a,r", [(9, 1, 3, 1), (21, 0, 2, 20),
                                       (5, 4, 1, 0)])
def test_expanded_budget_of_whole_video_is_dense(T, w, n_a, r):
    for C in (T, T + 1, 10 * T):
        assert (oracle.frame_mask_expanded(T, w, n_a, r, C) == 1).all()


@pytest.mark.parametrize("T", [1, 2, 5, 12, 21])
def test_expanded_without_anchors_is_the_nearest_run(T):
    """No anchors, w = 0: A(t) is the run of L = min(C, T) frames around t,
    one more frame before t than after when L is even, pushed inward at the
    ends of the video: lo = max(0, min(t - ceil((L-1)/2), T - L))."""
    for C in range(1, T + 3):
        L = min(C, T)
        for t in range(T):
            lo = max(0, min(t - (L // 2), T - L))
            want = set(range(lo, lo + L))
            assert oracle.frame_set_expanded(t, T, 0, 0, 0, C) == want, (C, t)


def test_expanded_window_is_balanced_and_minimal():
    """Properties of the growth order on a sweep of small cases: W(t) is one
    run [lo, hi] around t containing the plain window; away from the ends it
    reaches at most one frame further back than forward (earlier frame
    first); |A(t)| = max(min(C, T), |G u W_plain(t)|); and if the window grew
    at all, dropping the frame added last falls short of the target."""
    n = 0
    for T in (1, 2, 3, 6, 11, 16):
        for n_a in sorted({0, 1, 2, T // 3, T}):
            for w in (0, 1, 3):
                for r in (0, T // 2 + 1):
                    G = oracle.anchor_frames(T, n_a, r)
                    for C in range(0, T + 2):
                        target = min(C, T)
                        for t in range(T):
                            Wp = oracle.window_frames(t, T, w)
                            W = oracle.expanded_window_frames(t, T, w, n_a, r,
                                                              C)
                            lo, hi = min(W), max(W)
                            assert W == set(range(lo, hi + 1))
                            assert Wp <= W and lo <= t <= hi
                            A = G | W
                            assert len(A) == max(target, len(G | Wp))
                            if W == Wp:
                                continue
                            back, fwd = t - lo, hi - t
                            if lo > 0 and hi < T - 1:
                                assert back - fwd in (0, 1)
                            # the frame added last is the farthest from t,
                            # the later one of two equally far
                            last = max(W, key=lambda f: (abs(f - t), f))
                            assert len(G | (W - {last})) < target
                            n += 1
    assert n > 500


# ------------------------------------------------------------ block diagonal
def test_block_diagonal_by_hand():
    """5 tiles in runs of 2: {0, 1}, {2, 3}, {4}."""
    want = np.array([[1, 1, 0, 0, 0],
                     [1, 1, 0, 0, 0],
                     [0, 0, 1, 1, 0],
                     [0, 0, 1, 1, 0],
                     [0, 0, 0, 0, 1]], dtype=np.uint8)
    got = oracle.tile_mask(4, 1, 1, 300, 64, block_tiles=2, mask_heads=2)
    assert got.shape == (2, 5, 5)
    np.testing.assert_array_equal(got[0], want)
    np.testing.assert_array_equal(got[1], want)
    np.testing.assert_array_equal(oracle.tile_mask(4, 1, 1, 300, 64, block_tiles=1)[0],
                                  np.eye(5, dtype=np.uint8))
    assert (oracle.tile_mask(4, 1, 1, 300, 64, block_tiles=5)[0] == 1).all()
    with pytest.raises(ValueError):
        oracle.tile_mask(4, 1, 1, 300, 64, block_tiles=0)
