"""Pins for the oracle's index-branch variants (no GPU): the block mean-pool
summary and the forced local window, both after the sketch in section 3.3 of
chenxutan.com's "MiniMax M3 深度实战" (its block summary is the mean of the
block's keys; it always keeps the blocks nearest the query besides the
top-scored ones).

Mean pool: closed forms (constant blocks, one-token blocks, two-token means),
numpy's float64 mean of each block (to one fp32 rounding step), and the
ordering min <= mean <= max.  Window: window = 1 is the plain selection,
window = K is the pure sliding window, monotone scalar summaries give a closed
form, and a brute-force lexsort reference on random inputs.
"""
import numpy as np
import pytest


def test_pool_mean_closed_forms(orc):
    B, d = 8, 5
    # block 0 constant, block 1 two distinct values, block 2 one token
    x = np.zeros((17, d), np.float32)
    x[:8] = 1.25
    x[8:16] = np.array([[3.0, -1.0, 0.5, 7.0, -2.0]] * 4 + [[1.0, 1.0, 1.5, -7.0, 2.0]] * 4,
                       np.float32)
    x[16] = np.array([-0.5, 2.5, 9.0, 0.0, -3.25], np.float32)
    m = orc.pool_mean(x, B)
    assert m.shape == (3, d)
    assert np.all(m[0] == 1.25)
    assert m[1].tolist() == [2.0, 0.0, 1.0, 0.0, 0.0]
    assert np.array_equal(m[2], x[16])


def test_pool_mean_matches_float64_block_means(orc):
    rng = np.random.default_rng(5)
    for L, B, d in [(1000, 64, 16), (513, 512, 8), (77, 16, 3)]:
        x = rng.standard_normal((L, d)).astype(np.float32)
        m = orc.pool_mean(x, B)
        for b in range(m.shape[0]):
            blk = x[b * B:min(L, b * B + B)].astype(np.float64)
            want = blk.mean(axis=0).astype(np.float32)
            # two fp64 sums in different orders round to fp32 within one step
            assert np.all(np.abs(m[b] - want) <= np.spacing(np.abs(want)))
            assert np.all(m[b] >= blk.min(axis=0).astype(np.float32))
            assert np.all(m[b] <= blk.max(axis=0).astype(np.float32))


def _brute_window(idx_q, pos, kmax, B, K, w):
    rows = []
    for i, p in enumerate(pos):
        own = p // B
        first = max(0, own - w + 1)
        s = kmax[:first].astype(np.float64) @ idx_q[i].astype(np.float64)
        order = np.lexsort((np.arange(first), -s))
        kept = sorted(order[:min(K - w, first)].tolist())
        row = kept + list(range(first, own + 1))
        rows.append(row + [-1] * (K - len(row)))
    return np.array(rows, np.int32)


def test_window_one_is_the_plain_selection(orc):
    rng = np.random.default_rng(1)
    kmax = rng.standard_normal((50, 12)).astype(np.float32)
    q = rng.standard_normal((300, 12)).astype(np.float32)
    pos = rng.integers(0, 50 * 32, 300).astype(np.int64)
    a = orc.select(q, pos, kmax, 32, 6)
    b = orc.select(q, pos, kmax, 32, 6, window=1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


def test_window_k_is_the_sliding_window(orc):
    rng = np.random.default_rng(2)
    B, K = 16, 5
    kmax = rng.standard_normal((40, 8)).astype(np.float32)
    pos = np.arange(0, 40 * B, 7, dtype=np.int64)
    q = rng.standard_normal((len(pos), 8)).astype(np.float32)
    sel, gr, *_ = orc.select(q, pos, kmax, B, K, window=K)
    for i, p in enumerate(pos):
        own = p // B
        row = list(range(max(0, own - K + 1), own + 1))
        assert sel[i].tolist() == row + [-1] * (K - len(row))
    assert np.all(np.isnan(gr))


def test_window_monotone_closed_form(orc):
    # kmax[b] = b with q > 0: the kept candidates are the K-w blocks just
    # below the window; q < 0 keeps blocks 0 .. K-w-1.
    B, K, w, nb = 8, 6, 3, 30
    kmax = np.arange(nb, dtype=np.float32)[:, None]
    pos = np.array([0, 9, 23, 40, 100, 239], np.int64)
    for qv in (1.0, -1.0):
        q = np.full((len(pos), 1), qv, np.float32)
        sel, gr, ga, eb = orc.select(q, pos, kmax, B, K, window=w)
        for i, p in enumerate(pos):
            own = p // B
            first = max(0, own - w + 1)
            m = min(K - w, first)
            kept = list(range(first - m, first)) if qv > 0 else list(range(m))
            row = kept + list(range(first, own + 1))
            assert sel[i].tolist() == row + [-1] * (K - len(row))
            if first > K - w:
                a, z = (first - (K - w), first - (K - w) - 1) if qv > 0 else (K - w - 1, K - w)
                assert ga[i] == pytest.approx(qv * a - qv * z)


@pytest.mark.parametrize("B,K,w", [(16, 4, 2), (32, 8, 3), (64, 6, 6), (16, 5, 1)])
def test_window_brute_force(orc, B, K, w):
    rng = np.random.default_rng(B + K + w)
    nb = 45
    kmax = rng.standard_normal((nb, 10)).astype(np.float32)
    kmax[7] = kmax[3]            # a duplicated block: ties go to the lower index
    pos = rng.integers(0, nb * B, 400).astype(np.int64)
    q = rng.standard_normal((len(pos), 10)).astype(np.float32)
    sel, *_ = orc.select(q, pos, kmax, B, K, window=w)
    assert np.array_equal(sel, _brute_window(q, pos, kmax, B, K, w))
