"""Pins for the oracle's block max-pool (no GPU).

The pool is "elementwise max over the valid tokens of each block" (index
branch of the youleyou.com page "MiniMax M3模型算力成本大幅降低原因深度解析").
Pinned by hand-built blocks with a closed-form max, by numpy's own max over a
reshaped array, and by the partial-block and signed-zero readings.
"""
import numpy as np


def test_one_hot_rows(orc):
    # Block b holds the one-hot rows e_{(b + t) mod d} for t < B: the max is the
    # indicator of those columns.
    d, B, nb = 16, 4, 5
    x = np.zeros((nb * B, d), np.float32)
    for b in range(nb):
        for t in range(B):
            x[b * B + t, (b + t) % d] = 1.0
    got = orc.pool(x, B)
    want = np.zeros((nb, d), np.float32)
    for b in range(nb):
        want[b, [(b + t) % d for t in range(B)]] = 1.0
    assert np.array_equal(got, want)


def test_constant_block_and_single_token_tail(orc):
    d, B = 8, 16
    x = np.full((2 * B + 1, d), -3.25, np.float32)
    x[B:2 * B] = 7.5
    x[2 * B] = np.arange(d, dtype=np.float32) - 100.0   # 1-token last block
    got = orc.pool(x, B)
    assert got.shape == (3, d)
    assert np.all(got[0] == -3.25) and np.all(got[1] == 7.5)
    assert np.array_equal(got[2], x[2 * B])


def test_all_negative_partial_block_is_not_zero_padded(orc):
    # A partial last block of negative values keeps its (negative) max: the
    # pool runs over valid tokens only.
    d, B = 32, 64
    rng = np.random.default_rng(1)
    x = -np.abs(rng.standard_normal((B + 5, d)).astype(np.float32)) - 0.5
    got = orc.pool(x, B)
    assert np.all(got[1] < 0)
    assert np.array_equal(got[1], x[B:].max(axis=0))


def test_matches_numpy_max(orc):
    rng = np.random.default_rng(2)
    for L, B, d in [(4096, 64, 64), (1000, 128, 24), (17, 16, 3), (1, 16, 5)]:
        x = rng.standard_normal((L, d)).astype(np.float32)
        got = orc.pool(x, B)
        nb = -(-L // B)
        want = np.stack([x[b * B:min(L, b * B + B)].max(axis=0)
                         for b in range(nb)])
        assert np.array_equal(got, want)
        full = (L // B) * B
        if full:
            assert np.array_equal(got[:L // B],
                                  x[:full].reshape(-1, B, d).max(axis=1))


def test_signed_zero_order(orc):
    # -0 < +0 in the pool's total order, whichever comes first.
    x = np.array([[-0.0], [0.0], [-0.0], [-1.0]], np.float32)
    got = orc.pool(x, 4)
    assert got[0, 0] == 0.0 and not np.signbit(got[0, 0])
    y = np.array([[-0.0], [-0.0], [-2.0]], np.float32)
    got = orc.pool(y, 4)
    assert got[0, 0] == 0.0 and np.signbit(got[0, 0])
