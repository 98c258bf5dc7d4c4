"""Pins for the oracle's inverse map (queries per KV block, CSR) -- no GPU.

The KV-outer loop of section 2.2 ("KV Outer Gather Q：MSA 的关键设计") of
chenxutan.com's "MiniMax M3 深度实战" needs, per block, the queries that hit
it.  Pinned by the round trip (transposing the CSR gives back the selection),
ascending rows, nnz, the own-tokens-first structure of a causal selection, and
a hand-worked case.
"""
import numpy as np


def _roundtrip(sel, row_ptr, q_list, slot, nb):
    n_q, K = sel.shape
    assert row_ptr[0] == 0 and np.all(np.diff(row_ptr) >= 0)
    assert row_ptr[-1] == len(q_list) == np.count_nonzero(sel >= 0)
    for b in range(nb):
        row = q_list[row_ptr[b]:row_ptr[b + 1]]
        assert np.all(np.diff(row) > 0), "rows ascending, no repeats"
        for i in row:
            assert b in sel[i]
    for i in range(n_q):
        for k in range(K):
            b = sel[i, k]
            if b < 0:
                assert slot[i, k] == -1
            else:
                s = slot[i, k]
                assert row_ptr[b] <= s < row_ptr[b + 1] and q_list[s] == i


def test_hand_worked_case(orc):
    sel = np.array([[0, -1, -1],
                    [0, 1, -1],
                    [1, 2, -1],
                    [0, 2, 3]], np.int32)
    row_ptr, q_list, slot = orc.invert(sel, 4)
    # block 0 <- queries 0, 1, 3; block 1 <- 1, 2; block 2 <- 2, 3; block 3 <- 3
    assert row_ptr.tolist() == [0, 3, 5, 7, 8]
    assert q_list.tolist() == [0, 1, 3, 1, 2, 2, 3, 3]
    assert slot.tolist() == [[0, -1, -1], [1, 3, -1], [4, 5, -1], [2, 6, 7]]


def test_roundtrip_random_causal_selection(orc):
    rng = np.random.default_rng(6)
    B, K, L, d = 16, 5, 1500, 8
    kmax = orc.pool(rng.standard_normal((L, d)).astype(np.float32), B)
    pos = np.arange(L, dtype=np.int64)
    sel, *_ = orc.select(rng.standard_normal((L, d)).astype(np.float32), pos,
                         kmax, B, K)
    nb = kmax.shape[0]
    row_ptr, q_list, slot = orc.invert(sel, nb)
    _roundtrip(sel, row_ptr, q_list, slot, nb)
    # causal structure: row b starts with the block's own tokens b*B.., in order
    for b in range(nb):
        own = list(range(b * B, min(L, b * B + B)))
        assert q_list[row_ptr[b]:row_ptr[b] + len(own)].tolist() == own


def test_roundtrip_arbitrary_sets(orc):
    rng = np.random.default_rng(7)
    nb, K = 37, 6
    sel = np.full((500, K), -1, np.int32)
    for i in range(500):
        n = rng.integers(0, K + 1)
        sel[i, :n] = np.sort(rng.choice(nb, size=n, replace=False))
    row_ptr, q_list, slot = orc.invert(sel, nb)
    _roundtrip(sel, row_ptr, q_list, slot, nb)
