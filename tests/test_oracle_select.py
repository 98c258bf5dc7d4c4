"""Pins for the oracle's scores and causal top-K (no GPU).

Definition (index branch of "MiniMax M3模型算力成本大幅降低原因深度解析"; the
per-query scoring of the prefill/decode section 3.3 of chenxutan.com's
"MiniMax M3 深度实战"): for a query at position p, own = p // B; candidates are
blocks b < own scored by idx_q . kmax[b]; keep the best min(K-1, own) by
(score desc, index asc), add own, store ascending, pad -1.

Pins: closed forms (monotone summaries with d_idx = 1, one-hot summaries),
duplicated blocks (tie-break), optimality checked against scores computed
independently with numpy, the structural invariants, the cut-gap report, and
hand-worked fixtures under tests/golden/.
"""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check_invariants(sel, pos, B, K):
    for i, p in enumerate(pos):
        own = p // B
        n = min(K, own + 1)
        row = sel[i]
        assert np.all(row[n:] == -1)
        kept = row[:n]
        assert kept[-1] == own
        assert np.all(np.diff(kept) > 0)
        assert kept[0] >= 0


def test_monotone_scalar_summaries_closed_form(orc):
    # d_idx = 1, kmax[b] = b: score = q * b.  q > 0 keeps the K-1 blocks just
    # below own; q < 0 keeps blocks 0..K-2.
    B, K, nb = 16, 4, 40
    kmax = np.arange(nb, dtype=np.float32)[:, None]
    pos = np.array([0, 15, 16, 40, 63, 64, 200, 639], np.int64)
    for qv in (1.0, -1.0):
        q = np.full((len(pos), 1), qv, np.float32)
        sel, gr, ga, eb = orc.select(q, pos, kmax, B, K)
        _check_invariants(sel, pos, B, K)
        for i, p in enumerate(pos):
            own = p // B
            m = min(K - 1, own)
            want = (list(range(own - m, own)) if qv > 0 else list(range(m))) + [own]
            want += [-1] * (K - len(want))
            assert sel[i].tolist() == want
            if own > K - 1:
                # last kept vs first left out: (own-K+1, own-K) for q>0,
                # (K-2, K-1) for q<0 (scores -(K-2) and -(K-1)).
                a, z = (own - K + 1, own - K) if qv > 0 else (K - 2, K - 1)
                assert ga[i] == pytest.approx(qv * a - qv * z)
                den = max(abs(a), abs(z))
                assert gr[i] == pytest.approx(1.0 / den)
                u = 2.0 ** -24
                gamma = 1 * u / (1 - 1 * u)
                assert eb[i] == pytest.approx(gamma * (abs(a) + abs(z)))
            else:
                assert np.isnan(ga[i]) and np.isnan(gr[i]) and np.isnan(eb[i])


def test_one_hot_summaries_pick_largest_query_components(orc):
    # kmax[b] = e_b (d_idx = nb): score[b] = q[b].  The kept set is the K-1
    # largest q components among b < own (ties to the lower b), plus own.
    rng = np.random.default_rng(3)
    B, K, nb = 32, 6, 24
    kmax = np.eye(nb, dtype=np.float32)
    q = rng.standard_normal((50, nb)).astype(np.float32)
    q[0, :10] = 0.5                       # a row full of exact ties
    pos = rng.integers(0, nb * B, size=50).astype(np.int64)
    pos[0] = nb * B - 1
    sel, *_ = orc.select(q, pos, kmax, B, K)
    _check_invariants(sel, pos, B, K)
    for i, p in enumerate(pos):
        own = p // B
        cand = np.arange(own)
        order = sorted(cand.tolist(), key=lambda b: (-q[i, b], b))
        want = sorted(order[:K - 1]) + [own]
        got = [x for x in sel[i].tolist() if x >= 0]
        assert got == want


def test_duplicate_blocks_tie_to_lower_index(orc):
    # Every block has the same summary: all scores tie, so the kept
    # candidates are 0..K-2.
    rng = np.random.default_rng(4)
    B, K, nb, d = 64, 5, 30, 16
    kmax = np.tile(rng.standard_normal((1, d)).astype(np.float32), (nb, 1))
    q = rng.standard_normal((20, d)).astype(np.float32)
    pos = np.arange(20, dtype=np.int64) * 97
    sel, gr, ga, _ = orc.select(q, pos, kmax, B, K)
    for i, p in enumerate(pos):
        own = p // B
        m = min(K - 1, own)
        assert sel[i, :m + 1].tolist() == list(range(m)) + [own]
        if own > K - 1:
            assert ga[i] == 0.0 and gr[i] == 0.0


def test_optimal_against_independent_scores(orc):
    rng = np.random.default_rng(5)
    B, K, L, d = 16, 7, 2000, 32
    idx_k = rng.standard_normal((L, d)).astype(np.float32)
    kmax = orc.pool(idx_k, B)
    q = rng.standard_normal((300, d)).astype(np.float32)
    pos = rng.integers(0, L, size=300).astype(np.int64)
    sel, *_ = orc.select(q, pos, kmax, B, K)
    _check_invariants(sel, pos, B, K)
    scores = q.astype(np.float64) @ kmax.astype(np.float64).T     # [n_q, nb]
    for i, p in enumerate(pos):
        own = p // B
        kept = set(x for x in sel[i].tolist() if 0 <= x < own)
        left = [b for b in range(own) if b not in kept]
        assert len(kept) == min(K - 1, own)
        if kept and left:
            worst_kept = min(kept, key=lambda b: (scores[i, b], -b))
            best_left = max(left, key=lambda b: (scores[i, b], -b))
            assert (scores[i, worst_kept], -worst_kept) > (scores[i, best_left],
                                                            -best_left)


def test_future_blocks_never_chosen_and_own_forced(orc):
    # Future blocks carry huge summaries; the own block carries a very
    # negative one.  Neither changes the causal selection.
    B, K, nb, d = 16, 3, 10, 4
    kmax = np.full((nb, d), -1.0, np.float32)
    kmax[5:] = 1e6
    kmax[4] = -1e6
    q = np.ones((1, d), np.float32)
    pos = np.array([4 * B + 3], np.int64)
    sel, *_ = orc.select(q, pos, kmax, B, K)
    assert sel[0].tolist() == [0, 1, 4]


def _read_fixture(name):
    with open(os.path.join(GOLDEN, name)) as f:
        lines = [ln.split("#")[0].strip() for ln in f]
    return [ln for ln in lines if ln]


def test_golden_hand_worked_selection(orc):
    lines = _read_fixture("select_hand_worked.txt")
    it = iter(lines)
    B, K, d = (int(x) for x in next(it).split())
    nb = int(next(it))
    kmax = np.array([[float(x) for x in next(it).split()] for _ in range(nb)],
                    np.float32)
    n_q = int(next(it))
    q, pos, want = [], [], []
    for _ in range(n_q):
        parts = next(it).split("|")
        pos.append(int(parts[0]))
        q.append([float(x) for x in parts[1].split()])
        want.append([int(x) for x in parts[2].split()])
    sel, *_ = orc.select(np.array(q, np.float32), np.array(pos, np.int64), kmax,
                         B, K)
    assert sel.tolist() == want
