"""Shared test helpers: acceptance rules for selections and outputs.

Selections: the device result must equal the oracle's bit for bit, except on
queries the oracle flags as near-ties -- relative gap between the last kept
and first left-out candidate below 1e-3, or an absolute gap within the fp32
error bound of the two dot products.  There either choice is accepted, after
checking that the device row is itself a valid causal top-K (right size, own
block present, ascending, and optimal within that margin).
"""
from __future__ import annotations

import numpy as np

REL_TIE = 1e-3          # relative near-tie threshold on the oracle's cut gap
TOL_F32 = 1e-4          # max-abs output tolerance, fp32 inputs
TOL_BF16 = 1e-2         # max-abs output tolerance, bf16 inputs


def flagged(gap_rel, gap_abs, err_bnd):
    """Queries whose top-K cut is a near-tie (either rule)."""
    gr = np.nan_to_num(gap_rel, nan=np.inf)
    ga = np.nan_to_num(gap_abs, nan=np.inf)
    eb = np.nan_to_num(err_bnd, nan=0.0)
    return (gr < REL_TIE) | (ga <= eb)


def check_selection(dev_sel, orc_sel, gap_rel, gap_abs, err_bnd, idx_q, kmax,
                    q_pos, block, window=1):
    """Assert the acceptance rule; return (n_flagged, n_mismatch).  With a
    local window the forced blocks are own-window+1 .. own and only the
    blocks below them are ranked."""
    dev_sel = np.asarray(dev_sel)
    orc_sel = np.asarray(orc_sel)
    assert dev_sel.shape == orc_sel.shape
    flag = flagged(gap_rel, gap_abs, err_bnd)
    diff = np.any(dev_sel != orc_sel, axis=1)
    bad = np.nonzero(diff & ~flag)[0]
    assert bad.size == 0, (
        f"{bad.size} unflagged selection mismatches, first rows {bad[:5]}: "
        f"device {dev_sel[bad[:2]]}, oracle {orc_sel[bad[:2]]}")
    K = dev_sel.shape[1]
    for r in np.nonzero(diff)[0]:
        own = int(q_pos[r]) // block
        first = max(0, own - window + 1)
        n_cand = min(K - window, first)
        n = n_cand + own - first + 1
        row = dev_sel[r]
        assert np.all(row[n:] == -1)
        assert row[n_cand:n].tolist() == list(range(first, own + 1))
        assert np.all(np.diff(row[:n]) > 0) and row[0] >= 0
        s = kmax[:first].astype(np.float64) @ idx_q[r].astype(np.float64)
        kept = set(row[:n_cand].tolist())
        left = [b for b in range(first) if b not in kept]
        if kept and left:
            margin = max(REL_TIE * np.max(np.abs(s)), 2 * float(err_bnd[r]))
            assert min(s[list(kept)]) >= max(s[left]) - margin
    return int(flag.sum()), int(diff.sum())


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))
