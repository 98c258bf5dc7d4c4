"""Shared test helpers: acceptance rules for selections and outputs.

Selections: the device result must equal the oracle's bit for bit, except on
queries the oracle flags as near-ties -- relative gap between the last kept
and first left-out candidate below 1e-3 (the relative rule), or an absolute
gap within the fp32 error bound of the two dot products (the error-bound
rule).  There either choice is accepted, after checking that the device row
is itself a valid causal top-K: right size, forced blocks present, ascending,
and its own cut (lowest kept against highest left-out score) a near-tie by the
same two rules, computed for that pair of blocks.
"""
from __future__ import annotations

import numpy as np

REL_TIE = 1e-3          # relative near-tie threshold on the oracle's cut gap
TOL_F32 = 1e-4          # max-abs output tolerance, fp32 inputs
TOL_BF16 = 1e-2         # max-abs output tolerance, bf16 inputs
U32 = 2.0 ** -24        # unit roundoff of fp32


def flag_rules(gap_rel, gap_abs, err_bnd):
    """(relative-rule mask, error-bound-rule mask) of the oracle's cut."""
    gr = np.nan_to_num(np.asarray(gap_rel, np.float64), nan=np.inf)
    ga = np.nan_to_num(np.asarray(gap_abs, np.float64), nan=np.inf)
    eb = np.nan_to_num(np.asarray(err_bnd, np.float64), nan=0.0)
    return gr < REL_TIE, ga <= eb


def flagged(gap_rel, gap_abs, err_bnd):
    """Queries whose top-K cut is a near-tie (either rule)."""
    rel, bnd = flag_rules(gap_rel, gap_abs, err_bnd)
    return rel | bnd


def _pair_is_near_tie(q, kx, ky, sx, sy):
    """Block y (left out, score sy) beats block x (kept, score sx) by a gap
    that the near-tie rules accept."""
    gap = sy - sx
    if gap <= 0:
        return True
    den = max(abs(sx), abs(sy))
    if den > 0 and gap / den < REL_TIE:
        return True
    d = q.shape[0]
    gamma = d * U32 / (1 - d * U32)
    bound = gamma * (np.sum(np.abs(q * kx)) + np.sum(np.abs(q * ky)))
    return gap <= bound


def selection_report(dev_sel, orc_sel, gap_rel, gap_abs, err_bnd, idx_q, kmax, q_pos,
                     block, window=1):
    """Assert the acceptance rule on every row; return the counts:
    rows, flagged by the relative rule, flagged only by the error-bound rule,
    rows where device and oracle differ (all of them flagged)."""
    dev_sel = np.asarray(dev_sel)
    orc_sel = np.asarray(orc_sel)
    assert dev_sel.shape == orc_sel.shape
    rel, bnd = flag_rules(gap_rel, gap_abs, err_bnd)
    flag = rel | bnd
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
        q = idx_q[r].astype(np.float64)
        s = kmax[:first].astype(np.float64) @ q
        kept = row[:n_cand].tolist()
        left = sorted(set(range(first)) - set(kept))
        if kept and left:
            x = min(kept, key=lambda b: (s[b], -b))      # lowest-ranked kept block
            y = max(left, key=lambda b: (s[b], -b))      # highest-ranked left-out block
            assert _pair_is_near_tie(q, kmax[x].astype(np.float64),
                                     kmax[y].astype(np.float64), s[x], s[y]), (
                f"row {r}: device keeps block {x} (score {s[x]}) over block {y} "
                f"(score {s[y]}), not a near-tie")
    return {"rows": int(dev_sel.shape[0]), "flag_rel": int(rel.sum()),
            "flag_bound_only": int((bnd & ~rel).sum()), "differing": int(diff.sum())}


def check_selection(dev_sel, orc_sel, gap_rel, gap_abs, err_bnd, idx_q, kmax,
                    q_pos, block, window=1):
    """Assert the acceptance rule; return (n_flagged, n_mismatch).  With a
    local window the forced blocks are own-window+1 .. own and only the
    blocks below them are ranked."""
    r = selection_report(dev_sel, orc_sel, gap_rel, gap_abs, err_bnd, idx_q, kmax, q_pos,
                         block, window)
    return r["flag_rel"] + r["flag_bound_only"], r["differing"]


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))
