"""Pins for the work counters (no GPU): the (query, block) pair count and the
attended (query, key) pair count of an actual selection equal closed forms
that do not depend on which blocks were chosen."""
import os

import numpy as np

from block_sparse_attention_index_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def closed_form(T, B, K, q0=0):
    p = np.arange(q0, T, dtype=np.int64)
    keff = np.minimum(K, p // B + 1)
    return int(keff.sum()), int(((keff - 1) * B + p % B + 1).sum())


def test_counts_of_a_real_selection(orc):
    cfg = synth.CONFIGS["tiny"]
    x = synth.sequence_inputs(cfg, "cpu", 0)
    kmax = orc.pool(x["idx_k"].numpy(), cfg.block)
    pos = np.arange(cfg.T, dtype=np.int64)
    sel, *_ = orc.select(x["idx_q"].numpy(), pos, kmax, cfg.block, cfg.topk)
    nnz, att = orc.counts(sel, pos, cfg.block)
    assert (nnz, att) == closed_form(cfg.T, cfg.block, cfg.topk)


def test_golden_work_counts():
    with open(os.path.join(GOLDEN, "work_counts.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 4
    for name, T, B, K, nnz, att in rows:
        cfg = synth.CONFIGS[name]
        assert (cfg.T, cfg.block, cfg.topk) == (int(T), int(B), int(K))
        assert closed_form(int(T), int(B), int(K)) == (int(nnz), int(att))
