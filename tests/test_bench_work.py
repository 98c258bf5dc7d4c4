"""Pins for the benchmark's work counters (no GPU): the attended (query, key)
count that prices the sparse-GQA roofline equals the count of an actual
selection made by the oracle, and the decode byte count of the batched decode
workload adds up from its parts."""
import numpy as np

import bench
from block_sparse_attention_index_amd import synth


def test_attended_pairs_match_a_real_selection(orc):
    cfg = synth.CONFIGS["tiny"]
    x = synth.sequence_inputs(cfg, "cpu", 0)
    kmax = orc.pool(x["idx_k"].numpy(), cfg.block)
    for q0, n_q in [(0, cfg.T), (1000, 1500), (cfg.T - 70, 70)]:
        pos = np.arange(q0, q0 + n_q, dtype=np.int64)
        sel, *_ = orc.select(x["idx_q"].numpy()[q0:q0 + n_q], pos, kmax, cfg.block, cfg.topk)
        _, att = orc.counts(sel, pos, cfg.block)
        assert bench.attended_pairs(q0, n_q, cfg.block, cfg.topk) == att


def test_decode_bytes_of_the_batched_workload():
    cfg = synth.CONFIGS["dec16"]
    L = cfg.T
    keys = cfg.topk * cfg.block                      # every selected block is full
    kv = keys * cfg.Hkv * cfg.d * 2 * 2              # bf16 K and V
    summaries = (L // cfg.block) * cfg.d_idx * 4
    q = cfg.Hq * cfg.d * 2 + cfg.d_idx * 4
    out = cfg.Hq * (cfg.d + 1) * 4
    assert bench.decode_bytes(L, cfg) == kv + summaries + q + out
    assert cfg.n_seq * bench.decode_bytes(L, cfg) == 273428480   # 260.76 MiB per step
