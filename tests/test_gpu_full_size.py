"""Device parity at the full workload sizes (needs a GPU).

The whole device pipeline runs as the benchmark runs it (same entry points,
same query-chunking and workspaces), on the seeded synthetic inputs of each
workload; the oracle then recomputes sampled outputs one query at a time.
Acceptance: index summaries and CSR bit-exact; selections bit-exact except
flagged near-ties (which are counted and printed); outputs -- recomputed by
the oracle from the device's own selection, so ties cannot blur them --
within the bf16 tolerance.
"""
import time

import numpy as np
import pytest
import torch

from block_sparse_attention_index_amd import ops, pipeline, synth
from helpers import TOL_BF16, check_selection, max_abs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


def _say(msg):
    print(msg, flush=True)


def _rows(T, B, n, seed):
    """Sampled query rows: the first and last block and n random others."""
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([
        np.arange(min(T, B)), np.arange(max(0, T - B), T),
        rng.choice(T, size=min(T, n), replace=False)])).astype(np.int64)


def _attend_rows(orc, cfg, x, rows, pos, sel):
    q = synth.host(x["q"][torch.from_numpy(rows).to(x["q"].device)])
    return orc.attend(q, synth.host(x["k"]), synth.host(x["v"]),
                      np.arange(len(rows)), pos, sel, cfg.block, cfg.scale,
                      orc.BF16)


def _prefill_full(orc, name, n_sample, decode_steps=0, seed=0):
    cfg = synth.CONFIGS[name]
    T, B, K = cfg.T, cfg.block, cfg.topk
    t0 = time.perf_counter()
    x = synth.sequence_inputs(cfg, DEV, seed, length=T + decode_steps)
    torch.cuda.synchronize()
    _say(f"{name}: inputs generated in {time.perf_counter() - t0:.1f} s")
    t0 = time.perf_counter()
    bufs = pipeline.alloc_prefill(x["q"][:T], x["idx_q"][:T], B, K)
    o, lse, sel = pipeline.prefill(x["q"][:T], x["k"], x["v"], x["idx_q"][:T], x["idx_k"],
                                   B, K, cfg.scale, bufs=bufs)
    torch.cuda.synchronize()
    _say(f"{name}: device prefill in {time.perf_counter() - t0:.2f} s "
         f"(query chunk {bufs.chunk})")

    # index summaries: the whole table, bit for bit
    idx_k = _np(x["idx_k"])
    kmax_o = orc.pool(idx_k[:T], B)
    assert np.array_equal(_np(bufs.kmax), kmax_o)

    # CSR of the device's full selection, bit for bit
    sel_h = _np(sel)
    nb = -(-T // B)
    rp_d, ql_d, sl_d = ops.msa_invert_selection(sel, nb)
    rp_o, ql_o, sl_o = orc.invert(sel_h, nb)
    assert np.array_equal(_np(rp_d), rp_o)
    assert np.array_equal(_np(ql_d)[:rp_o[-1]], ql_o)
    assert np.array_equal(_np(sl_d), sl_o)

    # selections and outputs on sampled rows
    rows = _rows(T, B, n_sample, seed)
    idx_q = _np(x["idx_q"])
    so, gr, ga, eb = orc.select(idx_q[rows], rows, kmax_o, B, K)
    nf, nm = check_selection(sel_h[rows], so, gr, ga, eb, idx_q[rows], kmax_o, rows, B)
    oo, lo, _ = _attend_rows(orc, cfg, x, rows, rows, sel_h[rows])
    eo = max_abs(_np(o[torch.from_numpy(rows).to(DEV)]), oo)
    el = max_abs(_np(lse[torch.from_numpy(rows).to(DEV)]), lo)
    _say(f"{name}: {len(rows)} rows, near-ties flagged {nf}, differing {nm}; "
         f"max|do| {eo:.3g} max|dlse| {el:.3g}")
    assert eo <= TOL_BF16 and el <= TOL_BF16

    # decode steps against the prefilled cache (append-mode pooling)
    if decode_steps:
        kmax_d = torch.zeros((1, -(-(T + decode_steps) // B), cfg.d_idx),
                             dtype=torch.float32, device=DEV)
        kmax_d[0, :nb] = bufs.kmax
        dbufs = pipeline.alloc_decode(x["q"][:1], kmax_d, B, K)
        for s in range(decode_steps):
            L = T + s + 1
            seq_len = torch.tensor([L], dtype=torch.int64, device=DEV)
            od, ld, seld = pipeline.decode_step(
                x["q"][L - 1:L], x["idx_q"][L - 1:L], x["k"][None], x["v"][None],
                x["idx_k"][None], kmax_d, seq_len, B, K, cfg.scale, bufs=dbufs)
            kmo = orc.pool(idx_k[:L], B)
            nbl = -(-L // B)
            assert np.array_equal(_np(kmax_d)[0, :nbl], kmo)
            pos = np.array([L - 1], np.int64)
            so, gr, ga, eb = orc.select(idx_q[L - 1:L], pos, kmo, B, K)
            seld = _np(seld)
            check_selection(seld, so, gr, ga, eb, idx_q[L - 1:L], kmo, pos, B)
            oo, lo, _ = _attend_rows(orc, cfg, x, pos, pos, seld)
            eo, el = max_abs(_np(od)[0], oo[0]), max_abs(_np(ld)[0], lo[0])
            _say(f"{name}: decode at position {L - 1}: max|do| {eo:.3g} max|dlse| {el:.3g}")
            assert eo <= TOL_BF16 and el <= TOL_BF16
    del x, o, lse, sel, bufs
    torch.cuda.empty_cache()


def test_full_p32k(orc):
    _prefill_full(orc, "p32k", n_sample=512)


def test_full_p128k(orc):
    _prefill_full(orc, "p128k", n_sample=384)


def test_full_p1m_prefill_and_decode(orc):
    _prefill_full(orc, "p1m", n_sample=192, decode_steps=2)


def test_full_dec16(orc):
    cfg = synth.CONFIGS["dec16"]
    B, K, n = cfg.block, cfg.topk, cfg.n_seq
    t0 = time.perf_counter()
    x = synth.decode_inputs(cfg, DEV, 0)
    torch.cuda.synchronize()
    _say(f"dec16: inputs generated in {time.perf_counter() - t0:.1f} s")
    kmax = ops.msa_index_pool(x["idx_k"], B, seq_len=x["seq_len"], nb_max=cfg.nb)
    bufs = pipeline.alloc_decode(x["q"], kmax, B, K)
    sel = ops.msa_index_topk_decode(x["idx_q"], x["seq_len"], kmax, B, K,
                                    sel=bufs.sel, ws=bufs.topk_ws)
    o, lse = ops.msa_sparse_gqa_decode(x["q"], x["k_cache"], x["v_cache"], x["seq_len"],
                                       sel, B, cfg.scale, o=bufs.o, lse=bufs.lse,
                                       ws=bufs.attn_ws)
    torch.cuda.synchronize()
    kmax, sel, o, lse = _np(kmax), _np(sel), _np(o), _np(lse)
    idx_q = _np(x["idx_q"])
    nf_all = 0
    worst = (0.0, 0.0)
    for s in range(n):
        L = cfg.T
        kmo = orc.pool(_np(x["idx_k"][s]), B)
        assert np.array_equal(kmax[s], kmo)
        pos = np.array([L - 1], np.int64)
        so, gr, ga, eb = orc.select(idx_q[s:s + 1], pos, kmo, B, K)
        nf, _ = check_selection(sel[s:s + 1], so, gr, ga, eb, idx_q[s:s + 1], kmo, pos, B)
        nf_all += nf
        oo, lo, _ = orc.attend(synth.host(x["q"][s:s + 1]), synth.host(x["k_cache"][s]),
                               synth.host(x["v_cache"][s]), np.array([0]), pos,
                               sel[s:s + 1], B, cfg.scale, orc.BF16)
        eo, el = max_abs(o[s], oo[0]), max_abs(lse[s], lo[0])
        worst = (max(worst[0], eo), max(worst[1], el))
        assert eo <= TOL_BF16 and el <= TOL_BF16, (s, eo, el)
    _say(f"dec16: {n} sequences, near-ties flagged {nf_all}; "
         f"max|do| {worst[0]:.3g} max|dlse| {worst[1]:.3g}")
    # the fused step as it is timed: the last token appended again in place
    # (idempotent) gives the same selection and output bit for bit
    L = cfg.T - 1
    before = x["seq_len"] - 1
    kmax_f = ops.msa_index_pool(x["idx_k"], B, seq_len=x["seq_len"], nb_max=cfg.nb)
    fb = pipeline.alloc_decode_step(x["q"], kmax_f, B, K)
    o_f, lse_f, sel_f = pipeline.decode_append_step(
        x["q"], x["k_cache"][:, :, L].contiguous(), x["v_cache"][:, :, L].contiguous(),
        x["idx_q"], x["idx_k"][:, L].contiguous(), x["k_cache"], x["v_cache"], kmax_f, before,
        B, K, cfg.scale, idx_k_cache=x["idx_k"], bufs=fb)
    torch.cuda.synchronize()
    assert np.array_equal(_np(sel_f), sel)
    assert np.array_equal(_np(o_f), o) and np.array_equal(_np(lse_f), lse)
    _say("dec16: fused step matches the separate calls bit for bit")
