"""Device parity at the full workload sizes (needs a GPU).

The whole device pipeline runs as the benchmark runs it (same entry points,
same query-chunking and workspaces), on the seeded synthetic inputs of each
workload; the oracle then checks it:

* the index summaries, bit for bit, over the whole table;
* every query's selection: bit-exact except flagged near-ties, which are
  counted per rule (relative gap, error bound) and printed with the number of
  rows where device and oracle differ;
* the CSR of every query chunk the prefill built, bit for bit;
* outputs, recomputed by the oracle from the device's own selection (so a
  near-tie cannot blur them), within the bf16 tolerance: every query at
  32K tokens, a stratified sample of at least 8192 queries at 128K and 1M
  tokens (first and last blocks, both sides of each query-chunk boundary,
  queries that chose a planted hot block, random queries);
* the 1M-token decode loop exactly as the benchmark captures and replays it
  (256 fused steps appending tokens 2^20 .. 2^20+255), every step.
"""
import time

import numpy as np
import pytest
import torch

from block_sparse_attention_index_amd import ops, pipeline, synth
from helpers import TOL_BF16, max_abs, selection_report

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


def _say(msg):
    print(msg, flush=True)


def _stratified(T, B, chunk, sel_h, hot, n, seed):
    """At least n query rows: the first and last block, 64 rows on each side
    of every query-chunk boundary, up to n/4 rows that chose a hot block, and
    random rows up to n."""
    rng = np.random.default_rng(seed)
    parts = [np.arange(min(T, B)), np.arange(max(0, T - B), T)]
    for c0 in range(chunk, T, chunk):
        parts.append(np.arange(max(0, c0 - 64), min(T, c0 + 64)))
    if hot is not None and len(hot):
        chose_hot = np.nonzero(np.isin(sel_h, hot).any(axis=1))[0]
        if chose_hot.size:
            parts.append(rng.choice(chose_hot, size=min(n // 4, chose_hot.size), replace=False))
    rows = np.unique(np.concatenate(parts))
    need = n - rows.size
    if need > 0:
        rest = np.setdiff1d(np.arange(T), rows)
        rows = np.unique(np.concatenate([rows, rng.choice(rest, size=min(need, rest.size),
                                                          replace=False)]))
    return rows.astype(np.int64)


def _attend_rows(orc, cfg, q_dev, k_h, v_h, rows, pos, sel, batch=2048):
    """Oracle outputs for the given query rows (device tensor q, host k/v)."""
    outs, lses = [], []
    for i in range(0, len(rows), batch):
        r = rows[i:i + batch]
        q = synth.host(q_dev[torch.from_numpy(r).to(q_dev.device)])
        oo, lo, _ = orc.attend(q, k_h, v_h, np.arange(len(r)), pos[i:i + batch],
                               sel[i:i + batch], cfg.block, cfg.scale, orc.BF16)
        outs.append(oo)
        lses.append(lo)
    return np.concatenate(outs), np.concatenate(lses)


def _prefill_full(orc, name, n_attn=None, seed=0):
    cfg = synth.CONFIGS[name]
    T, B, K = cfg.T, cfg.block, cfg.topk
    t0 = time.perf_counter()
    x = synth.sequence_inputs(cfg, DEV, seed, length=T)
    torch.cuda.synchronize()
    _say(f"{name}: inputs generated in {time.perf_counter() - t0:.1f} s")
    t0 = time.perf_counter()
    bufs = pipeline.alloc_prefill(x["q"], x["idx_q"], B, K)
    o, lse, sel = pipeline.prefill(x["q"], x["k"], x["v"], x["idx_q"], x["idx_k"],
                                   B, K, cfg.scale, bufs=bufs)
    torch.cuda.synchronize()
    _say(f"{name}: device prefill in {time.perf_counter() - t0:.2f} s "
         f"(query chunk {bufs.chunk})")

    # index summaries: the whole table, bit for bit
    idx_k = _np(x["idx_k"])
    kmax_o = orc.pool(idx_k, B)
    assert np.array_equal(_np(bufs.kmax).view(np.uint32), kmax_o.view(np.uint32))
    del idx_k

    # every query's selection
    t0 = time.perf_counter()
    sel_h = _np(sel)
    idx_q = _np(x["idx_q"])
    pos = np.arange(T, dtype=np.int64)
    so, gr, ga, eb = orc.select(idx_q, pos, kmax_o, B, K)
    rep = selection_report(sel_h, so, gr, ga, eb, idx_q, kmax_o, pos, B)
    _say(f"{name}: selection of all {T} queries in {time.perf_counter() - t0:.1f} s: "
         f"near-ties flagged {rep['flag_rel']} (relative rule) + {rep['flag_bound_only']} "
         f"(error-bound rule only), differing rows {rep['differing']}")
    del so, gr, ga, eb

    # the CSR of each query chunk, as the prefill built it, bit for bit
    for c0 in range(0, T, bufs.chunk):
        c1 = min(T, c0 + bufs.chunk)
        nbc = -(-c1 // B)
        rp_d, ql_d, sl_d = ops.msa_invert_selection(sel[c0:c1], nbc)
        rp_o, ql_o, sl_o = orc.invert(sel_h[c0:c1], nbc)
        assert np.array_equal(_np(rp_d), rp_o)
        assert np.array_equal(_np(ql_d)[:rp_o[-1]], ql_o)
        assert np.array_equal(_np(sl_d), sl_o)
    _say(f"{name}: CSR of {-(-T // bufs.chunk)} query chunk(s) bit-exact")

    # outputs from the device's own selection
    t0 = time.perf_counter()
    hot = _np(x["hot"]) if cfg.n_hot else None
    rows = (np.arange(T, dtype=np.int64) if n_attn is None
            else _stratified(T, B, bufs.chunk, sel_h, hot, n_attn, seed))
    k_h, v_h = synth.host(x["k"]), synth.host(x["v"])
    oo, lo = _attend_rows(orc, cfg, x["q"], k_h, v_h, rows, rows, sel_h[rows])
    ridx = torch.from_numpy(rows).to(DEV)
    eo = max_abs(_np(o[ridx]), oo)
    el = max_abs(_np(lse[ridx]), lo)
    _say(f"{name}: outputs of {len(rows)} queries in {time.perf_counter() - t0:.1f} s: "
         f"max|do| {eo:.3g} max|dlse| {el:.3g}")
    assert eo <= TOL_BF16 and el <= TOL_BF16
    del x, o, lse, sel, bufs
    torch.cuda.empty_cache()


def test_full_p32k(orc):
    _prefill_full(orc, "p32k")


def test_full_p128k(orc):
    _prefill_full(orc, "p128k", n_attn=8192)


def test_full_p1m_prefill(orc):
    _prefill_full(orc, "p1m", n_attn=8192)


def test_full_p1m_decode_loop(orc):
    """The benchmark's 1M-token decode: 256 fused steps, each appending token
    2^20 + s (K/V rows, index key), updating block 2048's running max, and
    selecting and attending for that token's query -- captured in one graph
    as the benchmark captures it, except that step s writes its outputs to
    slot s so that every step can be checked.  The cache rows the steps append
    start zeroed, so the appends themselves are checked too; a second replay
    (the rows now present, as in the benchmark's repeated replays) must give
    the same outputs bit for bit."""
    cfg = synth.CONFIGS["p1m"]
    T, B, K, n_dec = cfg.T, cfg.block, cfg.topk, cfg.n_dec
    L_total = T + n_dec
    t0 = time.perf_counter()
    x = synth.sequence_inputs(cfg, DEV, 0, length=L_total)
    torch.cuda.synchronize()
    _say(f"p1m decode: inputs generated in {time.perf_counter() - t0:.1f} s")
    nb_max = -(-L_total // B)
    kmax = torch.zeros((1, nb_max, cfg.d_idx), dtype=torch.float32, device=DEV)
    ops.msa_index_pool(x["idx_k"][:T], B, kmax=kmax[0, :T // B])
    k_new = x["k"][:, T:L_total].permute(1, 0, 2).contiguous()      # [n_dec, Hkv, d]
    v_new = x["v"][:, T:L_total].permute(1, 0, 2).contiguous()
    ik_new = x["idx_k"][T:L_total].contiguous()
    k_cache, v_cache, ik_cache = x["k"].clone()[None], x["v"].clone()[None], x["idx_k"].clone()[None]
    k_cache[:, :, T:] = 0
    v_cache[:, :, T:] = 0
    ik_cache[:, T:] = 0
    seq_lens = torch.arange(T, L_total, dtype=torch.int64, device=DEV)
    dbufs = pipeline.alloc_decode_step(x["q"][:1], kmax, B, K)
    o_all = torch.empty((n_dec, 1, cfg.Hq, cfg.d), dtype=torch.float32, device=DEV)
    lse_all = torch.empty((n_dec, 1, cfg.Hq), dtype=torch.float32, device=DEV)
    sel_all = torch.empty((n_dec, 1, K), dtype=torch.int32, device=DEV)

    def decode_loop():
        for s in range(n_dec):
            dbufs.o, dbufs.lse, dbufs.sel = o_all[s], lse_all[s], sel_all[s]
            pipeline.decode_append_step(
                x["q"][T + s:T + s + 1], k_new[s:s + 1], v_new[s:s + 1],
                x["idx_q"][T + s:T + s + 1], ik_new[s:s + 1], k_cache, v_cache, kmax,
                seq_lens[s:s + 1], B, K, cfg.scale, idx_k_cache=ik_cache, bufs=dbufs)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_loop()
    graph.replay()
    torch.cuda.synchronize()
    o1, l1, s1 = _np(o_all)[:, 0], _np(lse_all)[:, 0], _np(sel_all)[:, 0]
    _say("p1m decode: 256 captured steps replayed")

    # the appends, bit for bit
    assert torch.equal(k_cache[0, :, T:], x["k"][:, T:])
    assert torch.equal(v_cache[0, :, T:], x["v"][:, T:])
    assert torch.equal(ik_cache[0, T:], x["idx_k"][T:])
    # the summaries: blocks 0..2047 from the prefix, block 2048 the running
    # max of the 256 appended keys -- a fresh pool of all 2^20 + 256 keys
    kmax_o = orc.pool(_np(x["idx_k"]), B)
    assert np.array_equal(_np(kmax)[0].view(np.uint32), kmax_o.view(np.uint32))
    # every step's selection (its own block 2048 is forced and never scored,
    # so all steps rank the same final summaries of blocks 0..2047)
    pos = np.arange(T, L_total, dtype=np.int64)
    idx_q = _np(x["idx_q"][T:L_total])
    so, gr, ga, eb = orc.select(idx_q, pos, kmax_o, B, K)
    rep = selection_report(s1, so, gr, ga, eb, idx_q, kmax_o, pos, B)
    _say(f"p1m decode: selections of {n_dec} steps: near-ties flagged {rep['flag_rel']} "
         f"(relative) + {rep['flag_bound_only']} (error bound only), differing {rep['differing']}")
    # every step's output, from its own selection
    t0 = time.perf_counter()
    oo, lo = _attend_rows(orc, cfg, x["q"], synth.host(x["k"]), synth.host(x["v"]), pos, pos, s1)
    eo, el = max_abs(o1, oo), max_abs(l1, lo)
    _say(f"p1m decode: outputs of {n_dec} steps in {time.perf_counter() - t0:.1f} s: "
         f"max|do| {eo:.3g} max|dlse| {el:.3g}")
    assert eo <= TOL_BF16 and el <= TOL_BF16
    # the benchmark replays the same graph again: identical outputs
    graph.replay()
    torch.cuda.synchronize()
    assert np.array_equal(_np(sel_all)[:, 0], s1)
    assert np.array_equal(_np(o_all)[:, 0], o1) and np.array_equal(_np(lse_all)[:, 0], l1)
    _say("p1m decode: second replay identical")
    del x, k_cache, v_cache, ik_cache, graph
    torch.cuda.empty_cache()


def test_full_dec16(orc):
    """The batched decode step at 16 x 262144 tokens: the separate calls and
    the fused step (as the benchmark times it: the last token appended again
    at its own position) against the oracle, every sequence."""
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
    # the fused step as it is timed
    L = cfg.T - 1
    before = x["seq_len"] - 1
    kmax_f = ops.msa_index_pool(x["idx_k"], B, seq_len=x["seq_len"], nb_max=cfg.nb)
    fb = pipeline.alloc_decode_step(x["q"], kmax_f, B, K)
    o_f, lse_f, sel_f = pipeline.decode_append_step(
        x["q"], x["k_cache"][:, :, L].contiguous(), x["v_cache"][:, :, L].contiguous(),
        x["idx_q"], x["idx_k"][:, L].contiguous(), x["k_cache"], x["v_cache"], kmax_f, before,
        B, K, cfg.scale, idx_k_cache=x["idx_k"], bufs=fb)
    torch.cuda.synchronize()
    kmax, sel, o, lse = _np(kmax), _np(sel), _np(o), _np(lse)
    sel_f, o_f, lse_f = _np(sel_f), _np(o_f), _np(lse_f)
    assert np.array_equal(_np(kmax_f).view(np.uint32), kmax.view(np.uint32))
    idx_q = _np(x["idx_q"])
    tot = {"flag_rel": 0, "flag_bound_only": 0, "differing": 0}
    worst = [0.0, 0.0, 0.0, 0.0]
    pos = np.array([cfg.T - 1], np.int64)
    for s in range(n):
        kmo = orc.pool(_np(x["idx_k"][s]), B)
        assert np.array_equal(kmax[s].view(np.uint32), kmo.view(np.uint32))
        so, gr, ga, eb = orc.select(idx_q[s:s + 1], pos, kmo, B, K)
        for dev_sel in (sel, sel_f):
            rep = selection_report(dev_sel[s:s + 1], so, gr, ga, eb, idx_q[s:s + 1], kmo,
                                   pos, B)
        for k_ in tot:
            tot[k_] += rep[k_]
        k_h, v_h = synth.host(x["k_cache"][s]), synth.host(x["v_cache"][s])
        q_h = synth.host(x["q"][s:s + 1])
        for i, (ds, do_, dl) in enumerate(((sel, o, lse), (sel_f, o_f, lse_f))):
            oo, lo, _ = orc.attend(q_h, k_h, v_h, np.array([0]), pos, ds[s:s + 1], B,
                                   cfg.scale, orc.BF16)
            eo, el = max_abs(do_[s], oo[0]), max_abs(dl[s], lo[0])
            worst[2 * i] = max(worst[2 * i], eo)
            worst[2 * i + 1] = max(worst[2 * i + 1], el)
            assert eo <= TOL_BF16 and el <= TOL_BF16, (s, i, eo, el)
    _say(f"dec16: {n} sequences: near-ties flagged {tot['flag_rel']} (relative) + "
         f"{tot['flag_bound_only']} (error bound only), differing {tot['differing']}; "
         f"separate calls max|do| {worst[0]:.3g} max|dlse| {worst[1]:.3g}; "
         f"fused step max|do| {worst[2]:.3g} max|dlse| {worst[3]:.3g}")
    assert np.array_equal(sel_f, sel)
    assert np.array_equal(o_f, o) and np.array_equal(lse_f, lse)
    _say("dec16: fused step matches the separate calls bit for bit")
