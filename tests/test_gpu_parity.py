"""Device parity: every entry point against the CPU oracle (needs a GPU).

Each stage is fed oracle-produced inputs (pooled summaries, selections, CSR)
so the device kernels are compared one by one; the end-to-end test then runs
the whole device pipeline and compares what is unique.  Acceptance:
pool and CSR bit-exact; selections bit-exact except flagged near-ties;
outputs within 1e-4 (fp32 inputs) or 1e-2 (bf16 inputs) max-abs.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_index_amd import ops, pipeline, synth
from helpers import TOL_BF16, TOL_F32, check_selection, max_abs, selection_report

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


def _say(msg):
    print(msg, flush=True)


# --------------------------------------------------------------------------
# pool
# --------------------------------------------------------------------------
@pytest.mark.parametrize("L,B,d", [(4096, 64, 64), (1000, 16, 128), (777, 128, 24),
                                   (1, 16, 4), (5000, 512, 128), (300, 32, 1024)])
def test_pool_bit_exact(orc, L, B, d):
    _say(f"pool L={L} B={B} d={d}")
    g = torch.Generator().manual_seed(L * 7 + B + d)
    x = torch.randn(L, d, generator=g)
    x[::5, 0] = -0.0
    x[1::5, 0] = 0.0
    kmax = ops.msa_index_pool(x.to(DEV), B)
    want = orc.pool(x.numpy(), B)
    assert np.array_equal(_np(kmax).view(np.uint32), want.view(np.uint32))


def test_pool_batched_ragged_and_last_block(orc):
    n, Lmax, B, d = 3, 1000, 64, 128
    g = torch.Generator().manual_seed(3)
    x = torch.randn(n, Lmax, d, generator=g)
    lens = [1000, 513, 64]
    nb_max = 17
    kmax = torch.full((n, nb_max, d), float("nan"), device=DEV)
    seq_len = torch.tensor(lens, dtype=torch.int64, device=DEV)
    ops.msa_index_pool(x.to(DEV), B, kmax=kmax, seq_len=seq_len, nb_max=nb_max)
    got = _np(kmax)
    for s, L in enumerate(lens):
        nb = -(-L // B)
        assert np.array_equal(got[s, :nb], orc.pool(x[s, :L].numpy(), B))
        assert np.all(np.isnan(got[s, nb:])), "blocks past the sequence stay untouched"
    # decode append: raise the newest token, re-pool only each last block
    x2 = x.clone()
    for s, L in enumerate(lens):
        x2[s, L - 1] += 3.0
    ops.msa_index_pool(x2.to(DEV), B, kmax=kmax, seq_len=seq_len, blk_begin=-1,
                       nb_max=nb_max)
    got = _np(kmax)
    for s, L in enumerate(lens):
        nb = -(-L // B)
        assert np.array_equal(got[s, :nb], orc.pool(x2[s, :L].numpy(), B))


def test_pool_append_mode_equals_full_pool(orc):
    # folding tokens one at a time into a running block max reproduces the
    # full pool (bit-exact), across block boundaries and for several sequences
    n, Lmax, B, d = 2, 700, 64, 128
    g = torch.Generator().manual_seed(4)
    x = torch.randn(n, Lmax, d, generator=g)
    x[:, ::7, 3] = -0.0
    start = [600, 250]
    nb_max = -(-Lmax // B)
    xd = x.to(DEV)
    kmax = torch.full((n, nb_max, d), float("nan"), device=DEV)
    ops.msa_index_pool(xd, B, kmax=kmax, nb_max=nb_max,
                       seq_len=torch.tensor(start, dtype=torch.int64, device=DEV))
    for step in range(1, 80):
        lens = torch.tensor([L + step for L in start], dtype=torch.int64, device=DEV)
        ops.msa_index_pool(xd, B, kmax=kmax, seq_len=lens, blk_begin=-2, nb_max=nb_max)
    got = _np(kmax)
    for s_, L in enumerate(start):
        Lf = L + 79
        nbf = -(-Lf // B)
        assert np.array_equal(got[s_, :nbf].view(np.uint32),
                              orc.pool(x[s_, :Lf].numpy(), B).view(np.uint32))


# --------------------------------------------------------------------------
# top-K (prefill)
# --------------------------------------------------------------------------
def _topk_case(orc, idx_q, idx_k, B, K, q_pos0=0):
    kmax = orc.pool(idx_k, B)
    n_q = idx_q.shape[0]
    pos = np.arange(q_pos0, q_pos0 + n_q, dtype=np.int64)
    sel_o, gr, ga, eb = orc.select(idx_q, pos, kmax, B, K)
    sel_d = ops.msa_index_topk(torch.from_numpy(idx_q).to(DEV),
                               torch.from_numpy(kmax).to(DEV), B, K, q_pos0=q_pos0)
    nf, nm = check_selection(_np(sel_d), sel_o, gr, ga, eb, idx_q, kmax, pos, B)
    _say(f"  near-ties flagged {nf}, device/oracle differing rows {nm}")
    return nf, nm


def test_topk_tiny_config(orc):
    cfg = synth.CONFIGS["tiny"]
    _say("topk tiny")
    x = synth.sequence_inputs(cfg, "cpu", 0)
    _topk_case(orc, x["idx_q"].numpy(), x["idx_k"].numpy(), cfg.block, cfg.topk)


@pytest.mark.parametrize("T,B,K,d,q0,hot", [
    (4096, 64, 16, 128, 0, 8),      # the 32K-token config's shape, scaled down
    (3000, 16, 1, 32, 0, 0),        # K = 1: own block only
    (2500, 32, 64, 24, 100, 0),     # K = 64 (max), d_idx not a multiple of 64
    (5000, 128, 16, 128, 1234, 6),  # chunk not aligned to anything
    (3000, 32, 8, 200, 0, 4),       # d_idx above one staged row: 64-column slices
    (2000, 32, 6, 130, 50, 3),      # sliced, d_idx not a multiple of 4 (scalar staging)
    (2000, 32, 5, 77, 0, 3),        # whole row staged, odd d_idx (zero-padded K step)
    (2500, 16, 20, 256, 0, 4),      # list longer than 16, sliced rows
])
def test_topk_shapes(orc, T, B, K, d, q0, hot):
    _say(f"topk T={T} B={B} K={K} d={d} q0={q0}")
    cfg = synth.Config("t", T, "f32", 1, 1, 64, d, B, K, hot)
    x = synth.sequence_inputs(cfg, "cpu", 1)
    _topk_case(orc, x["idx_q"].numpy()[q0:], x["idx_k"].numpy(), B, K, q_pos0=q0)


def test_topk_misaligned_rows(orc):
    """Row pointers that are not 16-byte aligned take the 4-byte staging path."""
    cfg = synth.Config("t", 3000, "f32", 1, 1, 64, 128, 64, 8, 4)
    x = synth.sequence_inputs(cfg, "cpu", 2)
    idx_q, idx_k = x["idx_q"].numpy(), x["idx_k"].numpy()
    B, K = cfg.block, cfg.topk
    kmax = orc.pool(idx_k, B)
    pos = np.arange(idx_q.shape[0], dtype=np.int64)
    sel_o, gr, ga, eb = orc.select(idx_q, pos, kmax, B, K)
    qbuf = torch.zeros(idx_q.size + 1, device=DEV)
    qbuf[1:] = torch.from_numpy(idx_q.ravel()).to(DEV)
    kbuf = torch.zeros(kmax.size + 1, device=DEV)
    kbuf[1:] = torch.from_numpy(kmax.ravel()).to(DEV)
    q_view, k_view = qbuf[1:].view(idx_q.shape), kbuf[1:].view(kmax.shape)
    assert q_view.data_ptr() % 16 != 0 and k_view.data_ptr() % 16 != 0
    sel_d = ops.msa_index_topk(q_view, k_view, B, K)
    check_selection(_np(sel_d), sel_o, gr, ga, eb, idx_q, kmax, pos, B)


def test_topk_ties_go_low(orc):
    # every summary identical: all scores tie exactly -> blocks 0..K-2
    B, K, nb, d = 64, 5, 40, 16
    kmax = np.tile(np.random.default_rng(0).standard_normal((1, d)).astype(np.float32),
                   (nb, 1))
    idx_q = np.random.default_rng(1).standard_normal((nb * B, d)).astype(np.float32)
    sel = _np(ops.msa_index_topk(torch.from_numpy(idx_q).to(DEV),
                                 torch.from_numpy(kmax).to(DEV), B, K))
    for p in range(nb * B):
        own = p // B
        m = min(K - 1, own)
        assert sel[p].tolist() == list(range(m)) + [own] + [-1] * (K - m - 1)


@pytest.mark.parametrize("lens,B,K,d", [
    ([9000, 4100, 700], 64, 16, 128),   # three chunk lists, the last sequences shorter
    ([5000, 2600], 32, 64, 77),         # K = 64 (max), odd d_idx (scalar scan)
    ([3000], 16, 1, 32),                # K = 1: own block only
    ([3000, 2000], 32, 8, 300),         # d_idx over two staged column slabs
])
@pytest.mark.parametrize("shuffle", [True, False])
def test_topk_batch(orc, lens, B, K, d, shuffle):
    """Queries of several sequences at scattered positions, each row against
    its own sequence's summaries; out-of-range sequence ids and positions get
    rows of -1, in a shuffled batch and in one ordered by sequence."""
    _say(f"topk batch lens={lens} B={B} K={K} d={d} shuffle={shuffle}")
    n_seq = len(lens)
    nb_max = -(-max(lens) // B) + 3          # summaries past every sequence's end
    kmax = np.zeros((n_seq, nb_max, d), np.float32)
    qrows, qs, qp = [], [], []
    rng = np.random.default_rng(7)
    for s_, L in enumerate(lens):
        cfg = synth.Config("t", L, "f32", 1, 1, 64, d, B, K, 4)
        x = synth.sequence_inputs(cfg, "cpu", 10 + s_)
        kmax[s_, :-(-L // B)] = orc.pool(x["idx_k"].numpy(), B)
        pos = np.unique(np.concatenate([[0, B - 1, B, L - 1], rng.integers(0, L, 120)]))
        qrows.append(x["idx_q"].numpy()[pos])
        qs += [s_] * len(pos)
        qp += pos.tolist()
    n_ok = len(qs)
    bad = [(-1, 0), (n_seq, 5), (0, -1), (0, nb_max * B), (n_seq - 1, 1 << 40)]
    qs += [b[0] for b in bad]
    qp += [b[1] for b in bad]
    idx_q = np.concatenate(qrows + [np.ones((len(bad), d), np.float32)])
    perm = rng.permutation(len(qs)) if shuffle else np.arange(len(qs))
    idx_q, qs, qp = idx_q[perm], np.array(qs, np.int32)[perm], np.array(qp, np.int64)[perm]
    ws = torch.empty(ops.load().msa_topk_batch_workspace_bytes(len(qs), nb_max, K),
                     dtype=torch.uint8, device=DEV)
    for rep in range(2):                      # the second call reuses the workspace
        sel_d = _np(ops.msa_index_topk_batch(torch.from_numpy(idx_q).to(DEV),
                                             torch.from_numpy(qs).to(DEV),
                                             torch.from_numpy(qp).to(DEV),
                                             torch.from_numpy(kmax).to(DEV), B, K, ws=ws))
    valid = perm < n_ok
    assert np.all(sel_d[~valid] == -1)
    for s_ in range(n_seq):
        rows = np.nonzero(valid & (qs == s_))[0]
        so, gr, ga, eb = orc.select(idx_q[rows], qp[rows], kmax[s_], B, K)
        check_selection(sel_d[rows], so, gr, ga, eb, idx_q[rows], kmax[s_], qp[rows], B)


# --------------------------------------------------------------------------
# CSR
# --------------------------------------------------------------------------
def _invert_case(orc, sel, nb):
    ro, qo, so = orc.invert(sel, nb)
    rd, qd, sd = ops.msa_invert_selection(torch.from_numpy(sel).to(DEV), nb)
    rd, qd, sd = _np(rd), _np(qd), _np(sd)
    assert np.array_equal(rd, ro)
    assert np.array_equal(qd[:ro[-1]], qo)
    assert np.array_equal(sd, so)


def test_invert_tiny_selection(orc):
    cfg = synth.CONFIGS["tiny"]
    x = synth.sequence_inputs(cfg, "cpu", 0)
    kmax = orc.pool(x["idx_k"].numpy(), cfg.block)
    pos = np.arange(cfg.T, dtype=np.int64)
    sel, *_ = orc.select(x["idx_q"].numpy(), pos, kmax, cfg.block, cfg.topk)
    _invert_case(orc, sel, cfg.nb)


@pytest.mark.parametrize("n_q,nb,K", [(5000, 9000, 6), (1, 1, 1), (2049, 3, 3),
                                      (70000, 300, 16)])
def test_invert_arbitrary_sets(orc, n_q, nb, K):
    _say(f"invert n_q={n_q} nb={nb} K={K}")
    rng = np.random.default_rng(n_q + nb)
    sel = np.full((n_q, K), -1, np.int32)
    for i in range(n_q):
        n = rng.integers(0, min(K, nb) + 1)
        sel[i, :n] = np.sort(rng.choice(nb, size=n, replace=False))
    _invert_case(orc, sel, nb)


# --------------------------------------------------------------------------
# sparse prefill
# --------------------------------------------------------------------------
def _prefill_case(orc, cfg, q_pos0=0, n_q=None, sample=None, seed=0):
    x = synth.sequence_inputs(cfg, "cpu", seed, length=cfg.T)
    T, B, K = cfg.T, cfg.block, cfg.topk
    n_q = T - q_pos0 if n_q is None else n_q
    kmax = orc.pool(x["idx_k"].numpy(), B)
    pos = np.arange(q_pos0, q_pos0 + n_q, dtype=np.int64)
    sel, *_ = orc.select(x["idx_q"].numpy()[q_pos0:q_pos0 + n_q], pos, kmax, B, K)
    nbc = -(-(q_pos0 + n_q) // B)
    row_ptr, q_list, slot = orc.invert(sel, nbc)
    dt = lambda a: torch.from_numpy(a).to(DEV)
    q = x["q"][q_pos0:q_pos0 + n_q].contiguous()
    o, lse = ops.msa_sparse_gqa_prefill(
        q.to(DEV), x["k"].to(DEV), x["v"].to(DEV), dt(sel), dt(row_ptr),
        dt(np.concatenate([q_list, np.zeros(1, np.int32)])), dt(slot), B, cfg.scale,
        q_pos0=q_pos0)
    o, lse = _np(o), _np(lse)
    rows = np.arange(n_q) if sample is None else np.unique(np.concatenate(
        [np.arange(min(n_q, B)), np.arange(max(0, n_q - B), n_q),
         np.random.default_rng(seed).choice(n_q, size=min(n_q, sample), replace=False)]))
    hq = synth.host(q)
    oo, lo, _ = orc.attend(hq, synth.host(x["k"]), synth.host(x["v"]), rows,
                           pos[rows], sel[rows], B, cfg.scale,
                           0 if cfg.dtype == "f32" else 1)
    tol = TOL_F32 if cfg.dtype == "f32" else TOL_BF16
    eo, el = max_abs(o[rows], oo), max_abs(lse[rows], lo)
    _say(f"  prefill {cfg.name}: rows {len(rows)} max|do| {eo:.3g} max|dlse| {el:.3g}")
    assert eo <= tol and el <= tol


def test_prefill_tiny_config_full(orc):
    _say("prefill tiny (all 4096 queries)")
    _prefill_case(orc, synth.CONFIGS["tiny"])


@pytest.mark.parametrize("name,over,q0,nq,sample", [
    ("bf16-p32k-shape", dict(T=4096, n_hot=8), 0, None, 600),
    ("bf16-ragged-chunk", dict(T=3000, n_hot=5, block=128, topk=6), 1000, 1500, 500),
    ("f32-G8-d128", dict(T=2000, dtype="f32", n_hot=3, topk=5, block=64), 0, None, 400),
    ("bf16-B512", dict(T=5000, block=512, topk=4, n_hot=2), 0, None, 300),
    ("bf16-B16-K1", dict(T=700, block=16, topk=1, n_hot=0), 0, None, None),
    ("bf16-G4-B32", dict(T=1500, Hq=16, Hkv=4, block=32, topk=6, n_hot=2), 0, None, 300),
    ("bf16-G16-B48", dict(T=1300, Hq=32, Hkv=2, block=48, topk=5, n_hot=2), 200, 1000, 300),
    ("bf16-G1-B64", dict(T=1200, Hq=4, Hkv=4, block=64, topk=4, n_hot=2), 0, None, None),
    ("bf16-G2-B16", dict(T=900, Hq=8, Hkv=4, block=16, topk=9, n_hot=2), 0, None, None),
    ("bf16-K24-B16", dict(T=1200, block=16, topk=24, n_hot=2), 300, 900, 300),   # merge of > 16 records
])
def test_prefill_shapes(orc, name, over, q0, nq, sample):
    _say(f"prefill {name}")
    cfg = synth.CONFIGS["p32k"].replace(name=name, **over)
    _prefill_case(orc, cfg, q_pos0=q0, n_q=nq, sample=sample)


def test_prefill_small_heads_d64(orc):
    _say("prefill G=2 d=64 bf16")
    cfg = synth.Config("g2", 1500, "bf16", 4, 2, 64, 32, 32, 5, 2)
    _prefill_case(orc, cfg)


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,hq,hkv,d,B,K,lens", [
    ("bf16", 16, 2, 128, 64, 8, [3000, 2049, 100]),     # matrix-core path
    ("bf16", 64, 8, 128, 512, 8, [3000, 1537, 600]),    # the 1M decode shape
    ("bf16", 64, 8, 128, 512, 8, [4700]),               # one sequence: two segments per block
    ("bf16", 32, 2, 128, 128, 5, [2000, 129, 1]),       # G = 16, one-token cache
    ("f32", 8, 2, 64, 64, 4, [1200, 700, 65]),          # VALU path
])
def test_decode_small(orc, dtype, hq, hkv, d, B, K, lens):
    T = max(lens)
    cfg = synth.Config("dec-small", T, dtype, hq, hkv, d, 128, B, K, 4,
                       n_seq=len(lens), mode="decode")
    _say(f"decode {dtype} G={hq // hkv} d={d} B={B} K={K} lens={lens}")
    x = synth.decode_inputs(cfg, "cpu", 0)
    lens = np.array(lens, np.int64)
    B, K = cfg.block, cfg.topk
    nb_max = cfg.nb
    seq_len = torch.from_numpy(lens).to(DEV)
    # pool (bit-exact per sequence)
    kmax_d = torch.full((cfg.n_seq, nb_max, cfg.d_idx), float("nan"), device=DEV)
    ops.msa_index_pool(x["idx_k"].to(DEV), B, kmax=kmax_d, seq_len=seq_len, nb_max=nb_max)
    kmax_o = np.zeros((cfg.n_seq, nb_max, cfg.d_idx), np.float32)
    for s, L in enumerate(lens):
        nb = -(-L // B)
        kmax_o[s, :nb] = orc.pool(x["idx_k"][s, :L].numpy(), B)
        assert np.array_equal(_np(kmax_d)[s, :nb], kmax_o[s, :nb])
    # top-K on the oracle's summaries; a second call on the same workspace
    # agrees with the first
    tws = torch.empty(ops.load().msa_topk_decode_workspace_bytes(cfg.n_seq, nb_max, K),
                      dtype=torch.uint8, device=DEV)
    sel_d = _np(ops.msa_index_topk_decode(x["idx_q"].to(DEV), seq_len,
                                          torch.from_numpy(kmax_o).to(DEV), B, K, ws=tws))
    sel_d2 = _np(ops.msa_index_topk_decode(x["idx_q"].to(DEV), seq_len,
                                           torch.from_numpy(kmax_o).to(DEV), B, K, ws=tws))
    assert np.array_equal(sel_d, sel_d2)
    for s, L in enumerate(lens):
        pos = np.array([L - 1])
        so, gr, ga, eb = orc.select(x["idx_q"][s:s + 1].numpy(), pos, kmax_o[s], B, K)
        check_selection(sel_d[s:s + 1], so, gr, ga, eb, x["idx_q"][s:s + 1].numpy(),
                        kmax_o[s], pos, B)
    # attention on the oracle's selection
    sels = []
    for s, L in enumerate(lens):
        so, *_ = orc.select(x["idx_q"][s:s + 1].numpy(), np.array([L - 1]), kmax_o[s], B, K)
        sels.append(so[0])
    sel_o = np.stack(sels).astype(np.int32)
    aws = torch.empty(ops.load().msa_decode_workspace_bytes(cfg.n_seq, cfg.Hq, cfg.d, B, K),
                      dtype=torch.uint8, device=DEV)
    for rep in range(2):                      # second call reuses the workspace
        o, lse = ops.msa_sparse_gqa_decode(x["q"].to(DEV), x["k_cache"].to(DEV),
                                           x["v_cache"].to(DEV), seq_len,
                                           torch.from_numpy(sel_o).to(DEV), B, cfg.scale,
                                           ws=aws)
    o, lse = _np(o), _np(lse)
    for s, L in enumerate(lens):
        oo, lo, _ = orc.attend(synth.host(x["q"][s:s + 1]), synth.host(x["k_cache"][s]),
                               synth.host(x["v_cache"][s]), np.array([0]),
                               np.array([L - 1]), sel_o[s:s + 1], B, cfg.scale,
                               0 if dtype == "f32" else 1)
        eo, el = max_abs(o[s], oo[0]), max_abs(lse[s], lo[0])
        _say(f"  seq {s} len {L}: max|do| {eo:.3g} max|dlse| {el:.3g}")
        tol = TOL_F32 if dtype == "f32" else TOL_BF16
        assert eo <= tol and el <= tol


# --------------------------------------------------------------------------
# end to end on the device
# --------------------------------------------------------------------------
def test_pipeline_end_to_end_tiny(orc):
    cfg = synth.CONFIGS["tiny"]
    _say("pipeline tiny end to end")
    x = synth.sequence_inputs(cfg, "cpu", 0)
    d = {k: v.to(DEV) for k, v in x.items() if k != "hot"}
    o, lse, sel = pipeline.prefill(d["q"], d["k"], d["v"], d["idx_q"], d["idx_k"],
                                   cfg.block, cfg.topk, cfg.scale)
    kmax = orc.pool(x["idx_k"].numpy(), cfg.block)
    pos = np.arange(cfg.T, dtype=np.int64)
    so, gr, ga, eb = orc.select(x["idx_q"].numpy(), pos, kmax, cfg.block, cfg.topk)
    sel = _np(sel)
    rep = selection_report(sel, so, gr, ga, eb, x["idx_q"].numpy(), kmax, pos, cfg.block)
    # every row's output against the oracle evaluated on the device's own
    # selection (a valid top-K wherever it differs from the oracle's)
    oo, lo, _ = orc.attend(synth.host(x["q"]), synth.host(x["k"]), synth.host(x["v"]),
                           pos, pos, sel, cfg.block, cfg.scale, 0)
    eo = max_abs(_np(o), oo)
    el = max_abs(_np(lse), lo)
    _say(f"  near-ties flagged {rep['flag_rel']} (relative) + {rep['flag_bound_only']} "
         f"(error bound only), differing {rep['differing']}; max|do| {eo:.3g} "
         f"max|dlse| {el:.3g}")
    assert eo <= TOL_F32 and el <= TOL_F32


def test_decode_steps_in_a_captured_graph(orc):
    # A chain of decode steps captured once and replayed must give the eager
    # results on every replay (eager work and synchronisation in between).
    cfg = synth.Config("dec-graph", 1500, "bf16", 16, 2, 128, 128, 64, 6, 3,
                       n_seq=2, mode="decode")
    _say("decode graph replay")
    x = synth.decode_inputs(cfg, "cpu", 3)
    B, K, n_steps = cfg.block, cfg.topk, 5
    nb_max = cfg.nb
    d = {k_: v_.to(DEV) for k_, v_ in x.items()}
    lens0 = [1500 - n_steps, 1000 - n_steps]
    seq_lens = [torch.tensor([a + s_ + 1 for a in lens0], dtype=torch.int64, device=DEV)
                for s_ in range(n_steps)]
    kmax0 = torch.empty((cfg.n_seq, nb_max, cfg.d_idx), device=DEV)
    ops.msa_index_pool(d["idx_k"], B, kmax=kmax0, nb_max=nb_max,
                       seq_len=torch.tensor(lens0, dtype=torch.int64, device=DEV))
    kmax = kmax0.clone()
    bufs = pipeline.alloc_decode(d["q"], kmax, B, K)
    outs = [torch.empty_like(bufs.o) for _ in range(n_steps)]

    def run():
        for s_ in range(n_steps):
            o, _, _ = pipeline.decode_step(d["q"], d["idx_q"], d["k_cache"], d["v_cache"],
                                           d["idx_k"], kmax, seq_lens[s_], B, K, cfg.scale,
                                           bufs=bufs)
            outs[s_].copy_(o)

    run()
    torch.cuda.synchronize()
    eager = [o_.cpu().clone() for o_ in outs]
    kmax.copy_(kmax0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        kmax.copy_(kmax0)                       # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for s_ in range(n_steps):
            assert torch.equal(outs[s_].cpu(), eager[s_]), f"replay {rep} step {s_}"



def test_fused_steps_in_a_captured_graph():
    # A chain of fused steps (each appends its token, so the caches and the
    # running block maxima change) captured once and replayed after restoring
    # the state must give the eager results on every replay, bit for bit.
    hq, hkv, d, di, B, K = 64, 8, 128, 128, 64, 6
    lens, steps = [300, 1000, 63], 4
    n, T = len(lens), max(lens) + steps
    cfg = synth.Config("dec-step-graph", T, "bf16", hq, hkv, d, di, B, K, 3, n_seq=n,
                       mode="decode")
    _say("fused decode step graph replay")
    x = synth.decode_inputs(cfg, "cpu", 5)
    nb_max = -(-T // B)
    kc0, vc0, ik0 = x["k_cache"].to(DEV), x["v_cache"].to(DEV), x["idx_k"].to(DEV)
    seq0 = torch.tensor(lens, dtype=torch.int64, device=DEV)
    kmax0 = torch.full((n, nb_max, di), float("nan"), device=DEV)
    for s, L in enumerate(lens):
        ops.msa_index_pool(ik0[s:s + 1, :L], B, kmax=kmax0[s:s + 1], seq_len=seq0[s:s + 1],
                           nb_max=nb_max)
    q_all = synth._normal_rows((steps, n, hq, d), torch.bfloat16, "cpu", 2, "q").to(DEV)
    iq_all = synth._normal_rows((steps, n, di), torch.float32, "cpu", 2, "idx_q").to(DEV)
    pos = [[L + t for L in lens] for t in range(steps)]
    k_new = [torch.stack([kc0[s, :, pos[t][s]] for s in range(n)]).contiguous() for t in range(steps)]
    v_new = [torch.stack([vc0[s, :, pos[t][s]] for s in range(n)]).contiguous() for t in range(steps)]
    ik_new = [torch.stack([ik0[s, pos[t][s]] for s in range(n)]).contiguous() for t in range(steps)]
    seqs = [seq0 + t for t in range(steps)]
    kc, vc, ik, kmax = kc0.clone(), vc0.clone(), ik0.clone(), kmax0.clone()
    bufs = pipeline.alloc_decode_step(q_all[0], kmax, B, K)
    outs = [torch.empty_like(bufs.o) for _ in range(steps)]
    sels = [torch.empty_like(bufs.sel) for _ in range(steps)]

    def reset():
        kc.copy_(kc0)
        vc.copy_(vc0)
        ik.copy_(ik0)
        kmax.copy_(kmax0)

    def run():
        for t in range(steps):
            o, _, sel = pipeline.decode_append_step(
                q_all[t], k_new[t], v_new[t], iq_all[t], ik_new[t], kc, vc, kmax, seqs[t], B, K,
                cfg.scale, idx_k_cache=ik, bufs=bufs)
            outs[t].copy_(o)
            sels[t].copy_(sel)

    reset()
    run()
    torch.cuda.synchronize()
    eager = [(o_.cpu().clone(), s_.cpu().clone()) for o_, s_ in zip(outs, sels)]
    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        reset()                                  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t in range(steps):
            assert torch.equal(outs[t].cpu(), eager[t][0]), f"replay {rep} step {t}"
            assert torch.equal(sels[t].cpu(), eager[t][1]), f"replay {rep} step {t}"


# --------------------------------------------------------------------------
# fused decode step (append + running block max + scan + top-K + attention)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("hq,hkv,B,K,lens", [
    (64, 8, 64, 6, [0, 63, 64, 200, 1000]),      # empty cache, block-opening tokens
    (16, 1, 128, 4, [1, 127, 300]),              # G = 16
    (8, 8, 512, 8, [511, 512, 3000]),            # G = 1, the 1M-token block size
    # the 1M-token decode shape (Hq 64 / Hkv 8, B 512, K 8): caches of 4..9
    # blocks, one sequence opening a block, one just short of full rows
    (64, 8, 512, 8, [4096, 4607, 3583, 1535]),
    # one sequence at that shape: blocks split into two 128-key segments, the
    # last workgroup of each KV head combining 16 partials (as at 1M tokens)
    (64, 8, 512, 8, [4700]),
    # 128 sequences with full rows (own block >= K - 1): the workgroups whose
    # range starts on an own-block unit fetch its first chunk before the
    # selection merge (own blocks from 7 to 512 keys)
    (8, 1, 512, 8, [3590 + 9 * i for i in range(128)]),
])
def test_decode_step_fused(orc, hq, hkv, B, K, lens):
    n, d, di, steps = len(lens), 128, 128, 3
    T = max(lens) + steps
    cfg = synth.Config("dec-step", T, "bf16", hq, hkv, d, di, B, K, 4, n_seq=n, mode="decode")
    _say(f"fused decode step G={hq // hkv} B={B} K={K} lens={lens[:8]}{' ...' if n > 8 else ''}")
    x = synth.decode_inputs(cfg, "cpu", 0)
    nb_max = -(-T // B)
    kc = x["k_cache"].to(DEV)
    vc = x["v_cache"].to(DEV)
    ik = x["idx_k"].to(DEV)
    # device caches hold only the first lens[s] tokens; later rows are garbage
    kc_d, vc_d = kc.clone(), vc.clone()
    ik_d = ik.clone()
    for s, L in enumerate(lens):
        kc_d[s, :, L:] = 0.5
        vc_d[s, :, L:] = -0.5
        ik_d[s, L:] = 7.0
    kmax = torch.full((n, nb_max, di), float("nan"), device=DEV)
    seq = torch.tensor(lens, dtype=torch.int64, device=DEV)
    for s, L in enumerate(lens):
        if L:
            ops.msa_index_pool(ik_d[s:s + 1, :L], B, kmax=kmax[s:s + 1],
                               seq_len=seq[s:s + 1], nb_max=nb_max)
    # queries of the new tokens: seed 1, so they differ from the cache's draws
    q_all = synth._normal_rows((steps, n, hq, d), torch.bfloat16, "cpu", 1, "q")
    iq_all = synth._normal_rows((steps, n, di), torch.float32, "cpu", 1, "idx_q")
    ws = torch.empty(ops.load().msa_decode_step_workspace_bytes(n, nb_max, hq, d, B, K),
                     dtype=torch.uint8, device=DEV)
    kc_h, vc_h, ik_h = synth.host(kc), synth.host(vc), _np(ik)
    for t in range(steps):
        pos = np.array(lens, np.int64) + t
        k_new = torch.stack([kc[s, :, pos[s]] for s in range(n)]).contiguous()
        v_new = torch.stack([vc[s, :, pos[s]] for s in range(n)]).contiguous()
        ik_new = torch.stack([ik[s, pos[s]] for s in range(n)]).contiguous()
        q = q_all[t].to(DEV)
        iq = iq_all[t].to(DEV)
        o, lse, sel = ops.msa_decode_step(q, k_new, v_new, iq, ik_new, kc_d, vc_d, kmax, seq,
                                          B, K, idx_k_cache=ik_d, ws=ws)
        o, lse, sel = _np(o), _np(lse), _np(sel)
        for s in range(n):
            L = int(pos[s])
            # the append, bit for bit
            assert torch.equal(kc_d[s, :, L], kc[s, :, L]) and torch.equal(vc_d[s, :, L], vc[s, :, L])
            assert torch.equal(ik_d[s, L], ik[s, L])
            # the running summaries equal a fresh pool of the first L+1 index keys
            kmo = orc.pool(ik_h[s, :L + 1], B)
            nbl = -(-(L + 1) // B)
            assert np.array_equal(_np(kmax[s, :nbl]), kmo)
            so, gr, ga, eb = orc.select(_np(iq)[s:s + 1], np.array([L]), kmo, B, K)
            check_selection(sel[s:s + 1], so, gr, ga, eb, _np(iq)[s:s + 1], kmo, np.array([L]), B)
            oo, lo, _ = orc.attend(synth.host(q[s:s + 1]), kc_h[s], vc_h[s], np.array([0]),
                                   np.array([L]), sel[s:s + 1], B, cfg.scale, orc.BF16)
            eo, el = max_abs(o[s], oo[0]), max_abs(lse[s], lo[0])
            assert eo <= TOL_BF16 and el <= TOL_BF16, (t, s, eo, el)
        # the composed path on the same (now appended) cache gives the same result
        seq1 = seq + 1
        sel_c = ops.msa_index_topk_decode(iq, seq1, kmax, B, K)
        o_c, lse_c = ops.msa_sparse_gqa_decode(q, kc_d, vc_d, seq1, sel_c, B)
        assert np.array_equal(_np(sel_c), sel)
        assert np.array_equal(_np(o_c), o) and np.array_equal(_np(lse_c), lse)
        seq += 1
    _say(f"  {steps} steps x {n} sequences checked")
