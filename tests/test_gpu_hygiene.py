"""Determinism and memory hygiene of the device path (needs a GPU).

* Run twice, bit for bit: the whole prefill (summaries, selection, CSR,
  outputs, log-sum-exps) at the full 32K-token workload, and the fused decode
  step, give identical results on every run -- no floating-point atomics or
  scheduling-dependent sums.
* Poisoned workspaces: every workspace filled with all-ones bytes (NaN floats,
  -1 integers) or with 0x7f bytes (large finite floats, large integers) gives
  the same outputs as a zeroed one, so no kernel reads a workspace word it did
  not write first.
* Canary bands: every output is a view into a larger buffer whose margins
  hold a fixed NaN pattern; the margins must be unchanged after each call, so
  no kernel writes outside its outputs.
* A selection whose CSR holds more pairs than the prefill workspace was sized
  for stays inside the workspace.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_index_amd import ops, pipeline, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
PAD = 4096                      # canary elements on each side of an output
CANARY = np.uint32(0x7FC0DEAD)  # a NaN with a payload no kernel produces


def _say(msg):
    print(msg, flush=True)


class Guarded:
    """A device tensor of `shape` inside a buffer with PAD canary words on
    either side (4-byte element types only)."""

    def __init__(self, shape, dtype):
        assert torch.empty(0, dtype=dtype).element_size() == 4
        n = int(np.prod(shape))
        self.raw = torch.full((n + 2 * PAD,), int(CANARY.view(np.int32)), dtype=torch.int32,
                              device=DEV)
        self.t = self.raw.view(dtype)[PAD:PAD + n].view(shape)

    def intact(self) -> bool:
        r = self.raw.cpu().numpy().view(np.uint32)
        return bool(np.all(r[:PAD] == CANARY) and np.all(r[-PAD:] == CANARY))


def _ws_variants(nbytes):
    out = []
    for fill in (0, 0xFF, 0x7F):
        out.append(torch.full((max(1, nbytes),), fill, dtype=torch.uint8, device=DEV))
    return out


def _cfg_small():
    return synth.CONFIGS["p32k"].replace(name="hyg", T=4096, n_hot=8)


def test_prefill_run_twice_bitwise_full_p32k():
    cfg = synth.CONFIGS["p32k"]
    _say("run twice: p32k prefill")
    x = synth.sequence_inputs(cfg, DEV, 0)
    B, K = cfg.block, cfg.topk
    runs = []
    for rep in range(2):
        bufs = pipeline.alloc_prefill(x["q"], x["idx_q"], B, K)
        bufs.attn_ws.fill_(0xFF if rep else 0)       # different workspace contents too
        o, lse, sel = pipeline.prefill(x["q"], x["k"], x["v"], x["idx_q"], x["idx_k"],
                                       B, K, cfg.scale, bufs=bufs)
        nrow = bufs.row_ptr[-1].item()
        runs.append([t.cpu() for t in (bufs.kmax, sel, bufs.row_ptr, bufs.q_list[:nrow],
                                       bufs.slot, o, lse)])
        del bufs, o, lse, sel
    names = ("kmax", "sel", "row_ptr", "q_list", "slot", "o", "lse")
    for nm, a, b in zip(names, runs[0], runs[1]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{nm} differs between runs"
    _say("  summaries, selection, CSR, outputs and log-sum-exps identical")


def test_prefill_poisoned_workspace_and_canaries():
    cfg = _cfg_small()
    _say("poisoned workspaces + canaries: prefill chain")
    x = synth.sequence_inputs(cfg, DEV, 1)
    T, B, K, hq, d = cfg.T, cfg.block, cfg.topk, cfg.Hq, cfg.d
    nb = -(-T // B)
    lib = ops.load()
    results = []
    for ws_p, ws_i, ws_a in zip(*(_ws_variants(n) for n in (
            0, lib.msa_invert_workspace_bytes(T, K, nb),
            lib.msa_prefill_workspace_bytes(ops.MSA_BF16, 0, T, hq, d, B, K)))):
        kmax = Guarded((nb, cfg.d_idx), torch.float32)
        sel = Guarded((T, K), torch.int32)
        rp, ql, sl = Guarded((nb + 1,), torch.int32), Guarded((T * K,), torch.int32), \
            Guarded((T, K), torch.int32)
        o, lse = Guarded((T, hq, d), torch.float32), Guarded((T, hq), torch.float32)
        ops.msa_index_pool(x["idx_k"], B, kmax=kmax.t)
        ops.msa_index_topk(x["idx_q"], kmax.t, B, K, sel=sel.t)
        ops.msa_invert_selection(sel.t, nb, row_ptr=rp.t, q_list=ql.t, slot=sl.t, ws=ws_i)
        ops.msa_sparse_gqa_prefill(x["q"], x["k"], x["v"], sel.t, rp.t, ql.t, sl.t, B,
                                   cfg.scale, o=o.t, lse=lse.t, ws=ws_a)
        torch.cuda.synchronize()
        for g, nm in ((kmax, "kmax"), (sel, "sel"), (rp, "row_ptr"), (ql, "q_list"),
                      (sl, "slot"), (o, "o"), (lse, "lse")):
            assert g.intact(), f"write outside {nm}"
        nnz = rp.t[-1].item()
        results.append([kmax.t.cpu(), sel.t.cpu(), rp.t.cpu(), ql.t[:nnz].cpu(), sl.t.cpu(),
                        o.t.cpu(), lse.t.cpu()])
    for r in results[1:]:
        for a, b in zip(results[0], r):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    _say("  outputs independent of workspace contents; all canaries intact")


def test_prefill_csr_beyond_workspace_bound():
    """A CSR with more non-own pairs than the workspace was sized for (every
    query lists blocks 0..K-1, so rows hold queries of later blocks too, and
    each query K - 1 non-own pairs even where the causal bound allows fewer):
    the tile table is clamped to the workspace's bound, the call returns OK,
    and nothing past the workspace or outside the outputs is written.  (The
    outputs of such a call are unspecified.)"""
    n_q, hq, hkv, d, B, K = 4096, 64, 8, 128, 512, 8
    nb = n_q // B
    _say(f"over-full CSR: n_q={n_q} B={B} K={K}")
    g = torch.Generator().manual_seed(7)
    q = torch.randn(n_q, hq, d, generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn(hkv, n_q, d, generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn(hkv, n_q, d, generator=g).to(torch.bfloat16).to(DEV)
    sel = torch.arange(K, dtype=torch.int32, device=DEV).repeat(n_q, 1).contiguous()
    rp, ql, sl = ops.msa_invert_selection(sel, nb)
    lib = ops.load()
    nbytes = lib.msa_prefill_workspace_bytes(ops.MSA_BF16, 0, n_q, hq, d, B, K)
    tail = 1 << 20
    big = torch.full((nbytes + tail,), 0xA5, dtype=torch.uint8, device=DEV)
    o, lse = Guarded((n_q, hq, d), torch.float32), Guarded((n_q, hq), torch.float32)
    ops.msa_sparse_gqa_prefill(q, k, v, sel, rp, ql, sl, B, d ** -0.5, o=o.t, lse=lse.t,
                               ws=big[:nbytes])
    torch.cuda.synchronize()
    assert bool((big[nbytes:] == 0xA5).all()), "write past the workspace"
    assert o.intact() and lse.intact(), "write outside the outputs"
    _say("  clamped: workspace tail and output canaries intact")


def test_prefill_f32_poisoned_workspace_and_canaries():
    cfg = synth.CONFIGS["tiny"].replace(name="hyg32", T=1500)
    _say("poisoned workspaces + canaries: fp32 prefill")
    x = synth.sequence_inputs(cfg, DEV, 2)
    T, B, K, hq, d = cfg.T, cfg.block, cfg.topk, cfg.Hq, cfg.d
    nb = -(-T // B)
    lib = ops.load()
    kmax = ops.msa_index_pool(x["idx_k"], B)
    sel = ops.msa_index_topk(x["idx_q"], kmax, B, K)
    rp, ql, sl = ops.msa_invert_selection(sel, nb)
    res = []
    for ws in _ws_variants(lib.msa_prefill_workspace_bytes(ops.MSA_F32, 0, T, hq, d, B, K)):
        o, lse = Guarded((T, hq, d), torch.float32), Guarded((T, hq), torch.float32)
        ops.msa_sparse_gqa_prefill(x["q"], x["k"], x["v"], sel, rp, ql, sl, B, cfg.scale,
                                   o=o.t, lse=lse.t, ws=ws)
        torch.cuda.synchronize()
        assert o.intact() and lse.intact()
        res.append((o.t.cpu(), lse.t.cpu()))
    for a, b in res[1:]:
        assert torch.equal(a, res[0][0]) and torch.equal(b, res[0][1])


@pytest.mark.parametrize("hq,hkv,B,K,lens", [
    (64, 8, 512, 8, [5000, 2600, 700]),
    (16, 2, 64, 6, [3000, 64, 1]),
])
def test_decode_poisoned_workspace_and_canaries(hq, hkv, B, K, lens):
    n = len(lens)
    T = max(lens) + 1
    cfg = synth.Config("hyg-dec", T, "bf16", hq, hkv, 128, 128, B, K, 3, n_seq=n,
                       mode="decode")
    _say(f"poisoned workspaces + canaries: decode G={hq // hkv} B={B} lens={lens}")
    x = {k_: v_.to(DEV) for k_, v_ in synth.decode_inputs(cfg, "cpu", 4).items()}
    nb_max = -(-T // B)
    lib = ops.load()
    seq = torch.tensor(lens, dtype=torch.int64, device=DEV)
    kmax0 = torch.zeros((n, nb_max, cfg.d_idx), device=DEV)
    ops.msa_index_pool(x["idx_k"], B, kmax=kmax0, seq_len=seq, nb_max=nb_max)
    # separate calls
    res = []
    for tws, aws in zip(_ws_variants(lib.msa_topk_decode_workspace_bytes(n, nb_max, K)),
                        _ws_variants(lib.msa_decode_workspace_bytes(n, hq, 128, B, K))):
        sel = Guarded((n, K), torch.int32)
        o, lse = Guarded((n, hq, 128), torch.float32), Guarded((n, hq), torch.float32)
        ops.msa_index_topk_decode(x["idx_q"], seq, kmax0, B, K, sel=sel.t, ws=tws)
        ops.msa_sparse_gqa_decode(x["q"], x["k_cache"], x["v_cache"], seq, sel.t, B,
                                  o=o.t, lse=lse.t, ws=aws)
        torch.cuda.synchronize()
        assert sel.intact() and o.intact() and lse.intact()
        res.append((sel.t.cpu(), o.t.cpu(), lse.t.cpu()))
    # fused step: append at seq_len (the token at L is already in the cache,
    # so repeating the step is idempotent)
    k_new = torch.stack([x["k_cache"][s, :, L] for s, L in enumerate(lens)]).contiguous()
    v_new = torch.stack([x["v_cache"][s, :, L] for s, L in enumerate(lens)]).contiguous()
    ik_new = torch.stack([x["idx_k"][s, L] for s, L in enumerate(lens)]).contiguous()
    res_f = []
    for ws in _ws_variants(lib.msa_decode_step_workspace_bytes(n, nb_max, hq, 128, B, K)):
        kmax = kmax0.clone()
        kc, vc, ik = x["k_cache"].clone(), x["v_cache"].clone(), x["idx_k"].clone()
        sel = Guarded((n, K), torch.int32)
        o, lse = Guarded((n, hq, 128), torch.float32), Guarded((n, hq), torch.float32)
        ops.msa_decode_step(x["q"], k_new, v_new, x["idx_q"], ik_new, kc, vc, kmax, seq, B, K,
                            idx_k_cache=ik, sel=sel.t, o=o.t, lse=lse.t, ws=ws)
        torch.cuda.synchronize()
        assert sel.intact() and o.intact() and lse.intact()
        # nothing but the appended rows changes in the caches
        assert torch.equal(kc, x["k_cache"]) and torch.equal(vc, x["v_cache"])
        assert torch.equal(ik, x["idx_k"])
        res_f.append((sel.t.cpu(), o.t.cpu(), lse.t.cpu(), kmax.cpu()))
    for r in res[1:]:
        for a, b in zip(res[0], r):
            assert torch.equal(a, b)
    for r in res_f[1:]:
        for a, b in zip(res_f[0], r):
            assert torch.equal(a, b)
    _say("  decode outputs independent of workspace contents; canaries intact")


def test_decode_step_run_twice_bitwise():
    hq, hkv, B, K, lens = 64, 8, 512, 8, [9000, 4097, 600, 20000]
    n, T = len(lens), max(lens) + 1
    cfg = synth.Config("twice-dec", T, "bf16", hq, hkv, 128, 128, B, K, 4, n_seq=n,
                       mode="decode")
    _say("run twice: fused decode step")
    x = {k_: v_.to(DEV) for k_, v_ in synth.decode_inputs(cfg, "cpu", 6).items()}
    nb_max = -(-T // B)
    seq = torch.tensor(lens, dtype=torch.int64, device=DEV)
    kmax0 = torch.zeros((n, nb_max, cfg.d_idx), device=DEV)
    ops.msa_index_pool(x["idx_k"], B, kmax=kmax0, seq_len=seq, nb_max=nb_max)
    k_new = torch.stack([x["k_cache"][s, :, L] for s, L in enumerate(lens)]).contiguous()
    v_new = torch.stack([x["v_cache"][s, :, L] for s, L in enumerate(lens)]).contiguous()
    ik_new = torch.stack([x["idx_k"][s, L] for s, L in enumerate(lens)]).contiguous()
    out = []
    for _ in range(2):
        kmax = kmax0.clone()
        o, lse, sel = ops.msa_decode_step(x["q"], k_new, v_new, x["idx_q"], ik_new,
                                          x["k_cache"], x["v_cache"], kmax, seq, B, K)
        out.append((o.cpu(), lse.cpu(), sel.cpu(), kmax.cpu()))
    for a, b in zip(*out):
        assert torch.equal(a, b)
