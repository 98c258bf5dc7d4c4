"""Device parity of the fused decode step over a paged bf16 cache (needs a
GPU): each step appends the new token's K and V rows into the page of its
block and attends through the block table (block-granular KV cache management
of section 3.3 of chenxutan.com's "MiniMax M3 深度实战").

The same steps run on the contiguous cache with msa_decode_step: selections,
outputs and log-sum-exps must agree bit for bit (same kernels, same
arithmetic), the pages must hold exactly the contiguous cache's rows after
the appends (and pages no sequence owns must be untouched), and every step is
checked against the oracle on the device's own selection.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_index_amd import ops, synth
from helpers import TOL_BF16, check_selection, max_abs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("hq,hkv,B,K,lens", [
    (16, 2, 128, 4, [300, 511, 1000, 0]),       # a block-opening append, an empty cache
    (64, 8, 512, 8, [4095, 3583, 1535]),         # the 1M-token decode shape
    (8, 8, 64, 6, [63, 64, 200]),                # G = 1
])
def test_decode_step_paged(orc, hq, hkv, B, K, lens):
    n, d, di, steps = len(lens), 128, 64, 3
    T = max(lens) + steps
    _say(f"paged fused decode step Hq={hq} Hkv={hkv} B={B} K={K} lens={lens}")
    cfg = synth.Config("dec-step-paged", T, "bf16", hq, hkv, d, di, B, K, 2, n_seq=n,
                       mode="decode")
    x = synth.decode_inputs(cfg, "cpu", 11)
    nb_max = -(-T // B)
    kc = x["k_cache"]                            # [n, Hkv, T, d] bf16 (rows past lens: future tokens)
    vc = x["v_cache"]
    ik = x["idx_k"]
    # contiguous device caches: rows past each length hold other values
    kc_d, vc_d, ik_d = kc.clone(), vc.clone(), ik.clone()
    for s, L in enumerate(lens):
        kc_d[s, :, L:] = 0.5
        vc_d[s, :, L:] = -0.5
        ik_d[s, L:] = 7.0
    kc_d, vc_d, ik_d = kc_d.to(DEV), vc_d.to(DEV), ik_d.to(DEV)
    ik_p = ik_d.clone()
    # paged pool: every block a sequence will use has a page (shuffled), plus
    # spare pages filled with noise that must stay untouched
    g = torch.Generator().manual_seed(7)
    n_pages = n * nb_max + 5
    perm = torch.randperm(n_pages, generator=g).to(torch.int32)
    table = torch.full((n, nb_max + 2), -1, dtype=torch.int32)
    kp = torch.randn(n_pages, hkv, B, d, generator=g).to(torch.bfloat16)
    vp = torch.randn(n_pages, hkv, B, d, generator=g).to(torch.bfloat16)
    used = set()
    kcd_h, vcd_h = kc_d.cpu(), vc_d.cpu()
    for s in range(n):
        for b in range(nb_max):
            pg = int(perm[s * nb_max + b])
            table[s, b] = pg
            used.add(pg)
            r = min(B, T - b * B)                 # the last page's tail stays noise
            kp[pg, :, :r] = kcd_h[s, :, b * B:b * B + r]
            vp[pg, :, :r] = vcd_h[s, :, b * B:b * B + r]
    spare = sorted(set(range(n_pages)) - used)
    kp_spare, vp_spare = kp[spare].clone(), vp[spare].clone()
    kp, vp, table = kp.to(DEV), vp.to(DEV), table.to(DEV)

    seq = torch.tensor(lens, dtype=torch.int64, device=DEV)
    kmax_c = torch.full((n, nb_max, di), float("nan"), device=DEV)
    for s, L in enumerate(lens):
        if L:
            ops.msa_index_pool(ik_d[s:s + 1, :L], B, kmax=kmax_c[s:s + 1], seq_len=seq[s:s + 1],
                               nb_max=nb_max)
    kmax_p = kmax_c.clone()
    q_all = synth._normal_rows((steps, n, hq, d), torch.bfloat16, "cpu", 1, "q")
    iq_all = synth._normal_rows((steps, n, di), torch.float32, "cpu", 1, "idx_q")
    kc_h, vc_h, ik_h = synth.host(kc), synth.host(vc), _np(ik)
    for t in range(steps):
        pos = np.array(lens, np.int64) + t
        k_new = torch.stack([kc[s, :, pos[s]] for s in range(n)]).contiguous().to(DEV)
        v_new = torch.stack([vc[s, :, pos[s]] for s in range(n)]).contiguous().to(DEV)
        ik_new = torch.stack([ik[s, pos[s]] for s in range(n)]).contiguous().to(DEV)
        q, iq = q_all[t].to(DEV), iq_all[t].to(DEV)
        o_c, l_c, s_c = ops.msa_decode_step(q, k_new, v_new, iq, ik_new, kc_d, vc_d, kmax_c, seq,
                                            B, K, idx_k_cache=ik_d)
        o_p, l_p, s_p = ops.msa_decode_step_paged(q, k_new, v_new, iq, ik_new, kp, vp, table,
                                                  kmax_p, seq, B, K, T, idx_k_cache=ik_p)
        torch.cuda.synchronize()
        assert torch.equal(s_p, s_c) and torch.equal(o_p, o_c) and torch.equal(l_p, l_c), t
        # bit patterns (unwritten summaries hold NaN on both sides)
        assert torch.equal(kmax_p.view(torch.int32), kmax_c.view(torch.int32))
        assert torch.equal(ik_p.view(torch.int32), ik_d.view(torch.int32))
        o, lse, sel = _np(o_p), _np(l_p), _np(s_p)
        for s in range(n):
            L = int(pos[s])
            kmo = orc.pool(ik_h[s, :L + 1], B)
            so, gr, ga, eb = orc.select(_np(iq)[s:s + 1], np.array([L]), kmo, B, K)
            check_selection(sel[s:s + 1], so, gr, ga, eb, _np(iq)[s:s + 1], kmo, np.array([L]), B)
            oo, lo, _ = orc.attend(synth.host(q[s:s + 1]), kc_h[s], vc_h[s], np.array([0]),
                                   np.array([L]), sel[s:s + 1], B, cfg.scale, orc.BF16)
            eo, el = max_abs(o[s], oo[0]), max_abs(lse[s], lo[0])
            assert eo <= TOL_BF16 and el <= TOL_BF16, (t, s, eo, el)
        seq += 1
    # the pages hold the contiguous cache block by block; spare pages untouched
    kp_h, vp_h, tb = kp.cpu(), vp.cpu(), table.cpu()
    kcd_h, vcd_h = kc_d.cpu(), vc_d.cpu()
    for s in range(n):
        for b in range(nb_max):
            pg, r = int(tb[s, b]), min(B, T - b * B)
            assert torch.equal(kp_h[pg, :, :r], kcd_h[s, :, b * B:b * B + r]), (s, b)
            assert torch.equal(vp_h[pg, :, :r], vcd_h[s, :, b * B:b * B + r]), (s, b)
    assert torch.equal(kp_h[spare], kp_spare) and torch.equal(vp_h[spare], vp_spare)
    _say(f"  {steps} steps x {n} sequences checked")
