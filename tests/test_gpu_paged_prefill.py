"""Device parity of the sparse prefill against a paged bf16 cache (needs a
GPU): a chunk of queries, the last tokens of a sequence whose keys and values
sit in block-granular pages addressed through a block table (prefill of a
request's next chunk against its cache; KV cache management of section 3.3
of chenxutan.com's "MiniMax M3 深度实战").

The pages are a shuffled pool holding the contiguous cache block by block
(spare pages and the unused tail of the last page hold other values, which
must not be read).  The paged result must equal the contiguous kernel's on
the same selection bit for bit (same kernels, same arithmetic), and match the
oracle on the device's own selection within the bf16 tolerance.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_index_amd import ops
from helpers import TOL_BF16, check_selection, max_abs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("hq,hkv,B,K,q_pos0,n_q,seed", [
    (64, 8, 64, 8, 1000, 700, 1),     # chunk after a cached prefix, ragged last block
    (16, 2, 128, 6, 0, 2500, 2),      # whole prompt
    (8, 8, 16, 4, 37, 300, 3),        # G = 1, small blocks
    (32, 2, 64, 16, 4096, 64, 4),     # short chunk, G = 16
])
def test_prefill_paged(orc, hq, hkv, B, K, q_pos0, n_q, seed):
    _say(f"paged prefill Hq={hq} Hkv={hkv} B={B} K={K} q_pos0={q_pos0} n_q={n_q}")
    d, di = 128, 64
    T = q_pos0 + n_q
    nb = -(-T // B)
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(hkv, T, d, generator=g).to(torch.bfloat16)
    v = torch.randn(hkv, T, d, generator=g).to(torch.bfloat16)
    q = torch.randn(n_q, hq, d, generator=g).to(torch.bfloat16)
    ik = torch.randn(T, di, generator=g)
    iq = torch.randn(n_q, di, generator=g)
    # shuffled pool with spare pages; everything not holding the cache is noise
    n_pages = nb + 7
    perm = torch.randperm(n_pages, generator=g)[:nb].to(torch.int32)
    kp = torch.randn(n_pages, hkv, B, d, generator=g).to(torch.bfloat16)
    vp = torch.randn(n_pages, hkv, B, d, generator=g).to(torch.bfloat16)
    for b in range(nb):
        r = min(B, T - b * B)
        kp[int(perm[b]), :, :r] = k[:, b * B:b * B + r]
        vp[int(perm[b]), :, :r] = v[:, b * B:b * B + r]
    table = torch.cat([perm, torch.full((3,), -1, dtype=torch.int32)])   # max_blocks > nb

    kd, vd = k.to(DEV), v.to(DEV)
    km = ops.msa_index_pool(ik.to(DEV), B)
    sel = ops.msa_index_topk(iq.to(DEV), km, B, K, q_pos0=q_pos0)
    rp, ql, sl = ops.msa_invert_selection(sel, nb)
    qd = q.to(DEV)
    o_c, l_c = ops.msa_sparse_gqa_prefill(qd, kd, vd, sel, rp, ql, sl, B, q_pos0=q_pos0)
    o_p, l_p = ops.msa_sparse_gqa_prefill_paged(qd, kp.to(DEV), vp.to(DEV), table.to(DEV), sel,
                                                rp, ql, sl, B, q_pos0=q_pos0)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_c) and torch.equal(l_p, l_c)

    # the oracle on the device's own selection
    pos = np.arange(q_pos0, T, dtype=np.int64)
    kmax = orc.pool(ik.numpy(), B)
    so, gr, ga, eb = orc.select(iq.numpy(), pos, kmax, B, K)
    sel_h = _np(sel)
    nf, nm = check_selection(sel_h, so, gr, ga, eb, iq.numpy(), kmax, pos, B)
    oo, lo, _ = orc.attend(q.view(torch.uint16).numpy(), k.view(torch.uint16).numpy(),
                           v.view(torch.uint16).numpy(), np.arange(n_q), pos, sel_h, B,
                           d ** -0.5, orc.BF16)
    eo, el = max_abs(_np(o_p), oo), max_abs(_np(l_p), lo)
    _say(f"  near-ties {nf}, differing {nm}, max|do| {eo:.3g} max|dlse| {el:.3g}")
    assert eo <= TOL_BF16 and el <= TOL_BF16
