"""Device parity of the several-sequences prefill (needs a GPU): each
sequence of the packed batch against the oracle (selection bit-exact except
flagged near-ties, outputs within the tolerance, evaluated on the device's
own selection), and against the single-sequence entry points on the same
data, which must agree bit for bit (same kernels, same arithmetic).
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_index_amd import ops, pipeline
from helpers import TOL_BF16, TOL_F32, check_selection, max_abs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


def _say(msg):
    print(msg, flush=True)


def _many_short(n, seed):
    """n requests of a serving batch: mostly short prompts (some only a few
    tokens), a few longer ones, a few continuing a cached prefix."""
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        kvn = int(r.choice([r.integers(1, 64), r.integers(64, 400), r.integers(400, 1200)],
                           p=[0.3, 0.55, 0.15]))
        qn = kvn if r.random() < 0.8 else int(r.integers(0, kvn + 1))
        out.append((qn, kvn))
    return out


@pytest.mark.parametrize("dtype,hq,hkv,d,B,K,seqs", [
    # (queries, cached tokens) per sequence; queries are each cache's last tokens
    ("bf16", 64, 8, 128, 64, 8, [(1000, 1000), (300, 2000), (0, 500), (1, 1), (700, 700)]),
    # more sequences than one chain holds (64): two chains
    ("bf16", 16, 2, 128, 64, 8, _many_short(70, 5)),
    ("bf16", 16, 2, 128, 128, 6, [(129, 4000), (2500, 2500)]),
    ("f32", 8, 2, 64, 64, 4, [(640, 640), (64, 900), (33, 33)]),
])
def test_prefill_varlen(orc, dtype, hq, hkv, d, B, K, seqs):
    _say(f"varlen {dtype} Hq={hq} Hkv={hkv} d={d} B={B} K={K} seqs={seqs}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    di = 64
    cu_q = np.concatenate([[0], np.cumsum([s[0] for s in seqs])]).astype(np.int64)
    cu_kv = np.concatenate([[0], np.cumsum([s[1] for s in seqs])]).astype(np.int64)
    nq, nkv = int(cu_q[-1]), int(cu_kv[-1])
    g = torch.Generator().manual_seed(hq + B + K)
    k = torch.randn(hkv, nkv, d, generator=g).to(tdt)
    v = torch.randn(hkv, nkv, d, generator=g).to(tdt)
    ik = torch.randn(nkv, di, generator=g)
    # each sequence's queries belong to its last tokens
    q = torch.randn(nq, hq, d, generator=g).to(tdt)
    iq = torch.randn(nq, di, generator=g)
    o, lse, sel = ops.msa_prefill_varlen(q.to(DEV), k.to(DEV), v.to(DEV), iq.to(DEV),
                                         ik.to(DEV), cu_q, cu_kv, B, K)
    o, lse, sel = _np(o), _np(lse), _np(sel)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for s, (qn, kvn) in enumerate(seqs):
        if qn == 0:
            continue
        a, b = int(cu_q[s]), int(cu_q[s + 1])
        ka, kb = int(cu_kv[s]), int(cu_kv[s + 1])
        pos = np.arange(kvn - qn, kvn, dtype=np.int64)
        kmax = orc.pool(ik[ka:kb].numpy(), B)
        so, gr, ga, eb = orc.select(iq[a:b].numpy(), pos, kmax, B, K)
        nf, nm = check_selection(sel[a:b], so, gr, ga, eb, iq[a:b].numpy(), kmax, pos, B)
        if dtype == "bf16":
            qh = q[a:b].view(torch.uint16).numpy()
            kh = k[:, ka:kb].contiguous().view(torch.uint16).numpy()
            vh = v[:, ka:kb].contiguous().view(torch.uint16).numpy()
            dt = orc.BF16
        else:
            qh, kh, vh, dt = q[a:b].numpy(), k[:, ka:kb].contiguous().numpy(), \
                v[:, ka:kb].contiguous().numpy(), orc.F32
        oo, lo, _ = orc.attend(qh, kh, vh, np.arange(qn), pos, sel[a:b], B, d ** -0.5, dt)
        eo, el = max_abs(o[a:b], oo), max_abs(lse[a:b], lo)
        _say(f"  seq {s}: {qn} queries / {kvn} tokens, near-ties {nf}, differing {nm}, "
             f"max|do| {eo:.3g} max|dlse| {el:.3g}")
        assert eo <= tol and el <= tol
        # the single-sequence entry points on the same sequence, bit for bit
        kd, vd = k[:, ka:kb].contiguous().to(DEV), v[:, ka:kb].contiguous().to(DEV)
        km = ops.msa_index_pool(ik[ka:kb].to(DEV), B)
        s1 = ops.msa_index_topk(iq[a:b].to(DEV), km, B, K, q_pos0=kvn - qn)
        assert np.array_equal(_np(s1), sel[a:b])
        nb = -(-kvn // B)
        rp, ql, sl = ops.msa_invert_selection(s1, nb)
        o1, l1 = ops.msa_sparse_gqa_prefill(q[a:b].to(DEV), kd, vd, s1, rp, ql, sl, B,
                                            d ** -0.5, q_pos0=kvn - qn)
        assert np.array_equal(_np(o1), o[a:b]) and np.array_equal(_np(l1), lse[a:b])
