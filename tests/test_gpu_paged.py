"""Device parity of the paged decode (needs a GPU): bf16 and FP8 (e4m3) page
pools addressed through a block table (KV cache management of section 3.3 of
chenxutan.com's "MiniMax M3 深度实战": block-granular pages, reduced-precision
KV).

The oracle attends over the contiguous cache the pages stand for: for bf16
pages the cache itself (and the paged result must equal the contiguous
kernel's bit for bit: same units, same arithmetic); for FP8 pages the
oracle's dequantised values (scale * e4m3 value in fp32), against which the
tolerance is the bf16 one (e4m3 values are exact in bf16; only the scaled
products round).  The FP8 codes and scales are inputs: they are made here by
torch's fp32 -> e4m3 cast of amax-scaled pages.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_index_amd import ops
from helpers import TOL_BF16, max_abs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


def _say(msg):
    print(msg, flush=True)


def _paged_case(orc, hq, hkv, B, K, lens, fp8, seed):
    d = 128
    n = len(lens)
    max_blocks = -(-max(lens) // B)
    L = max_blocks * B
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(n, hkv, L, d, generator=g).to(torch.bfloat16)
    v = torch.randn(n, hkv, L, d, generator=g).to(torch.bfloat16)
    q = torch.randn(n, hq, d, generator=g).to(torch.bfloat16)
    # a shuffled page pool with spare pages; unused table entries point nowhere
    n_pages = n * max_blocks + 5
    perm = torch.randperm(n_pages, generator=g)
    table = torch.full((n, max_blocks), -1, dtype=torch.int32)
    kp = torch.zeros(n_pages, hkv, B, d, dtype=torch.bfloat16)
    vp = torch.zeros(n_pages, hkv, B, d, dtype=torch.bfloat16)
    for s, Ls in enumerate(lens):
        for b in range(-(-Ls // B)):
            pg = int(perm[s * max_blocks + b])
            table[s, b] = pg
            kp[pg] = k[s, :, b * B:(b + 1) * B]
            vp[pg] = v[s, :, b * B:(b + 1) * B]
    ks = vs = None
    if fp8:
        amax_k = kp.float().abs().amax(dim=(2, 3)).clamp_min(1e-6)
        amax_v = vp.float().abs().amax(dim=(2, 3)).clamp_min(1e-6)
        ks, vs = amax_k / 448.0, amax_v / 448.0
        kp8 = (kp.float() / ks[:, :, None, None]).to(torch.float8_e4m3fn)
        vp8 = (vp.float() / vs[:, :, None, None]).to(torch.float8_e4m3fn)
        # the cache the pages stand for: the oracle's dequantisation of the
        # codes (scale * e4m3 value, rounded once), laid out contiguously
        kd = torch.from_numpy(orc.dequant_e4m3(kp8.view(torch.uint8).numpy(), ks.numpy()))
        vd = torch.from_numpy(orc.dequant_e4m3(vp8.view(torch.uint8).numpy(), vs.numpy()))
        kc = torch.zeros(n, hkv, L, d)
        vc = torch.zeros(n, hkv, L, d)
        for s, Ls in enumerate(lens):
            for b in range(-(-Ls // B)):
                pg = int(table[s, b])
                kc[s, :, b * B:(b + 1) * B] = kd[pg]
                vc[s, :, b * B:(b + 1) * B] = vd[pg]
        kp, vp = kp8, vp8
    # a valid selection per sequence: the own block and K-1 random earlier ones
    sel = torch.full((n, K), -1, dtype=torch.int32)
    for s, Ls in enumerate(lens):
        own = (Ls - 1) // B
        pick = sorted(torch.randperm(own, generator=g)[:K - 1].tolist()) if own else []
        row = pick + [own]
        sel[s, :len(row)] = torch.tensor(row, dtype=torch.int32)
    seq = torch.tensor(lens, dtype=torch.int64)
    o, lse = ops.msa_sparse_gqa_decode_paged(
        q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), seq.to(DEV), sel.to(DEV), B,
        k_scale=None if ks is None else ks.contiguous().to(DEV),
        v_scale=None if vs is None else vs.contiguous().to(DEV))
    o, lse = _np(o), _np(lse)
    if not fp8:
        # bit for bit the contiguous kernel
        oc, lc = ops.msa_sparse_gqa_decode(q.to(DEV), k.to(DEV), v.to(DEV), seq.to(DEV),
                                           sel.to(DEV), B)
        assert np.array_equal(o, _np(oc)) and np.array_equal(lse, _np(lc))
    worst = 0.0
    for s, Ls in enumerate(lens):
        pos = np.array([Ls - 1], np.int64)
        if fp8:
            oo, lo, _ = orc.attend(q[s:s + 1].float().numpy(), kc[s].numpy(), vc[s].numpy(),
                                   np.array([0]), pos, _np(sel[s:s + 1]), B, d ** -0.5, orc.F32)
        else:
            oo, lo, _ = orc.attend(q[s:s + 1].view(torch.uint16).numpy(),
                                   k[s].view(torch.uint16).numpy(),
                                   v[s].view(torch.uint16).numpy(), np.array([0]), pos,
                                   _np(sel[s:s + 1]), B, d ** -0.5, orc.BF16)
        eo, el = max_abs(o[s], oo[0]), max_abs(lse[s], lo[0])
        worst = max(worst, eo, el)
        assert eo <= TOL_BF16 and el <= TOL_BF16, (s, eo, el)
    _say(f"  max error {worst:.3g}")


@pytest.mark.parametrize("hq,hkv,B,K,lens", [
    (64, 8, 64, 8, [1, 64, 65, 700, 3000]),
    (16, 1, 512, 4, [511, 512, 2049]),      # G = 16
    (8, 8, 128, 6, [128, 1000]),            # G = 1
    # 40 sequences: ~10 one-chunk units per workgroup, so the copies run
    # several units ahead of the computation
    (64, 8, 64, 8, [50 + 37 * i for i in range(40)]),
])
@pytest.mark.parametrize("fp8", [False, True])
def test_paged_decode(orc, hq, hkv, B, K, lens, fp8):
    _say(f"paged decode fp8={fp8} Hq={hq} Hkv={hkv} B={B} K={K} lens={lens}")
    _paged_case(orc, hq, hkv, B, K, lens, fp8, seed=hq + B + K)
