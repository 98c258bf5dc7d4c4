"""Device parity of the index-branch variants (needs a GPU): the block
mean-pool summary and the forced local window, after the sketch in section
3.3 of chenxutan.com's "MiniMax M3 深度实战".

Mean pool: fp32 sums in the kernel's order against the oracle's fp64 mean,
within (n+1) * 2^-24 * sum|x| / n + 2^-24 * |mean| per element for a block of
n tokens (the classical bound of recursive summation plus the division's
rounding).  Window selections: bit-exact except flagged near-ties, on
summaries produced by the device (max-pool, itself bit-exact, or mean-pool,
fed to the oracle as they are).
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_index_amd import ops, synth
from helpers import check_selection

pytestmark = pytest.mark.gpu
DEV = "cuda"
U = 2.0 ** -24


def _np(t):
    return t.detach().cpu().numpy()


def _say(msg):
    print(msg, flush=True)


def _mean_bound(x, B):
    """Per-element error bound of the device mean for each block of x."""
    L = x.shape[0]
    out = []
    for b in range(-(-L // B)):
        blk = np.abs(x[b * B:min(L, b * B + B)].astype(np.float64))
        n = blk.shape[0]
        out.append((n + 1) * U * blk.sum(axis=0) / n + U * np.abs(blk.mean(axis=0)) + 1e-30)
    return np.array(out)


@pytest.mark.parametrize("L,B,d", [(4096, 64, 64), (1000, 16, 128), (777, 128, 24),
                                   (1, 16, 4), (5000, 512, 128), (300, 32, 1024),
                                   (260, 64, 5)])
def test_pool_mean_within_bound(orc, L, B, d):
    _say(f"pool mean L={L} B={B} d={d}")
    g = torch.Generator().manual_seed(L + 3 * B + d)
    x = torch.randn(L, d, generator=g) * 3 + 1
    got = _np(ops.msa_index_pool_mean(x.to(DEV), B))
    want = orc.pool_mean(x.numpy(), B)
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    assert np.all(err <= _mean_bound(x.numpy(), B) + U * np.abs(want))


def test_pool_mean_batched_ragged_and_last_block(orc):
    n, Lmax, B, d = 3, 1000, 64, 128
    g = torch.Generator().manual_seed(9)
    x = torch.randn(n, Lmax, d, generator=g)
    lens = [1000, 513, 64]
    nb_max = 17
    km = torch.full((n, nb_max, d), float("nan"), device=DEV)
    seq_len = torch.tensor(lens, dtype=torch.int64, device=DEV)
    ops.msa_index_pool_mean(x.to(DEV), B, kmean=km, seq_len=seq_len, nb_max=nb_max)
    got = _np(km)
    for s, L in enumerate(lens):
        nb = -(-L // B)
        want = orc.pool_mean(x[s, :L].numpy(), B)
        assert np.all(np.abs(got[s, :nb] - want) <= _mean_bound(x[s, :L].numpy(), B)
                      + U * np.abs(want))
        assert np.all(np.isnan(got[s, nb:])), "blocks past the sequence stay untouched"
    # last-block form: change each sequence's newest token, re-pool only that block
    x2 = x.clone()
    for s, L in enumerate(lens):
        x2[s, L - 1] += 5.0
    ops.msa_index_pool_mean(x2.to(DEV), B, kmean=km, seq_len=seq_len, blk_begin=-1,
                            nb_max=nb_max)
    got = _np(km)
    for s, L in enumerate(lens):
        want = orc.pool_mean(x2[s, :L].numpy(), B)
        b = (L - 1) // B
        assert np.all(np.abs(got[s, b] - want[b]) <= _mean_bound(x2[s, :L].numpy(), B)[b]
                      + U * np.abs(want[b]))


@pytest.mark.parametrize("T,B,K,w,d,q0,mean", [
    (4096, 64, 16, 4, 128, 0, False),
    (3000, 16, 4, 4, 32, 0, False),      # window = K: pure sliding window
    (2500, 32, 64, 9, 24, 100, False),   # K = 64, d_idx not a multiple of 64
    (5000, 128, 8, 2, 128, 1234, True),  # mean-pool summaries
    (2000, 64, 6, 1, 64, 0, True),       # window 1 on mean summaries
])
def test_topk_window_prefill(orc, T, B, K, w, d, q0, mean):
    _say(f"topk window T={T} B={B} K={K} w={w} d={d} q0={q0} mean={mean}")
    cfg = synth.Config("tw", T, "f32", 1, 1, 64, d, B, K, 6)
    x = synth.sequence_inputs(cfg, "cpu", 2)
    idx_k = x["idx_k"].to(DEV)
    summ = ops.msa_index_pool_mean(idx_k, B) if mean else ops.msa_index_pool(idx_k, B)
    kmax = _np(summ)
    idx_q = x["idx_q"].numpy()[q0:]
    pos = np.arange(q0, T, dtype=np.int64)
    sel_o, gr, ga, eb = orc.select(idx_q, pos, kmax, B, K, window=w)
    sel_d = ops.msa_index_topk_window(torch.from_numpy(idx_q).to(DEV), summ, B, K, w,
                                      q_pos0=q0)
    nf, nm = check_selection(_np(sel_d), sel_o, gr, ga, eb, idx_q, kmax, pos, B, window=w)
    _say(f"  near-ties flagged {nf}, differing rows {nm}")


@pytest.mark.parametrize("B,K,w,lens", [
    (64, 8, 3, [1, 64, 65, 200, 1000, 5000]),
    (512, 8, 2, [511, 512, 3000, 40000]),
    (16, 5, 5, [7, 16, 100, 3000]),
    (16, 16, 1, [4096, 70000]),          # more than 64 scan chunks: staged tournament
    (16, 8, 2, [300000]),                # more than 256 chunks: running-list merge
])
def test_topk_window_decode(orc, B, K, w, lens):
    _say(f"topk window decode B={B} K={K} w={w} lens={lens}")
    n, d = len(lens), 128
    Lmax = max(lens)
    g = torch.Generator().manual_seed(B + K + w)
    ik = torch.randn(n, Lmax, d, generator=g)
    iq = torch.randn(n, d, generator=g)
    nb_max = -(-Lmax // B)
    seq = torch.tensor(lens, dtype=torch.int64, device=DEV)
    kmax = ops.msa_index_pool(ik.to(DEV), B, seq_len=seq, nb_max=nb_max)
    sel = _np(ops.msa_index_topk_decode_window(iq.to(DEV), seq, kmax, B, K, w))
    km = _np(kmax)
    for s, L in enumerate(lens):
        pos = np.array([L - 1], np.int64)
        so, gr, ga, eb = orc.select(iq[s:s + 1].numpy(), pos, km[s], B, K, window=w)
        check_selection(sel[s:s + 1], so, gr, ga, eb, iq[s:s + 1].numpy(), km[s], pos, B,
                        window=w)
