"""Pins for the oracle's sparse attention (no GPU).

Definition: standard GQA over the union of the selected blocks (sparse branch
of "MiniMax M3模型算力成本大幅降低原因深度解析"; the softmax over gathered keys
of section 2.3 "MSA 算法实现" of chenxutan.com's "MiniMax M3 深度实战").

Pins: (1) K >= number of blocks reproduces dense causal GQA attention from
torch's scaled_dot_product_attention in fp64; (2) K = 1 reproduces
block-diagonal causal attention (the same library routine with a mask);
(3) p = 0 gives o = v[0] and lse = scale * q.k[0]; (4) identical keys give the
mean of the attended values; (5) log-sum-exp merging per-block partials over
any partition equals the whole; (6) bf16 bit inputs equal their exact fp32
upcast.
"""
import numpy as np
import torch

F32, BF16 = 0, 1


def _rand(shape, rng):
    return rng.standard_normal(shape).astype(np.float32)


def _sdpa(q, k, v, mask, scale):
    """Reference attention in fp64 with torch's library routine.
    q [L, Hq, d]; k/v [Hkv, L, d]; mask [L, L] bool (True = attend)."""
    Hq, Hkv = q.shape[1], k.shape[0]
    G = Hq // Hkv
    qt = torch.from_numpy(q).double().permute(1, 0, 2)[None]            # [1,Hq,L,d]
    kt = torch.from_numpy(k).double().repeat_interleave(G, 0)[None]     # [1,Hq,L,d]
    vt = torch.from_numpy(v).double().repeat_interleave(G, 0)[None]
    m = torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=m, scale=scale)[0].permute(1, 0, 2)        # [L,Hq,d]
    s = (qt @ kt.transpose(-1, -2))[0] * scale                          # [Hq,L,L]
    s = s.masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(s, dim=-1).T                                  # [L,Hq]
    return o.numpy(), lse.numpy()


def _setup(L=300, Hq=4, Hkv=2, d=16, seed=8):
    rng = np.random.default_rng(seed)
    return _rand((L, Hq, d), rng), _rand((Hkv, L, d), rng), _rand((Hkv, L, d), rng)


def test_all_blocks_equals_dense_causal(orc):
    L, B = 300, 16
    q, k, v = _setup(L)
    nb = -(-L // B)
    K = nb
    pos = np.arange(L, dtype=np.int64)
    sel = np.full((L, K), -1, np.int32)
    for p in range(L):
        sel[p, :p // B + 1] = np.arange(p // B + 1)
    scale = 0.3
    o, lse, nk = orc.attend(q, k, v, pos, pos, sel, B, scale, F32)
    mask = np.tril(np.ones((L, L), bool))
    ro, rlse = _sdpa(q, k, v, mask, scale)
    np.testing.assert_allclose(o, ro, rtol=2e-6, atol=2e-6)
    np.testing.assert_allclose(lse, rlse, rtol=2e-6, atol=2e-6)
    assert np.array_equal(nk, pos + 1)


def test_own_block_only_equals_block_diagonal(orc):
    L, B = 200, 32
    q, k, v = _setup(L, Hq=6, Hkv=3, d=8, seed=9)
    pos = np.arange(L, dtype=np.int64)
    sel = (pos // B).astype(np.int32)[:, None]
    o, lse, _ = orc.attend(q, k, v, pos, pos, sel, B, 0.25, F32)
    t = np.arange(L)
    mask = (t[:, None] // B == t[None, :] // B) & (t[None, :] <= t[:, None])
    ro, rlse = _sdpa(q, k, v, mask, 0.25)
    np.testing.assert_allclose(o, ro, rtol=2e-6, atol=2e-6)
    np.testing.assert_allclose(lse, rlse, rtol=2e-6, atol=2e-6)


def test_first_token_and_identical_keys(orc):
    L, B, Hq, Hkv, d = 64, 16, 4, 1, 8
    q, k, v = _setup(L, Hq, Hkv, d, seed=10)
    sel = np.array([[0, -1]], np.int32)
    o, lse, _ = orc.attend(q, k, v, np.array([0]), np.array([0]), sel, B, 0.5, F32)
    for h in range(Hq):
        assert np.array_equal(o[0, h], v[0, 0])
        assert lse[0, h] == np.float32(0.5 * np.dot(q[0, h].astype(np.float64),
                                                   k[0, 0].astype(np.float64)))
    # identical keys: uniform weights -> mean of the attended values
    k2 = np.tile(k[:, :1], (1, L, 1))
    p = 50                                       # own block 3, keys 48..50 + block 1
    sel = np.array([[1, 3]], np.int32)
    o, lse, nk = orc.attend(q, k2, v, np.array([p]), np.array([p]), sel, B, 0.5, F32)
    keys = list(range(16, 32)) + [48, 49, 50]
    assert nk[0] == len(keys)
    want = v[0, keys].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(o[0, 0], want, rtol=1e-6, atol=1e-6)
    s = 0.5 * np.dot(q[p, 0].astype(np.float64), k2[0, 0].astype(np.float64))
    np.testing.assert_allclose(lse[0, 0], s + np.log(len(keys)), rtol=1e-6)


def test_lse_merge_of_partials_equals_whole(orc):
    # Partials over any partition of a query's blocks, merged by
    # lse = log sum exp(lse_i), o = sum exp(lse_i - lse) o_i, give the whole.
    L, B, K = 512, 32, 6
    q, k, v = _setup(L, Hq=8, Hkv=2, d=16, seed=11)
    rng = np.random.default_rng(12)
    pos = np.array([500, 333, 64, 255], np.int64)
    for p in pos:
        own = p // B
        blocks = sorted(rng.choice(own, size=min(K - 1, own), replace=False).tolist()) + [own]
        sel = np.array([blocks + [-1] * (K - len(blocks))], np.int32)
        o, lse, _ = orc.attend(q, k, v, np.array([p]), np.array([p]), sel, B, 0.2, F32)
        parts = [blocks[:1], blocks[1:3], blocks[3:]]
        parts = [x for x in parts if x]
        po, pl = [], []
        for part in parts:
            s1 = np.array([part + [-1] * (K - len(part))], np.int32)
            a, b, _ = orc.attend(q, k, v, np.array([p]), np.array([p]), s1, B, 0.2, F32)
            po.append(a[0].astype(np.float64))
            pl.append(b[0].astype(np.float64))
        pl = np.stack(pl)                                  # [n_part, Hq]
        m = pl.max(axis=0)
        tot = m + np.log(np.exp(pl - m).sum(axis=0))
        mo = sum(np.exp(pl[i] - tot)[:, None] * po[i] for i in range(len(po)))
        np.testing.assert_allclose(lse[0], tot, rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(o[0], mo, rtol=1e-5, atol=1e-6)


def test_bf16_bits_equal_exact_upcast(orc):
    L, B = 128, 16
    q, k, v = _setup(L, Hq=4, Hkv=2, d=16, seed=13)
    tq, tk, tv = (torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))
    bits = [t.view(torch.int16).numpy().view(np.uint16) for t in (tq, tk, tv)]
    ups = [t.float().numpy() for t in (tq, tk, tv)]
    pos = np.arange(L, dtype=np.int64)
    sel = np.stack([pos // B, np.maximum(pos // B - 2, 0)], 1).astype(np.int32)
    sel = np.sort(sel, axis=1)
    sel[sel[:, 0] == sel[:, 1], 0] = -1
    sel = np.sort(sel, axis=1)[:, ::-1].copy()          # padding first: any order is accepted
    ob, lb, _ = orc.attend(*bits, pos, pos, sel, B, 0.25, BF16)
    of, lf, _ = orc.attend(*ups, pos, pos, sel, B, 0.25, F32)
    assert np.array_equal(ob, of) and np.array_equal(lb, lf)


def test_rejects_future_block(orc):
    q, k, v = _setup(64, 2, 1, 4)
    import pytest
    with pytest.raises(ValueError):
        orc.attend(q, k, v, np.array([3]), np.array([3]), np.array([[0, 1]], np.int32),
                   16, 1.0, F32)
