"""msa_decode_step_noalloc (the decode step on the library's static scratch)
against msa_decode_step with a caller workspace, through the C ABI (needs a
GPU): bit for bit on two calls in a row, the second with a smaller input, and
a shape beyond the scratch maximum refused without a launch."""
import numpy as np
import pytest
import torch

from block_sparse_attention_index_amd import ops, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(hq, hkv, B, K, lens, seed):
    n, T = len(lens), max(lens) + 1
    cfg = synth.Config("noalloc", T, "bf16", hq, hkv, 128, 128, B, K, 3, n_seq=n,
                       mode="decode")
    x = {k_: v_.to(DEV) for k_, v_ in synth.decode_inputs(cfg, "cpu", seed).items()}
    nb_max = -(-T // B)
    seq = torch.tensor(lens, dtype=torch.int64, device=DEV)
    kmax = torch.zeros((n, nb_max, cfg.d_idx), device=DEV)
    ops.msa_index_pool(x["idx_k"], B, kmax=kmax, seq_len=seq, nb_max=nb_max)
    # the new token of each sequence (a fresh draw) is appended at position len
    g = torch.Generator().manual_seed(seed + 100)
    k_new = torch.randn((n, hkv, 128), generator=g).to(torch.bfloat16).to(DEV)
    v_new = torch.randn((n, hkv, 128), generator=g).to(torch.bfloat16).to(DEV)
    ik_new = torch.randn((n, cfg.d_idx), generator=g).to(DEV)
    return cfg, x, seq, kmax, k_new, v_new, ik_new


def _run_both(hq, hkv, B, K, lens, seed):
    cfg, x, seq, kmax, k_new, v_new, ik_new = _case(hq, hkv, B, K, lens, seed)
    n = len(lens)
    res = []
    for noalloc in (False, True):
        kc, vc, ik, km = (x["k_cache"].clone(), x["v_cache"].clone(), x["idx_k"].clone(),
                          kmax.clone())
        sel = torch.empty((n, K), dtype=torch.int32, device=DEV)
        o = torch.empty((n, hq, 128), dtype=torch.float32, device=DEV)
        lse = torch.empty((n, hq), dtype=torch.float32, device=DEV)
        if noalloc:
            ops.msa_decode_step_noalloc(x["q"], k_new, v_new, x["idx_q"], ik_new, kc, vc, km, seq,
                                        B, K, idx_k_cache=ik, sel=sel, o=o, lse=lse)
        else:
            ops.msa_decode_step(x["q"], k_new, v_new, x["idx_q"], ik_new, kc, vc, km, seq, B, K,
                                idx_k_cache=ik, sel=sel, o=o, lse=lse)
        torch.cuda.synchronize()
        res.append([t.cpu() for t in (sel, o, lse, km, kc, vc, ik)])
    for name, a, b in zip(("sel", "o", "lse", "kmax", "k_cache", "v_cache", "idx_k"), *res):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                           b.view(torch.uint8) if b.dtype != torch.int32 else b), name
    return res[0]


def test_noalloc_decode_step_matches_workspace_call():
    print("no-alloc decode step: call 1 (4 sequences, block 512)", flush=True)
    _run_both(64, 8, 512, 8, [5000, 9000, 2047, 700], seed=1)
    print("no-alloc decode step: call 2 (smaller: 2 sequences, block 64)", flush=True)
    _run_both(16, 2, 64, 6, [1000, 300], seed=2)


def test_noalloc_refuses_beyond_the_maximum():
    lib = ops.load()
    cap = lib.msa_decode_step_noalloc_max_bytes()
    assert cap == 32 << 20
    # 512 sequences x 64 heads at block 512, top-K 8: about 270 MB of scratch
    assert lib.msa_decode_step_workspace_bytes(512, 2048, 64, 128, 512, 8) > cap
    P = ctypes_p = __import__("ctypes").c_void_p(0x1000)
    st = lib.msa_decode_step_noalloc(P, P, P, P, P, P, P, None, P, 1, 512, 1 << 20, 2048, P,
                                     64, 8, 128, 128, 512, 8, 0.1, P, P, None, None)
    assert st == -3, st
