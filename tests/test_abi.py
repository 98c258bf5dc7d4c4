"""C-ABI checks that need no GPU: every function include/msa.h declares is
exported by libmsa.so, and argument validation returns the documented
status before anything is enqueued (the calls below never reach a launch:
each fails a check first, so fake non-null pointers are never dereferenced).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

OK, EINVAL, EUNSUP, EWS, EHIP = 0, -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  (loads the HIP runtime the library links)
    from block_sparse_attention_index_amd import ops
    if not os.path.exists(ops.LIB_PATH):
        pytest.fail("libmsa.so is not built: run __graft_entry__.build()")
    return ops.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 11
    from block_sparse_attention_index_amd import ops
    assert sorted(ops.ENTRY_POINTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, word in [(OK, b"MSA_OK"), (EINVAL, b"INVALID_ARG"), (EUNSUP, b"UNSUPPORTED"),
                       (EWS, b"WORKSPACE"), (EHIP, b"HIP")]:
        assert word in lib.msa_status_string(code)
    assert lib.msa_status_string(12345)


def test_pool_validation(lib):
    P = FAKE
    assert lib.msa_index_pool(None, 1, 100, None, 64, 64, 0, 2, P, 2, None) == EINVAL
    assert lib.msa_index_pool(P, 1, 100, None, 64, 60, 0, 2, P, 2, None) == EINVAL   # B % 16
    assert lib.msa_index_pool(P, 1, 100, None, 64, 64, 0, 2, P, 1, None) == EINVAL   # nb_max
    assert lib.msa_index_pool(P, 1, 100, None, 64, 64, 2, 2, P, 2, None) == EINVAL   # range
    assert lib.msa_index_pool(P, 1, 100, None, 64, 64, -3, 0, P, 2, None) == EINVAL  # mode
    assert lib.msa_index_pool(P, 1, 100, None, 2000, 64, 0, 2, P, 2, None) == EINVAL  # d_idx
    assert lib.msa_index_pool(P, 0, 100, None, 64, 64, 0, 2, P, 2, None) == EINVAL   # n_seq


def test_topk_validation(lib):
    P = FAKE
    assert lib.msa_index_topk(P, 10, 0, P, 1, 64, 64, 0, P, None) == EINVAL      # topk 0
    assert lib.msa_index_topk(P, 10, 0, P, 1, 64, 64, 65, P, None) == EINVAL     # topk > 64
    assert lib.msa_index_topk(P, 200, 0, P, 2, 64, 64, 4, P, None) == EINVAL     # own >= nb
    assert lib.msa_index_topk(P, 0, 0, P, 1, 64, 64, 4, P, None) == OK           # empty: no-op
    need = lib.msa_topk_decode_workspace_bytes(2, 100, 8)
    assert need > 0
    assert lib.msa_index_topk_decode(P, 2, P, P, 100, 64, 64, 8, P, P, need - 1, None) == EWS
    assert lib.msa_index_topk_decode(P, 2, None, P, 100, 64, 64, 8, P, P, need, None) == EINVAL
    f = lib.msa_index_topk_batch
    need = lib.msa_topk_batch_workspace_bytes(300, 100, 8)
    assert need > 0
    assert lib.msa_topk_batch_workspace_bytes(300, 65535 * 64 + 1, 8) == 0   # grid y
    assert f(P, 300, P, P, P, 2, 100, 64, 64, 8, P, P, need - 1, None) == EWS
    assert f(P, 300, None, P, P, 2, 100, 64, 64, 8, P, P, need, None) == EINVAL  # q_seq
    assert f(P, 300, P, P, P, 0, 100, 64, 64, 8, P, P, need, None) == EINVAL     # n_seq
    assert f(P, 300, P, P, P, 2, 100, 64, 64, 65, P, P, need, None) == EINVAL    # topk
    assert f(P, 300, P, P, P, 2, 65535 * 64 + 1, 64, 64, 8, P, P, need, None) == EINVAL
    assert f(None, 0, None, None, None, 2, 100, 64, 64, 8, None, None, 0, None) == OK


def test_invert_validation(lib):
    P = FAKE
    need = lib.msa_invert_workspace_bytes(5000, 8, 100)
    assert need >= 100 * 4
    assert lib.msa_invert_selection(P, 5000, 8, 100, P, P, P, P, need - 1, None) == EWS
    assert lib.msa_invert_selection(P, 5000, 8, 0, P, P, P, P, need, None) == EINVAL
    assert lib.msa_invert_selection(P, 1 << 30, 8, 100, P, P, P, P, 1 << 40, None) == EINVAL


def test_prefill_validation(lib):
    P = FAKE
    f = lib.msa_sparse_gqa_prefill
    args = lambda **kw: dict(dict(q=P, k=P, v=P, dt=1, kvs=4096, q0=0, nq=4096, hq=64, hkv=8,
                                  d=128, B=64, sel=P, K=16, rp=P, ql=P, sl=P, sc=0.1, o=P,
                                  lse=None, ws=P, wsb=1 << 40, st=None), **kw)
    call = lambda a: f(a["q"], a["k"], a["v"], a["dt"], a["kvs"], a["q0"], a["nq"], a["hq"],
                       a["hkv"], a["d"], a["B"], a["sel"], a["K"], a["rp"], a["ql"], a["sl"],
                       a["sc"], a["o"], a["lse"], a["ws"], a["wsb"], a["st"])
    assert call(args(q=None)) == EINVAL
    assert call(args(hq=60)) == EINVAL                    # Hq % Hkv
    assert call(args(dt=2)) == EINVAL                     # dtype
    assert call(args(q0=10)) == EINVAL                    # q_pos0 + n_q > kv_stride
    assert call(args(sc=float("inf"))) == EINVAL
    assert call(args(d=96)) == EUNSUP                     # no kernel for d = 96
    assert call(args(hq=24, hkv=8)) == EUNSUP             # group 3
    need = lib.msa_prefill_workspace_bytes(1, 0, 4096, 64, 128, 64, 16)
    assert call(args(wsb=need - 1)) == EWS
    assert lib.msa_prefill_workspace_bytes(2, 0, 4096, 64, 128, 64, 16) == 0


def test_prefill_workspace_holds_the_partials(lib):
    # the KV-outer pass keeps one partial record per (non-own pair, query
    # head): fp32 (d values + lse) for fp32 inputs, fp16 values + (lse, e) for
    # the bf16 d = 128 path; non-own pairs have a closed form
    for q0, n, B, K in [(0, 32768, 64, 16), (1000, 3000, 128, 6), (0, 1 << 20, 512, 8)]:
        p = sum((min(K, (pos // B) + 1) - 1) for pos in range(q0, q0 + n)) if n < 100000 else \
            sum((min(K, b + 1) - 1) * min(B, q0 + n - b * B) for b in range((q0 + n + B - 1) // B))
        assert lib.msa_prefill_workspace_bytes(0, q0, n, 64, 128, B, K) >= p * 64 * 129 * 4
        assert lib.msa_prefill_workspace_bytes(1, q0, n, 64, 128, B, K) >= p * 64 * (128 * 2 + 8)


def test_decode_validation(lib):
    P = FAKE
    need = lib.msa_decode_workspace_bytes(4, 64, 128, 512, 8)
    assert need > 0
    f = lib.msa_sparse_gqa_decode
    assert f(P, P, P, 1, 4, 1000, P, 64, 8, 128, 512, P, 8, 0.1, P, None, P, need - 1, None) == EWS
    assert f(P, P, P, 1, 4, 1000, None, 64, 8, 128, 512, P, 8, 0.1, P, None, P, need, None) == EINVAL
    assert f(P, P, P, 1, 4, 1000, P, 64, 8, 96, 512, P, 8, 0.1, P, None, P, need, None) == EUNSUP
    assert f(P, P, P, 0, 4, 1000, P, 64, 8, 256, 512, P, 8, 0.1, P, None, P, need, None) == EUNSUP


def test_index_variant_validation(lib):
    P = FAKE
    f = lib.msa_index_topk_window
    assert f(P, 10, 0, P, 1, 64, 64, 4, 0, P, None) == EINVAL       # window 0
    assert f(P, 10, 0, P, 1, 64, 64, 4, 5, P, None) == EINVAL       # window > K
    assert f(P, 0, 0, P, 1, 64, 64, 4, 4, P, None) == OK            # empty: no-op
    g = lib.msa_index_topk_decode_window
    need = lib.msa_topk_decode_workspace_bytes(2, 100, 8)
    assert g(P, 2, P, P, 100, 64, 64, 8, 9, P, P, need, None) == EINVAL
    assert g(P, 2, P, P, 100, 64, 64, 8, 2, P, P, need - 1, None) == EWS
    m = lib.msa_index_pool_mean
    assert m(P, 1, 100, None, 64, 64, -2, 0, P, 2, None) == EINVAL   # no append form
    assert m(P, 1, 100, None, 64, 60, 0, 2, P, 2, None) == EINVAL    # B % 16
    assert m(None, 1, 100, None, 64, 64, 0, 2, P, 2, None) == EINVAL


def test_paged_decode_validation(lib):
    P = FAKE
    f = lib.msa_sparse_gqa_decode_paged
    need = lib.msa_decode_workspace_bytes(4, 64, 128, 512, 8)
    a = dict(q=P, kp=P, vp=P, dt=2, ks=P, vs=P, npg=100, bt=P, mb=10, n=4, sl=P, hq=64, hkv=8,
             d=128, B=512, sel=P, K=8, sc=0.1, o=P, lse=None, ws=P, wsb=need)
    call = lambda **kw: f(*dict(a, **kw).values(), None)
    assert call(wsb=need - 1) == EWS
    assert call(dt=0) == EINVAL                  # fp32 pages: no
    assert call(ks=None) == EINVAL               # FP8 needs scales
    assert call(npg=0) == EINVAL
    assert call(d=64) == EUNSUP
    assert call(hq=24) == EUNSUP                 # group 3


def test_varlen_validation(lib):
    P = FAKE
    c = lambda xs: (ctypes.c_int64 * len(xs))(*xs)
    wsb = lib.msa_prefill_varlen_workspace_bytes
    assert wsb(1, 2, c([0, 100, 300]), c([0, 100, 500]), 64, 128, 128, 64, 8) > 0
    assert wsb(1, 2, c([1, 100, 300]), c([0, 100, 500]), 64, 128, 128, 64, 8) == 0   # cu[0]
    assert wsb(1, 2, c([0, 200, 300]), c([0, 100, 500]), 64, 128, 128, 64, 8) == 0   # qn > kvn
    assert wsb(1, 2, c([0, 100, 90]), c([0, 100, 500]), 64, 128, 128, 64, 8) == 0    # decreasing
    f = lib.msa_prefill_varlen
    cq, ckv = c([0, 100, 300]), c([0, 100, 500])
    need = wsb(1, 2, cq, ckv, 64, 128, 128, 64, 8)
    args = [P, P, P, P, P, 1, 2, cq, ckv, 64, 8, 128, 128, 64, 8, 0.1, P, P, None, P]
    assert f(*args, need - 1, None) == EWS
    bad = list(args)
    bad[7] = c([0, 200, 300])
    assert f(*bad, need, None) == EINVAL
    bad = list(args)
    bad[11] = 96                                   # d = 96: no kernel
    assert f(*bad, need, None) == EUNSUP


def test_varlen_chain_grouping(lib):
    """bf16 / d = 128 runs the sequences in chains of at most 64, each chain's
    workspace covering all its sequences at once: one more sequence grows the
    workspace until the 65th, which opens a second (smaller) chain; empty
    sequences add nothing."""
    c = lambda xs: (ctypes.c_int64 * len(xs))(*xs)
    wsb = lib.msa_prefill_varlen_workspace_bytes

    def ws(n, qn=300, kvn=1000, dtype=1, d=128):
        cq = c([i * qn for i in range(n + 1)])
        ckv = c([i * kvn for i in range(n + 1)])
        return wsb(dtype, n, cq, ckv, 64, d, 128, 64, 8)

    one, two, w64, w65 = ws(1), ws(2), ws(64), ws(65)
    assert 0 < one < two < w64
    assert w65 == w64
    # an empty sequence between two others changes nothing
    cq, ckv = c([0, 300, 300, 600]), c([0, 1000, 1500, 2500])
    assert wsb(1, 3, cq, ckv, 64, 128, 128, 64, 8) == two
    # the per-sequence path (fp32, or another head size) sizes for one sequence
    assert ws(1, dtype=0) == ws(8, dtype=0)
    assert ws(1, d=64) == ws(8, d=64)


def test_paged_prefill_validation(lib):
    P = FAKE
    f = lib.msa_sparse_gqa_prefill_paged
    args = lambda **kw: dict(dict(q=P, kp=P, vp=P, npg=100, bt=P, mb=64, q0=0, nq=4096, hq=64,
                                  hkv=8, d=128, B=64, sel=P, K=16, rp=P, ql=P, sl=P, sc=0.1,
                                  o=P, lse=None, ws=P, wsb=1 << 40, st=None), **kw)
    call = lambda a: f(a["q"], a["kp"], a["vp"], a["npg"], a["bt"], a["mb"], a["q0"], a["nq"],
                       a["hq"], a["hkv"], a["d"], a["B"], a["sel"], a["K"], a["rp"], a["ql"],
                       a["sl"], a["sc"], a["o"], a["lse"], a["ws"], a["wsb"], a["st"])
    assert call(args(bt=None)) == EINVAL
    assert call(args(npg=0)) == EINVAL
    assert call(args(mb=63)) == EINVAL                    # table shorter than the blocks used
    assert call(args(q0=10)) == EINVAL                    # 65 blocks > 64 table entries
    assert call(args(hq=60)) == EINVAL
    assert call(args(sc=float("nan"))) == EINVAL
    assert call(args(d=64)) == EUNSUP                     # bf16 matrix-core path only
    assert call(args(hq=24, hkv=8)) == EUNSUP
    need = lib.msa_prefill_workspace_bytes(1, 0, 4096, 64, 128, 64, 16)
    assert call(args(wsb=need - 1)) == EWS
    assert call(args(nq=0)) == 0                          # nothing to do


def test_paged_decode_step_validation(lib):
    P = FAKE
    f = lib.msa_decode_step_paged
    args = lambda **kw: dict(dict(q=P, kn=P, vn=P, iq=P, ikn=P, kp=P, vp=P, npg=64, bt=P, mb=8,
                                  ikc=None, km=P, n=4, lm=4096, nbm=8, sl=P, hq=64, hkv=8,
                                  d=128, di=128, B=512, K=8, sc=0.1, sel=P, o=P, lse=None, ws=P,
                                  wsb=1 << 40, st=None), **kw)
    keys = ["q", "kn", "vn", "iq", "ikn", "kp", "vp", "npg", "bt", "mb", "ikc", "km", "n", "lm",
            "nbm", "sl", "hq", "hkv", "d", "di", "B", "K", "sc", "sel", "o", "lse", "ws", "wsb",
            "st"]
    call = lambda a: f(*[a[k_] for k_ in keys])
    assert call(args(bt=None)) == EINVAL
    assert call(args(npg=0)) == EINVAL
    assert call(args(mb=0)) == EINVAL
    assert call(args(hq=60)) == EINVAL
    assert call(args(d=64)) == EUNSUP
    need = lib.msa_decode_step_workspace_bytes(4, 8, 64, 128, 512, 8)
    assert call(args(wsb=need - 1)) == EWS
