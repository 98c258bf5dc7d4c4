"""CPU oracle for MiniMax Sparse Attention (MSA) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never imports, loads or calls it, and it imports nothing from the
product package.

The arithmetic lives in ``msa_oracle.c`` (plain C, fp64, OpenMP over queries);
this module builds it with gcc and wraps it for numpy arrays.  Each function
states the passage it follows; the pages are:

* [YLY] "MiniMax M3模型算力成本大幅降低原因深度解析" (youleyou.com/wenzhang/3016623.html)
* [CXT] "MiniMax M3 深度实战：当稀疏注意力打破百万 Token 墙 ..." (chenxutan.com/d/3746.html)

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, brute force or a library routine; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile ``msa_oracle.c`` into ``liboracle.so`` with gcc (-O3 without fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O3", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
            "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_pool.argtypes = [P, i64, i32, i32, P]
        lib.oracle_pool_mean.argtypes = [P, i64, i32, i32, P]
        lib.oracle_select.argtypes = [P, i64, P, P, i64, i32, i32, i32, P, P, P, P]
        lib.oracle_select_window.argtypes = [P, i64, P, P, i64, i32, i32, i32, i32, P, P,
                                             P, P]
        lib.oracle_invert.argtypes = [P, i64, i32, i64, P, P, P]
        lib.oracle_invert.restype = ctypes.c_int64
        lib.oracle_attend.argtypes = [P, P, P, i32, i64, P, P, P, i32, i32, i32,
                                      i32, i32, i64, f64, P, P, P]
        lib.oracle_counts.argtypes = [P, i64, i32, P, i32, P, P]
        lib.oracle_dequant_e4m3.argtypes = [P, i64, i32, i64, P, P]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def threads() -> int:
    """Number of OpenMP threads the oracle uses."""
    return _load().oracle_threads()


def pool(idx_k: np.ndarray, block: int) -> np.ndarray:
    """Block max-pool of index keys [YLY, "索引分支（Index Branch）"].

    ``idx_k`` [L, d_idx] fp32 -> ``kmax`` [ceil(L/B), d_idx] fp32, the
    elementwise max over the valid tokens of each block (exact).
    """
    idx_k = np.ascontiguousarray(idx_k, dtype=np.float32)
    L, d = idx_k.shape
    out = np.empty(((L + block - 1) // block, d), np.float32)
    rc = _load().oracle_pool(_ptr(idx_k), L, d, block, _ptr(out))
    if rc:
        raise ValueError("oracle_pool: invalid arguments")
    return out


def pool_mean(idx_k: np.ndarray, block: int) -> np.ndarray:
    """Block mean-pool of index keys (the block summary of CXT §3.3's sketch).

    ``idx_k`` [L, d_idx] fp32 -> ``kmean`` [ceil(L/B), d_idx] fp32: the mean
    over the valid tokens of each block, summed in fp64, rounded once.
    """
    idx_k = np.ascontiguousarray(idx_k, dtype=np.float32)
    L, d = idx_k.shape
    out = np.empty(((L + block - 1) // block, d), np.float32)
    rc = _load().oracle_pool_mean(_ptr(idx_k), L, d, block, _ptr(out))
    if rc:
        raise ValueError("oracle_pool_mean: invalid arguments")
    return out


def select(idx_q: np.ndarray, q_pos: np.ndarray, kmax: np.ndarray, block: int,
           topk: int, window: int = 1):
    """Causal top-K per query [YLY, "索引分支（Index Branch）"; CXT §3.3].

    Returns ``(sel [n_q, K] int32, gap_rel, gap_abs, err_bound)``: ``sel`` is
    ascending and -1 padded; the gap arrays describe the cut between the last
    kept and the first left-out candidate (NaN when nothing is left out).
    ``window`` > 1 forces the blocks own-window+1 .. own (the local window of
    CXT §3.3's sketch) and ranks only the blocks below them.
    """
    idx_q = np.ascontiguousarray(idx_q, dtype=np.float32)
    kmax = np.ascontiguousarray(kmax, dtype=np.float32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int64)
    n_q, d = idx_q.shape
    assert kmax.shape[1] == d and q_pos.shape == (n_q,)
    sel = np.empty((n_q, topk), np.int32)
    gr = np.empty(n_q, np.float64)
    ga = np.empty(n_q, np.float64)
    eb = np.empty(n_q, np.float64)
    rc = _load().oracle_select_window(_ptr(idx_q), n_q, _ptr(q_pos), _ptr(kmax),
                                      kmax.shape[0], d, block, topk, window, _ptr(sel),
                                      _ptr(gr), _ptr(ga), _ptr(eb))
    if rc:
        raise ValueError("oracle_select: invalid arguments")
    return sel, gr, ga, eb


def invert(sel: np.ndarray, n_blocks: int):
    """Queries per KV block as CSR [CXT §2.2 "KV Outer Gather Q"].

    Returns ``(row_ptr [nb+1], q_list [nnz], slot [n_q, K])``, all int32,
    with each row ascending by query index.
    """
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    n_q, topk = sel.shape
    row_ptr = np.empty(n_blocks + 1, np.int32)
    q_list = np.empty(max(1, n_q * topk), np.int32)
    slot = np.empty((n_q, topk), np.int32)
    nnz = _load().oracle_invert(_ptr(sel), n_q, topk, n_blocks, _ptr(row_ptr),
                                _ptr(q_list), _ptr(slot))
    if nnz < 0:
        raise ValueError("oracle_invert: invalid arguments")
    return row_ptr, q_list[:nnz].copy(), slot


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_row: np.ndarray,
           q_pos: np.ndarray, sel: np.ndarray, block: int, scale: float,
           dtype: int):
    """GQA over the union of the selected blocks [YLY, "稀疏分支（Sparse Branch）"].

    ``q`` [n_rows, Hq, d], ``k``/``v`` [Hkv, kv_stride, d], as float32 arrays
    (dtype F32) or uint16 bf16 bit patterns (dtype BF16).  ``sel`` holds one
    row per evaluated query.  Returns ``(o [n_eval, Hq, d] fp32,
    lse [n_eval, Hq] fp32, n_keys [n_eval] int64)``.
    """
    want = np.float32 if dtype == F32 else np.uint16
    q = np.ascontiguousarray(q, dtype=want)
    k = np.ascontiguousarray(k, dtype=want)
    v = np.ascontiguousarray(v, dtype=want)
    q_row = np.ascontiguousarray(q_row, dtype=np.int64)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int64)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    _, hq, d = q.shape
    hkv, kv_stride, dk = k.shape
    assert dk == d and v.shape == k.shape
    n_eval, topk = sel.shape
    assert q_row.shape == (n_eval,) and q_pos.shape == (n_eval,)
    o = np.empty((n_eval, hq, d), np.float32)
    lse = np.empty((n_eval, hq), np.float32)
    nk = np.empty(n_eval, np.int64)
    rc = _load().oracle_attend(_ptr(q), _ptr(k), _ptr(v), dtype, n_eval,
                               _ptr(q_row), _ptr(q_pos), _ptr(sel), topk, hq,
                               hkv, d, block, kv_stride, float(scale), _ptr(o),
                               _ptr(lse), _ptr(nk))
    if rc:
        raise ValueError("oracle_attend: invalid arguments")
    return o, lse, nk


def counts(sel: np.ndarray, q_pos: np.ndarray, block: int):
    """(nnz, attended pairs) of an actual selection."""
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int64)
    n_q, topk = sel.shape
    nnz = ctypes.c_int64()
    att = ctypes.c_int64()
    rc = _load().oracle_counts(_ptr(sel), n_q, topk, _ptr(q_pos), block,
                               ctypes.byref(nnz), ctypes.byref(att))
    if rc:
        raise ValueError("oracle_counts: invalid arguments")
    return nnz.value, att.value


def dequant_e4m3(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """FP8 E4M3 KV pages to fp32 [CXT §3.3: KV kept in blocks, in reduced
    precision].  ``codes`` [n_pages, Hkv, ...] uint8 (OCP e4m3 bit patterns,
    no infinities), ``scale`` [n_pages, Hkv] fp32 -> fp32 of the shape of
    ``codes``: scale times the code's value, rounded once to fp32."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    n_pages, hkv = codes.shape[0], codes.shape[1]
    assert scale.shape == (n_pages, hkv)
    row = int(np.prod(codes.shape[2:])) if codes.ndim > 2 else 1
    out = np.empty(codes.shape, np.float32)
    rc = _load().oracle_dequant_e4m3(_ptr(codes), n_pages, hkv, row, _ptr(scale), _ptr(out))
    if rc:
        raise ValueError("oracle_dequant_e4m3: invalid arguments")
    return out
