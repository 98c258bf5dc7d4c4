"""Thin Python binding of ``libmsa.so`` (the C ABI in ``include/msa.h``).

Each function has the name of the C entry point it calls and only marshals
arguments: it checks devices, dtypes and contiguity, allocates outputs and
workspaces with torch when the caller does not pass them, and passes raw
device pointers plus torch's current HIP stream.  Every step of the path runs
in the library's HIP kernels.  If the library is not built, every call raises:
there is no other implementation behind these names.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmsa.so")
_lib = None

MSA_F32, MSA_BF16, MSA_FP8_E4M3 = 0, 1, 2
_STATUS = {0: "MSA_OK", -1: "MSA_ERR_INVALID_ARG", -2: "MSA_ERR_UNSUPPORTED",
           -3: "MSA_ERR_WORKSPACE", -4: "MSA_ERR_HIP"}

ENTRY_POINTS = (
    "msa_status_string", "msa_index_pool", "msa_index_topk",
    "msa_topk_decode_workspace_bytes", "msa_index_topk_decode",
    "msa_invert_workspace_bytes", "msa_invert_selection",
    "msa_prefill_workspace_bytes", "msa_sparse_gqa_prefill",
    "msa_decode_workspace_bytes", "msa_sparse_gqa_decode",
    "msa_decode_step_workspace_bytes", "msa_decode_step",
    "msa_index_pool_mean", "msa_index_topk_window", "msa_index_topk_decode_window",
    "msa_sparse_gqa_decode_paged", "msa_prefill_varlen_workspace_bytes",
    "msa_prefill_varlen", "msa_decode_step_noalloc_max_bytes", "msa_decode_step_noalloc",
    "msa_sparse_gqa_prefill_paged", "msa_decode_step_paged",
    "msa_topk_batch_workspace_bytes", "msa_index_topk_batch",
)


class MsaError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {status} ({_STATUS.get(status, '?')})")


def load():
    """Load ``libmsa.so`` (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m "
            "block_sparse_attention_index_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    sz = ctypes.c_size_t
    sig = {
        "msa_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "msa_index_pool": ([P, i32, i64, P, i32, i32, i64, i64, P, i64, P], ctypes.c_int),
        "msa_index_pool_mean": ([P, i32, i64, P, i32, i32, i64, i64, P, i64, P],
                                ctypes.c_int),
        "msa_index_topk": ([P, i64, i64, P, i64, i32, i32, i32, P, P], ctypes.c_int),
        "msa_index_topk_window": ([P, i64, i64, P, i64, i32, i32, i32, i32, P, P],
                                  ctypes.c_int),
        "msa_index_topk_decode_window": ([P, i32, P, P, i64, i32, i32, i32, i32, P, P, sz,
                                          P], ctypes.c_int),
        "msa_topk_decode_workspace_bytes": ([i32, i64, i32], sz),
        "msa_topk_batch_workspace_bytes": ([i64, i64, i32], sz),
        "msa_index_topk_batch": ([P, i64, P, P, P, i32, i64, i32, i32, i32, P, P, sz, P],
                                 i32),
        "msa_index_topk_decode": ([P, i32, P, P, i64, i32, i32, i32, P, P, sz, P],
                                  ctypes.c_int),
        "msa_invert_workspace_bytes": ([i64, i32, i64], sz),
        "msa_invert_selection": ([P, i64, i32, i64, P, P, P, P, sz, P], ctypes.c_int),
        "msa_prefill_workspace_bytes": ([i32, i64, i64, i32, i32, i32, i32], sz),
        "msa_sparse_gqa_prefill": ([P, P, P, i32, i64, i64, i64, i32, i32, i32, i32,
                                    P, i32, P, P, P, f32, P, P, P, sz, P],
                                   ctypes.c_int),
        "msa_sparse_gqa_prefill_paged": ([P, P, P, i64, P, i32, i64, i64, i32, i32, i32, i32,
                                          P, i32, P, P, P, f32, P, P, P, sz, P], ctypes.c_int),
        "msa_decode_workspace_bytes": ([i32, i32, i32, i32, i32], sz),
        "msa_sparse_gqa_decode": ([P, P, P, i32, i32, i64, P, i32, i32, i32, i32, P,
                                   i32, f32, P, P, P, sz, P], ctypes.c_int),
        "msa_sparse_gqa_decode_paged": ([P, P, P, i32, P, P, i64, P, i32, i32, P, i32, i32,
                                         i32, i32, P, i32, f32, P, P, P, sz, P], ctypes.c_int),
        "msa_prefill_varlen_workspace_bytes": ([i32, i32, P, P, i32, i32, i32, i32, i32], sz),
        "msa_prefill_varlen": ([P, P, P, P, P, i32, i32, P, P, i32, i32, i32, i32, i32, i32,
                                f32, P, P, P, P, sz, P], ctypes.c_int),
        "msa_decode_step_workspace_bytes": ([i32, i64, i32, i32, i32, i32], sz),
        "msa_decode_step": ([P, P, P, P, P, P, P, P, P, i32, i32, i64, i64, P, i32, i32,
                             i32, i32, i32, i32, f32, P, P, P, P, sz, P], ctypes.c_int),
        "msa_decode_step_paged": ([P, P, P, P, P, P, P, i64, P, i32, P, P, i32, i64, i64, P,
                                   i32, i32, i32, i32, i32, i32, f32, P, P, P, P, sz, P],
                                  ctypes.c_int),
        "msa_decode_step_noalloc_max_bytes": ([], sz),
        "msa_decode_step_noalloc": ([P, P, P, P, P, P, P, P, P, i32, i32, i64, i64, P, i32,
                                     i32, i32, i32, i32, i32, f32, P, P, P, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MsaError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _shape(t, want, name: str) -> None:
    """Raise ValueError unless ``t`` has ``len(want)`` dimensions matching
    ``want`` (None: any extent).  The C calls receive sizes, not shapes, so a
    tensor of another layout would be read as if it had the stated one."""
    got = tuple(t.shape)
    if len(got) != len(want) or any(w is not None and g != w for g, w in zip(got, want)):
        exp = tuple("*" if w is None else w for w in want)
        raise ValueError(f"{name} has shape {got}, expected {exp}")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ws(nbytes: int, like: torch.Tensor, ws):
    if ws is not None:
        _dev(ws, "ws", torch.uint8)
        return ws
    return torch.empty(max(1, nbytes), dtype=torch.uint8, device=like.device)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MSA_F32
    if t.dtype == torch.bfloat16:
        return MSA_BF16
    raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def status_string(status: int) -> str:
    return load().msa_status_string(status).decode()


# --------------------------------------------------------------------------
# Index branch
# --------------------------------------------------------------------------
def msa_index_pool(idx_k: torch.Tensor, block: int, kmax: torch.Tensor | None = None,
                   seq_len: torch.Tensor | None = None, blk_begin: int = 0,
                   blk_end: int | None = None, nb_max: int | None = None):
    """Block max-pool of index keys.  ``idx_k`` [L, d_idx] or [n_seq, L, d_idx]
    fp32 -> ``kmax`` [nb_max, d_idx] or [n_seq, nb_max, d_idx] fp32.
    ``blk_begin = -1`` re-pools each sequence's last block; ``-2`` folds only
    the newest token into it (decode append)."""
    _dev(idx_k, "idx_k", torch.float32)
    batched = idx_k.dim() == 3
    n_seq = idx_k.shape[0] if batched else 1
    L, d = idx_k.shape[-2], idx_k.shape[-1]
    nb = -(-L // block)
    nb_max = nb if nb_max is None else nb_max
    if kmax is None:
        shape = (n_seq, nb_max, d) if batched else (nb_max, d)
        kmax = torch.empty(shape, dtype=torch.float32, device=idx_k.device)
    _dev(kmax, "kmax", torch.float32)
    if seq_len is not None:
        _dev(seq_len, "seq_len", torch.int64)
    if blk_end is None:
        blk_end = nb
    st = load().msa_index_pool(_ptr(idx_k), n_seq, L, _ptr(seq_len), d, block,
                               blk_begin, blk_end, _ptr(kmax), nb_max, _stream(idx_k))
    _check("msa_index_pool", st)
    return kmax


def msa_index_pool_mean(idx_k: torch.Tensor, block: int, kmean: torch.Tensor | None = None,
                        seq_len: torch.Tensor | None = None, blk_begin: int = 0,
                        blk_end: int | None = None, nb_max: int | None = None):
    """Block mean-pool of index keys (ablation summary); arguments and shapes
    as :func:`msa_index_pool` (``blk_begin`` >= 0 or -1)."""
    _dev(idx_k, "idx_k", torch.float32)
    batched = idx_k.dim() == 3
    n_seq = idx_k.shape[0] if batched else 1
    L, d = idx_k.shape[-2], idx_k.shape[-1]
    nb = -(-L // block)
    nb_max = nb if nb_max is None else nb_max
    if kmean is None:
        shape = (n_seq, nb_max, d) if batched else (nb_max, d)
        kmean = torch.empty(shape, dtype=torch.float32, device=idx_k.device)
    _dev(kmean, "kmean", torch.float32)
    if seq_len is not None:
        _dev(seq_len, "seq_len", torch.int64)
    if blk_end is None:
        blk_end = nb
    st = load().msa_index_pool_mean(_ptr(idx_k), n_seq, L, _ptr(seq_len), d, block,
                                    blk_begin, blk_end, _ptr(kmean), nb_max, _stream(idx_k))
    _check("msa_index_pool_mean", st)
    return kmean


def msa_index_topk(idx_q: torch.Tensor, kmax: torch.Tensor, block: int, topk: int,
                   q_pos0: int = 0, sel: torch.Tensor | None = None):
    """Prefill causal top-K: ``idx_q`` [n_q, d_idx] at positions q_pos0 + i,
    ``kmax`` [nb, d_idx] -> ``sel`` [n_q, topk] int32 (ascending, -1 padded)."""
    _dev(idx_q, "idx_q", torch.float32)
    _dev(kmax, "kmax", torch.float32)
    n_q, d = idx_q.shape
    if sel is None:
        sel = torch.empty((n_q, topk), dtype=torch.int32, device=idx_q.device)
    _dev(sel, "sel", torch.int32)
    st = load().msa_index_topk(_ptr(idx_q), n_q, q_pos0, _ptr(kmax), kmax.shape[0],
                               d, block, topk, _ptr(sel), _stream(idx_q))
    _check("msa_index_topk", st)
    return sel


def msa_index_topk_window(idx_q: torch.Tensor, kmax: torch.Tensor, block: int, topk: int,
                          window: int, q_pos0: int = 0, sel: torch.Tensor | None = None):
    """Prefill top-K with a forced local window of ``window`` blocks ending at
    the own block; the other ``topk - window`` are chosen by score."""
    _dev(idx_q, "idx_q", torch.float32)
    _dev(kmax, "kmax", torch.float32)
    n_q, d = idx_q.shape
    if sel is None:
        sel = torch.empty((n_q, topk), dtype=torch.int32, device=idx_q.device)
    _dev(sel, "sel", torch.int32)
    st = load().msa_index_topk_window(_ptr(idx_q), n_q, q_pos0, _ptr(kmax), kmax.shape[0],
                                      d, block, topk, window, _ptr(sel), _stream(idx_q))
    _check("msa_index_topk_window", st)
    return sel


def msa_index_topk_decode(idx_q: torch.Tensor, seq_len: torch.Tensor,
                          kmax: torch.Tensor, block: int, topk: int,
                          sel: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Decode top-K: one query per sequence at position seq_len[s]-1.
    ``idx_q`` [n_seq, d_idx], ``kmax`` [n_seq, nb_max, d_idx] -> ``sel`` [n_seq, topk]."""
    _dev(idx_q, "idx_q", torch.float32)
    _dev(seq_len, "seq_len", torch.int64)
    _dev(kmax, "kmax", torch.float32)
    n_seq, d = idx_q.shape
    nb_max = kmax.shape[1]
    lib = load()
    ws = _ws(lib.msa_topk_decode_workspace_bytes(n_seq, nb_max, topk), idx_q, ws)
    if sel is None:
        sel = torch.empty((n_seq, topk), dtype=torch.int32, device=idx_q.device)
    _dev(sel, "sel", torch.int32)
    st = lib.msa_index_topk_decode(_ptr(idx_q), n_seq, _ptr(seq_len), _ptr(kmax),
                                   nb_max, d, block, topk, _ptr(sel), _ptr(ws),
                                   ws.numel(), _stream(idx_q))
    _check("msa_index_topk_decode", st)
    return sel


def msa_index_topk_decode_window(idx_q: torch.Tensor, seq_len: torch.Tensor,
                                 kmax: torch.Tensor, block: int, topk: int, window: int,
                                 sel: torch.Tensor | None = None,
                                 ws: torch.Tensor | None = None):
    """Decode top-K with the forced local window of
    :func:`msa_index_topk_window`."""
    _dev(idx_q, "idx_q", torch.float32)
    _dev(seq_len, "seq_len", torch.int64)
    _dev(kmax, "kmax", torch.float32)
    n_seq, d = idx_q.shape
    nb_max = kmax.shape[1]
    lib = load()
    ws = _ws(lib.msa_topk_decode_workspace_bytes(n_seq, nb_max, topk), idx_q, ws)
    if sel is None:
        sel = torch.empty((n_seq, topk), dtype=torch.int32, device=idx_q.device)
    _dev(sel, "sel", torch.int32)
    st = lib.msa_index_topk_decode_window(_ptr(idx_q), n_seq, _ptr(seq_len), _ptr(kmax),
                                          nb_max, d, block, topk, window, _ptr(sel),
                                          _ptr(ws), ws.numel(), _stream(idx_q))
    _check("msa_index_topk_decode_window", st)
    return sel


def msa_index_topk_batch(idx_q: torch.Tensor, q_seq: torch.Tensor, q_pos: torch.Tensor,
                         kmax: torch.Tensor, block: int, topk: int,
                         sel: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Top-K for a batch of queries of several sequences, each at its own
    position: ``idx_q`` [n_q, d_idx] fp32, ``q_seq`` [n_q] int32, ``q_pos``
    [n_q] int64, ``kmax`` [n_seq, nb_max, d_idx] -> ``sel`` [n_q, topk]."""
    _dev(idx_q, "idx_q", torch.float32)
    _dev(q_seq, "q_seq", torch.int32)
    _dev(q_pos, "q_pos", torch.int64)
    _dev(kmax, "kmax", torch.float32)
    n_q, d = idx_q.shape
    n_seq, nb_max = kmax.shape[0], kmax.shape[1]
    _shape(q_seq, (n_q,), "q_seq")
    _shape(q_pos, (n_q,), "q_pos")
    _shape(kmax, (n_seq, nb_max, d), "kmax")
    lib = load()
    ws = _ws(lib.msa_topk_batch_workspace_bytes(n_q, nb_max, topk), idx_q, ws)
    if sel is None:
        sel = torch.empty((n_q, topk), dtype=torch.int32, device=idx_q.device)
    _dev(sel, "sel", torch.int32)
    _shape(sel, (n_q, topk), "sel")
    st = lib.msa_index_topk_batch(_ptr(idx_q), n_q, _ptr(q_seq), _ptr(q_pos), _ptr(kmax),
                                  n_seq, nb_max, d, block, topk, _ptr(sel), _ptr(ws),
                                  ws.numel(), _stream(idx_q))
    _check("msa_index_topk_batch", st)
    return sel


def msa_invert_selection(sel: torch.Tensor, n_blocks: int, row_ptr=None, q_list=None,
                         slot=None, ws=None):
    """CSR of queries per block: returns ``(row_ptr [nb+1], q_list [n_q*K]
    (capacity; the first row_ptr[-1] entries are used), slot [n_q, K])``."""
    _dev(sel, "sel", torch.int32)
    n_q, topk = sel.shape
    dev = sel.device
    lib = load()
    ws = _ws(lib.msa_invert_workspace_bytes(n_q, topk, n_blocks), sel, ws)
    if row_ptr is None:
        row_ptr = torch.empty(n_blocks + 1, dtype=torch.int32, device=dev)
    if q_list is None:
        q_list = torch.empty(max(1, n_q * topk), dtype=torch.int32, device=dev)
    if slot is None:
        slot = torch.empty((n_q, topk), dtype=torch.int32, device=dev)
    for t, nm in ((row_ptr, "row_ptr"), (q_list, "q_list"), (slot, "slot")):
        _dev(t, nm, torch.int32)
    st = lib.msa_invert_selection(_ptr(sel), n_q, topk, n_blocks, _ptr(row_ptr),
                                  _ptr(q_list), _ptr(slot), _ptr(ws), ws.numel(),
                                  _stream(sel))
    _check("msa_invert_selection", st)
    return row_ptr, q_list, slot


# --------------------------------------------------------------------------
# Sparse branch
# --------------------------------------------------------------------------
def prefill_workspace_bytes(dtype: int, q_pos0: int, n_q: int, hq: int, d: int,
                            block: int, topk: int) -> int:
    return load().msa_prefill_workspace_bytes(dtype, q_pos0, n_q, hq, d, block, topk)


def msa_sparse_gqa_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           sel: torch.Tensor, row_ptr: torch.Tensor,
                           q_list: torch.Tensor, slot: torch.Tensor, block: int,
                           scale: float | None = None, q_pos0: int = 0,
                           o=None, lse=None, ws=None, want_lse: bool = True):
    """Sparse GQA prefill, KV outer.  ``q`` [n_q, Hq, d]; ``k``/``v``
    [Hkv, kv_stride, d] (fp32 or bf16); returns ``(o [n_q, Hq, d] fp32,
    lse [n_q, Hq] fp32 or None)``."""
    _shape(q, (None, None, None), "q")
    _shape(k, (None, None, q.shape[2]), "k")
    _shape(v, tuple(k.shape), "v")
    _shape(sel, (q.shape[0], None), "sel")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, nm)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    for t, nm in ((sel, "sel"), (row_ptr, "row_ptr"), (q_list, "q_list"),
                  (slot, "slot")):
        _dev(t, nm, torch.int32)
    n_q, hq, d = q.shape
    hkv, kv_stride, _ = k.shape
    topk = sel.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load()
    ws = _ws(lib.msa_prefill_workspace_bytes(_dtype_code(q), q_pos0, n_q, hq, d, block,
                                             topk), q, ws)
    if o is None:
        o = torch.empty((n_q, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((n_q, hq), dtype=torch.float32, device=q.device)
    _dev(o, "o", torch.float32)
    st = lib.msa_sparse_gqa_prefill(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), kv_stride, q_pos0, n_q, hq, hkv,
        d, block, _ptr(sel), topk, _ptr(row_ptr), _ptr(q_list), _ptr(slot), scale,
        _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(q))
    _check("msa_sparse_gqa_prefill", st)
    return o, lse


def msa_sparse_gqa_prefill_paged(q, k_pages, v_pages, block_table, sel, row_ptr, q_list, slot,
                                 block: int, scale: float | None = None, q_pos0: int = 0,
                                 o=None, lse=None, ws=None, want_lse: bool = True):
    """Sparse GQA prefill of a query chunk against a paged bf16 cache.
    ``q`` [n_q, Hq, d] bf16; ``k_pages``/``v_pages`` [n_pages, Hkv, B, d]
    bf16; ``block_table`` [max_blocks] int32.  Returns ``(o, lse)`` as
    msa_sparse_gqa_prefill."""
    _shape(q, (None, None, None), "q")
    _shape(k_pages, (None, None, block, q.shape[2]), "k_pages")
    _shape(v_pages, tuple(k_pages.shape), "v_pages")
    _shape(block_table, (None,), "block_table")
    _shape(sel, (q.shape[0], None), "sel")
    for t, nm in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _dev(t, nm, torch.bfloat16)
    for t, nm in ((block_table, "block_table"), (sel, "sel"), (row_ptr, "row_ptr"),
                  (q_list, "q_list"), (slot, "slot")):
        _dev(t, nm, torch.int32)
    n_q, hq, d = q.shape
    n_pages, hkv = k_pages.shape[0], k_pages.shape[1]
    topk = sel.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load()
    ws = _ws(lib.msa_prefill_workspace_bytes(MSA_BF16, q_pos0, n_q, hq, d, block, topk), q, ws)
    if o is None:
        o = torch.empty((n_q, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((n_q, hq), dtype=torch.float32, device=q.device)
    _dev(o, "o", torch.float32)
    st = lib.msa_sparse_gqa_prefill_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), n_pages, _ptr(block_table), block_table.numel(),
        q_pos0, n_q, hq, hkv, d, block, _ptr(sel), topk, _ptr(row_ptr), _ptr(q_list),
        _ptr(slot), scale, _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(q))
    _check("msa_sparse_gqa_prefill_paged", st)
    return o, lse


def decode_workspace_bytes(n_seq: int, hq: int, d: int, block: int, topk: int) -> int:
    return load().msa_decode_workspace_bytes(n_seq, hq, d, block, topk)


def msa_sparse_gqa_decode(q: torch.Tensor, k_cache: torch.Tensor,
                          v_cache: torch.Tensor, seq_len: torch.Tensor,
                          sel: torch.Tensor, block: int, scale: float | None = None,
                          o=None, lse=None, ws=None, want_lse: bool = True):
    """Sparse GQA decode.  ``q`` [n_seq, Hq, d]; caches [n_seq, Hkv, len_max, d];
    returns ``(o [n_seq, Hq, d] fp32, lse [n_seq, Hq] fp32 or None)``."""
    _shape(q, (None, None, None), "q")
    _shape(k_cache, (q.shape[0], None, None, q.shape[2]), "k_cache")
    _shape(v_cache, tuple(k_cache.shape), "v_cache")
    _shape(sel, (q.shape[0], None), "sel")
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, nm)
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q and the caches must share a dtype")
    _dev(seq_len, "seq_len", torch.int64)
    _dev(sel, "sel", torch.int32)
    n_seq, hq, d = q.shape
    _, hkv, len_max, _ = k_cache.shape
    topk = sel.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load()
    ws = _ws(lib.msa_decode_workspace_bytes(n_seq, hq, d, block, topk), q, ws)
    if o is None:
        o = torch.empty((n_seq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((n_seq, hq), dtype=torch.float32, device=q.device)
    st = lib.msa_sparse_gqa_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(q), n_seq, len_max,
        _ptr(seq_len), hq, hkv, d, block, _ptr(sel), topk, scale, _ptr(o), _ptr(lse),
        _ptr(ws), ws.numel(), _stream(q))
    _check("msa_sparse_gqa_decode", st)
    return o, lse



def msa_prefill_varlen(q, k, v, idx_q, idx_k, cu_q, cu_kv, block: int, topk: int,
                       scale: float | None = None, sel=None, o=None, lse=None, ws=None,
                       want_lse: bool = True):
    """Prefill of several sequences in one call.  ``q`` [Nq, Hq, d], ``idx_q``
    [Nq, d_idx] packed by ``cu_q``; ``k``/``v`` [Hkv, Nkv, d], ``idx_k``
    [Nkv, d_idx] packed by ``cu_kv`` (host integer sequences of n_seq + 1
    offsets); each sequence's queries are its last tokens.  Returns
    ``(o, lse, sel)``."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, nm)
    _dev(idx_q, "idx_q", torch.float32)
    _dev(idx_k, "idx_k", torch.float32)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share a dtype")
    code = _dtype_code(q)
    nq, hq, d = q.shape
    hkv = k.shape[0]
    cq = (ctypes.c_int64 * len(cu_q))(*[int(x) for x in cu_q])
    ckv = (ctypes.c_int64 * len(cu_kv))(*[int(x) for x in cu_kv])
    n_seq = len(cu_q) - 1
    if len(cu_kv) != n_seq + 1:
        raise ValueError("cu_q and cu_kv must have the same length")
    scale = d ** -0.5 if scale is None else scale
    lib = load()
    ws = _ws(lib.msa_prefill_varlen_workspace_bytes(code, n_seq, cq, ckv, hq, d,
                                                    idx_q.shape[1], block, topk), q, ws)
    if sel is None:
        sel = torch.empty((nq, topk), dtype=torch.int32, device=q.device)
    if o is None:
        o = torch.empty((nq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((nq, hq), dtype=torch.float32, device=q.device)
    st = lib.msa_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(idx_q), _ptr(idx_k), code,
                                n_seq, cq, ckv, hq, hkv, d, idx_q.shape[1], block, topk, scale,
                                _ptr(sel), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(q))
    _check("msa_prefill_varlen", st)
    return o, lse, sel


def msa_sparse_gqa_decode_paged(q, k_pages, v_pages, block_table, seq_len, sel, block: int,
                                scale: float | None = None, k_scale=None, v_scale=None,
                                o=None, lse=None, ws=None, want_lse: bool = True):
    """Sparse GQA decode over a paged cache.  ``q`` [n_seq, Hq, d] bf16;
    ``k_pages``/``v_pages`` [n_pages, Hkv, B, d] bf16 or float8_e4m3fn (then
    ``k_scale``/``v_scale`` [n_pages, Hkv] fp32); ``block_table``
    [n_seq, max_blocks] int32.  Returns ``(o, lse)`` as msa_sparse_gqa_decode."""
    _shape(q, (None, None, None), "q")
    _shape(k_pages, (None, None, block, q.shape[2]), "k_pages")
    _shape(v_pages, tuple(k_pages.shape), "v_pages")
    _shape(block_table, (q.shape[0], None), "block_table")
    _shape(sel, (q.shape[0], None), "sel")
    for t, nm in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _dev(t, nm)
    _dev(block_table, "block_table", torch.int32)
    _dev(seq_len, "seq_len", torch.int64)
    _dev(sel, "sel", torch.int32)
    if q.dtype != torch.bfloat16:
        raise ValueError("q must be bf16")
    if k_pages.dtype != v_pages.dtype:
        raise ValueError("k_pages and v_pages must share a dtype")
    if k_pages.dtype == torch.bfloat16:
        kvd = MSA_BF16
    elif k_pages.dtype == torch.float8_e4m3fn:
        kvd = MSA_FP8_E4M3
        _dev(k_scale, "k_scale", torch.float32)
        _dev(v_scale, "v_scale", torch.float32)
    else:
        raise ValueError("pages must be bf16 or float8_e4m3fn")
    n_seq, hq, d = q.shape
    n_pages, hkv = k_pages.shape[0], k_pages.shape[1]
    topk = sel.shape[1]
    scale = d ** -0.5 if scale is None else scale
    lib = load()
    ws = _ws(lib.msa_decode_workspace_bytes(n_seq, hq, d, block, topk), q, ws)
    if o is None:
        o = torch.empty((n_seq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((n_seq, hq), dtype=torch.float32, device=q.device)
    st = lib.msa_sparse_gqa_decode_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), kvd, _ptr(k_scale if kvd == MSA_FP8_E4M3 else None),
        _ptr(v_scale if kvd == MSA_FP8_E4M3 else None), n_pages, _ptr(block_table),
        block_table.shape[1], n_seq, _ptr(seq_len), hq, hkv, d, block, _ptr(sel), topk,
        scale, _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(q))
    _check("msa_sparse_gqa_decode_paged", st)
    return o, lse

def _step_shapes(q, k_new, v_new, idx_q, idx_k_new, kmax) -> None:
    """The shapes every fused-step binding shares: q [n_seq, Hq, d], the new
    rows [n_seq, Hkv, d], idx_q / idx_k_new [n_seq, d_idx], kmax [n_seq,
    nb_max, d_idx]."""
    _shape(q, (None, None, None), "q")
    n_seq, d = q.shape[0], q.shape[2]
    _shape(k_new, (n_seq, None, d), "k_new")
    _shape(v_new, tuple(k_new.shape), "v_new")
    _shape(idx_q, (n_seq, None), "idx_q")
    _shape(idx_k_new, tuple(idx_q.shape), "idx_k_new")
    _shape(kmax, (n_seq, None, idx_q.shape[1]), "kmax")


def msa_decode_step(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                    idx_q: torch.Tensor, idx_k_new: torch.Tensor, k_cache: torch.Tensor,
                    v_cache: torch.Tensor, kmax: torch.Tensor, seq_len: torch.Tensor,
                    block: int, topk: int, scale: float | None = None,
                    idx_k_cache: torch.Tensor | None = None, sel=None, o=None, lse=None,
                    ws=None, want_lse: bool = True):
    """Fused decode step: append the new token at ``seq_len[s]`` (K/V, index
    key), update its block's running max, select and attend.  ``q`` [n_seq,
    Hq, d]; ``k_new``/``v_new`` [n_seq, Hkv, d]; ``idx_q``/``idx_k_new``
    [n_seq, d_idx]; caches [n_seq, Hkv, len_max, d]; ``kmax`` [n_seq, nb_max,
    d_idx].  ``seq_len`` is not advanced.  Returns ``(o, lse, sel)``."""
    _step_shapes(q, k_new, v_new, idx_q, idx_k_new, kmax)
    _shape(k_cache, (q.shape[0], k_new.shape[1], None, q.shape[2]), "k_cache")
    _shape(v_cache, tuple(k_cache.shape), "v_cache")
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                  (v_cache, "v_cache")):
        _dev(t, nm)
    if not (q.dtype == k_new.dtype == v_new.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, the new rows and the caches must share a dtype")
    for t, nm in ((idx_q, "idx_q"), (idx_k_new, "idx_k_new"), (kmax, "kmax")):
        _dev(t, nm, torch.float32)
    if idx_k_cache is not None:
        _dev(idx_k_cache, "idx_k_cache", torch.float32)
    _dev(seq_len, "seq_len", torch.int64)
    n_seq, hq, d = q.shape
    _, hkv, len_max, _ = k_cache.shape
    nb_max, d_idx = kmax.shape[1], kmax.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load()
    ws = _ws(lib.msa_decode_step_workspace_bytes(n_seq, nb_max, hq, d, block, topk), q, ws)
    if sel is None:
        sel = torch.empty((n_seq, topk), dtype=torch.int32, device=q.device)
    if o is None:
        o = torch.empty((n_seq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((n_seq, hq), dtype=torch.float32, device=q.device)
    st = lib.msa_decode_step(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(idx_q), _ptr(idx_k_new), _ptr(k_cache),
        _ptr(v_cache), _ptr(idx_k_cache), _ptr(kmax), _dtype_code(q), n_seq, len_max, nb_max,
        _ptr(seq_len), hq, hkv, d, d_idx, block, topk, scale, _ptr(sel), _ptr(o), _ptr(lse),
        _ptr(ws), ws.numel(), _stream(q))
    _check("msa_decode_step", st)
    return o, lse, sel


def msa_decode_step_paged(q, k_new, v_new, idx_q, idx_k_new, k_pages, v_pages, block_table,
                          kmax, seq_len, block: int, topk: int, len_max: int,
                          scale: float | None = None, idx_k_cache=None, sel=None, o=None,
                          lse=None, ws=None, want_lse: bool = True):
    """Fused decode step over a paged bf16 cache: ``k_pages``/``v_pages``
    [n_pages, Hkv, B, d]; ``block_table`` [n_seq, max_blocks] int32; the new
    token's rows go to row ``L % B`` of page ``block_table[s][L // B]``.
    ``len_max`` bounds L (and is the row capacity of ``idx_k_cache`` [n_seq,
    len_max, d_idx] when given).  Otherwise as :func:`msa_decode_step`."""
    _step_shapes(q, k_new, v_new, idx_q, idx_k_new, kmax)
    _shape(k_pages, (None, k_new.shape[1], block, q.shape[2]), "k_pages")
    _shape(v_pages, tuple(k_pages.shape), "v_pages")
    _shape(block_table, (q.shape[0], None), "block_table")
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_pages, "k_pages"),
                  (v_pages, "v_pages")):
        _dev(t, nm, torch.bfloat16)
    for t, nm in ((idx_q, "idx_q"), (idx_k_new, "idx_k_new"), (kmax, "kmax")):
        _dev(t, nm, torch.float32)
    if idx_k_cache is not None:
        _dev(idx_k_cache, "idx_k_cache", torch.float32)
    _dev(block_table, "block_table", torch.int32)
    _dev(seq_len, "seq_len", torch.int64)
    n_seq, hq, d = q.shape
    n_pages, hkv = k_pages.shape[0], k_pages.shape[1]
    nb_max, d_idx = kmax.shape[1], kmax.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = load()
    ws = _ws(lib.msa_decode_step_workspace_bytes(n_seq, nb_max, hq, d, block, topk), q, ws)
    if sel is None:
        sel = torch.empty((n_seq, topk), dtype=torch.int32, device=q.device)
    if o is None:
        o = torch.empty((n_seq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((n_seq, hq), dtype=torch.float32, device=q.device)
    st = lib.msa_decode_step_paged(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(idx_q), _ptr(idx_k_new), _ptr(k_pages),
        _ptr(v_pages), n_pages, _ptr(block_table), block_table.shape[1], _ptr(idx_k_cache),
        _ptr(kmax), n_seq, len_max, nb_max, _ptr(seq_len), hq, hkv, d, d_idx, block, topk,
        scale, _ptr(sel), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(q))
    _check("msa_decode_step_paged", st)
    return o, lse, sel


def msa_decode_step_noalloc(q, k_new, v_new, idx_q, idx_k_new, k_cache, v_cache, kmax,
                            seq_len, block: int, topk: int, scale: float | None = None,
                            idx_k_cache=None, sel=None, o=None, lse=None,
                            want_lse: bool = True):
    """:func:`msa_decode_step` on the library's static scratch (no workspace
    argument; the C call allocates nothing).  Outputs not passed in are
    allocated here by torch; pass them to keep the whole call allocation-free."""
    _step_shapes(q, k_new, v_new, idx_q, idx_k_new, kmax)
    _shape(k_cache, (q.shape[0], k_new.shape[1], None, q.shape[2]), "k_cache")
    _shape(v_cache, tuple(k_cache.shape), "v_cache")
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                  (v_cache, "v_cache")):
        _dev(t, nm)
    if not (q.dtype == k_new.dtype == v_new.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, the new rows and the caches must share a dtype")
    for t, nm in ((idx_q, "idx_q"), (idx_k_new, "idx_k_new"), (kmax, "kmax")):
        _dev(t, nm, torch.float32)
    if idx_k_cache is not None:
        _dev(idx_k_cache, "idx_k_cache", torch.float32)
    _dev(seq_len, "seq_len", torch.int64)
    n_seq, hq, d = q.shape
    _, hkv, len_max, _ = k_cache.shape
    nb_max, d_idx = kmax.shape[1], kmax.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if sel is None:
        sel = torch.empty((n_seq, topk), dtype=torch.int32, device=q.device)
    if o is None:
        o = torch.empty((n_seq, hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((n_seq, hq), dtype=torch.float32, device=q.device)
    st = load().msa_decode_step_noalloc(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(idx_q), _ptr(idx_k_new), _ptr(k_cache),
        _ptr(v_cache), _ptr(idx_k_cache), _ptr(kmax), _dtype_code(q), n_seq, len_max, nb_max,
        _ptr(seq_len), hq, hkv, d, d_idx, block, topk, scale, _ptr(sel), _ptr(o), _ptr(lse),
        _stream(q))
    _check("msa_decode_step_noalloc", st)
    return o, lse, sel

