"""Whole-path drivers: chain the C-ABI entry points for one prefill or one
decode step.  They only order calls and size buffers; all arithmetic runs in
the library's kernels.

Prefill ([CXT] section 3.3: every query scores every earlier block): pool the
index keys, select per query, then build the CSR and run the sparse GQA --
over all queries at once when the partial outputs of the KV-outer pass fit in
free HBM (so each KV block is read by one pass), else per chunk of queries.  Decode (same section: only the new query is scored): re-pool the
block that holds each sequence's newest token, select for the new query, and
attend over the selected blocks.

[CXT] = "MiniMax M3 深度实战：当稀疏注意力打破百万 Token 墙 ..."
(chenxutan.com/d/3746.html).
"""
from __future__ import annotations

import dataclasses
import math

import torch

from . import ops


@dataclasses.dataclass
class PrefillBuffers:
    """Device buffers for a chunked prefill (reusable across calls)."""
    kmax: torch.Tensor
    sel: torch.Tensor
    row_ptr: torch.Tensor
    q_list: torch.Tensor
    slot: torch.Tensor
    inv_ws: torch.Tensor
    attn_ws: torch.Tensor
    o: torch.Tensor
    lse: torch.Tensor
    chunk: int


def default_chunk(dtype: int, T: int, hq: int, d: int, block: int, topk: int,
                  budget_bytes: int) -> int:
    """Largest power-of-two query chunk (>= one block) whose prefill
    workspace fits ``budget_bytes``; the whole sequence when it fits."""
    c = 1 << max(0, (T - 1).bit_length())
    while c > block and ops.prefill_workspace_bytes(dtype, T - c if T > c else 0, min(c, T),
                                                     hq, d, block, topk) > budget_bytes:
        c //= 2
    return max(min(c, T), 1)


def alloc_prefill(q, idx_q, block: int, topk: int, chunk: int | None = None,
                  budget_bytes: int | None = None, headroom_bytes: int = 8 << 30) -> PrefillBuffers:
    """Buffers for :func:`prefill`.  With no ``chunk`` and no
    ``budget_bytes``, the partial-record workspace may take the device memory
    that is free once the outputs are allocated, less ``headroom_bytes``: one
    chunk covers the whole sequence whenever it fits (each KV block is then
    streamed by a single pass over all queries), and long sequences fall back
    to query chunks, which re-stream the blocks before each chunk."""
    T, hq, d = q.shape
    dev = q.device
    nb = -(-T // block)
    code = ops._dtype_code(q)
    if chunk is None:
        if budget_bytes is None:
            free, _ = torch.cuda.mem_get_info(dev)
            outputs = T * hq * (d + 1) * 4 + T * topk * 4 * 3 + nb * idx_q.shape[1] * 4
            budget_bytes = max(1 << 30, free - outputs - headroom_bytes)
        chunk = default_chunk(code, T, hq, d, block, topk, budget_bytes)
    lib = ops.load()
    # the largest workspace is the last chunk's (most non-own pairs)
    ws_attn = max(lib.msa_prefill_workspace_bytes(code, c0, min(chunk, T - c0), hq, d, block,
                                                  topk)
                  for c0 in range(0, T, chunk))
    ws_inv = lib.msa_invert_workspace_bytes(chunk, topk, nb)
    return PrefillBuffers(
        kmax=torch.empty((nb, idx_q.shape[1]), dtype=torch.float32, device=dev),
        sel=torch.empty((T, topk), dtype=torch.int32, device=dev),
        row_ptr=torch.empty(nb + 1, dtype=torch.int32, device=dev),
        q_list=torch.empty(chunk * topk, dtype=torch.int32, device=dev),
        slot=torch.empty((chunk, topk), dtype=torch.int32, device=dev),
        inv_ws=torch.empty(max(1, ws_inv), dtype=torch.uint8, device=dev),
        attn_ws=torch.empty(max(1, ws_attn), dtype=torch.uint8, device=dev),
        o=torch.empty((T, hq, d), dtype=torch.float32, device=dev),
        lse=torch.empty((T, hq), dtype=torch.float32, device=dev),
        chunk=chunk)


def prefill(q, k, v, idx_q, idx_k, block: int, topk: int, scale: float | None = None,
            bufs: PrefillBuffers | None = None):
    """Full causal MSA prefill of one sequence.

    ``q`` [T, Hq, d]; ``k``/``v`` [Hkv, kv_stride >= T, d]; ``idx_q`` [T, d_idx];
    ``idx_k`` [>= T, d_idx].  Returns ``(o [T, Hq, d], lse [T, Hq], sel [T, K])``.
    """
    T, hq, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    bufs = bufs or alloc_prefill(q, idx_q, block, topk)
    nb = -(-T // block)
    ops.msa_index_pool(idx_k[:T], block, kmax=bufs.kmax)
    ops.msa_index_topk(idx_q[:T], bufs.kmax, block, topk, sel=bufs.sel)
    for c0 in range(0, T, bufs.chunk):
        c1 = min(T, c0 + bufs.chunk)
        nbc = -(-c1 // block)
        n = c1 - c0
        ops.msa_invert_selection(bufs.sel[c0:c1], nbc, row_ptr=bufs.row_ptr[:nbc + 1],
                                 q_list=bufs.q_list[:n * topk], slot=bufs.slot[:n],
                                 ws=bufs.inv_ws)
        ops.msa_sparse_gqa_prefill(q[c0:c1], k, v, bufs.sel[c0:c1], bufs.row_ptr[:nbc + 1],
                                   bufs.q_list[:n * topk], bufs.slot[:n], block, scale,
                                   q_pos0=c0, o=bufs.o[c0:c1], lse=bufs.lse[c0:c1],
                                   ws=bufs.attn_ws)
    assert nb >= 1
    return bufs.o, bufs.lse, bufs.sel


@dataclasses.dataclass
class DecodeBuffers:
    sel: torch.Tensor
    topk_ws: torch.Tensor
    attn_ws: torch.Tensor
    o: torch.Tensor
    lse: torch.Tensor


def alloc_decode(q, kmax, block: int, topk: int) -> DecodeBuffers:
    n_seq, hq, d = q.shape
    dev = q.device
    lib = ops.load()
    return DecodeBuffers(
        sel=torch.empty((n_seq, topk), dtype=torch.int32, device=dev),
        topk_ws=torch.empty(max(1, lib.msa_topk_decode_workspace_bytes(
            n_seq, kmax.shape[1], topk)), dtype=torch.uint8, device=dev),
        attn_ws=torch.empty(max(1, lib.msa_decode_workspace_bytes(
            n_seq, hq, d, block, topk)), dtype=torch.uint8, device=dev),
        o=torch.empty((n_seq, hq, d), dtype=torch.float32, device=dev),
        lse=torch.empty((n_seq, hq), dtype=torch.float32, device=dev))


def decode_step(q, idx_q, k_cache, v_cache, idx_k, kmax, seq_len, block: int,
                topk: int, scale: float | None = None, bufs: DecodeBuffers | None = None):
    """One decode step for ``n_seq`` sequences whose newest token (position
    seq_len[s]-1, already in the caches) is the query.

    ``q`` [n_seq, Hq, d]; ``idx_q`` [n_seq, d_idx]; caches [n_seq, Hkv, len_max, d];
    ``idx_k`` [n_seq, len_max, d_idx]; ``kmax`` [n_seq, nb_max, d_idx] (updated in
    place: the newest token is folded into its block's running max, which
    assumes the previous token was already pooled).  Returns ``(o, lse, sel)``.
    """
    d = q.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    bufs = bufs or alloc_decode(q, kmax, block, topk)
    ops.msa_index_pool(idx_k, block, kmax=kmax, seq_len=seq_len, blk_begin=-2,
                       nb_max=kmax.shape[1])
    ops.msa_index_topk_decode(idx_q, seq_len, kmax, block, topk, sel=bufs.sel,
                              ws=bufs.topk_ws)
    ops.msa_sparse_gqa_decode(q, k_cache, v_cache, seq_len, bufs.sel, block, scale,
                              o=bufs.o, lse=bufs.lse, ws=bufs.attn_ws)
    return bufs.o, bufs.lse, bufs.sel


@dataclasses.dataclass
class DecodeStepBuffers:
    sel: torch.Tensor
    o: torch.Tensor
    lse: torch.Tensor
    ws: torch.Tensor


def alloc_decode_step(q, kmax, block: int, topk: int) -> DecodeStepBuffers:
    n_seq, hq, d = q.shape
    dev = q.device
    lib = ops.load()
    return DecodeStepBuffers(
        sel=torch.empty((n_seq, topk), dtype=torch.int32, device=dev),
        o=torch.empty((n_seq, hq, d), dtype=torch.float32, device=dev),
        lse=torch.empty((n_seq, hq), dtype=torch.float32, device=dev),
        ws=torch.empty(max(1, lib.msa_decode_step_workspace_bytes(
            n_seq, kmax.shape[1], hq, d, block, topk)), dtype=torch.uint8, device=dev))


def decode_append_step(q, k_new, v_new, idx_q, idx_k_new, k_cache, v_cache, kmax, seq_len,
                       block: int, topk: int, scale: float | None = None, idx_k_cache=None,
                       bufs: DecodeStepBuffers | None = None):
    """One generation step with the fused entry point: the new token (K/V rows
    ``k_new``/``v_new`` [n_seq, Hkv, d], index key ``idx_k_new``) is appended
    at position ``seq_len[s]`` (not advanced here), its block's running max
    updated, and its query (``q``, ``idx_q``) selects and attends.  Returns
    ``(o, lse, sel)``; no allocation when ``bufs`` is given."""
    bufs = bufs or alloc_decode_step(q, kmax, block, topk)
    return ops.msa_decode_step(q, k_new, v_new, idx_q, idx_k_new, k_cache, v_cache, kmax,
                               seq_len, block, topk, scale, idx_k_cache=idx_k_cache,
                               sel=bufs.sel, o=bufs.o, lse=bufs.lse, ws=bufs.ws)
