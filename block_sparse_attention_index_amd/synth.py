"""Seeded synthetic inputs for the MSA index and sparse branches.

This module only draws random tensors; it holds none of the method's
arithmetic.  Both the HIP path and the CPU oracle consume the same buffers
(the oracle gets host copies), so it is the one module the two sides share.

Recipe (all configurations): values are fp32 N(0, 1); bf16 tensors are the
round-to-nearest-even bf16 of the same fp32 draws.  Planted structure, so that
the top-K is not trivial: a shared unit vector ``u`` (a normalised N(0, I)
draw); ``n_hot`` blocks chosen uniformly without replacement get ``+2u`` added
to every index key they hold; every index query independently gets ``+2u``
with probability 1/2.  Every tensor (and every chunk of a large one) is drawn
from its own generator, seeded from ``(seed, tensor id, chunk)``, so a tensor
does not depend on what was drawn before it and any device reproduces the
same structure.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

# Tensor ids for seeding: adding a tensor never changes the others.
_TID = {"q": 1, "k": 2, "v": 3, "idx_q": 4, "idx_k": 5, "u": 6, "hot": 7,
        "bern": 8}


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload.  ``T`` is the prefill length; decode configurations set
    ``n_seq`` sequences of ``T`` cached tokens each and ``n_dec`` steps."""
    name: str
    T: int
    dtype: str          # "f32" or "bf16": q, k, v precision
    Hq: int
    Hkv: int
    d: int
    d_idx: int
    block: int
    topk: int
    n_hot: int = 0
    n_seq: int = 1
    n_dec: int = 0      # decode steps after the prefill (one new token each)
    mode: str = "prefill"   # "prefill" or "decode"

    @property
    def nb(self) -> int:
        return -(-self.T // self.block)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # 1 sequence, 4096 tokens, fp32, 8/2 heads, d 64, B 64, K 4, no planting.
    "tiny": Config("tiny", 4096, "f32", 8, 2, 64, 64, 64, 4, 0),
    # 32768 tokens, bf16, 64/8 heads, d 128, B 64 (512 blocks), K 16, 32 hot.
    "p32k": Config("p32k", 32768, "bf16", 64, 8, 128, 128, 64, 16, 32),
    # 131072 tokens, B 128 (1024 blocks), K 16, 64 hot.
    "p128k": Config("p128k", 131072, "bf16", 64, 8, 128, 128, 128, 16, 64),
    # 16 sequences x 262144 cached tokens, B 512, K 8, 16 hot per sequence.
    "dec16": Config("dec16", 262144, "bf16", 64, 8, 128, 128, 512, 8, 16,
                    n_seq=16, mode="decode"),
    # 1048576-token prefill (2048 blocks of 512, K 8, 128 hot) + 256 decode steps.
    "p1m": Config("p1m", 1 << 20, "bf16", 64, 8, 128, 128, 512, 8, 128,
                  n_dec=256),
}


def _seed(seed: int, tensor: str, chunk: int = 0, sub: int = 0) -> int:
    ss = np.random.SeedSequence([int(seed), _TID[tensor], int(chunk), int(sub)])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(device, seed: int, tensor: str, chunk: int = 0, sub: int = 0):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, tensor, chunk, sub))
    return g


def _normal_rows(shape, dtype, device, seed, tensor, sub=0,
                 chunk_elems: int = 1 << 28):
    """N(0,1) tensor of ``shape``, drawn in row chunks of at most
    ``chunk_elems`` fp32 values (bounded temporary memory)."""
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    per_row = max(1, int(np.prod(shape[1:])))
    step = max(1, chunk_elems // per_row)
    for ci, r0 in enumerate(range(0, rows, step)):
        r1 = min(rows, r0 + step)
        g = _gen(device, seed, tensor, ci, sub)
        x = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g,
                        dtype=torch.float32, device=device)
        out[r0:r1].copy_(x)          # fp32 -> bf16 is round-to-nearest-even
        del x
    return out


def _unit(d_idx, device, seed):
    g = _gen(device, seed, "u")
    u = torch.randn(d_idx, generator=g, dtype=torch.float32, device=device)
    return u / torch.linalg.vector_norm(u)


def _hot_blocks(nb, n_hot, device, seed, sub=0):
    if n_hot <= 0:
        return torch.empty(0, dtype=torch.int64, device=device)
    g = _gen("cpu", seed, "hot", 0, sub)
    return torch.randperm(nb, generator=g)[:n_hot].to(device)


def _plant_keys(idx_k, hot, block, u):
    """idx_k [L, d_idx]: add 2u to every token of each hot block."""
    L = idx_k.shape[0]
    for b in hot.tolist():
        idx_k[b * block:min(L, (b + 1) * block)] += 2.0 * u


def _plant_queries(idx_q, u, device, seed, sub=0):
    g = _gen(device, seed, "bern", 0, sub)
    hit = torch.rand(idx_q.shape[0], generator=g, device=device) < 0.5
    idx_q += hit.to(torch.float32)[:, None] * (2.0 * u)[None, :]


def sequence_inputs(cfg: Config, device="cpu", seed: int = 0,
                    length: int | None = None):
    """One sequence of ``length`` tokens (default ``cfg.T + cfg.n_dec``).

    Returns a dict: ``q`` [L, Hq, d], ``k``/``v`` [Hkv, L, d] (cfg dtype),
    ``idx_q``/``idx_k`` [L, d_idx] fp32, ``hot`` (planted block ids).
    Hot blocks are drawn among the first ``cfg.T`` tokens' blocks.
    """
    L = cfg.T + cfg.n_dec if length is None else int(length)
    dt = cfg.torch_dtype
    out = {
        "q": _normal_rows((L, cfg.Hq, cfg.d), dt, device, seed, "q"),
        "k": torch.stack([_normal_rows((L, cfg.d), dt, device, seed, "k", h)
                          for h in range(cfg.Hkv)]),
        "v": torch.stack([_normal_rows((L, cfg.d), dt, device, seed, "v", h)
                          for h in range(cfg.Hkv)]),
        "idx_q": _normal_rows((L, cfg.d_idx), torch.float32, device, seed,
                              "idx_q"),
        "idx_k": _normal_rows((L, cfg.d_idx), torch.float32, device, seed,
                              "idx_k"),
    }
    hot = _hot_blocks(-(-min(L, cfg.T) // cfg.block), cfg.n_hot, device, seed)
    if cfg.n_hot > 0:
        u = _unit(cfg.d_idx, device, seed)
        _plant_keys(out["idx_k"], hot, cfg.block, u)
        _plant_queries(out["idx_q"], u, device, seed)
    out["hot"] = hot
    return out


def decode_inputs(cfg: Config, device="cpu", seed: int = 0):
    """Batched decode: ``n_seq`` caches of ``cfg.T`` tokens, one new query each.

    Returns ``k_cache``/``v_cache`` [n_seq, Hkv, T, d], ``idx_k``
    [n_seq, T, d_idx], ``q`` [n_seq, Hq, d], ``idx_q`` [n_seq, d_idx],
    ``seq_len`` [n_seq] int64 (all ``T``; the query sits at position T-1 and its
    own key, value and index key are already in the cache).
    """
    n, L, dt = cfg.n_seq, cfg.T, cfg.torch_dtype
    k = torch.empty((n, cfg.Hkv, L, cfg.d), dtype=dt, device=device)
    v = torch.empty_like(k)
    idx_k = torch.empty((n, L, cfg.d_idx), dtype=torch.float32, device=device)
    u = _unit(cfg.d_idx, device, seed) if cfg.n_hot > 0 else None
    for s in range(n):
        for h in range(cfg.Hkv):
            k[s, h] = _normal_rows((L, cfg.d), dt, device, seed, "k",
                                   s * cfg.Hkv + h)
            v[s, h] = _normal_rows((L, cfg.d), dt, device, seed, "v",
                                   s * cfg.Hkv + h)
        idx_k[s] = _normal_rows((L, cfg.d_idx), torch.float32, device, seed,
                                "idx_k", s)
        if u is not None:
            _plant_keys(idx_k[s], _hot_blocks(cfg.nb, cfg.n_hot, device, seed,
                                              s), cfg.block, u)
    q = _normal_rows((n, cfg.Hq, cfg.d), dt, device, seed, "q")
    idx_q = _normal_rows((n, cfg.d_idx), torch.float32, device, seed, "idx_q")
    if u is not None:
        _plant_queries(idx_q, u, device, seed)
    seq_len = torch.full((n,), L, dtype=torch.int64, device=device)
    return {"k_cache": k, "v_cache": v, "idx_k": idx_k, "q": q,
            "idx_q": idx_q, "seq_len": seq_len}


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 view of a bf16 tensor (the oracle's bf16 input format)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy in the oracle's input format (fp32, or bf16 bits)."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().cpu().contiguous().numpy()
