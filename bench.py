"""Benchmark: the MSA hot path at 1M-token context on one MI355X.

One step = the whole path over one synthetic sequence: the causal prefill of
1,048,576 tokens (index-key max-pool, q.blockmax top-K, CSR inversion, sparse
GQA with the KV-outer pass and the log-sum-exp merge) followed by 256
sequential decode steps against the 1M-token cache (re-pool of the newest
block, top-K of the new query, split-KV sparse attention, merge).

Inputs are generated on the device before timing (seeded N(0,1), bf16 q/k/v,
fp32 index vectors, 128 planted hot blocks) and stay resident in HBM.

Printed (rank 0, one JSON line): ``value`` = attended TFLOP/s of the whole
step (4*d*Hq FLOP per attended (query, key) pair, prefill and decode);
``prefill_tflops`` and ``decode_us_per_step`` break it down (the 256 decode
steps run as one captured HIP graph, replayed each step); ``roofline`` is
for the sparse-GQA prefill (its two kernels per call, timed with HIP events on
the launch stream) against the dense bf16 MFMA peak; ``cpu_baseline`` times
the CPU oracle on the same step (index branch and decode steps in full, the
prefill attention on a stratified sample extrapolated by attended pairs);
``selection_vs_oracle`` counts the near-ties and differing rows of the
device's selection of all queries against the oracle's.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_sparse_attention_index_amd import ops, pipeline, synth  # noqa: E402

PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "sparse_gqa_prefill_p1m_traffic.md")
KERNEL_SOURCES = ("prefill_mfma.hip", "prefill_common.h", "mfma_common.h", "seqtab.h")

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (vector / MFMA)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def attended_pairs(q_pos0: int, n_q: int, block: int, topk: int) -> int:
    """Sum over queries of the keys each attends (every non-own selected
    block is full): (min(K, own+1) - 1) * B + (p mod B) + 1."""
    p = np.arange(q_pos0, q_pos0 + n_q, dtype=np.int64)
    keff = np.minimum(topk, p // block + 1)
    return int(((keff - 1) * block + p % block + 1).sum())


def index_work(T: int, cfg, n_calls: int) -> dict:
    """Algorithmic work of the index stages of one T-token prefill: the pool
    reads every index key and writes the block summaries; the top-K scores
    2*d_idx FLOP per (query, earlier block) -- sum over p of own(p); the
    inversion reads K selections per query and writes the CSR row pointers,
    one query entry and one slot per selected pair."""
    B, K, di = cfg.block, cfg.topk, cfg.d_idx
    nb = -(-T // B)
    p = np.arange(T, dtype=np.int64)
    pairs = int(np.minimum(K, p // B + 1).sum())
    return {"pool_bytes": T * di * 4 + nb * di * 4,
            "topk_flop": 2 * di * int((p // B).sum()),
            "invert_bytes": T * K * 4 + pairs * 8 + (nb + 1) * 4 * n_calls}


def index_roofline(w: dict, pool_ms: float, topk_ms: float, invert_ms: float) -> dict:
    """Each index stage against the roofline that bounds it: the pool and the
    inversion against HBM, the top-K scores against the fp32 peak."""
    def hbm(b, t):
        g = b / (t * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(g, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(g / PEAK_HBM_GBS, 4)}
    tf = w["topk_flop"] / (topk_ms * 1e-3) / 1e12
    return {"pool": hbm(w["pool_bytes"], pool_ms),
            "topk": {"bound": "fp32 mfma", "achieved": round(tf, 2), "peak": PEAK_F32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_F32_TFLOPS, 4)},
            "invert": hbm(w["invert_bytes"], invert_ms)}


def decode_bytes(L: int, cfg) -> int:
    """Algorithmic HBM bytes of one decode step for a sequence of length L
    (query at L-1): K and V of the attended keys, the block summaries scanned,
    the query, the index query, and the output."""
    n_keys = attended_pairs(L - 1, 1, cfg.block, cfg.topk)
    nb = -(-L // cfg.block)
    elt = 2 if cfg.dtype == "bf16" else 4
    return (n_keys * cfg.Hkv * cfg.d * elt * 2 + nb * cfg.d_idx * 4 +
            cfg.Hq * cfg.d * elt + cfg.d_idx * 4 + cfg.Hq * (cfg.d + 1) * 4)


def kernel_source_hash() -> str:
    """sha256 over the sources of the sparse-GQA prefill kernels: a stored
    counter reading is only reported while these are unchanged."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_attention_index_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload: str):
    """HBM bytes per sparse-GQA prefill call from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated), or None if the summary is
    missing, for another workload, or older than the kernel sources."""
    try:
        text = open(PROFILE_TRAFFIC).read()
    except OSError:
        return None
    fields = dict(re.findall(r"^- (\w+): (\S+)\s*$", text, flags=re.M))
    if fields.get("workload") != workload or fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def calibrate_copy(mib: int) -> None:
    """One plain device copy of `mib` MiB, repeated 3 times: the reference
    run that scales FETCH_SIZE / WRITE_SIZE to bytes."""
    dev = torch.device("cuda:0")
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)


def measure_dec16(dev, seed: int, reps: int = 100, with_cpu: bool = False):
    """Batched decode at the 16 x 256K-token cache workload: one fused decode
    step per sequence (append of the 262144th token, its block's running max,
    the index scan over every cached block summary, top-K, split-KV attention
    and merge), captured once as a HIP graph of `reps` repetitions and
    replayed (each repetition appends the same token again: idempotent);
    bytes are the algorithmic ones (attended K/V, summaries, q, o)."""
    cfg = synth.CONFIGS["dec16"]
    x = synth.decode_inputs(cfg, dev, seed)
    kmax = ops.msa_index_pool(x["idx_k"], cfg.block, seq_len=x["seq_len"], nb_max=cfg.nb)
    bufs = pipeline.alloc_decode_step(x["q"], kmax, cfg.block, cfg.topk)
    L = cfg.T - 1                                    # tokens before the new one
    before = x["seq_len"] - 1
    k_new = x["k_cache"][:, :, L].contiguous()
    v_new = x["v_cache"][:, :, L].contiguous()
    ik_new = x["idx_k"][:, L].contiguous()

    def one():
        pipeline.decode_append_step(x["q"], k_new, v_new, x["idx_q"], ik_new, x["k_cache"],
                                    x["v_cache"], kmax, before, cfg.block, cfg.topk, cfg.scale,
                                    idx_k_cache=x["idx_k"], bufs=bufs)

    one()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            one()
    g.replay()                     # warm-up replay
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    times = []
    for _ in range(3):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e3 / reps)
    us = min(times)
    nbytes = cfg.n_seq * decode_bytes(cfg.T, cfg)
    gbs = nbytes / (us * 1e-6) / 1e9
    res = {"workload": "dec16: 16 sequences x 262144-token bf16 cache, Hq 64 / Hkv 8, d 128, "
                       "block 512, top-K 8; one fused decode step repeated "
                       f"{reps}x in a graph, best of 3 replays",
           "us_per_step": round(us, 3), "bytes_per_step": int(nbytes),
           "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    del kmax, bufs, g
    if with_cpu:
        res["cpu_baseline"] = dec16_cpu_baseline(x, cfg)
    del x
    torch.cuda.empty_cache()
    return res


def dec16_cpu_baseline(x, cfg):
    """The CPU oracle on the whole batched decode step (every sequence: pool of
    its index keys, selection for the query at the last position, attention
    over the selected blocks, fp64); host copies of the caches are not
    timed."""
    import oracle
    oracle.build(force=False)
    B, K, L = cfg.block, cfg.topk, cfg.T
    pos = np.array([L - 1], np.int64)
    dt = 0.0
    for s in range(cfg.n_seq):
        idx_k = x["idx_k"][s].cpu().numpy()
        idx_q = x["idx_q"][s:s + 1].cpu().numpy()
        q_h = synth.host(x["q"][s:s + 1])
        k_h, v_h = synth.host(x["k_cache"][s]), synth.host(x["v_cache"][s])
        t0 = time.perf_counter()
        kmax = oracle.pool(idx_k, B)
        sel, *_ = oracle.select(idx_q, pos, kmax, B, K)
        oracle.attend(q_h, k_h, v_h, np.array([0]), pos, sel, B, cfg.scale, oracle.BF16)
        dt += time.perf_counter() - t0
        del k_h, v_h
    return {"value": round(dt * 1e6, 1), "unit": "us/step", "cores": oracle.threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"the whole step, all {cfg.n_seq} sequences (pool of each "
                      f"sequence's {L} index keys, selection, attention), {dt:.2f} s"}


def _graph_us(fn, reps: int = 20) -> float:
    """Best of three replays of `reps` captured calls, µs per call."""
    st = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(st)
        g.replay()
        b.record(st)
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) * 1e3 / reps)
    return best


def _event_ms(fn, reps: int = 5) -> float:
    """Mean over `reps` eager calls after one warm-up, ms per call."""
    fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def decode_cache_residency(dev, seed: int, reps: int = 10) -> dict:
    """The fused decode step at 1M cached tokens (one sequence, the 1M-token
    workload's shape), timed two ways: back to back, as the bench's decode
    loop runs it (a step may find the previous step's blocks in the L2 or in
    the last-level cache in front of HBM), and after streaming 1 GiB through
    a scratch copy before each step (both caches evicted). The gap between
    the two is what cache residency is worth to the step; the L2-side
    counters cannot tell a last-level-cache hit from an HBM read."""
    cfg = synth.CONFIGS["dec16"].replace(name="dec1m", n_seq=1, T=1 << 20, n_hot=128)
    x = synth.decode_inputs(cfg, dev, seed)
    kmax = ops.msa_index_pool(x["idx_k"], cfg.block, seq_len=x["seq_len"], nb_max=cfg.nb)
    bufs = pipeline.alloc_decode_step(x["q"], kmax, cfg.block, cfg.topk)
    L = cfg.T - 1
    before = x["seq_len"] - 1
    k_new = x["k_cache"][:, :, L].contiguous()
    v_new = x["v_cache"][:, :, L].contiguous()
    ik_new = x["idx_k"][:, L].contiguous()

    def one():
        pipeline.decode_append_step(x["q"], k_new, v_new, x["idx_q"], ik_new, x["k_cache"],
                                    x["v_cache"], kmax, before, cfg.block, cfg.topk, cfg.scale,
                                    idx_k_cache=x["idx_k"], bufs=bufs)

    warm = _graph_us(one)
    g1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        one()
    src = torch.ones(1 << 29, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream(dev)
    times = []
    for _ in range(reps):
        dst.copy_(src)                      # 512 MiB read + 512 MiB written
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(st)
        g1.replay()
        b.record(st)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    nbytes = decode_bytes(cfg.T, cfg)
    res = {"workload": f"1 sequence x {cfg.T}-token bf16 cache, Hq {cfg.Hq} / Hkv {cfg.Hkv}, "
                       f"d {cfg.d}, block {cfg.block}, top-K {cfg.topk}; fused decode step",
           "bytes_per_step": int(nbytes), "us_back_to_back": round(warm, 2),
           "us_caches_evicted": round(float(np.median(times)), 2)}
    del x, kmax, bufs, g1, src, dst
    torch.cuda.empty_cache()
    return res


def measure_next(dev, seed: int) -> dict:
    """The rows past the default path, each against its own roofline:
    several sequences per prefill call (chunks of queries against their
    caches, and many short requests), the paged bf16 / FP8 decode attention
    at the batched decode shape, the 1M-token decode step with and without
    warm caches, and the index variants (mean-pool, forced local window)
    beside the default max-pool and top-K."""
    out = {"metric": "next-row measurements (one GPU)", "data": "synthetic, seeded"}
    # -- several sequences per call: the 32K-token workload's sequence packed
    cfg = synth.CONFIGS["p32k"]
    x = synth.sequence_inputs(cfg, dev, seed)
    B, K, d, hq = cfg.block, cfg.topk, cfg.d, cfg.Hq
    for name, n_seq, L, nq in (("chunks", 8, cfg.T, 8192), ("short", 64, 2048, 2048)):
        cu_q = np.arange(n_seq + 1, dtype=np.int64) * nq
        cu_kv = np.arange(n_seq + 1, dtype=np.int64) * L
        q = x["q"][L - nq:L].repeat(n_seq, 1, 1).contiguous()
        iq = x["idx_q"][L - nq:L].repeat(n_seq, 1).contiguous()
        k = x["k"][:, :L].repeat(1, n_seq, 1).contiguous()
        v = x["v"][:, :L].repeat(1, n_seq, 1).contiguous()
        ik = x["idx_k"][:L].repeat(n_seq, 1).contiguous()
        ms = _event_ms(lambda: ops.msa_prefill_varlen(q, k, v, iq, ik, cu_q, cu_kv, B, K,
                                                      cfg.scale))
        flop = 4.0 * d * hq * n_seq * attended_pairs(L - nq, nq, B, K)
        out[f"varlen_{name}"] = {
            "workload": f"{n_seq} sequences x {L}-token cache, last {nq} tokens as queries, "
                        f"Hq {hq} / Hkv {cfg.Hkv}, d {d}, block {B}, top-K {K}",
            "ms_per_call": round(ms, 3), "attended_tflops": round(flop / ms / 1e9, 1),
            "frac_bf16_peak": round(flop / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
        del q, iq, k, v, ik
    del x
    torch.cuda.empty_cache()
    # -- paged bf16 / FP8 decode attention at the batched decode shape
    cfg = synth.CONFIGS["dec16"]
    n, B, K, hq, hkv, d = cfg.n_seq, cfg.block, cfg.topk, cfg.Hq, cfg.Hkv, cfg.d
    nb = cfg.T // B
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    q = torch.randn((n, hq, d), device=dev, generator=g).to(torch.bfloat16)
    seq = torch.full((n,), cfg.T, dtype=torch.int64, device=dev)
    sel = torch.stack([torch.sort(torch.randperm(nb - 1, device=dev, generator=g)[:K - 1]).values
                       for _ in range(n)])
    sel = torch.cat([sel, torch.full((n, 1), nb - 1, device=dev)], 1).to(torch.int32).contiguous()
    table = torch.randperm(n * nb, device=dev, generator=g).to(torch.int32).view(n, nb).contiguous()
    ws = torch.empty(ops.load().msa_decode_workspace_bytes(n, hq, d, B, K), dtype=torch.uint8,
                     device=dev)
    o = torch.empty((n, hq, d), device=dev)
    lse = torch.empty((n, hq), device=dev)
    kv_elems = n * hkv * K * B * d
    kp = torch.randn((n * nb, hkv, B, d), device=dev, generator=g).to(torch.bfloat16)
    vp = torch.randn((n * nb, hkv, B, d), device=dev, generator=g).to(torch.bfloat16)
    us = _graph_us(lambda: ops.msa_sparse_gqa_decode_paged(q, kp, vp, table, seq, sel, B,
                                                           o=o, lse=lse, ws=ws))
    out["paged_bf16"] = {"workload": f"{n} sequences x {cfg.T} tokens in {B}-key pages, top-K {K}",
                         "us_per_step": round(us, 2),
                         "kv_gbs": round(kv_elems * 4 / (us * 1e-6) / 1e9, 1),
                         "hbm_frac": round(kv_elems * 4 / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    del kp, vp
    torch.cuda.empty_cache()
    kp = torch.randn((n * nb, hkv, B, d), device=dev, generator=g).to(torch.float8_e4m3fn)
    vp = torch.randn((n * nb, hkv, B, d), device=dev, generator=g).to(torch.float8_e4m3fn)
    ks = torch.rand((n * nb, hkv), device=dev, generator=g) + 0.5
    vs = torch.rand((n * nb, hkv), device=dev, generator=g) + 0.5
    us = _graph_us(lambda: ops.msa_sparse_gqa_decode_paged(q, kp, vp, table, seq, sel, B,
                                                           k_scale=ks, v_scale=vs, o=o, lse=lse,
                                                           ws=ws))
    out["paged_fp8"] = {"workload": out["paged_bf16"]["workload"] + ", e4m3 K/V",
                        "us_per_step": round(us, 2),
                        "kv_gbs": round(kv_elems * 2 / (us * 1e-6) / 1e9, 1),
                        "hbm_frac": round(kv_elems * 2 / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    del kp, vp, ks, vs, q, o, lse, ws
    torch.cuda.empty_cache()
    out["decode_1m_caches"] = decode_cache_residency(dev, seed)
    # -- index variants next to the default rule
    T1, B1, di = 1 << 20, 512, 128
    ik = torch.randn((T1, di), device=dev, generator=g)
    nb1 = T1 // B1
    pool_bytes = T1 * di * 4 + nb1 * di * 4
    km = torch.empty((nb1, di), device=dev)
    for name, fn in (("pool_max", lambda: ops.msa_index_pool(ik, B1, kmax=km)),
                     ("pool_mean", lambda: ops.msa_index_pool_mean(ik, B1, kmean=km))):
        us = _graph_us(fn)
        out[name] = {"workload": f"{T1} index keys, d_idx {di}, block {B1}",
                     "us": round(us, 2), "gbs": round(pool_bytes / (us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(pool_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    del ik, km
    cfg = synth.CONFIGS["p128k"]
    T2, B2, K2 = cfg.T, cfg.block, cfg.topk
    iq = torch.randn((T2, di), device=dev, generator=g)
    kmax = torch.randn((T2 // B2, di), device=dev, generator=g)
    p = np.arange(T2, dtype=np.int64)
    flop = 2 * di * int((p // B2).sum())
    for name, fn in (("topk", lambda: ops.msa_index_topk(iq, kmax, B2, K2)),
                     ("topk_window4", lambda: ops.msa_index_topk_window(iq, kmax, B2, K2, 4))):
        ms = _event_ms(fn)
        out[name] = {"workload": f"{T2} queries x {T2 // B2} blocks, d_idx {di}, top-K {K2}",
                     "ms": round(ms, 3), "tflops": round(flop / ms / 1e9, 2),
                     "frac_fp32_peak": round(flop / ms / 1e9 / PEAK_F32_TFLOPS, 4)}
    # -- a batch of queries of 16 sequences at scattered positions
    n_s, per = 16, 256
    nbs = T2 // B2
    kms = torch.randn((n_s, nbs, di), device=dev, generator=g)
    qs = torch.arange(n_s, dtype=torch.int32, device=dev).repeat_interleave(per)
    qp = torch.randint(0, T2, (n_s * per,), device=dev, generator=g)
    iqb = torch.randn((n_s * per, di), device=dev, generator=g)
    flop = 2 * di * int((qp // B2).sum().item())
    ms = _event_ms(lambda: ops.msa_index_topk_batch(iqb, qs, qp, kms, B2, K2))
    out["topk_batch"] = {"workload": f"{n_s} sequences x {nbs} blocks, {per} queries each at "
                                     f"uniform positions, d_idx {di}, top-K {K2}",
                         "ms": round(ms, 3), "tflops": round(flop / ms / 1e9, 2),
                         "frac_fp32_peak": round(flop / ms / 1e9 / PEAK_F32_TFLOPS, 4)}
    del iq, kmax, kms, qs, qp, iqb
    return out


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or 'unknown'."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, cfg, dev_sel, n_dec: int, attn_budget_s: float = 10.0):
    """The CPU oracle (fp64, every host core) on the same 1M-token step as the
    GPU: the index branch in full (pool of all index keys, selection of every
    query), the prefill attention on a stratified sample of queries (blocks 0
    and 1 and the last block in full, plus random queries, about
    `attn_budget_s` of work) extrapolated to all queries by attended pairs,
    and every decode step in full (each: re-pool of the newest token's block,
    selection and attention for its query).  The device's selection is also
    compared with the oracle's here: near-ties flagged per rule, and rows
    where the two differ."""
    import oracle
    oracle.build(force=False)
    T, B, K = cfg.T, cfg.block, cfg.topk
    L_all = x["idx_k"].shape[0]
    idx_k = x["idx_k"].cpu().numpy()
    idx_q = x["idx_q"].cpu().numpy()
    k_h, v_h = synth.host(x["k"]), synth.host(x["v"])
    # index branch, whole
    t0 = time.perf_counter()
    kmax = oracle.pool(idx_k[:T], B)
    t_pool = time.perf_counter() - t0
    pos = np.arange(T, dtype=np.int64)
    t0 = time.perf_counter()
    so, gr, ga, eb = oracle.select(idx_q[:T], pos, kmax, B, K)
    t_sel = time.perf_counter() - t0
    rel = np.nan_to_num(gr, nan=np.inf) < 1e-3
    bnd = np.nan_to_num(ga, nan=np.inf) <= np.nan_to_num(eb, nan=0.0)
    diff = np.any(np.asarray(dev_sel) != so, axis=1)
    ties = {"rows": T, "flag_rel": int(rel.sum()), "flag_bound_only": int((bnd & ~rel).sum()),
            "differing": int(diff.sum()), "differing_unflagged": int((diff & ~(rel | bnd)).sum())}
    # prefill attention on a stratified sample, extrapolated by attended pairs
    rng = np.random.default_rng(0)
    fixed = np.unique(np.concatenate([np.arange(min(T, 2 * B)), np.arange(max(0, T - B), T)]))

    def attend(rows):
        t1 = time.perf_counter()
        q_h = synth.host(x["q"][torch.from_numpy(rows).to(x["q"].device)])
        _, _, nk = oracle.attend(q_h, k_h, v_h, np.arange(len(rows)), rows, so[rows], B,
                                 cfg.scale, oracle.BF16)
        return time.perf_counter() - t1, int(nk.sum())

    t_fix, keys_fix = attend(fixed)
    per_key = t_fix / max(1, keys_fix)
    mean_keys = attended_pairs(0, T, B, K) / T
    n_rand = int(max(64, min(T, attn_budget_s / max(per_key * mean_keys, 1e-9))))
    rand = np.sort(rng.choice(np.setdiff1d(np.arange(T), fixed), size=n_rand, replace=False))
    t_rand, keys_rand = attend(rand)
    t_attn = (t_fix + t_rand) / (keys_fix + keys_rand) * attended_pairs(0, T, B, K)
    # every decode step
    t0 = time.perf_counter()
    km = np.concatenate([kmax, np.zeros((1, cfg.d_idx), np.float32)]) if n_dec else kmax
    for s in range(n_dec):
        L = T + s + 1
        own = (L - 1) // B
        km[own:own + 1] = oracle.pool(idx_k[own * B:L], B)
        p = np.array([L - 1], np.int64)
        sel1, *_ = oracle.select(idx_q[L - 1:L], p, km[:own + 1], B, K)
        oracle.attend(synth.host(x["q"][L - 1:L]), k_h, v_h, np.array([0]), p, sel1, B,
                      cfg.scale, oracle.BF16)
    t_dec = time.perf_counter() - t0
    assert L_all >= T + n_dec
    step_s = t_pool + t_sel + t_attn + t_dec
    flops = 4.0 * cfg.d * cfg.Hq * (attended_pairs(0, T, B, K) +
                                    sum(attended_pairs(T + s, 1, B, K) for s in range(n_dec)))
    n_att = len(fixed) + n_rand
    return {"value": flops / step_s / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": (f"index branch in full (pool {t_pool:.2f} s, selection of all {T} "
                       f"queries {t_sel:.1f} s); prefill attention measured on {n_att} queries "
                       f"(blocks 0-1 and the last block in full + {n_rand} random) in "
                       f"{t_fix + t_rand:.1f} s and extrapolated by attended pairs to "
                       f"{t_attn:.0f} s (extrapolated); all {n_dec} decode steps in full "
                       f"{t_dec:.1f} s ({t_dec / max(1, n_dec) * 1e3:.1f} ms/step); step "
                       f"{step_s:.0f} s"),
            "step_s": round(step_s, 2), "extrapolated_s": round(t_attn, 2),
            "decode_ms_per_step": round(t_dec / max(1, n_dec) * 1e3, 2),
            "selection_vs_oracle": ties}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="p1m", choices=["p1m", "p32k", "p128k"])
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dec16", action="store_true",
                    help="skip the batched-decode (16 x 256K cache) measurement")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--next", action="store_true",
                    help="only measure the rows past the default path (several sequences per "
                         "call, paged / FP8 decode, index variants); prints one JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(sharding is described in DESIGN.md); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.next:
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        ops.load()
        print(json.dumps(measure_next(dev, args.seed)), flush=True)
        return

    cfg = synth.CONFIGS[args.config]
    n_dec = cfg.n_dec if args.decode_steps is None else args.decode_steps
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ops.load()
    T, B, K = cfg.T, cfg.block, cfg.topk
    L_total = T + n_dec
    print(f"[bench] generating {cfg.name}: {L_total} tokens", file=sys.stderr, flush=True)
    x = synth.sequence_inputs(cfg, dev, args.seed, length=L_total)
    torch.cuda.synchronize()

    nb_max = -(-L_total // B)
    kmax_dec = torch.zeros((1, nb_max, cfg.d_idx), dtype=torch.float32, device=dev)
    bufs = pipeline.alloc_prefill(x["q"][:T], x["idx_q"][:T], B, K)
    bufs.kmax = kmax_dec[0, :-(-T // B)]
    k_cache, v_cache = x["k"][None], x["v"][None]
    idx_k_cache = x["idx_k"][None]
    # decode: one fused step per new token (append at position T + s, running
    # block max, scan, top-K, attention, merge); the new tokens' rows are
    # gathered contiguous once, outside the timed region
    seq_lens = torch.arange(T, T + n_dec, dtype=torch.int64, device=dev)  # before each step
    dbufs = None
    if n_dec:
        k_new = x["k"][:, T:T + n_dec].permute(1, 0, 2).contiguous()      # [n_dec, Hkv, d]
        v_new = x["v"][:, T:T + n_dec].permute(1, 0, 2).contiguous()
        ik_new = x["idx_k"][T:T + n_dec].contiguous()
        dbufs = pipeline.alloc_decode_step(x["q"][:1], kmax_dec, B, K)
    stream = torch.cuda.current_stream(dev)

    def decode_loop():
        for s in range(n_dec):
            pipeline.decode_append_step(
                x["q"][T + s:T + s + 1], k_new[s:s + 1], v_new[s:s + 1],
                x["idx_q"][T + s:T + s + 1], ik_new[s:s + 1], k_cache, v_cache, kmax_dec,
                seq_lens[s:s + 1], B, K, cfg.scale, idx_k_cache=idx_k_cache, bufs=dbufs)

    # The decode steps are launch-bound at batch 1: capture them once in a HIP
    # graph (no allocation or memset inside) and replay it.
    dec_graph = None
    if n_dec:
        decode_loop()                      # eager warm-up of the decode kernels
        torch.cuda.synchronize()
        dec_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dec_graph):
            decode_loop()
        torch.cuda.synchronize()

    ev = {"pre": [], "attn": [], "dec": [], "pool": [], "topk": [], "invert": []}

    def event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def step(record: bool):
        e0 = event()
        # prefill: pool, top-K, then per chunk CSR + sparse GQA (timed per call)
        q, k, v = x["q"][:T], x["k"], x["v"]
        ops.msa_index_pool(x["idx_k"][:T], B, kmax=bufs.kmax)
        ep = event()
        ops.msa_index_topk(x["idx_q"][:T], bufs.kmax, B, K, sel=bufs.sel)
        et = event()
        if record:
            ev["pool"].append((e0, ep))
            ev["topk"].append((ep, et))
        for c0 in range(0, T, bufs.chunk):
            c1 = min(T, c0 + bufs.chunk)
            nbc = -(-c1 // B)
            n = c1 - c0
            i0 = event()
            ops.msa_invert_selection(bufs.sel[c0:c1], nbc, row_ptr=bufs.row_ptr[:nbc + 1],
                                     q_list=bufs.q_list[:n * K], slot=bufs.slot[:n],
                                     ws=bufs.inv_ws)
            if record:
                ev["invert"].append((i0, event()))
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            ops.msa_sparse_gqa_prefill(q[c0:c1], k, v, bufs.sel[c0:c1],
                                       bufs.row_ptr[:nbc + 1], bufs.q_list[:n * K],
                                       bufs.slot[:n], B, cfg.scale, q_pos0=c0,
                                       o=bufs.o[c0:c1], lse=bufs.lse[c0:c1],
                                       ws=bufs.attn_ws)
            a1.record(stream)
            if record:
                ev["attn"].append((a0, a1))
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record(stream)
        if dec_graph is not None:
            dec_graph.replay()
        e2 = torch.cuda.Event(enable_timing=True)
        e2.record(stream)
        if record:
            ev["pre"].append((e0, e1))
            ev["dec"].append((e1, e2))

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms = lambda pairs: sum(a.elapsed_time(b) for a, b in pairs)
    pre_ms = ms(ev["pre"]) / args.steps
    dec_ms = ms(ev["dec"]) / args.steps
    attn_ms = ms(ev["attn"]) / len(ev["attn"])           # per prefill-attention call
    n_calls = len(ev["attn"]) // args.steps
    pre_pairs = attended_pairs(0, T, B, K)
    dec_pairs = sum(attended_pairs(T + s, 1, B, K) for s in range(n_dec))
    fl = 4.0 * cfg.d * cfg.Hq
    step_s = wall / args.steps
    value = fl * (pre_pairs + dec_pairs) / step_s / 1e12
    attn_tflops = fl * pre_pairs / n_calls / (attn_ms * 1e-3) / 1e12
    dec_us = dec_ms * 1e3 / max(1, n_dec)
    dec_gbs = (sum(decode_bytes(T + s + 1, cfg) for s in range(n_dec)) /
               max(1e-12, dec_ms * 1e-3) / 1e9) if n_dec else None
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS

    out = {
        "metric": "prefill attended TFLOP/s + decode us/step at 1M ctx; % of MFMA/HBM roofline",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1), planted hot blocks), generated on device",
        "config": {"workload": f"{cfg.name}: 1 sequence, {T}-token causal prefill + "
                               f"{n_dec} decode steps, {cfg.dtype} q/k/v, fp32 index, "
                               f"Hq {cfg.Hq} / Hkv {cfg.Hkv}, d {cfg.d}, d_idx {cfg.d_idx}, "
                               f"block {B}, top-K {K}, {cfg.n_hot} hot blocks",
                   "seq_len": T, "decode_steps": n_dec, "global_batch": 1,
                   "parallelism": "none (1 GPU)"},
        "prefill_ms": round(pre_ms, 3),
        "prefill_tflops": round(fl * pre_pairs / (pre_ms * 1e-3) / 1e12, 3),
        "decode_us_per_step": round(dec_us, 3) if n_dec else None,
        "decode_hbm_gbs": round(dec_gbs, 1) if dec_gbs else None,
        "index_ms": {"pool": round(ms(ev["pool"]) / args.steps, 3),
                     "topk": round(ms(ev["topk"]) / args.steps, 3),
                     "invert": round(ms(ev["invert"]) / args.steps, 3)},
        "index_roofline": index_roofline(index_work(T, cfg, n_calls),
                                         ms(ev["pool"]) / args.steps,
                                         ms(ev["topk"]) / args.steps,
                                         ms(ev["invert"]) / args.steps),
        "roofline": {"kernel": "msa_sparse_gqa_prefill (KV-outer pass + own-block/merge pass)",
                     "bound": "mfma", "achieved": round(attn_tflops, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 5),
                     "traffic": stored_traffic(cfg.name),
                     "launch_ms": round(attn_ms, 3), "launches_per_step": n_calls},
    }
    sel_final = bufs.sel.cpu().numpy()
    if not args.no_dec16:
        print("[bench] batched decode (dec16)", file=sys.stderr, flush=True)
        del bufs, dbufs, dec_graph
        out["decode16"] = measure_dec16(dev, args.seed, with_cpu=not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(x, cfg, sel_final, n_dec)
        out["selection_vs_oracle"] = out["cpu_baseline"].pop("selection_vs_oracle")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
