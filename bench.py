"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the whole path over one batch: prepare_seqlens (device metadata),
kv_cache_append (this step's K/V rows into the paged cache) and paged_attention_fwd
(split-K decode over the block table, merge with sinks), made by one paged_decode_step
call (the split-K kernel derives the lengths and writes the new rows itself, then the
merge).  The same step as prepare_and_append -> paged_attention_fwd is reported beside
it.  Workload: GQA paged decode,
fp16, B=32 requests with key counts ~ U{0..8192} (one forced empty), H_q=64, H_kv=8,
head_dim 64, block 16, a 20000-block pool, sinks ~ N(0,1).  Inputs are resident in HBM
before the timed region; three copies of the KV pool are rotated so that consecutive
steps never find their 260 MB of keys/values in the 256 MB Infinity Cache.

value = decode KV bytes per step / time per step (GB/s, 1 GB = 1e9 B).  The prefill
TFLOP/s of the windowed paged prefill workload (B=4, lengths 1024/512/2048/1536, W=128)
and of the same without a window are reported alongside, as the metric names both; so
are the selected-token and local-plus-auxiliary decode, the QKV prologue and the TopK
selection.  Each of these calls is preceded by a 1 GiB read outside its events, so the
caches hold none of its inputs.

`--gpus N` with N > 1 is not supported: the benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2516.6    # MI355X dense fp16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
METRIC = "decode KV GB/s (% HBM peak) + prefill TFLOP/s (% MFMA peak), GQA paged attn"

# HBM bytes per paged_decode_step call on the decode workload, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE counter passes scaled by the same counters' reading on a plain device copy of
# known size (profiles/decode_gqa_paged_f16_traffic.md).  Valid only for the kernel sources
# whose digest is recorded with it; any other source reports traffic = null.
MEASURED_TRAFFIC = {"sources_sha1": "45ff4aabb1b04412e83b69e250adef8a36a0ecc9",
                    "bytes_per_call": 278401400}
KERNEL_SOURCES = ("selected_token_sparse_amd/csrc/decode.hip", "selected_token_sparse_amd/csrc/common.h",
                  "selected_token_sparse_amd/csrc/launch.h", "selected_token_sparse_amd/csrc/append.h")


def kernel_sources_sha1():
    h = hashlib.sha1()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _kv_bytes(case):
    """Algorithmic K+V bytes the decode step must read: every visible key of every row,
    once per (row, KV head); the GQA group shares it."""
    esize = 2 if case.cache_dtype in (1, 2) else (4 if case.cache_dtype == 0 else 1)
    total = 0
    cu = case.cu_seqlens_q
    for b in range(case.B):
        q_len = int(cu[b + 1] - cu[b])
        kv = int(case.seqlens_k[b]) + 1
        for i in range(q_len):
            p = kv - q_len + i
            lo = max(0, p - case.local_window + 1) if case.local_window > 0 else 0
            total += max(0, p - lo + 1)
    return total * case.H_kv * case.D * esize * 2


def _prefill_flops(case):
    """4*D flops per visible (row, query head, key): QK^T and PV."""
    pairs = 0
    cu = case.cu_seqlens_q
    for b in range(case.B):
        q_len = int(cu[b + 1] - cu[b])
        kv = int(case.seqlens_k[b]) + 1
        for i in range(q_len):
            p = kv - q_len + i
            lo = max(0, p - case.local_window + 1) if case.local_window > 0 else 0
            pairs += max(0, p - lo + 1)
    return pairs * case.H_q * 4 * case.D


def _prefill_bytes(case):
    """Algorithmic HBM bytes of a prefill call: Q and out once, and the K+V rows of every
    key some row of the request sees, once per (request, KV head): positions
    max(0, p_first - W + 1) .. p_last."""
    esize = {0: 4, 1: 2, 2: 2, 3: 1, 4: 1}[case.cache_dtype]
    qo = 2 * case.T * case.H_q * case.D * (4 if case.dtype == 0 else 2)
    keys = 0
    cu = case.cu_seqlens_q
    for b in range(case.B):
        q_len = int(cu[b + 1] - cu[b])
        if q_len == 0:
            continue
        kv = int(case.seqlens_k[b]) + 1
        p_first, p_last = kv - q_len, kv - 1
        lo = max(0, p_first - case.local_window + 1) if case.local_window > 0 else 0
        keys += max(0, p_last - lo + 1)
    return qo + keys * case.H_kv * case.D * esize * 2


def _queue_ahead():
    """A short device spin before a timed loop, so that the host has queued the loop's
    launches before the GPU reaches them and the events time the GPU, not the launches."""
    import torch
    torch.cuda._sleep(4_000_000)


class ColdCache:
    """Before each timed call: read (not write) a 1 GiB buffer, so neither the L2 nor the
    256 MB Infinity Cache holds the call's inputs, and neither holds dirty lines that the
    call would have to write back (a 1 GiB write leaves up to 256 MB of them, which cost
    the sparse and prologue calls 10-40 us of extra HBM writes)."""

    def __init__(self):
        import torch
        self.buf = torch.empty(1 << 27, dtype=torch.int64, device="cuda")
        self.buf.zero_()
        self.out = torch.empty(1, dtype=torch.int64, device="cuda")

    def __call__(self):
        import torch
        torch.sum(self.buf, dim=0, keepdim=True, out=self.out)


def _p10_p90(ms_sorted):
    """10th and 90th percentiles (us) of sorted per-call times in ms."""
    n = len(ms_sorted)
    return (round(ms_sorted[min(n - 1, n // 10)] * 1e3, 2),
            round(ms_sorted[min(n - 1, (9 * n) // 10)] * 1e3, 2))


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def bench_decode(steps, warmup, copies=3, cache_dtype=None, fused=False):
    """The GQA paged decode step, `steps` timed after `warmup`.  fused: one paged_decode_step
    call per step (events around it); otherwise prepare_and_append, then paged_attention_fwd
    (events around the attention call)."""
    import torch

    import selected_token_sparse_amd as sta
    import synth
    from synth.device import case_tensors, tensor

    case = synth.config_gqa_paged_decode(cache_dtype=synth.F16 if cache_dtype is None else cache_dtype)
    base = case_tensors(case)
    sets = [base]
    for _ in range(copies - 1):
        sets.append(dict(base, k_cache=base["k_cache"].clone(), v_cache=base["v_cache"].clone()))
    B, T = case.B, case.T
    sq = torch.empty(B, dtype=torch.int32, device="cuda")
    sk = torch.empty(B, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty((T, case.H_q, case.D), dtype=torch.float16, device="cuda")
    need = sta.attention_workspace_bytes(sta.KIND_PAGED, sta.F16, B, T, case.max_seqlen_q,
                                         case.max_seqlen_k, 0, case.local_window, case.H_q,
                                         case.H_kv, case.D)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def step(i, ev=None):
        t = sets[i % copies]
        if fused:
            if ev is not None:
                ev[0].record()
            sta.paged_decode_step(t["cu"], t["past"], T, sq, sk, t["q"], t["k_new"], t["v_new"],
                                  t["k_cache"], t["v_cache"], case.max_seqlen_q, case.max_seqlen_k,
                                  out, block_table=t["block_table"], key_scale=t["key_scale"],
                                  value_scale=t["value_scale"], scale=case.scale, sinks=t["sinks"],
                                  workspace=ws, status=status)
            if ev is not None:
                ev[1].record()
            return
        # metadata and the cache append of this step's rows: one launch
        sta.prepare_and_append(t["cu"], t["past"], T, sq, sk, t["k_new"], t["v_new"], t["k_cache"],
                               t["v_cache"], t["block_table"], key_scale=t["key_scale"],
                               value_scale=t["value_scale"], status=status)
        if ev is not None:
            ev[0].record()
        sta.paged_attention_fwd(t["q"], t["k_cache"], t["v_cache"], t["cu"], sk, case.max_seqlen_q,
                                case.max_seqlen_k, out, block_table=t["block_table"],
                                key_scale=t["key_scale"], value_scale=t["value_scale"],
                                scale=case.scale, sinks=t["sinks"], workspace=ws, status=status)
        if ev is not None:
            ev[1].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # the timed steps, back to back with nothing recorded between them
    t0, t1 = _events()
    _queue_ahead()
    t0.record()
    for i in range(steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    # the same steps again with events around each call: its duration distribution (the
    # event records between calls would lengthen the steps timed above)
    evs = [_events() for _ in range(steps)]
    _queue_ahead()
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    attn_ms = sorted(a.elapsed_time(b) for a, b in evs)
    st = int(status.item())
    return case, total_ms / steps, attn_ms, st


def bench_decode_graph(layers=24, steps=20, warmup=3, copies=3):
    """A decode step of a `layers`-layer model (per layer one paged_decode_step: the
    metadata, the cache append and the attention) on the GQA paged decode workload, eager
    and replayed from one HIP graph.  Layer i uses the i % 3 copy of the KV pool, so
    consecutive layers read different 655 MB pools as a real model's layers would."""
    import torch

    import selected_token_sparse_amd as sta
    import synth
    from synth.device import case_tensors

    case = synth.config_gqa_paged_decode()
    base = case_tensors(case)
    sets = [base] + [dict(base, k_cache=base["k_cache"].clone(), v_cache=base["v_cache"].clone())
                     for _ in range(copies - 1)]
    B, T = case.B, case.T
    sq = torch.empty(B, dtype=torch.int32, device="cuda")
    sk = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty((T, case.H_q, case.D), dtype=torch.float16, device="cuda")
    need = sta.attention_workspace_bytes(sta.KIND_PAGED, sta.F16, B, T, case.max_seqlen_q,
                                         case.max_seqlen_k, 0, case.local_window, case.H_q,
                                         case.H_kv, case.D)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def step():
        for layer in range(layers):
            t = sets[layer % copies]
            sta.paged_decode_step(t["cu"], t["past"], T, sq, sk, t["q"], t["k_new"], t["v_new"],
                                  t["k_cache"], t["v_cache"], case.max_seqlen_q,
                                  case.max_seqlen_k, out, block_table=t["block_table"],
                                  scale=case.scale, sinks=t["sinks"], workspace=ws)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = _events()
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps * 1e3

    eager_us = timed(step)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    graph_us = timed(g.replay)
    kv = _kv_bytes(case) * layers
    return {"workload": f"{case.name} x {layers} layers", "layers": layers,
            "eager_us_per_step": round(eager_us, 1), "graph_us_per_step": round(graph_us, 1),
            "graph_us_per_layer": round(graph_us / layers, 2),
            "graph_kv_gbs": round(kv / (graph_us * 1e-6) / 1e9, 1)}


def bench_prefill(window, steps, warmup, cache_dtype=None):
    import torch

    import selected_token_sparse_amd as sta
    import synth
    from synth.device import case_tensors

    case = synth.config_paged_prefill_window(window=window, cache_dtype=cache_dtype)
    t = case_tensors(case)
    # the prompt rows are appended once, outside the timed region
    sta.kv_cache_append(t["k_new"], t["v_new"], t["cu"], t["seqlens_k"], t["k_cache"], t["v_cache"],
                        t["block_table"], t["key_scale"], t["value_scale"])
    out = torch.empty((case.T, case.H_q, case.D), dtype=torch.float16, device="cuda")

    def call():
        sta.paged_attention_fwd(t["q"], t["k_cache"], t["v_cache"], t["cu"], t["seqlens_k"],
                                case.max_seqlen_q, case.max_seqlen_k, out,
                                block_table=t["block_table"], key_scale=t["key_scale"],
                                value_scale=t["value_scale"], scale=case.scale,
                                local_window=case.local_window, sinks=t["sinks"])

    flush = ColdCache()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [_events() for _ in range(steps)]
    for a, b in evs:
        flush()                # outside the events: Q, the cache and out start in HBM
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    med = ms[len(ms) // 2]
    flops = _prefill_flops(case)
    alg = _prefill_bytes(case)
    tfl = flops / (med * 1e-3) / 1e12
    gbs = alg / (med * 1e-3) / 1e9
    return {
        "workload": case.name, "window": window, "median_us": round(med * 1e3, 2),
        "p10_p90_us": _p10_p90(ms),
        "tflops": round(tfl, 2), "frac_mfma_peak": round(tfl / MFMA_F16_PEAK_TFLOPS, 4),
        "algorithmic_gflop": round(flops / 1e9, 3),
        "algorithmic_bytes": alg, "gbs": round(gbs, 1),
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
    }


def _sparse_bytes(case):
    """Algorithmic bytes of a sparse call: K+V of every key a row sees, once per (row, KV
    head) (visible selected main positions j <= p, window positions, in-range auxiliary
    rows), plus Q and out."""
    import numpy as np
    cu = case.cu_seqlens_q
    T, H_kv, D = case.T, case.H_kv, case.D
    main_es = 1 if case.cache_dtype == 3 else 2
    req = np.searchsorted(cu, np.arange(T), side="right") - 1
    kv = case.seqlens_k[req].astype(np.int64) + 1
    p = kv - (cu[req + 1] - cu[req]) + (np.arange(T) - cu[req])           # [T]
    sel = case.sel_idx.astype(np.int64)                                   # [T, H_kv, S]
    t = np.arange(sel.shape[2])[None, None, :]
    cnt = np.clip(case.sel_count.astype(np.int64), 0, case.max_selected)[:, :, None]
    inside = t < cnt
    if case.mode == 0:
        vis = inside & (sel >= 0) & (sel <= p[:, None, None]) & (sel < kv[:, None, None])
        main_keys = int(vis.sum())
        aux_keys = 0
    else:
        W = case.local_window
        main_keys = int(np.minimum(p + 1, W).sum()) * H_kv
        aux_keys = int((inside & (sel >= 0) & (sel < case.aux_len)).sum())
    qo = 2 * T * case.H_q * D * 2
    return main_keys * 2 * D * main_es + aux_keys * 2 * D * 2 + qo, main_keys, aux_keys


def bench_sparse(which, steps, warmup):
    """Selected-token grouped decode (mode 0) or local-plus-aux INT8 (mode 1)."""
    import torch

    import selected_token_sparse_amd as sta
    import synth
    from synth.device import case_tensors

    case = synth.config_selected_decode() if which == "selected" else synth.config_local_plus_aux_int8()
    t = case_tensors(case)
    out = torch.empty((case.T, case.H_q, case.D), dtype=torch.float16, device="cuda")
    kind = sta.KIND_SELECTED if case.mode == 0 else sta.KIND_LOCAL_AUX
    need = sta.attention_workspace_bytes(kind, sta.F16, case.B, case.T, case.max_seqlen_q, 0,
                                         case.max_selected, case.local_window, case.H_q,
                                         case.H_kv, case.D)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    flush = ColdCache()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call():
        sta.sparse_attention_fwd(t["q"], case.mode, t["k_cache"], t["v_cache"], t["cu"],
                                 t["seqlens_k"], case.max_seqlen_q, t["sel_idx"], out,
                                 sel_count=t["sel_count"], key_scale=t["key_scale"],
                                 value_scale=t["value_scale"], local_window=case.local_window,
                                 aux_k=t["aux_k"], aux_v=t["aux_v"],
                                 aux_batch_stride=case.aux_batch_stride if case.mode == 1 else None,
                                 scale=case.scale, sinks=t["sinks"], workspace=ws, status=status)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [_events() for _ in range(steps)]
    for a, b in evs:
        flush()                # outside the events: the caches hold none of the rows
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    med = ms[len(ms) // 2]
    alg, main_keys, aux_keys = _sparse_bytes(case)
    gbs = alg / (med * 1e-3) / 1e9
    return {"workload": case.name, "median_us": round(med * 1e3, 2),
            "avg_us": round(sum(ms) / len(ms) * 1e3, 2), "p10_p90_us": _p10_p90(ms),
            "algorithmic_bytes": alg,
            "main_keys": main_keys, "aux_keys": aux_keys, "gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "status": int(status.item())}


def _prologue_bytes(case):
    """Algorithmic bytes of one qkv_prologue call: each row's packed Q/K/V read once, its
    cos / sin table rows, the query row written, the key and value rows written to the
    cache, the two norm weight vectors."""
    es = 2 if case.dtype != 0 else 4
    ces = {0: 4, 1: 2, 2: 2, 3: 1, 4: 1}[case.cache_dtype]
    per_row = ((case.H_q + 2 * case.H_kv) * case.D * es + case.H_q * case.D * es
               + 2 * case.H_kv * case.D * ces + (case.rotary_dim // 2) * 4 * 2)
    return case.T * per_row + 2 * case.D * 4


def bench_prologue(shape, steps, warmup):
    """qkv_prologue (packed f16 rows, QK RMSNorm, full-width rotation, f16 paged cache) at the
    GQA decode shape (31 rows) or the windowed prefill shape (5120 rows)."""
    import numpy as np
    import torch

    import selected_token_sparse_amd as sta
    import synth
    from synth.device import tensor

    if shape == "decode":
        base = synth.config_gqa_paged_decode()
        kv, ql = base.seqlens_k + 1, np.diff(base.cu_seqlens_q)
        name = "prologue_gqa_decode_f16 (31 rows, H 64/8, D 64)"
    else:
        kv = ql = np.array([1024, 512, 2048, 1536])
        name = "prologue_prefill_f16 (5120 rows, H 64/8, D 64)"
    case = synth.prologue_case(seed=1006, kv_lens=kv, q_lens=ql, H_q=64, H_kv=8, D=64,
                               dtype=synth.F16, packed=True, rotary_dim=64, qk_norm=True,
                               poison=False)
    d = lambda x, dt=None: tensor(x, dt)   # noqa: E731
    qkv, cu, sk = d(case.qkv, case.dtype), d(case.cu_seqlens_q), d(case.seqlens_k)
    kc, vc, bt = d(case.k_cache, case.cache_dtype), d(case.v_cache, case.cache_dtype), d(case.block_table)
    qw, kw, cos, sin = d(case.q_norm_weight), d(case.k_norm_weight), d(case.cos_table), d(case.sin_table)
    q_out = torch.empty((case.T, case.H_q, case.D), dtype=torch.float16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    flush = ColdCache()

    def call():
        sta.qkv_prologue(q_out, kc, vc, cu, sk, H_q=case.H_q, H_kv=case.H_kv, qkv=qkv, qk_norm=True,
                         q_norm_weight=qw, k_norm_weight=kw, rotary_dim=64, cos_table=cos,
                         sin_table=sin, block_table=bt, status=status)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [_events() for _ in range(steps)]
    for a, b in evs:
        flush()                # outside the events: the caches hold none of the rows
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    med = ms[len(ms) // 2]
    alg = _prologue_bytes(case)
    gbs = alg / (med * 1e-3) / 1e9
    return {"workload": name, "median_us": round(med * 1e3, 2),
            "avg_us": round(sum(ms) / len(ms) * 1e3, 2), "p10_p90_us": _p10_p90(ms),
            "algorithmic_bytes": alg,
            "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "status": int(status.item())}


def bench_topk(steps, warmup):
    """topk_select at the selected grouped decode shape: 128 rows x 4 KV heads, 65536
    candidates each (float32 scores, 134 MB), k = 2048 with a 64-key causal tail."""
    import torch

    import selected_token_sparse_amd as sta
    import synth
    from synth.device import tensor

    case = synth.topk_case(1007, kv_lens=[65536] * 16, q_lens=[8] * 16, H_kv=4, L=65536, k=2048,
                           tail=64, capacity=2048, ties=0.05, specials=0.001)
    scores, cu, sk = tensor(case.scores), tensor(case.cu_seqlens_q), tensor(case.seqlens_k)
    sel = torch.empty((case.T, case.H_kv, case.capacity), dtype=torch.int32, device="cuda")
    cnt = torch.empty((case.T, case.H_kv), dtype=torch.int32, device="cuda")
    flush = ColdCache()

    def call():
        sta.topk_select(scores, cu, sk, case.k, sel, cnt, tail=case.tail)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [_events() for _ in range(steps)]
    for a, b in evs:
        flush()                # outside the events: the caches hold none of the scores
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    med = ms[len(ms) // 2]
    alg = case.scores.nbytes + sel.numel() * 4 + cnt.numel() * 4
    gbs = alg / (med * 1e-3) / 1e9
    return {"workload": "topk_selected_decode (128 rows x 4 KV heads, 65536 scores, k 2048, tail 64)",
            "median_us": round(med * 1e3, 2), "avg_us": round(sum(ms) / len(ms) * 1e3, 2),
            "p10_p90_us": _p10_p90(ms),
            "algorithmic_bytes": alg, "gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def copy_calibration(mib, reps=4):
    """A plain device-to-device copy of `mib` MiB, for scaling the HBM byte counters: the
    copy reads and writes exactly mib * 2^20 bytes each."""
    import torch
    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy calibration: {reps} copies of {mib << 20} bytes", file=sys.stderr, flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds=10.0):
    """The oracle (numpy float64) on the host cores, as a process pool over rows (all cores
    this process may use, at most 16: the machine's CPU share for one GPU), each worker on one
    BLAS thread.  Two legs on the same workloads as the GPU lines:
    - decode: the attention rows of the GQA paged decode step, after one oracle metadata +
      append pass (not timed), cycled until `seconds` have passed; GB/s of the rows' KV bytes;
    - prefill: rows of the windowed paged prefill (W=128), cycled likewise; TFLOP/s of the
      rows' algorithmic flops (4 D per visible (row, query head, key)).
    Must run before the GPU is initialised: the pool forks, sharing the arrays."""
    import numpy as np

    import oracle
    import synth
    from oracle import pool

    workers = pool.default_workers()
    legs = {}
    for leg in ("decode", "prefill"):
        case = synth.config_gqa_paged_decode() if leg == "decode" else synth.config_paged_prefill_window()
        cu = case.cu_seqlens_q
        _, sk, _, _, _ = oracle.prepare_seqlens(cu, case.past_seqlens, case.T)
        kc, vc, _ = oracle.kv_cache_append(case.k_new, case.v_new, cu, sk, case.k_cache,
                                           case.v_cache, case.block_table, case.block_size)
        # per-row work: visible keys of each row
        req = np.searchsorted(cu, np.arange(case.T), side="right") - 1
        q_len = (cu[req + 1] - cu[req]).astype(np.int64)
        p = (sk[req].astype(np.int64) + 1) - q_len + (np.arange(case.T) - cu[req])
        lo = np.maximum(0, p - case.local_window + 1) if case.local_window > 0 else 0
        keys = np.maximum(0, p - lo + 1)
        args = (case.q, kc, vc, cu, sk)
        kw = dict(H_kv=case.H_kv, block_table=case.block_table, block_size=case.block_size,
                  max_seqlen_q=case.max_seqlen_q, max_seqlen_k=case.max_seqlen_k, scale=case.scale,
                  local_window=case.local_window, sinks=case.sinks)
        chunk = 1 if leg == "decode" else 16
        done, dt = pool.run_for("paged_attention", args, kw, range(case.T), workers, seconds,
                                chunk=chunk, method="fork")
        k = keys[np.asarray(done, dtype=np.int64)]
        if leg == "decode":
            kv_bytes = int(k.sum()) * case.H_kv * case.D * 2 * 2
            legs[leg] = {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s",
                         "sample": f"{len(done)} row evaluations (the 31 rows cycled) of the GQA "
                                   f"paged decode workload, {dt:.1f} s wall, KV bytes of those rows"}
        else:
            flops = int(k.sum()) * case.H_q * 4 * case.D
            legs[leg] = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
                         "sample": f"{len(done)} row evaluations (rows cycled in order) of the "
                                   f"windowed paged prefill workload, {dt:.1f} s wall, "
                                   f"algorithmic flops of those rows"}
        del case, kc, vc
    out = dict(legs["decode"])
    out.update({"cores": workers, "kind": "oracle", "host_cpus": os.cpu_count(),
                "cpu_model": _cpu_model(), "prefill": legs["prefill"]})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-sparse", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-prologue", action="store_true")
    ap.add_argument("--no-topk", action="store_true")
    ap.add_argument("--no-quant", action="store_true", help="skip the INT8 / FP8-cache workloads")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: bench.py measures one GPU "
              "(the path shards by request or by KV head with no exchange; a key range split over "
              "GPUs needs one all-gather of split partials before the merge)",
              file=sys.stderr)
        sys.exit(2)
    # the oracle's CPU baseline first: its process pool forks, which must happen before
    # anything initialises the GPU in this process
    cpu = None if args.no_cpu_baseline else cpu_baseline()
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib)
    case, ms_step, attn_ms, st = bench_decode(args.steps, args.warmup, fused=True)
    kv = _kv_bytes(case)
    gbs = kv / (ms_step * 1e-3) / 1e9
    attn_med = attn_ms[len(attn_ms) // 2]
    attn_avg = sum(attn_ms) / len(attn_ms)
    # algorithmic bytes of one step call: K/V of visible keys, Q, out, block-table entries,
    # and the new K/V rows read once and written once into the cache
    q_bytes = case.T * case.H_q * case.D * 2
    bt_bytes = sum((int(s) + 1 + 15) // 16 for s in case.seqlens_k if s >= 0) * 4
    new_bytes = 2 * (2 * case.T * case.H_kv * case.D * 2)
    alg = kv + 2 * q_bytes + bt_bytes + new_bytes
    achieved = alg / (attn_avg * 1e-3) / 1e9
    digest = kernel_sources_sha1()
    traffic = (MEASURED_TRAFFIC["bytes_per_call"]
               if MEASURED_TRAFFIC["sources_sha1"] == digest else None)
    line = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "GQA paged decode fp16: B=32, S_q=1, H_q=64, H_kv=8, D=64, "
                               "block 16, key counts U{0..8192} (one empty), 20000-block pool, sinks",
                   "kv_bytes_per_step": kv, "global_batch": case.B, "rows": case.T,
                   "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "status": st},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "paged_decode_step call: split-K kernel (with the metadata and "
                               "the append of the new rows) + merge kernel",
                     "kernel_sources_sha1": digest,
                     "avg_us": round(attn_avg * 1e3, 2), "median_us": round(attn_med * 1e3, 2),
                     "p10_p90_us": _p10_p90(attn_ms),
                     "algorithmic_bytes": alg},
    }
    _, ms2, attn2, st2 = bench_decode(args.steps, args.warmup)
    attn2_avg = sum(attn2) / len(attn2)
    line["decode_two_calls"] = {
        "workload": "the same step as prepare_and_append, then paged_attention_fwd",
        "us_per_step": round(ms2 * 1e3, 2), "gbs": round(kv / (ms2 * 1e-3) / 1e9, 1),
        "attention_call_avg_us": round(attn2_avg * 1e3, 2),
        "attention_call_gbs": round((alg - new_bytes) / (attn2_avg * 1e-3) / 1e9, 1),
        "attention_p10_p90_us": _p10_p90(attn2), "status": st2}
    if not args.no_prefill:
        line["prefill"] = bench_prefill(128, 50, 5)
        line["prefill_no_window"] = bench_prefill(-1, 30, 3)
    if not args.no_graph:
        line["decode_graph"] = bench_decode_graph()
    if not args.no_quant:
        import synth
        for tag, cdt, what in (("int8", synth.I8, "an INT8 cache"),
                               ("fp8", synth.FP8, "an FP8 E4M3 cache")):
            qcase, _, q_attn, q_st = bench_decode(50, 5, cache_dtype=cdt)
            q_kv = _kv_bytes(qcase)
            q_avg = sum(q_attn) / len(q_attn)
            line[f"decode_{tag}"] = {
                "workload": f"the GQA paged decode with {what} (per-channel scales), attention call",
                "kv_bytes_per_step": q_kv, "avg_us": round(q_avg * 1e3, 2),
                "median_us": round(q_attn[len(q_attn) // 2] * 1e3, 2),
                "p10_p90_us": _p10_p90(q_attn), "gbs": round(q_kv / (q_avg * 1e-3) / 1e9, 1),
                "frac_hbm_peak": round(q_kv / (q_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "status": q_st}
            if not args.no_prefill:
                line[f"prefill_{tag}_no_window"] = bench_prefill(-1, 20, 3, cache_dtype=cdt)
    if not args.no_sparse:
        line["selected_decode"] = bench_sparse("selected", 50, 5)
        line["local_plus_aux"] = bench_sparse("local_aux", 50, 5)
    if not args.no_prologue:
        line["prologue_decode"] = bench_prologue("decode", 50, 5)
        line["prologue_prefill"] = bench_prologue("prefill", 50, 5)
    if not args.no_topk:
        line["topk"] = bench_topk(30, 3)
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
