"""Shared helpers of the GPU parity tests: run the HIP path through the Python binding of
the C ABI, run the oracle on the same host arrays, and compare with the tolerance the
arithmetic allows."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import selected_token_sparse_amd as sta
import synth
from synth.device import TORCH_DTYPE, case_tensors

# |gpu - ref| <= ATOL + RTOL * |ref|, per output element, ref = float64 oracle
TOL = {
    synth.F32: (1e-5, 1e-5),
    synth.F16: (2e-3, 2e-3),
    synth.BF16: (2e-3, 2e-3),
}


def assert_close(gpu: torch.Tensor, ref: np.ndarray, dtype: int, what: str = ""):
    """f32 / f16 outputs: |gpu - ref| <= atol + rtol |ref|.  bf16 outputs are compared with
    the oracle rounded to bf16: the bf16 value the GPU wrote must be the rounding of some
    value within atol + rtol |ref| of the oracle, i.e. lie in [bf16(ref - tol),
    bf16(ref + tol)] (round to nearest even is monotonic; the bounds are rounded from
    float64 once, by the oracle's pinned bf16 rounding).  No slack is added for the
    kernel's own intermediate roundings."""
    g = gpu.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    atol, rtol = TOL[dtype]
    finite = np.isfinite(ref)
    assert np.all(np.isfinite(g[finite])), f"{what}: non-finite GPU values where the oracle is finite"
    tol = atol + rtol * np.abs(ref)
    err = np.abs(g - ref)
    if dtype == synth.BF16:
        lo = oracle.round_to(ref - tol, "bf16").astype(np.float64)
        hi = oracle.round_to(ref + tol, "bf16").astype(np.float64)
        bad = (g < lo) | (g > hi)
    else:
        bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance "
            f"(max err {err.max():.3e}); first at {idx.tolist()}: gpu {g[tuple(idx[0])]} ref {ref[tuple(idx[0])]}")
    return float(err.max()) if err.size else 0.0


def status_tensor():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


def run_paged_step(case, t=None, append=True, use_prepare=True, status=None, out=None):
    """prepare_seqlens -> kv_cache_append -> paged_attention_fwd on the GPU.
    Returns (out, seqlens_k used, tensors)."""
    t = t if t is not None else case_tensors(case)
    status = status if status is not None else status_tensor()
    if use_prepare:
        sq = torch.empty(case.B, dtype=torch.int32, device="cuda")
        sk = torch.empty(case.B, dtype=torch.int32, device="cuda")
        sta.prepare_seqlens(t["cu"], t["past"], case.T, sq, sk, status=status)
    else:
        sk = t["seqlens_k"]
    if append and case.T > 0:
        sta.kv_cache_append(t["k_new"], t["v_new"], t["cu"], sk, t["k_cache"], t["v_cache"],
                            t["block_table"], t["key_scale"], t["value_scale"], status=status)
    if out is None:
        out = torch.empty((case.T, case.H_q, case.D), dtype=TORCH_DTYPE[case.dtype], device="cuda")
    sta.paged_attention_fwd(t["q"], t["k_cache"], t["v_cache"], t["cu"], sk, case.max_seqlen_q,
                            case.max_seqlen_k, out, block_table=t["block_table"],
                            key_scale=t["key_scale"], value_scale=t["value_scale"],
                            scale=case.scale, local_window=case.local_window, sinks=t["sinks"],
                            status=status)
    return out, sk, t, status


def oracle_paged_step(case, rows=None, append=True, workers=1):
    """The oracle's view of the same step: metadata, append, attention (the attention rows
    spread over `workers` processes by oracle.pool when workers > 1)."""
    sq, sk, _, _, st0 = oracle.prepare_seqlens(case.cu_seqlens_q, case.past_seqlens, case.T)
    kc, vc = case.k_cache, case.v_cache
    st1 = 0
    if append:
        kc, vc, st1 = oracle.kv_cache_append(case.k_new, case.v_new, case.cu_seqlens_q, sk, kc, vc,
                                             case.block_table, case.block_size, case.key_scale,
                                             case.value_scale)
    kw = dict(H_kv=case.H_kv, block_table=case.block_table, block_size=case.block_size,
              key_scale=case.key_scale, value_scale=case.value_scale,
              max_seqlen_q=case.max_seqlen_q, max_seqlen_k=case.max_seqlen_k, scale=case.scale,
              local_window=case.local_window, sinks=case.sinks, rows=rows)
    if workers > 1:
        from oracle import pool
        todo = range(case.T) if rows is None else sorted(rows)
        del kw["rows"]
        out, st2 = pool.map_rows("paged_attention", (case.q, kc, vc, case.cu_seqlens_q, sk), kw,
                                 todo, workers)
    else:
        out, st2 = oracle.paged_attention(case.q, kc, vc, case.cu_seqlens_q, sk, **kw)
    return out, st0 | st1 | st2


def run_sparse(case, t=None, status=None, out=None):
    t = t if t is not None else case_tensors(case)
    status = status if status is not None else status_tensor()
    if out is None:
        out = torch.empty((case.T, case.H_q, case.D), dtype=TORCH_DTYPE[case.dtype], device="cuda")
    sta.sparse_attention_fwd(t["q"], case.mode, t["k_cache"], t["v_cache"], t["cu"], t["seqlens_k"],
                             case.max_seqlen_q, t["sel_idx"], out, sel_count=t["sel_count"],
                             block_table=t["block_table"], key_scale=t["key_scale"],
                             value_scale=t["value_scale"], local_window=case.local_window,
                             aux_k=t["aux_k"], aux_v=t["aux_v"],
                             aux_batch_stride=case.aux_batch_stride if case.mode == 1 else None,
                             scale=case.scale, sinks=t["sinks"], status=status)
    return out, t, status


def oracle_sparse(case, rows=None):
    """(out, status) of the oracle."""
    return oracle.sparse_attention(
        case.q, case.mode, case.k_cache, case.v_cache, case.cu_seqlens_q, case.seqlens_k,
        case.sel_idx, case.sel_count, case.max_selected, H_kv=case.H_kv,
        block_table=case.block_table, block_size=case.block_size, key_scale=case.key_scale,
        value_scale=case.value_scale, max_seqlen_q=case.max_seqlen_q,
        local_window=case.local_window, aux_k=case.aux_k, aux_v=case.aux_v, aux_len=case.aux_len,
        aux_batch_stride=case.aux_batch_stride, scale=case.scale, sinks=case.sinks, rows=rows)
