"""Upload a synthetic case to device tensors (torch is only the memory allocator here)."""
from __future__ import annotations

import numpy as np
import torch

from .workloads import BF16, F16, F32, FP8, I8

TORCH_DTYPE = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16, I8: torch.int8,
               FP8: torch.float8_e4m3fn}


def tensor(x, dtype: int = None, device="cuda"):
    """numpy -> device tensor; bf16 data (carried as float32) is converted exactly, FP8
    E4M3 codes (carried as uint8) are reinterpreted as float8_e4m3fn."""
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == BF16:
        t = t.to(torch.bfloat16)
    elif dtype == FP8:
        t = t.view(torch.float8_e4m3fn)
    return t.to(device)


def case_tensors(case, device="cuda") -> dict:
    """Every array of a PagedCase / SparseCase as a device tensor (None stays None)."""
    d = {
        "q": tensor(case.q, case.dtype, device),
        "cu": tensor(case.cu_seqlens_q, None, device),
        "seqlens_k": tensor(case.seqlens_k, None, device),
        "k_cache": tensor(case.k_cache, case.cache_dtype, device),
        "v_cache": tensor(case.v_cache, case.cache_dtype, device),
        "block_table": tensor(case.block_table, None, device),
        "key_scale": tensor(case.key_scale, None, device),
        "value_scale": tensor(case.value_scale, None, device),
        "sinks": tensor(case.sinks, None, device),
    }
    if hasattr(case, "past_seqlens"):
        d["past"] = tensor(case.past_seqlens, None, device)
        d["k_new"] = tensor(case.k_new, case.dtype, device)
        d["v_new"] = tensor(case.v_new, case.dtype, device)
    if hasattr(case, "sel_idx"):
        d["sel_idx"] = tensor(case.sel_idx, None, device)
        d["sel_count"] = tensor(case.sel_count, None, device)
        d["aux_k"] = tensor(case.aux_k, case.aux_dtype, device)
        d["aux_v"] = tensor(case.aux_v, case.aux_dtype, device)
    return d
