"""Seeded synthetic inputs shared by the tests, the oracle checks and the benchmark.

This package only draws input arrays (lengths, block tables, index lists, Q/K/V values,
sinks, scales).  It holds none of the attention arithmetic: the metadata, the cache append
and the attention itself are computed separately by ``oracle/`` (CPU) and by the HIP
library (GPU).  The value of ``seqlens_k`` it emits is an *input* of the attention
operators (the total key count minus one, the convention the PagedAttention metadata page
uses for its worked examples), chosen together with the other lengths it draws.
"""
from .workloads import (  # noqa: F401
    BF16, F16, F32, I8, FP8, QUANTISED, DTYPE_NAMES,
    PagedCase, SparseCase, PrologueCase, TopkCase,
    paged_case, prologue_case, rotary_tables, topk_case, sparse_selected_case, sparse_local_aux_case,
    config_tiny_paged_decode, config_gqa_paged_decode, config_paged_prefill_window,
    config_selected_decode, config_local_plus_aux_int8,
    round_bf16,
)
