"""CPU oracle for paged and selected-token sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, headers, tables or constants with the HIP
library in ``selected_token_sparse_amd/``.

The oracle is the plain definition of what the operators compute, written out in numpy
with float64 arithmetic and no blocking, fusion or reordering beyond what the definition
states.  Where the pages leave a step open, the reading taken here is documented in the
function that takes it.  Pages cited (by title and section):

* "[WebGPU] Add PagedAttention metadata and GPT-OSS support" (onnxruntime PR 32277):
  Description, Changes, review findings T1 and Q3.
* "[WebGPU] Add SparsePagedAttention" (onnxruntime PR 32533): pull-request overview and
  file summaries (scatter, token metadata, main/auxiliary partials, finalize).
* "[WebGPU] Add DynamicSparseAttention" (onnxruntime PR 32529): Description (selected
  main-cache and local-plus-auxiliary modes, joint FP32 softmax with sink, guarded int32
  indices, GQA head mapping; packed QKV, QK RMSNorm, partial / interleaved RoPE with
  offsets and position IDs) and the review comments on the count-bounded loop and on
  reducing each head's RMS once.
* DynamicSparseAttention INT8 KV cache / grouped decode (onnxruntime PR 33472): Key
  Changes table (INT8 per-channel K/V with key_scale / value_scale; hierarchical / compact
  TopK selection) and its follow-up description (TopK properties: stable keys, causal
  tails, capacity padding).
* "ai.onnx.LinearAttention" kernel page: Attributes table (scale 0 selects 1/sqrt(d)).

Parity status of each function is stated in its docstring; functions whose results no
page fixes (the sanitisation of malformed inputs and the status bits) are marked
"parity unpinned".
"""
from .status import (  # noqa: F401
    STATUS_BAD_CU, STATUS_Q_BOUND, STATUS_K_BOUND, STATUS_CAPACITY, STATUS_BAD_BLOCK,
    STATUS_BAD_INDEX, STATUS_BAD_COUNT, STATUS_SHORT_KV, STATUS_CURSOR, STATUS_POSITION,
)
from .metadata import prepare_seqlens  # noqa: F401
from .append import quantize_int8, quantize_fp8_e4m3, decode_fp8_e4m3, kv_cache_append  # noqa: F401
from .attention import attend, paged_attention, sparse_attention  # noqa: F401
from .prologue import qkv_prologue, round_to  # noqa: F401
from .topk import topk_select  # noqa: F401
