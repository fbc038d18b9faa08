"""Device-side sequence metadata, defined on the CPU.

"[WebGPU] Add PagedAttention metadata and GPT-OSS support", Description and Changes: the
exact per-request query length and key length are derived on the device from the
cumulative query offsets and the past (cached) lengths, so no host readback is needed;
review finding T1 gives the worked examples (new lengths [2, 0] -> seqlens_q [2, 0],
seqlen_k [1, -1]; new lengths [1, 2] -> seqlens_q [1, 2], seqlen_k [0, 1]).
"[WebGPU] Add SparsePagedAttention", file summaries: a token-metadata stage resolves, per
packed token, its request and position (the review flags a per-token linear scan; the
result is the same whatever the search).
"""
from __future__ import annotations

import numpy as np

from .status import STATUS_BAD_CU


def prepare_seqlens(cu_seqlens_q, past_seqlens, T: int):
    """Per-request lengths and per-token (request, position) from cumulative offsets.

    For a well-formed ``cu`` (``cu[0] = 0``, non-decreasing, ``cu[B] = T``) and
    ``past >= 0`` (pinned by the page's worked examples and by the definitions):

    * ``seqlens_q[b] = cu[b+1] - cu[b]``
    * ``seqlens_k[b] = past[b] + seqlens_q[b] - 1`` (total keys minus one; -1 = empty)
    * for ``cu[b] <= t < cu[b+1]``: ``token_req[t] = b`` and
      ``token_pos[t] = past[b] + (t - cu[b])`` (the key position of the row).

    Malformed input (parity unpinned, this library's own reading): the status bit
    STATUS_BAD_CU is set; each boundary is replaced by the running maximum of
    ``cu[0..b]`` clamped to ``[0, T]`` and a negative ``past`` by 0, and the definitions
    above are applied to the sanitised values; rows outside every request get
    ``token_req = token_pos = -1``.

    Returns ``(seqlens_q, seqlens_k, token_req, token_pos, status)``.
    """
    cu = [int(x) for x in np.asarray(cu_seqlens_q).reshape(-1)]
    past = [int(x) for x in np.asarray(past_seqlens).reshape(-1)]
    B = len(past)
    assert len(cu) == B + 1
    status = 0
    well_formed = cu[0] == 0 and cu[B] == T and all(cu[b] <= cu[b + 1] for b in range(B))
    if not well_formed or any(p < 0 for p in past):
        status |= STATUS_BAD_CU

    bound = []
    running = cu[0]
    for b in range(B + 1):
        running = max(running, cu[b])
        bound.append(min(max(running, 0), T))

    seqlens_q = np.zeros(B, dtype=np.int32)
    seqlens_k = np.zeros(B, dtype=np.int32)
    token_req = np.full(T, -1, dtype=np.int32)
    token_pos = np.full(T, -1, dtype=np.int32)
    for b in range(B):
        q_len = bound[b + 1] - bound[b]
        p0 = max(past[b], 0)
        seqlens_q[b] = q_len
        seqlens_k[b] = p0 + q_len - 1
        for t in range(bound[b], bound[b + 1]):
            token_req[t] = b
            token_pos[t] = p0 + (t - bound[b])
    return seqlens_q, seqlens_k, token_req, token_pos, status
