"""Status bits reported for malformed device-side inputs (this library's own contract).

The DynamicSparseAttention INT8 page (onnxruntime PR 33472, Key Changes table) adds a
device ``validation_status`` output but never defines its codes, so the bits below are
ours.  Each bit is informational: the affected keys are excluded or the affected rows are
written as zeros, never read or written out of bounds.  Parity unpinned (no page fixes
these values; the GPU path is compared with this definition bit for bit).
"""
STATUS_BAD_CU = 1 << 0      # cu_seqlens_q not 0 = cu[0] <= ... <= cu[B] = T, or past < 0
STATUS_Q_BOUND = 1 << 1     # a request's query length exceeds max_seqlen_q: its rows are 0
STATUS_K_BOUND = 1 << 2     # a request's key count exceeds max_seqlen_k: its rows are 0
STATUS_CAPACITY = 1 << 3    # a needed key position lies beyond the cache capacity
STATUS_BAD_BLOCK = 1 << 4   # a needed block-table entry is outside [0, num_blocks)
STATUS_BAD_INDEX = 1 << 5   # a selected index (inside the count) is neither -1 nor in range
STATUS_BAD_COUNT = 1 << 6   # a selected count outside [0, max_selected] (clamped)
STATUS_SHORT_KV = 1 << 7    # a request has fewer keys than query rows
STATUS_CURSOR = 1 << 8      # committed_length disagrees with the append position: nothing appended
STATUS_POSITION = 1 << 9    # a rotary position outside [0, max_position): row's Q is 0, K/V not appended
