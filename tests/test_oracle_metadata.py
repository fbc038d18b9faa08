"""Pins of the oracle's metadata definition (CPU only).

Against: the worked examples of the PagedAttention metadata page (golden fixture), a
library search (numpy.searchsorted) for the token-to-request map, and closed-form
relations between the outputs.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_page_worked_examples():
    with open(os.path.join(GOLDEN, "metadata_examples.json")) as f:
        data = json.load(f)
    for case in data["cases"]:
        sq, sk, req, pos, st = oracle.prepare_seqlens(case["cu_seqlens_q"], case["past_seqlens"], case["T"])
        assert sq.tolist() == case["seqlens_q"], case["note"]
        assert sk.tolist() == case["seqlens_k"], case["note"]
        assert st == 0


@pytest.mark.parametrize("seed", range(20))
def test_well_formed_random(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 12))
    q_lens = rng.integers(0, 6, size=B)
    past = rng.integers(0, 50, size=B).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(cu[-1])
    sq, sk, req, pos, st = oracle.prepare_seqlens(cu, past, T)
    assert st == 0
    assert sq.tolist() == q_lens.tolist()
    # the key count is past + new rows; an empty request (no past, no rows) is -1
    assert (sk + 1).tolist() == (past + q_lens).tolist()
    assert all(sk[b] == -1 for b in range(B) if past[b] == 0 and q_lens[b] == 0)
    # token -> request agrees with a library search over the offsets
    t = np.arange(T)
    assert req.tolist() == (np.searchsorted(cu, t, side="right") - 1).tolist()
    # positions: the last row of each non-empty request is its newest key (seqlens_k),
    # and rows of a request occupy consecutive positions
    for b in range(B):
        if q_lens[b]:
            assert pos[cu[b + 1] - 1] == sk[b]
            assert np.all(np.diff(pos[cu[b]:cu[b + 1]]) == 1)


@pytest.mark.parametrize("cu,past,T", [
    ([1, 2, 3], [0, 0], 3),          # cu[0] != 0
    ([0, 3, 2, 4], [0, 0, 0], 4),    # decreasing
    ([0, 2, 9], [0, 0], 5),          # cu[B] > T
    ([0, 2, 3], [0, 0], 5),          # cu[B] < T
    ([0, 1, 2], [-4, 0], 2),         # negative past
    ([-3, 5, 1, 7], [1, 2, 3], 6),   # several faults at once
])
def test_malformed_is_flagged_and_in_range(cu, past, T):
    sq, sk, req, pos, st = oracle.prepare_seqlens(cu, past, T)
    assert st & oracle.STATUS_BAD_CU
    assert np.all(sq >= 0) and int(sq.sum()) <= T
    assert np.all((req >= -1) & (req < len(past)))
    assert np.all((req == -1) == (pos == -1))
    for t in range(T):
        if req[t] >= 0:
            assert 0 <= pos[t] <= sk[req[t]]
