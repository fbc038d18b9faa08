"""GPU parity of topk_select against the oracle: index work, so bit-exact (every selected
position, the -1 padding and every count).  Scores are compared, never computed, so both
sides take every decision on the same float32 values."""
import numpy as np
import pytest
import torch

import oracle
import selected_token_sparse_amd as sta
import synth
from synth.device import tensor

from harness import assert_close, status_tensor

pytestmark = pytest.mark.gpu


def _run(case):
    sel = torch.full((case.T, case.H_kv, case.capacity), 12345, dtype=torch.int32, device="cuda")
    cnt = torch.full((case.T, case.H_kv), 12345, dtype=torch.int32, device="cuda")
    st = status_tensor()
    sta.topk_select(tensor(case.scores), tensor(case.cu_seqlens_q), tensor(case.seqlens_k), case.k,
                    sel, cnt, tail=case.tail, status=st)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), cnt.cpu().numpy(), int(st.item())


def _check(case, what):
    print("topk", what, flush=True)
    sel, cnt, st = _run(case)
    want_sel, want_cnt = oracle.topk_select(case.scores, case.cu_seqlens_q, case.seqlens_k,
                                            k=case.k, tail=case.tail, capacity=case.capacity)
    assert st == 0
    assert np.array_equal(cnt, want_cnt), f"{what}: counts differ"
    if not np.array_equal(sel, want_sel):
        bad = np.argwhere((sel != want_sel).any(axis=-1))[:3]
        t, c = bad[0]
        raise AssertionError(f"{what}: selections differ at {bad.tolist()}: gpu {sel[t, c][:12]} "
                             f"oracle {want_sel[t, c][:12]}")


VARIANTS = [
    # (name, kv_lens, q_lens, H_kv, L, k, tail, capacity, ties, specials)
    ("tiny_L_kpt4", [60, 9], [4, 9], 2, 64, 16, 3, 20, 0.5, 0.1),
    ("L3000_ties", [3000, 2000], [8, 8], 4, 3000, 512, 0, 512, 0.6, 0.0),
    ("L5000_kpt8_specials_tail", [5000, 4000], [3, 5], 2, 5000, 600, 32, 640, 0.3, 0.05),
    ("L4998_unaligned", [4998, 4000], [4, 4], 2, 4998, 700, 8, 700, 0.3, 0.02),
    ("L12000_kpt16", [12000, 9000], [8, 8], 2, 12000, 1024, 0, 1030, 0.3, 0.01),
    ("L20000_kpt32", [20000, 12000], [8, 8], 4, 20000, 2048, 64, 2048, 0.2, 0.01),
    ("L65536_kpt64", [65536], [8], 4, 65536, 2048, 16, 2048, 0.3, 0.01),
    ("tail_ge_k", [3000], [4], 2, 3000, 100, 150, 100, 0.0, 0.0),
    ("k0", [300], [3], 1, 300, 0, 5, 4, 0.0, 0.0),
    ("all_fit", [100, 40], [100, 40], 1, 128, 128, 4, 130, 0.0, 0.0),
    ("prefill_rows_vary", [700, 300, 1], [700, 50, 1], 3, 700, 128, 16, 128, 0.4, 0.02),
]


@pytest.mark.parametrize("v", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_topk_variants(v):
    name, kv, ql, H, L, k, tail, cap, ties, spec = v
    case = synth.topk_case(sum(map(ord, name)), kv_lens=kv, q_lens=ql, H_kv=H, L=L, k=k, tail=tail,
                           capacity=cap, ties=ties, specials=spec, name=name)
    _check(case, name)


# Rows longer than 16384 candidates take the streaming path (persistent workgroups, the
# next segment's scores copied under the current one's selection); these cases walk its
# branches: several segments a workgroup with rows that select everything in between, one-
# and two-word rows, ranked counts on both sides of the 32768-position word edge, no
# ranked selection (tail >= k, k = 0), no tail, NaN / -0 scores and the shortest row
# length that takes the path.
STREAM_VARIANTS = [
    # (name, kv_lens, q_lens, H_kv, L, k, tail, capacity, ties, specials)
    ("stream_many_segments", [20000, 100, 17000, 2500], [40, 30, 20, 10], 4, 20000, 1024, 16,
     1100, 0.2, 0.01),
    ("stream_two_words_mixed", [65536, 30000, 32833, 40000], [8, 8, 3, 8], 4, 65536, 2048, 64,
     2048, 0.1, 0.005),
    ("stream_tail_covers_k", [30000, 25000], [3, 2], 2, 30000, 100, 150, 128, 0.0, 0.0),
    ("stream_k0", [30000], [2], 2, 30000, 0, 5, 4, 0.0, 0.0),
    ("stream_no_tail_specials", [50000, 49000], [4, 4], 2, 50000, 3000, 0, 3000, 0.3, 0.05),
    ("stream_L16388", [16388, 16000], [4, 4], 3, 16388, 700, 8, 700, 0.3, 0.02),
]


@pytest.mark.parametrize("v", STREAM_VARIANTS, ids=[v[0] for v in STREAM_VARIANTS])
def test_topk_stream_variants(v):
    name, kv, ql, H, L, k, tail, cap, ties, spec = v
    case = synth.topk_case(sum(map(ord, name)), kv_lens=kv, q_lens=ql, H_kv=H, L=L, k=k, tail=tail,
                           capacity=cap, ties=ties, specials=spec, name=name)
    _check(case, name)


@pytest.mark.parametrize("L", [3000, 40000], ids=["L3000", "L40000"])
def test_rows_owned_by_no_request(L):
    """Rows past cu[B] belong to no request: count 0, every slot -1 and the BAD_CU status
    bit; the owned rows still match the oracle."""
    case = synth.topk_case(L, kv_lens=[L, L // 2], q_lens=[3, 2], H_kv=2, L=L, k=256, tail=8,
                           capacity=260, ties=0.1, specials=0.01)
    extra = 3
    scores = np.concatenate([case.scores, np.ones((extra,) + case.scores.shape[1:], np.float32)])
    sel = torch.full((case.T + extra, 2, 260), 777, dtype=torch.int32, device="cuda")
    cnt = torch.full((case.T + extra, 2), 777, dtype=torch.int32, device="cuda")
    st = status_tensor()
    print("topk rows owned by no request", L, flush=True)
    sta.topk_select(tensor(scores), tensor(case.cu_seqlens_q), tensor(case.seqlens_k), case.k,
                    sel, cnt, tail=case.tail, status=st)
    torch.cuda.synchronize()
    sel, cnt = sel.cpu().numpy(), cnt.cpu().numpy()
    assert int(st.item()) & sta.STATUS_BAD_CU
    assert (cnt[case.T:] == 0).all() and (sel[case.T:] == -1).all()
    want_sel, want_cnt = oracle.topk_select(case.scores, case.cu_seqlens_q, case.seqlens_k,
                                            k=case.k, tail=case.tail, capacity=260)
    assert np.array_equal(cnt[:case.T], want_cnt)
    assert np.array_equal(sel[:case.T], want_sel)


def test_all_equal_scores_take_the_lowest_positions():
    case = synth.topk_case(3, kv_lens=[40000], q_lens=[2], H_kv=2, L=40000, k=1000, tail=10)
    case.scores[:] = 0.5
    case.scores[0, 1, ::7] = -0.0
    case.scores[1, 0, 5::3] = np.nan
    _check(case, "all equal")
    sel, cnt, _ = _run(case)
    assert sel[0, 0, :990].tolist() == list(range(990))


def test_selected_decode_shape():
    """The selected grouped decode workload's shape: 128 rows (16 requests x 8), 4 KV heads,
    65536 candidates, k = 2048 with a 64-key causal tail."""
    case = synth.topk_case(1004, kv_lens=[65536] * 16, q_lens=[8] * 16, H_kv=4, L=65536, k=2048,
                           tail=64, capacity=2048, ties=0.05, specials=0.001)
    _check(case, "selected decode shape")


def test_topk_feeds_sparse_attention():
    """TopK then selected-token attention on the GPU against the oracle's TopK then attention."""
    sc = synth.sparse_selected_case(31, B=3, S_q=4, H_q=24, H_kv=2, D=128, capacity=3000,
                                    max_selected=256, dtype=synth.F16, sinks=True)
    tk = synth.topk_case(32, kv_lens=sc.seqlens_k + 1, q_lens=np.diff(sc.cu_seqlens_q), H_kv=2,
                         L=3000, k=256, tail=8, capacity=256, ties=0.2, specials=0.01)
    sel = torch.empty((tk.T, 2, 256), dtype=torch.int32, device="cuda")
    cnt = torch.empty((tk.T, 2), dtype=torch.int32, device="cuda")
    sta.topk_select(tensor(tk.scores), tensor(tk.cu_seqlens_q), tensor(tk.seqlens_k), 256, sel, cnt, tail=8)
    want_sel, want_cnt = oracle.topk_select(tk.scores, tk.cu_seqlens_q, tk.seqlens_k, k=256, tail=8,
                                            capacity=256)
    out = torch.empty((sc.T, sc.H_q, sc.D), dtype=torch.float16, device="cuda")
    sta.sparse_attention_fwd(tensor(sc.q, sc.dtype), 0, tensor(sc.k_cache, sc.dtype),
                             tensor(sc.v_cache, sc.dtype), tensor(sc.cu_seqlens_q), tensor(sc.seqlens_k),
                             sc.max_seqlen_q, sel, out, sel_count=cnt, scale=sc.scale,
                             sinks=tensor(sc.sinks))
    torch.cuda.synchronize()
    ref, _ = oracle.sparse_attention(sc.q, 0, sc.k_cache, sc.v_cache, sc.cu_seqlens_q, sc.seqlens_k,
                                     want_sel, want_cnt, 256, H_kv=2, max_seqlen_q=sc.max_seqlen_q,
                                     scale=sc.scale, sinks=sc.sinks)
    assert_close(out, ref, sc.dtype, "topk + sparse attention")
