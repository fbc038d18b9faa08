"""Host logic of bench.py (CPU only): the algorithmic byte and flop counts its roofline and
throughput figures divide by, pinned to closed forms and to figures derived from the
workload definitions, and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_decode_kv_bytes_is_every_key_once_per_kv_head():
    # one new row per request sees its whole history: K + V of L keys x 8 KV heads x 64 dims
    # x 2 bytes = 2048 L bytes per request
    case = synth.config_gqa_paged_decode(B=8, max_len=1500, seed=11)
    L = case.seqlens_k.astype(np.int64) + 1
    assert bench._kv_bytes(case) == int(L.sum()) * 2048


def test_prefill_flops_match_the_visible_pair_counts():
    # fresh prompts of 1024, 512, 2048 and 1536 tokens: a causal row at position p sees p + 1
    # keys, so a prompt of n tokens has n (n + 1) / 2 pairs; with a 128-key window a row
    # sees min(p + 1, 128), i.e. n (n + 1) / 2 - (n - 128) (n - 127) / 2 pairs
    lens = (1024, 512, 2048, 1536)
    causal = sum(n * (n + 1) // 2 for n in lens)
    window = sum(n * (n + 1) // 2 - (n - 128) * (n - 127) // 2 for n in lens)
    assert causal == 3_934_720 and window == 622_848
    for w, pairs in ((-1, causal), (128, window)):
        case = synth.config_paged_prefill_window(window=w)
        assert bench._prefill_flops(case) == pairs * 64 * 4 * 64


def test_local_plus_aux_bytes():
    # every row sits at p >= 127 of its request, so it sees a full 128-key INT8 window; all
    # 1024 selected auxiliary rows are in range
    case = synth.config_local_plus_aux_int8(B=2, capacity=4096)
    T, H_kv, D = case.T, case.H_kv, case.D
    total, main_keys, aux_keys = bench._sparse_bytes(case)
    assert main_keys == T * 128 * H_kv
    assert aux_keys == T * H_kv * 1024
    assert total == main_keys * 2 * D * 1 + aux_keys * 2 * D * 2 + 2 * T * case.H_q * D * 2


def test_selected_bytes_count_visible_entries_one_by_one():
    case = synth.sparse_selected_case(7, B=3, S_q=4, H_q=24, H_kv=2, D=128, capacity=900,
                                      max_selected=300, dtype=synth.F16, oor_frac=0.05)
    cu = case.cu_seqlens_q
    visible = 0
    for b in range(case.B):
        q_len = int(cu[b + 1] - cu[b])
        kv = int(case.seqlens_k[b]) + 1
        for i in range(q_len):
            r, p = int(cu[b]) + i, kv - q_len + i
            for c in range(case.H_kv):
                n = min(max(int(case.sel_count[r, c]), 0), case.max_selected)
                for t in range(n):
                    j = int(case.sel_idx[r, c, t])
                    if 0 <= j <= p and j < kv:
                        visible += 1
    total, main_keys, aux_keys = bench._sparse_bytes(case)
    assert main_keys == visible and aux_keys == 0
    assert total == visible * 2 * case.D * 2 + 2 * case.T * case.H_q * case.D * 2


def test_percentiles_of_sorted_call_times():
    ms = [0.001 * (i + 1) for i in range(100)]        # 1 .. 100 us
    assert bench._p10_p90(ms) == (11.0, 91.0)
    assert bench._p10_p90([0.005]) == (5.0, 5.0)


def test_prefill_bytes_are_q_out_and_each_visible_key_once():
    # fresh prompts: Q and out 5120 rows x 64 heads x 64 dims x 2 bytes each; every key of
    # a prompt is seen by some row, so K + V once per KV head: 5120 x 8 x 64 x 2 x 2
    for w in (128, -1):
        case = synth.config_paged_prefill_window(window=w)
        assert bench._prefill_bytes(case) == 2 * 5120 * 64 * 64 * 2 + 5120 * 8 * 64 * 4
    # a chunk of 40 rows after 160 past keys with a 50-key window sees positions 111..199
    case = synth.paged_case(3, kv_lens=[200], q_lens=[40], H_q=8, H_kv=2, D=64,
                            dtype=synth.F16, local_window=50)
    assert bench._prefill_bytes(case) == 2 * 40 * 8 * 64 * 2 + 89 * 2 * 64 * 2 * 2
