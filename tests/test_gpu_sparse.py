"""GPU parity: sparse_attention_fwd (selected main-cache rows; local window plus selected
auxiliary rows with an INT8 main cache) against the oracle."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import selected_token_sparse_amd as sta
import synth
from synth.device import case_tensors, tensor

from harness import assert_close, oracle_sparse, run_sparse

pytestmark = pytest.mark.gpu


def _check(case, what, rows=None):
    print("sparse", what, flush=True)
    out, _, st = run_sparse(case)
    torch.cuda.synchronize()
    ref, ost = oracle_sparse(case, rows=rows)
    g = out if rows is None else out[rows]
    err = assert_close(g, ref, case.dtype, what)
    if rows is None:
        assert int(st.item()) == ost, (int(st.item()), ost)
    return err


SELECTED = [
    ("f16_g12_d128_sink", dict(B=2, S_q=8, H_q=24, H_kv=2, D=128, capacity=3000, max_selected=300, dtype=synth.F16, sinks=True, oor_frac=0.05)),
    ("f16_g12_nosink", dict(B=3, S_q=8, H_q=12, H_kv=1, D=128, capacity=2000, max_selected=700, dtype=synth.F16, sinks=False, oor_frac=0.01)),
    ("bf16_g4_d64", dict(B=2, S_q=3, H_q=8, H_kv=2, D=64, capacity=500, max_selected=64, dtype=synth.BF16, sinks=True, oor_frac=0.1)),
    ("f16_nocount", dict(B=2, S_q=2, H_q=8, H_kv=2, D=64, capacity=400, max_selected=40, dtype=synth.F16, sinks=True, pass_count=False)),
    ("f16_i8_main", dict(B=2, S_q=4, H_q=12, H_kv=1, D=128, capacity=900, max_selected=200, dtype=synth.F16, cache_dtype=synth.I8, sinks=True, oor_frac=0.02)),
    ("f16_fp8_main", dict(B=2, S_q=4, H_q=12, H_kv=1, D=128, capacity=900, max_selected=200, dtype=synth.F16, cache_dtype=synth.FP8, sinks=True, oor_frac=0.02)),
    ("f32_g3", dict(B=2, S_q=2, H_q=6, H_kv=2, D=64, capacity=300, max_selected=50, dtype=synth.F32, sinks=True, oor_frac=0.05)),
    ("f16_paged_main", dict(B=3, S_q=2, H_q=16, H_kv=2, D=64, capacity=600, kv_lens=[600, 250, 17], max_selected=128, dtype=synth.F16, sinks=True, block_size=16, oor_frac=0.03)),
    ("f16_g20_two_tiles", dict(B=1, S_q=2, H_q=40, H_kv=2, D=64, capacity=300, max_selected=90, dtype=synth.F16, sinks=True)),
    # 16384 selected positions of a 100k-key cache
    ("f16_16k_of_100k", dict(B=1, S_q=2, H_q=12, H_kv=1, D=128, capacity=100000, max_selected=16384, dtype=synth.F16, sinks=True, oor_frac=0.01)),
]


@pytest.mark.parametrize("name,kw", SELECTED, ids=[s[0] for s in SELECTED])
def test_selected_variants(name, kw):
    case = synth.sparse_selected_case(zlib.crc32(name.encode()) % 1000, poison=True, **kw)
    _check(case, name)


def test_selected_batch_beyond_staged_metadata():
    """520 requests of one row each: the request lookup runs in global memory (more than
    512 staged boundaries); ragged key counts, paged and contiguous main caches."""
    kv = np.random.default_rng(520).integers(1, 300, size=520)
    case = synth.sparse_selected_case(520, B=520, S_q=1, H_q=8, H_kv=2, D=64, capacity=300,
                                      kv_lens=kv, max_selected=96, dtype=synth.F16, sinks=True,
                                      oor_frac=0.02, poison=True)
    _check(case, "f16_B520")
    case = synth.sparse_selected_case(521, B=520, S_q=1, H_q=8, H_kv=2, D=64, capacity=300,
                                      kv_lens=kv, max_selected=64, dtype=synth.F16, sinks=True,
                                      block_size=16)
    _check(case, "f16_B520_paged")


def test_selected_counts_zero_and_full_and_bad():
    T, H_kv = 6, 2
    counts = np.array([[0, 40], [40, 0], [-3, 17], [55, 1], [40, 40], [2, 0]])
    case = synth.sparse_selected_case(61, B=2, S_q=3, H_q=8, H_kv=2, D=64, capacity=200,
                                      max_selected=40, counts=np.clip(counts, 0, 40),
                                      dtype=synth.F16, sinks=True, poison=True)
    case.sel_count = counts.astype(np.int32)        # out-of-range counts are clamped + flagged
    _check(case, "counts")


LOCAL_AUX = [
    ("i8_main_f16_aux", dict(B=2, S_q=8, H_q=24, H_kv=2, D=128, capacity=700, local_window=128, aux_len=600, n_selected=100, dtype=synth.F16, cache_dtype=synth.I8)),
    ("f16_main_shared_aux", dict(B=3, S_q=2, H_q=8, H_kv=2, D=64, capacity=300, kv_lens=[300, 100, 5], local_window=20, aux_len=90, n_selected=30, max_selected=40, dtype=synth.F16, cache_dtype=synth.F16, shared_aux=True)),
    ("bf16_i8_main", dict(B=2, S_q=4, H_q=8, H_kv=2, D=64, capacity=200, local_window=7, aux_len=50, n_selected=9, max_selected=16, dtype=synth.BF16, cache_dtype=synth.I8, oor_frac=0.1)),
    ("f32_i8_main", dict(B=1, S_q=3, H_q=4, H_kv=1, D=64, capacity=64, local_window=10, aux_len=40, n_selected=12, dtype=synth.F32, cache_dtype=synth.I8)),
    ("fp8_main_f16_aux", dict(B=2, S_q=8, H_q=24, H_kv=2, D=128, capacity=700, local_window=128, aux_len=600, n_selected=100, dtype=synth.F16, cache_dtype=synth.FP8)),
    ("bf16_fp8_main", dict(B=2, S_q=4, H_q=8, H_kv=2, D=64, capacity=200, local_window=7, aux_len=50, n_selected=9, max_selected=16, dtype=synth.BF16, cache_dtype=synth.FP8, oor_frac=0.1)),
    ("f16_long_window", dict(B=1, S_q=2, H_q=12, H_kv=1, D=128, capacity=1000, local_window=600, aux_len=700, n_selected=500, max_selected=520, dtype=synth.F16, cache_dtype=synth.F16)),
]


@pytest.mark.parametrize("name,kw", LOCAL_AUX, ids=[s[0] for s in LOCAL_AUX])
def test_local_aux_variants(name, kw):
    case = synth.sparse_local_aux_case(zlib.crc32(name.encode()) % 1000, sinks=True, **kw)
    _check(case, name)


def test_selected_single_key_is_the_value_row():
    # one selected, visible entry and no sink: out equals that V row bit for bit
    case = synth.sparse_selected_case(62, B=2, S_q=2, H_q=8, H_kv=2, D=64, capacity=100,
                                      max_selected=8, counts=np.ones((4, 2)), dtype=synth.F16,
                                      sinks=False)
    out, _, _ = run_sparse(case)
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    for r in range(case.T):
        b = r // 2
        for c in range(2):
            j = int(case.sel_idx[r, c, 0])
            p = 99 - 1 + (r % 2)
            want = case.v_cache[b, c, j] if j <= p else np.zeros(64, np.float16)
            for h in range(4 * c, 4 * c + 4):
                assert np.array_equal(g[r, h].view(np.int16), want.view(np.int16))


def test_sparse_argument_errors():
    case = synth.sparse_selected_case(63, B=1, S_q=1, H_q=4, H_kv=2, D=64, capacity=10,
                                      max_selected=4, dtype=synth.F16)
    t = case_tensors(case)
    out = torch.empty((1, 4, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(sta.SpattnError) as e:   # mode 0 takes no window
        sta.sparse_attention_fwd(t["q"], 0, t["k_cache"], t["v_cache"], t["cu"], t["seqlens_k"], 1,
                                 t["sel_idx"], out, local_window=4)
    assert e.value.rc == -4
    with pytest.raises(sta.SpattnError) as e:   # mode 1 needs a window and an aux store
        sta.sparse_attention_fwd(t["q"], 1, t["k_cache"], t["v_cache"], t["cu"], t["seqlens_k"], 1,
                                 t["sel_idx"], out, local_window=4)
    assert e.value.rc == -1


# ---------------- full-size workloads, every row ----------------

def test_full_selected_decode_every_row():
    for sinks in (True, False):
        _check(synth.config_selected_decode(sinks=sinks), f"selected_decode_f16 sink={sinks} (full)")


def test_full_local_plus_aux_int8_every_row():
    _check(synth.config_local_plus_aux_int8(), "local_plus_aux_int8 (full)")
