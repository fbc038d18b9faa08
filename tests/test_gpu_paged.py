"""GPU parity: the paged step (prepare_seqlens -> kv_cache_append -> paged_attention_fwd)
against the oracle, at small sizes and at the workloads' full sizes (every row); decode
(split-K) and prefill (MFMA tile) regimes, paged and contiguous caches, windows, sinks, GQA
groups, INT8 / FP8 caches, batches past the staged-metadata limit, empty and degenerate
requests."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle import pool
import selected_token_sparse_amd as sta
import synth
from synth.device import case_tensors, tensor

from harness import assert_close, oracle_paged_step, run_paged_step, status_tensor

pytestmark = pytest.mark.gpu


def _check_full(case, what):
    print("paged", what, flush=True)
    out, _, _, st = run_paged_step(case)
    torch.cuda.synchronize()
    ref, ost = oracle_paged_step(case)
    err = assert_close(out, ref, case.dtype, what)
    assert int(st.item()) == ost, (int(st.item()), ost)
    return err


def test_tiny_paged_decode_f32():
    _check_full(synth.config_tiny_paged_decode(poison=True), "tiny_paged_decode_f32")


def test_gqa_paged_decode_reduced():
    _check_full(synth.config_gqa_paged_decode(poison=True, B=8, max_len=1500, seed=77),
                "gqa_paged_decode_f16_reduced")


DECODE = [
    # name, kwargs
    ("f16_g8_sink", dict(kv_lens=[1, 2, 17, 33, 200, 0, 511], q_lens=[1, 1, 1, 1, 1, 0, 1], H_q=16, H_kv=2, D=64, dtype=synth.F16, sinks=True)),
    ("bf16_g8_w5", dict(kv_lens=[40, 3, 129], q_lens=[1, 1, 1], H_q=16, H_kv=2, D=64, dtype=synth.BF16, sinks=True, local_window=5)),
    ("f16_d128_g12", dict(kv_lens=[300, 77], q_lens=[1, 1], H_q=24, H_kv=2, D=128, dtype=synth.F16, sinks=True)),
    ("f16_g1_mtp4", dict(kv_lens=[9, 100], q_lens=[4, 4], H_q=3, H_kv=3, D=64, dtype=synth.F16)),
    ("f16_g20_two_tiles", dict(kv_lens=[64, 5], q_lens=[2, 1], H_q=40, H_kv=2, D=64, dtype=synth.F16, sinks=True)),
    ("f16_g3_bs12", dict(kv_lens=[50, 13], q_lens=[8, 1], H_q=6, H_kv=2, D=64, dtype=synth.F16, block_size=12)),
    ("f16_i8_cache", dict(kv_lens=[70, 260], q_lens=[1, 3], H_q=12, H_kv=1, D=128, dtype=synth.F16, cache_dtype=synth.I8, sinks=True)),
    ("bf16_i8_cache_w9", dict(kv_lens=[70, 33], q_lens=[2, 1], H_q=8, H_kv=2, D=64, dtype=synth.BF16, cache_dtype=synth.I8, local_window=9)),
    ("f32_g4_w3_sink", dict(kv_lens=[31, 2, 90], q_lens=[1, 2, 3], H_q=8, H_kv=2, D=128, dtype=synth.F32, sinks=True, local_window=3)),
    ("f32_i8_cache", dict(kv_lens=[45], q_lens=[2], H_q=4, H_kv=2, D=64, dtype=synth.F32, cache_dtype=synth.I8)),
    ("f16_contig", dict(kv_lens=[120, 7, 64], q_lens=[1, 1, 1], H_q=8, H_kv=1, D=64, dtype=synth.F16, contiguous=True, capacity=128, sinks=True)),
    ("f16_long_splits", dict(kv_lens=[8192, 4000, 1], q_lens=[1, 1, 1], H_q=64, H_kv=8, D=64, dtype=synth.F16, sinks=True)),
    ("f16_fp8_cache", dict(kv_lens=[70, 260], q_lens=[1, 3], H_q=12, H_kv=1, D=128, dtype=synth.F16, cache_dtype=synth.FP8, sinks=True)),
    ("bf16_fp8_cache_w9", dict(kv_lens=[70, 33], q_lens=[2, 1], H_q=8, H_kv=2, D=64, dtype=synth.BF16, cache_dtype=synth.FP8, local_window=9)),
    ("f32_fp8_cache", dict(kv_lens=[45, 130], q_lens=[2, 1], H_q=4, H_kv=2, D=64, dtype=synth.F32, cache_dtype=synth.FP8, sinks=True)),
    ("f16_fp8_contig_long", dict(kv_lens=[3000, 9], q_lens=[1, 1], H_q=16, H_kv=2, D=64, dtype=synth.F16, cache_dtype=synth.FP8, contiguous=True, capacity=3000, sinks=True)),
    # long contexts: 100k keys (391 splits of the key range) and a 4096-key window at 70k
    ("f16_long_context_100k", dict(kv_lens=[100000, 3, 40000], q_lens=[1, 1, 2], H_q=8, H_kv=1, D=64, dtype=synth.F16, sinks=True)),
    ("bf16_d128_70k_w4096", dict(kv_lens=[70000], q_lens=[3], H_q=12, H_kv=1, D=128, dtype=synth.BF16, local_window=4096)),
]


@pytest.mark.parametrize("name,kw", DECODE, ids=[d[0] for d in DECODE])
def test_decode_variants(name, kw):
    case = synth.paged_case(zlib.crc32(name.encode()) % 1000, poison=True, **kw)
    _check_full(case, name)


PREFILL = [
    ("f16_w128_sink", dict(kv_lens=[160, 64, 300, 97], q_lens=[160, 64, 300, 97], H_q=16, H_kv=2, D=64, dtype=synth.F16, sinks=True, local_window=128)),
    ("f16_causal", dict(kv_lens=[130, 33, 257], q_lens=[130, 33, 257], H_q=8, H_kv=2, D=64, dtype=synth.F16, sinks=True)),
    ("bf16_causal_d128", dict(kv_lens=[100, 70], q_lens=[100, 70], H_q=8, H_kv=2, D=128, dtype=synth.BF16)),
    ("f16_chunked_prefill", dict(kv_lens=[300, 90], q_lens=[45, 90], H_q=8, H_kv=1, D=64, dtype=synth.F16, sinks=True, local_window=50)),
    ("f16_g1", dict(kv_lens=[200, 9], q_lens=[150, 9], H_q=2, H_kv=2, D=64, dtype=synth.F16)),
    ("f16_g2", dict(kv_lens=[100], q_lens=[77], H_q=4, H_kv=2, D=128, dtype=synth.F16, local_window=16)),
    ("f16_g12_d128", dict(kv_lens=[64, 40], q_lens=[64, 40], H_q=24, H_kv=2, D=128, dtype=synth.F16, sinks=True)),
    ("f16_i8_prefill", dict(kv_lens=[90, 40], q_lens=[90, 20], H_q=8, H_kv=2, D=64, dtype=synth.F16, cache_dtype=synth.I8, sinks=True)),
    ("f16_w1", dict(kv_lens=[40], q_lens=[40], H_q=8, H_kv=2, D=64, dtype=synth.F16, local_window=1)),
    ("f16_bs5", dict(kv_lens=[61, 20], q_lens=[61, 12], H_q=8, H_kv=2, D=64, dtype=synth.F16, block_size=5, sinks=True)),
    ("f16_empty_mixed", dict(kv_lens=[0, 50, 0, 9], q_lens=[0, 50, 0, 9], H_q=8, H_kv=2, D=64, dtype=synth.F16, sinks=True)),
    ("f16_fp8_prefill", dict(kv_lens=[90, 40], q_lens=[90, 20], H_q=8, H_kv=2, D=64, dtype=synth.F16, cache_dtype=synth.FP8, sinks=True)),
    ("bf16_fp8_prefill_d128_w20", dict(kv_lens=[120], q_lens=[70], H_q=8, H_kv=2, D=128, dtype=synth.BF16, cache_dtype=synth.FP8, local_window=20)),
    # a key range of more than 512 blocks (block size 4): block ids read from the table in
    # global memory instead of the staged copy
    ("f16_bs4_long_table", dict(kv_lens=[2100, 70], q_lens=[40, 70], H_q=8, H_kv=2, D=64, dtype=synth.F16, block_size=4, sinks=True)),
    ("bf16_bs4_long_table_d128", dict(kv_lens=[2300], q_lens=[33], H_q=4, H_kv=1, D=128, dtype=synth.BF16, block_size=4)),
    # a chunk of 700 rows appended at position 5300 of a 6000-key history, window 256
    ("f16_long_history_chunk_w256", dict(kv_lens=[6000], q_lens=[700], H_q=8, H_kv=2, D=64, dtype=synth.F16, local_window=256, sinks=True)),
    # contiguous per-request caches [B, H_kv, capacity, D] (no block table): fresh prompts
    # and chunked prefill (rows appended after a history), with and without a window
    ("f16_contig_w64", dict(kv_lens=[300, 97, 160], q_lens=[300, 97, 40], H_q=16, H_kv=2, D=64, dtype=synth.F16, contiguous=True, capacity=320, sinks=True, local_window=64)),
    # the windowed span kernel's block ids: read per lane for a block size that is not a
    # power of two of at least 8 (5, 4), by scalar loads otherwise (32, with D = 128)
    ("f16_w96_bs5", dict(kv_lens=[150, 61, 230], q_lens=[150, 40, 100], H_q=16, H_kv=2, D=64, dtype=synth.F16, block_size=5, sinks=True, local_window=96)),
    ("f16_w40_bs4_g4", dict(kv_lens=[130, 77], q_lens=[130, 60], H_q=8, H_kv=2, D=64, dtype=synth.F16, block_size=4, local_window=40)),
    ("bf16_w128_bs32_d128", dict(kv_lens=[300, 45], q_lens=[260, 45], H_q=16, H_kv=2, D=128, dtype=synth.BF16, block_size=32, sinks=True, local_window=128)),
    # the causal kernel's DMA: one uniform block per instruction (block sizes of at least
    # 8 keys at D = 64, 4 at D = 128), per lane at range edges
    ("f16_causal_bs8", dict(kv_lens=[200, 77], q_lens=[200, 50], H_q=8, H_kv=2, D=64, dtype=synth.F16, block_size=8, sinks=True)),
    ("f16_chunk_bs64_w70", dict(kv_lens=[300, 150], q_lens=[260, 150], H_q=8, H_kv=2, D=64, dtype=synth.F16, block_size=64, local_window=70)),
    ("bf16_causal_bs128_d128", dict(kv_lens=[400, 130], q_lens=[300, 130], H_q=8, H_kv=2, D=128, dtype=synth.BF16, block_size=128, sinks=True)),
    # the windowed kernel's first and last span tiles in one pass (fp16, a window that is a
    # multiple of 32, full row blocks past the sequence start): W = 32 (the pair alone),
    # W = 64 at D = 128, W = 96 in a chunk after a history
    ("f16_w32_pair", dict(kv_lens=[130, 70], q_lens=[130, 70], H_q=8, H_kv=2, D=64, dtype=synth.F16, sinks=True, local_window=32)),
    ("f16_w64_d128_pair", dict(kv_lens=[200, 90], q_lens=[200, 70], H_q=8, H_kv=2, D=128, dtype=synth.F16, sinks=True, local_window=64)),
    ("f16_w96_chunk_pair", dict(kv_lens=[400, 160], q_lens=[100, 160], H_q=16, H_kv=2, D=64, dtype=synth.F16, local_window=96)),
    # 8-bit caches: a wave's tile load in one block by a scalar table read (block size 8
    # at D = 64, 4 keys a load at D = 128), per lane at range edges and for block size 4
    ("f16_i8_bs8_chunk", dict(kv_lens=[300, 120], q_lens=[200, 120], H_q=8, H_kv=2, D=64, dtype=synth.F16, cache_dtype=synth.I8, block_size=8, sinks=True)),
    ("bf16_fp8_bs4_d128", dict(kv_lens=[150, 60], q_lens=[150, 40], H_q=8, H_kv=2, D=128, dtype=synth.BF16, cache_dtype=synth.FP8, block_size=4)),
    ("f16_contig_causal_chunked", dict(kv_lens=[500, 200, 33], q_lens=[120, 200, 9], H_q=8, H_kv=2, D=64, dtype=synth.F16, contiguous=True, capacity=512)),
    ("bf16_contig_d128_chunked_sink", dict(kv_lens=[260, 70], q_lens=[100, 70], H_q=8, H_kv=2, D=128, dtype=synth.BF16, contiguous=True, capacity=300, sinks=True)),
    ("f16_i8_contig", dict(kv_lens=[200, 90], q_lens=[150, 30], H_q=8, H_kv=2, D=64, dtype=synth.F16, cache_dtype=synth.I8, contiguous=True, capacity=256, sinks=True)),
    ("f16_i8_contig_w40_d128", dict(kv_lens=[230, 64], q_lens=[100, 64], H_q=12, H_kv=1, D=128, dtype=synth.F16, cache_dtype=synth.I8, contiguous=True, capacity=240, local_window=40, sinks=True)),
    ("f16_fp8_contig", dict(kv_lens=[180, 130], q_lens=[180, 50], H_q=8, H_kv=2, D=64, dtype=synth.F16, cache_dtype=synth.FP8, contiguous=True, capacity=192, sinks=True)),
    ("bf16_fp8_contig_w33_d128", dict(kv_lens=[150], q_lens=[60], H_q=8, H_kv=2, D=128, dtype=synth.BF16, cache_dtype=synth.FP8, contiguous=True, capacity=160, local_window=33)),
]


@pytest.mark.parametrize("name,kw", PREFILL, ids=[d[0] for d in PREFILL])
def test_prefill_variants(name, kw):
    case = synth.paged_case(zlib.crc32(name.encode()) % 1000, poison=True, **kw)
    assert case.max_seqlen_q > 8
    _check_full(case, name)


def test_decode_batch_beyond_staged_metadata():
    """600 requests: more boundaries than the split kernel stages in LDS (512), so the row's
    request and key count are binary-searched in global memory; several splits and the
    merge; one empty request."""
    rng = np.random.default_rng(600)
    kv = rng.integers(1, 400, size=600)
    kv[17] = 0
    ql = (kv > 0).astype(np.int64)
    case = synth.paged_case(600, kv_lens=kv, q_lens=ql, H_q=16, H_kv=2, D=64, dtype=synth.F16,
                            sinks=True, poison=True)
    _check_full(case, "f16_B600")
    case = synth.paged_case(601, kv_lens=kv, q_lens=ql, H_q=8, H_kv=2, D=64, dtype=synth.F16,
                            cache_dtype=synth.I8, local_window=50, poison=True)
    _check_full(case, "f16_i8_B600_w50")


def test_single_visible_key_is_the_value_row():
    # window 1, no sink: the softmax weight is exactly 1, so out == the row's own V (bit-exact)
    for q_lens, dt in (([1, 1], synth.F16), ([30, 12], synth.F16), ([1, 3], synth.BF16), ([20], synth.BF16)):
        kv = [x + 5 for x in q_lens]
        case = synth.paged_case(5, kv_lens=kv, q_lens=q_lens, H_q=8, H_kv=2, D=64, dtype=dt,
                                local_window=1, poison=True)
        print("single key", q_lens, dt, flush=True)
        out, _, _, _ = run_paged_step(case)
        torch.cuda.synchronize()
        g = out.cpu()
        want = tensor(np.repeat(case.v_new, 4, axis=1), dt, "cpu")
        assert torch.equal(g.view(torch.int16), want.view(torch.int16))


def test_block_table_permutation_gives_identical_bits():
    case = synth.paged_case(9, kv_lens=[300, 45], q_lens=[1, 1], H_q=16, H_kv=2, D=64,
                            dtype=synth.F16, sinks=True, num_blocks=40)
    out1, _, _, _ = run_paged_step(case)
    perm = np.random.default_rng(3).permutation(case.num_blocks)
    kc = np.empty_like(case.k_cache)
    vc = np.empty_like(case.v_cache)
    kc[perm] = case.k_cache
    vc[perm] = case.v_cache
    case.block_table = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    case.k_cache, case.v_cache = kc, vc
    out2, _, _, _ = run_paged_step(case)
    torch.cuda.synchronize()
    assert torch.equal(out1.cpu().view(torch.int16), out2.cpu().view(torch.int16))


def test_deterministic_repeat():
    case = synth.config_gqa_paged_decode(B=6, max_len=3000, seed=5)
    t = case_tensors(case)
    a, _, _, _ = run_paged_step(case, t=t)
    b, _, _, _ = run_paged_step(case, t=t)
    torch.cuda.synchronize()
    assert torch.equal(a.cpu().view(torch.int16), b.cpu().view(torch.int16))


def test_host_bounds_change_only_the_plan():
    """The host bounds size the launch, not the result: a loose key bound (more, partly empty
    splits) and a query bound above 8 (the MFMA prefill kernel on decode rows) both match the
    oracle on the same decode step."""
    base = synth.paged_case(41, kv_lens=[700, 1, 0, 2500, 64], q_lens=[1, 1, 0, 1, 1], H_q=16,
                            H_kv=2, D=64, dtype=synth.F16, sinks=True, poison=True)
    for mq, mk in ((base.max_seqlen_q, base.max_seqlen_k), (base.max_seqlen_q, 8 * base.max_seqlen_k),
                   (16, base.max_seqlen_k)):
        case = synth.paged_case(41, kv_lens=[700, 1, 0, 2500, 64], q_lens=[1, 1, 0, 1, 1], H_q=16,
                                H_kv=2, D=64, dtype=synth.F16, sinks=True, poison=True)
        case.max_seqlen_q, case.max_seqlen_k = mq, mk
        _check_full(case, f"bounds_q{mq}_k{mk}")


def test_bound_violations_zero_rows():
    for mq in (4, 40):
        case = synth.paged_case(31, kv_lens=[40, 100, 30], q_lens=[10, 1, 30], H_q=8, H_kv=2, D=64,
                                dtype=synth.F16, sinks=True)
        case.max_seqlen_q = 30 if mq == 40 else 4    # request 0 (and 2) exceed the bound
        case.max_seqlen_k = 60                        # request 1 exceeds the key bound
        print("bounds", mq, flush=True)
        _check_full(case, f"bounds_{mq}")


def test_short_kv_and_bad_blocks():
    case = synth.paged_case(32, kv_lens=[40, 100, 30], q_lens=[10, 1, 30], H_q=8, H_kv=2, D=64,
                            dtype=synth.F16, sinks=True, num_blocks=20)
    case.block_table = case.block_table.copy()
    case.block_table[1, 2] = 77       # beyond the pool
    case.block_table[1, 4] = -5
    print("short kv / bad blocks", flush=True)
    # request 2 holds fewer keys than rows: seqlens_k passed directly (no metadata kernel)
    sk = case.seqlens_k.copy()
    sk[2] = 19
    t = case_tensors(case)
    t["seqlens_k"] = tensor(sk, None)
    st = status_tensor()
    out = torch.empty((case.T, case.H_q, case.D), dtype=torch.float16, device="cuda")
    sta.paged_attention_fwd(t["q"], t["k_cache"], t["v_cache"], t["cu"], t["seqlens_k"],
                            case.max_seqlen_q, case.max_seqlen_k, out, block_table=t["block_table"],
                            scale=case.scale, sinks=t["sinks"], status=st)
    torch.cuda.synchronize()
    ref, ost = oracle.paged_attention(case.q, case.k_cache, case.v_cache, case.cu_seqlens_q, sk,
                                      H_kv=2, block_table=case.block_table, block_size=16,
                                      max_seqlen_q=case.max_seqlen_q, max_seqlen_k=case.max_seqlen_k,
                                      scale=case.scale, sinks=case.sinks)
    assert_close(out, ref, synth.F16, "short_kv_bad_blocks")
    assert int(st.item()) == ost
    assert ost & oracle.STATUS_BAD_BLOCK and ost & oracle.STATUS_SHORT_KV


@pytest.mark.parametrize("bs", [16, 5])
def test_windowed_short_kv_bad_blocks_and_bounds(bs):
    """The windowed span kernel (window 24, 8 query heads per KV head) over a table with a
    block id past the pool and a negative one, a request with fewer keys than rows and one
    over the query bound (zero rows): outputs and status bits against the oracle.  Block
    size 16 reads the block ids by scalar loads, 5 per lane."""
    kv, ql = [60, 160, 45, 50], [20, 60, 45, 30]
    case = synth.paged_case(33 + bs, kv_lens=kv, q_lens=ql, H_q=16, H_kv=2, D=64,
                            dtype=synth.F16, sinks=True, block_size=bs, local_window=24)
    case.block_table = case.block_table.copy()
    case.block_table[2, 1] = case.block_table.max() + 1000   # beyond the pool (keys in view)
    case.block_table[2, 2] = -5
    case.max_seqlen_q = 50                                     # request 2 (45) fits, 1 (60) does not
    print("windowed short kv / bad blocks / bounds", bs, flush=True)
    sk = case.seqlens_k.copy()
    sk[3] = 19                                                 # request 3: 20 keys for 30 rows
    t = case_tensors(case)
    t["seqlens_k"] = tensor(sk, None)
    st = status_tensor()
    out = torch.empty((case.T, case.H_q, case.D), dtype=torch.float16, device="cuda")
    sta.paged_attention_fwd(t["q"], t["k_cache"], t["v_cache"], t["cu"], t["seqlens_k"],
                            case.max_seqlen_q, case.max_seqlen_k, out, block_table=t["block_table"],
                            scale=case.scale, local_window=24, sinks=t["sinks"], status=st)
    torch.cuda.synchronize()
    ref, ost = oracle.paged_attention(case.q, case.k_cache, case.v_cache, case.cu_seqlens_q, sk,
                                      H_kv=2, block_table=case.block_table, block_size=bs,
                                      max_seqlen_q=case.max_seqlen_q, max_seqlen_k=case.max_seqlen_k,
                                      scale=case.scale, local_window=24, sinks=case.sinks)
    assert_close(out, ref, synth.F16, f"windowed_short_kv_bad_blocks_bs{bs}")
    assert int(st.item()) == ost
    assert ost & oracle.STATUS_BAD_BLOCK and ost & oracle.STATUS_SHORT_KV and ost & oracle.STATUS_Q_BOUND


def test_argument_errors_enqueue_nothing():
    case = synth.config_tiny_paged_decode()
    t = case_tensors(case)
    out = torch.full((case.T, case.H_q, case.D), 7.0, device="cuda")
    with pytest.raises(sta.SpattnError) as e:
        sta.paged_attention_fwd(t["q"], t["k_cache"], t["v_cache"], t["cu"], t["seqlens_k"], 1, 100,
                                out, block_table=t["block_table"], is_causal=0)
    assert e.value.rc == -4
    with pytest.raises(sta.SpattnError) as e:
        sta.paged_attention_fwd(t["q"].half(), t["k_cache"], t["v_cache"], t["cu"], t["seqlens_k"], 1,
                                100, out.half(), block_table=t["block_table"])
    assert e.value.rc == -3
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


# ---------------- full-size workloads, every row ----------------

def _full(case, what, workers=1):
    print("paged full-size", what, flush=True)
    out, _, _, st = run_paged_step(case)
    torch.cuda.synchronize()
    ref, ost = oracle_paged_step(case, workers=workers)
    err = assert_close(out, ref, case.dtype, what)
    assert int(st.item()) == ost, (int(st.item()), ost)
    return err


def test_full_gqa_paged_decode_every_row():
    _full(synth.config_gqa_paged_decode(poison=True), "gqa_paged_decode_f16 (full)")


def test_full_windowed_prefill_every_row():
    _full(synth.config_paged_prefill_window(), "paged_prefill_w128_f16 (full)",
          workers=pool.default_workers())


def test_full_causal_prefill_every_row():
    _full(synth.config_paged_prefill_window(window=-1), "paged_prefill_f16 no window (full)",
          workers=pool.default_workers())


def test_workspace_reuse():
    # one uninitialised workspace across many calls: every call gives the same bits
    case = synth.config_gqa_paged_decode(B=12, max_len=6000, seed=21)
    t = case_tensors(case)
    need = sta.attention_workspace_bytes(sta.KIND_PAGED, sta.F16, case.B, case.T, case.max_seqlen_q,
                                         case.max_seqlen_k, 0, -1, case.H_q, case.H_kv, case.D)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN-pattern garbage
    sta.kv_cache_append(t["k_new"], t["v_new"], t["cu"], t["seqlens_k"], t["k_cache"], t["v_cache"],
                        t["block_table"])
    outs = []
    for it in range(4):
        out = torch.empty((case.T, case.H_q, case.D), dtype=torch.float16, device="cuda")
        sta.paged_attention_fwd(t["q"], t["k_cache"], t["v_cache"], t["cu"], t["seqlens_k"],
                                case.max_seqlen_q, case.max_seqlen_k, out, block_table=t["block_table"],
                                scale=case.scale, sinks=t["sinks"], workspace=ws)
        outs.append(out)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.cpu().view(torch.int16), outs[0].cpu().view(torch.int16))
    ref, _ = oracle_paged_step(case)
    assert_close(outs[0], ref, case.dtype, "workspace reuse")
