"""paged_decode_step: the metadata pass, the cache append and the split-K attention of a
decode step in one call.  For well-formed metadata its outputs, every cache byte, the
lengths and the status must equal those of prepare_and_append followed by
paged_attention_fwd bit for bit (same poisoned caches: unreferenced slots hold NaN), and
the attention rows must match the oracle's metadata -> append -> attention step.
("[WebGPU] Add PagedAttention metadata and GPT-OSS support", Description: lengths derived
on the device; "[WebGPU] Add SparsePagedAttention", file summaries: the step's K/V
scattered through the block table before attention reads it.)"""
import numpy as np
import pytest
import torch

import oracle
import selected_token_sparse_amd as sta
import synth
from synth.device import TORCH_DTYPE, case_tensors, tensor

from harness import assert_close, oracle_paged_step, status_tensor

pytestmark = pytest.mark.gpu


def _bits(t):
    n = t.element_size()
    return t.view(torch.uint8 if n == 1 else torch.int16 if n == 2 else torch.int32)


def _ws(case, T=None):
    n = sta.attention_workspace_bytes(sta.KIND_PAGED, case.dtype, case.B,
                                      case.T if T is None else T, case.max_seqlen_q,
                                      case.max_seqlen_k, 0, case.local_window, case.H_q,
                                      case.H_kv, case.D)
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")


def _run(case, t, mode, cu_t, past_t, ws, committed=None):
    """One step on fresh copies of the caches; returns every output as host tensors."""
    B, T = int(past_t.shape[0]), case.T
    kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
    sq = torch.full((B,), 777, dtype=torch.int32, device="cuda")
    sk = torch.full((B,), 777, dtype=torch.int32, device="cuda")
    out = torch.full((T, case.H_q, case.D), float("nan"), dtype=TORCH_DTYPE[case.dtype],
                     device="cuda")
    st = status_tensor()
    kw = dict(block_table=t["block_table"], key_scale=t["key_scale"],
              value_scale=t["value_scale"], scale=case.scale, local_window=case.local_window,
              sinks=t["sinks"], workspace=ws, status=st)
    if mode == "step":
        sta.paged_decode_step(cu_t, past_t, T, sq, sk, t["q"], t["k_new"], t["v_new"], kc, vc,
                              case.max_seqlen_q, case.max_seqlen_k, out,
                              committed_length=committed, **kw)
    else:
        sta.prepare_and_append(cu_t, past_t, T, sq, sk, t["k_new"], t["v_new"], kc, vc,
                               t["block_table"], key_scale=t["key_scale"],
                               value_scale=t["value_scale"], committed_length=committed,
                               status=st)
        sta.paged_attention_fwd(t["q"], kc, vc, cu_t, sk, case.max_seqlen_q, case.max_seqlen_k,
                                out, **kw)
    torch.cuda.synchronize()
    return dict(out=out, sq=sq.cpu(), sk=sk.cpu(), k=_bits(kc).cpu(), v=_bits(vc).cpu(),
                st=int(st.item()))


def _step_vs_calls(case, cu=None, past=None, committed=None):
    """The step and the two calls on the same inputs: identical bit for bit."""
    t = case_tensors(case)
    cu_t = tensor(np.asarray(case.cu_seqlens_q if cu is None else cu, dtype=np.int32))
    past_t = tensor(np.asarray(case.past_seqlens if past is None else past, dtype=np.int32))
    cm_t = None if committed is None else tensor(np.asarray(committed, dtype=np.int32))
    ws = _ws(case)
    a = _run(case, t, "step", cu_t, past_t, ws, cm_t)
    b = _run(case, t, "calls", cu_t, past_t, ws, cm_t)
    for name in ("sq", "sk", "k", "v"):
        assert torch.equal(a[name], b[name]), name
    assert torch.equal(_bits(a["out"]).cpu(), _bits(b["out"]).cpu()), "out"
    assert a["st"] == b["st"], (a["st"], b["st"])
    return a


def _against_oracle(case, got, what):
    ref, ost = oracle_paged_step(case)
    assert_close(got["out"], ref, case.dtype, what)
    assert got["st"] == ost, (got["st"], ost)


@pytest.mark.parametrize("cache_dtype", [synth.F16, synth.I8, synth.FP8])
def test_gqa_decode_step(cache_dtype):
    """B=32 decode rows over up to 3000 keys (several splits and the merge), H 64/8, D 64,
    sinks, one empty request; 16-bit, INT8 and FP8 caches."""
    print("decode step gqa", cache_dtype, flush=True)
    case = synth.config_gqa_paged_decode(poison=True, B=32, max_len=3000, seed=301,
                                         cache_dtype=cache_dtype)
    got = _step_vs_calls(case)
    _against_oracle(case, got, f"step_gqa_{cache_dtype}")


def test_multi_row_window_contiguous_bf16():
    """Up to 4 new rows per request (each row sees the new keys before it), a 100-key
    window, a contiguous cache, bf16, D 128, group 12."""
    print("decode step multi-row window", flush=True)
    case = synth.paged_case(302, kv_lens=[700, 4, 260, 1, 129, 0], q_lens=[4, 4, 3, 1, 2, 0],
                            H_q=48, H_kv=4, D=128, dtype=synth.BF16, contiguous=True,
                            capacity=720, sinks=True, local_window=100, poison=True,
                            max_seqlen_q=4)
    got = _step_vs_calls(case)
    _against_oracle(case, got, "step_multi_row")


@pytest.mark.parametrize("cache_dtype", [synth.I8, synth.FP8])
def test_bf16_quantised_cache_d128_window(cache_dtype):
    """bf16 activations over an INT8 / FP8 cache at D 128 with a 256-key window and two new
    rows per request: the codes the step writes and the rows it returns."""
    print("decode step bf16 quantised d128", cache_dtype, flush=True)
    case = synth.paged_case(310, kv_lens=[1500, 300, 2, 700], q_lens=[2, 2, 2, 1], H_q=16,
                            H_kv=2, D=128, dtype=synth.BF16, cache_dtype=cache_dtype, sinks=True,
                            local_window=256, poison=True, max_seqlen_q=2)
    got = _step_vs_calls(case)
    _against_oracle(case, got, f"step_bf16_d128_{cache_dtype}")


def test_head_tiles_and_one_split():
    """Group 20 (two head tiles write the same new keys) and a key range short enough for
    one split, whose workgroup writes the output directly."""
    print("decode step head tiles", flush=True)
    case = synth.paged_case(303, kv_lens=[90, 17, 128], q_lens=[2, 1, 1], H_q=40, H_kv=2, D=64,
                            dtype=synth.F16, sinks=True, poison=True, max_seqlen_q=2,
                            max_seqlen_k=128)
    got = _step_vs_calls(case)
    _against_oracle(case, got, "step_head_tiles")


def test_rows_beyond_the_bounds_still_append():
    """A request over max_seqlen_k and one over max_seqlen_q get zero rows and their flags,
    and their new keys are still written, as the separate calls write them."""
    print("decode step bounds", flush=True)
    case = synth.paged_case(304, kv_lens=[40, 300, 30, 64], q_lens=[1, 1, 3, 2], H_q=8, H_kv=2,
                            D=64, dtype=synth.F16, sinks=True, poison=True)
    case.max_seqlen_q = 2            # request 2 exceeds it
    case.max_seqlen_k = 200          # request 1 exceeds it
    got = _step_vs_calls(case)
    assert got["st"] & sta.STATUS_Q_BOUND and got["st"] & sta.STATUS_K_BOUND
    _against_oracle(case, got, "step_bounds")


@pytest.mark.parametrize("cache_dtype", [synth.F16, synth.I8])
def test_cursor_mismatch_appends_nothing(cache_dtype):
    """committed_length on the fused step: requests whose cursor disagrees with their past
    length (including one beyond the key bound) flag STATUS_CURSOR and write no key; their
    rows are attended over the unchanged cache; the rest append normally.  Bit for bit the
    two calls with the same cursor, and the oracle's append with the cursor, then attention."""
    print("decode step cursor", cache_dtype, flush=True)
    case = synth.paged_case(311, kv_lens=[700, 40, 2600, 1, 90, 0], q_lens=[1, 1, 1, 1, 2, 0],
                            H_q=16, H_kv=2, D=64, dtype=synth.F16, cache_dtype=cache_dtype,
                            sinks=True, poison=cache_dtype == synth.F16, max_seqlen_q=2,
                            max_seqlen_k=2000)
    committed = case.past_seqlens.copy()
    committed[1] += 1            # stale cursor
    committed[2] -= 3            # beyond the key bound as well
    committed[4] = 0
    committed[5] = 77            # no rows: not checked
    got = _step_vs_calls(case, committed=committed)
    assert got["st"] & sta.STATUS_CURSOR
    _, sk, _, _, st0 = oracle.prepare_seqlens(case.cu_seqlens_q, case.past_seqlens, case.T)
    kc, vc, st1 = oracle.kv_cache_append(case.k_new, case.v_new, case.cu_seqlens_q, sk,
                                         case.k_cache, case.v_cache, case.block_table,
                                         case.block_size, case.key_scale, case.value_scale,
                                         committed_length=committed)
    assert np.array_equal(got["k"].numpy().view(kc.dtype).reshape(kc.shape), kc, equal_nan=True)
    ref, st2 = oracle.paged_attention(case.q, kc, vc, case.cu_seqlens_q, sk, H_kv=case.H_kv,
                                      block_table=case.block_table, block_size=case.block_size,
                                      key_scale=case.key_scale, value_scale=case.value_scale,
                                      max_seqlen_q=case.max_seqlen_q,
                                      max_seqlen_k=case.max_seqlen_k, scale=case.scale,
                                      sinks=case.sinks)
    assert_close(got["out"], ref, case.dtype, f"step_cursor_{cache_dtype}")
    assert got["st"] == st0 | st1 | st2, (got["st"], st0 | st1 | st2)


def test_missing_slots_flagged():
    """New keys whose block id lies outside the pool are flagged and skipped."""
    print("decode step bad blocks", flush=True)
    case = synth.paged_case(305, kv_lens=[40, 100, 33], q_lens=[1, 2, 1], H_q=8, H_kv=2, D=64,
                            dtype=synth.F16, sinks=True, num_blocks=16)
    case.block_table = case.block_table.copy()
    case.block_table[1, 6] = 99      # holds positions 96..99: both new keys of request 1
    case.block_table[2, 2] = -3      # the new key of request 2
    got = _step_vs_calls(case)
    assert got["st"] & sta.STATUS_BAD_BLOCK


@pytest.mark.parametrize("cu,past", [
    ([0, 2, 1, 3], [5, 5, 5]),          # decreasing boundary
    ([1, 2, 3], [5, 5]),                # cu[0] != 0
    ([0, 1, 4], [5, 5]),                # cu[B] != T
    ([0, 1, 3], [-2, 5]),               # negative past
])
def test_malformed_metadata_is_an_empty_step(cu, past):
    """Malformed metadata: BAD_CU, lengths as prepare_seqlens writes them, no cache byte
    changed, every row zero."""
    print("decode step malformed", cu, past, flush=True)
    case = synth.paged_case(306, kv_lens=[8, 9], q_lens=[1, 2], H_q=4, H_kv=2, D=64,
                            dtype=synth.F16, num_blocks=8, max_seqlen_q=2)
    t = case_tensors(case)
    cu_t, past_t = tensor(np.asarray(cu, dtype=np.int32)), tensor(np.asarray(past, dtype=np.int32))
    got = _run(case, t, "step", cu_t, past_t, _ws(case))
    sq, sk, _, _, ost = oracle.prepare_seqlens(np.asarray(cu, dtype=np.int32),
                                              np.asarray(past, dtype=np.int32), case.T)
    assert np.array_equal(got["sq"].numpy(), sq) and np.array_equal(got["sk"].numpy(), sk)
    assert got["st"] == sta.STATUS_BAD_CU == ost
    assert torch.equal(got["k"], _bits(t["k_cache"]).cpu())
    assert torch.equal(got["v"], _bits(t["v_cache"]).cpu())
    assert bool((got["out"] == 0).all())


def test_no_rows_writes_the_metadata_only():
    case = synth.paged_case(307, kv_lens=[5, 0], q_lens=[0, 0], H_q=4, H_kv=2, D=64,
                            dtype=synth.F16, max_seqlen_q=1)
    print("decode step T=0", flush=True)
    t = case_tensors(case)
    sq = torch.full((2,), 7, dtype=torch.int32, device="cuda")
    sk = torch.full((2,), 7, dtype=torch.int32, device="cuda")
    out = torch.empty((0, 4, 64), dtype=torch.float16, device="cuda")
    sta.paged_decode_step(t["cu"], t["past"], 0, sq, sk, t["q"], t["k_new"], t["v_new"],
                          t["k_cache"], t["v_cache"], 1, 16, out, block_table=t["block_table"])
    torch.cuda.synchronize()
    assert sq.tolist() == [0, 0] and sk.tolist() == [4, -1]


def test_unsupported_shapes_enqueue_nothing():
    case = synth.paged_case(308, kv_lens=[40, 30], q_lens=[20, 1], H_q=4, H_kv=2, D=64,
                            dtype=synth.F16)
    print("decode step unsupported", flush=True)
    t = case_tensors(case)
    sq = torch.full((2,), 7, dtype=torch.int32, device="cuda")
    sk = torch.full((2,), 7, dtype=torch.int32, device="cuda")
    out = torch.full((case.T, 4, 64), 3.0, dtype=torch.float16, device="cuda")
    with pytest.raises(sta.SpattnError) as e:     # a 20-row block takes the prefill kernel
        sta.paged_decode_step(t["cu"], t["past"], case.T, sq, sk, t["q"], t["k_new"], t["v_new"],
                              t["k_cache"], t["v_cache"], 20, 40, out, block_table=t["block_table"])
    assert e.value.rc == -4
    torch.cuda.synchronize()
    assert sq.tolist() == [7, 7] and bool((out == 3.0).all())


def test_step_in_a_graph_replays_bit_exactly():
    """The step recorded into a HIP graph: every replay (after eager work, outputs first
    overwritten with NaN) reproduces the eager outputs and cache bit for bit."""
    print("decode step graph", flush=True)
    case = synth.config_gqa_paged_decode(poison=True, B=8, max_len=3000, seed=309)
    t = case_tensors(case)
    ws = _ws(case)
    eager = _run(case, t, "step", t["cu"], t["past"], ws)
    kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
    sq = torch.empty(case.B, dtype=torch.int32, device="cuda")
    sk = torch.empty(case.B, dtype=torch.int32, device="cuda")
    out = torch.empty((case.T, case.H_q, case.D), dtype=torch.float16, device="cuda")
    st = status_tensor()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sta.paged_decode_step(t["cu"], t["past"], case.T, sq, sk, t["q"], t["k_new"],
                                  t["v_new"], kc, vc, case.max_seqlen_q, case.max_seqlen_k, out,
                                  block_table=t["block_table"], scale=case.scale,
                                  sinks=t["sinks"], workspace=ws, status=st)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        junk = torch.randn(1 << 20, device="cuda").sum()
        out.fill_(float("nan"))
        sq.fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out).cpu(), _bits(eager["out"]).cpu()), rep
        assert torch.equal(sq.cpu(), eager["sq"]) and torch.equal(sk.cpu(), eager["sk"])
        assert torch.equal(_bits(kc).cpu(), eager["k"]) and torch.equal(_bits(vc).cpu(), eager["v"])
        del junk


def test_full_size_decode_step_every_row():
    """The GQA decode workload at full size (B=32, up to 8192 keys, a 20000-block pool, NaN
    in every unreferenced slot): bit-identical to the two calls, and every row against the
    oracle."""
    print("decode step full size", flush=True)
    case = synth.config_gqa_paged_decode(poison=True)
    got = _step_vs_calls(case)
    _against_oracle(case, got, "step_full_size")
