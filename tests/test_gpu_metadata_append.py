"""GPU parity: prepare_seqlens and kv_cache_append against the oracle, bit for bit."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import selected_token_sparse_amd as sta
import synth
from synth.device import TORCH_DTYPE, case_tensors, tensor

from harness import status_tensor

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _gpu_meta(cu, past, T):
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
    past_t = torch.tensor(past, dtype=torch.int32, device="cuda")
    B = len(past)
    sq = torch.full((B,), 12345, dtype=torch.int32, device="cuda")
    sk = torch.full((B,), 12345, dtype=torch.int32, device="cuda")
    req = torch.full((max(T, 1),), 12345, dtype=torch.int32, device="cuda")
    pos = torch.full((max(T, 1),), 12345, dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    sta.prepare_seqlens(cu_t, past_t, T, sq, sk, req[:T] if T else None, pos[:T] if T else None, st)
    torch.cuda.synchronize()
    return (sq.cpu().numpy(), sk.cpu().numpy(), req[:T].cpu().numpy(), pos[:T].cpu().numpy(),
            int(st.item()))


def _check_meta(cu, past, T):
    g = _gpu_meta(cu, past, T)
    o = oracle.prepare_seqlens(cu, past, T)
    for name, a, b in zip(["seqlens_q", "seqlens_k", "token_req", "token_pos"], g[:4], o[:4]):
        assert np.array_equal(a, b), (name, a, b)
    assert g[4] == o[4]


def test_metadata_page_examples():
    with open(os.path.join(GOLDEN, "metadata_examples.json")) as f:
        for case in json.load(f)["cases"]:
            print("metadata example", case["cu_seqlens_q"], flush=True)
            g = _gpu_meta(case["cu_seqlens_q"], case["past_seqlens"], case["T"])
            assert g[0].tolist() == case["seqlens_q"]
            assert g[1].tolist() == case["seqlens_k"]
            _check_meta(case["cu_seqlens_q"], case["past_seqlens"], case["T"])


@pytest.mark.parametrize("seed", range(6))
def test_metadata_random(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 3000 if seed % 2 else 40))
    q_lens = rng.integers(0, 9 if seed % 3 else 300, size=B)
    past = rng.integers(0, 70000, size=B)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    print("metadata random", seed, B, int(cu[-1]), flush=True)
    _check_meta(cu, past.astype(np.int32), int(cu[-1]))


@pytest.mark.parametrize("cu,past,T", [
    ([1, 2, 3], [0, 0], 3), ([0, 3, 2, 4], [0, 0, 0], 4), ([0, 2, 9], [0, 0], 5),
    ([0, 2, 3], [0, 0], 5), ([0, 1, 2], [-4, 0], 2), ([-3, 5, 1, 7], [1, 2, 3], 6), ([0], [], 0),
    ([0], [], 4),
])
def test_metadata_malformed(cu, past, T):
    print("metadata malformed", cu, past, T, flush=True)
    _check_meta(cu, past, T)


def test_metadata_max_batch():
    rng = np.random.default_rng(7)
    q_lens = rng.integers(0, 3, size=8192)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    _check_meta(cu, rng.integers(0, 100, size=8192).astype(np.int32), int(cu[-1]))
    # beyond the limit: rejected on the host
    with pytest.raises(sta.SpattnError):
        _gpu_meta(np.zeros(8194, dtype=np.int32), np.zeros(8193, dtype=np.int32), 0)


APPEND_CASES = [
    dict(name="paged_f16", kv_lens=[5, 0, 40, 17, 1], q_lens=[2, 0, 40, 1, 1], dtype=synth.F16),
    dict(name="paged_bf16_bs12", kv_lens=[30, 7], q_lens=[9, 7], dtype=synth.BF16, block_size=12),
    dict(name="paged_f32", kv_lens=[3, 64], q_lens=[3, 2], dtype=synth.F32, D=128),
    dict(name="contig_f16", kv_lens=[5, 48, 20], q_lens=[2, 8, 20], dtype=synth.F16, contiguous=True, capacity=48),
    dict(name="paged_i8_from_f16", kv_lens=[9, 33, 3], q_lens=[3, 8, 3], dtype=synth.F16, cache_dtype=synth.I8, D=128),
    dict(name="paged_i8_from_bf16", kv_lens=[20], q_lens=[20], dtype=synth.BF16, cache_dtype=synth.I8),
    dict(name="contig_i8_from_f32", kv_lens=[16, 4], q_lens=[16, 4], dtype=synth.F32, cache_dtype=synth.I8, contiguous=True, capacity=16),
    dict(name="paged_fp8_from_f16", kv_lens=[5, 0, 40, 17], q_lens=[2, 0, 40, 1], dtype=synth.F16, cache_dtype=synth.FP8, D=128),
    dict(name="paged_fp8_from_bf16", kv_lens=[20], q_lens=[20], dtype=synth.BF16, cache_dtype=synth.FP8),
    dict(name="contig_fp8_from_f32", kv_lens=[16, 4], q_lens=[16, 4], dtype=synth.F32, cache_dtype=synth.FP8, contiguous=True, capacity=16),
]


def _bits(t):
    """Raw bits of a tensor, for bit-exact comparison of any element type."""
    n = t.element_size()
    return t.view(torch.uint8 if n == 1 else torch.int16 if n == 2 else torch.int32)


@pytest.mark.parametrize("spec", APPEND_CASES, ids=[c["name"] for c in APPEND_CASES])
def test_append_bit_exact(spec):
    spec = dict(spec)
    name = spec.pop("name")
    D = spec.pop("D", 64)
    print("append", name, flush=True)
    case = synth.paged_case(21, H_q=4, H_kv=2, D=D, poison=True, **spec)
    t = case_tensors(case)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    sta.kv_cache_append(t["k_new"], t["v_new"], t["cu"], t["seqlens_k"], t["k_cache"], t["v_cache"],
                        t["block_table"], t["key_scale"], t["value_scale"], status=st)
    torch.cuda.synchronize()
    kc, vc, ost = oracle.kv_cache_append(case.k_new, case.v_new, case.cu_seqlens_q, case.seqlens_k,
                                         case.k_cache, case.v_cache, case.block_table, case.block_size,
                                         case.key_scale, case.value_scale)
    for got, want in ((t["k_cache"], kc), (t["v_cache"], vc)):
        g = got.cpu()
        w = tensor(want, case.cache_dtype, "cpu")
        assert torch.equal(_bits(g), _bits(w))
    assert int(st.item()) == ost


def test_append_missing_slots_flagged_and_skipped():
    case = synth.paged_case(22, kv_lens=[20, 20, 20], q_lens=[4, 4, 4], H_q=2, H_kv=1, D=64,
                            block_size=16, dtype=synth.F16, num_blocks=6)
    bt = case.block_table.copy()
    bt[1, 1] = 99
    sk = case.seqlens_k.copy()
    sk[2] = 40
    t = case_tensors(case)
    t["block_table"] = tensor(bt, None)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    sta.kv_cache_append(t["k_new"], t["v_new"], t["cu"], tensor(sk, None), t["k_cache"], t["v_cache"],
                        t["block_table"], status=st)
    torch.cuda.synchronize()
    kc, vc, ost = oracle.kv_cache_append(case.k_new, case.v_new, case.cu_seqlens_q, sk, case.k_cache,
                                         case.v_cache, bt, case.block_size)
    assert ost == oracle.STATUS_BAD_BLOCK | oracle.STATUS_CAPACITY
    assert int(st.item()) == ost
    assert np.array_equal(t["k_cache"].cpu().numpy().view(np.int16), kc.view(np.int16))


def test_append_quantisation_hand_worked_codes():
    # one row of eight hand-worked values through the device quantiser
    with open(os.path.join(GOLDEN, "int8_codes.json")) as f:
        cases = json.load(f)["cases"]
    n = len(cases)
    D = 64
    x = np.zeros((1, 1, D), dtype=np.float32)
    s = np.ones((1, D), dtype=np.float32)
    want = np.zeros(D, dtype=np.int8)
    for i, c in enumerate(cases):
        x[0, 0, i] = np.float32(float(c["x"]))
        s[0, i] = np.float32(float(c["s"]))
        want[i] = c["code"]
    cu = tensor(np.array([0, 1], dtype=np.int32), None)
    sk = tensor(np.array([0], dtype=np.int32), None)
    kc = torch.zeros((1, 1, 1, D), dtype=torch.int8, device="cuda")
    vc = torch.zeros_like(kc)
    xt = tensor(x, None)
    st_ = tensor(s, None)
    sta.kv_cache_append(xt, xt, cu, sk, kc, vc, None, st_, st_)
    torch.cuda.synchronize()
    assert kc.cpu().numpy().reshape(-1)[:n].tolist() == want[:n].tolist()


def test_append_cursor_page_example():
    """The DynamicSparseAttention INT8 page's strict-mode cursor case (batch 1, one new row,
    capacity 2, seqlens_k = {0}, committed_length = {1}): flagged, nothing written."""
    print("append cursor page example", flush=True)
    rng = np.random.default_rng(21)
    kc0 = rng.standard_normal((1, 1, 2, 64)).astype(np.float32)
    k_new = rng.standard_normal((1, 1, 64)).astype(np.float32)
    kc, vc = tensor(kc0, None), tensor(kc0.copy(), None)
    kn = tensor(k_new, None)
    cu = tensor(np.array([0, 1], np.int32), None)
    sk = tensor(np.array([0], np.int32), None)
    st = status_tensor()
    sta.kv_cache_append(kn, kn, cu, sk, kc, vc, status=st,
                        committed_length=tensor(np.array([1], np.int32), None))
    torch.cuda.synchronize()
    assert int(st.item()) == oracle.STATUS_CURSOR
    assert np.array_equal(kc.cpu().numpy(), kc0) and np.array_equal(vc.cpu().numpy(), kc0)


@pytest.mark.parametrize("contiguous", [False, True])
def test_append_cursor_check_bit_exact(contiguous):
    print("append cursor mixed batch", contiguous, flush=True)
    case = synth.paged_case(31, kv_lens=[20, 33, 7, 64], q_lens=[3, 1, 7, 2], H_q=4, H_kv=2, D=64,
                            block_size=16, dtype=synth.F16, contiguous=contiguous, capacity=64,
                            poison=True)
    committed = case.past_seqlens.copy()
    committed[1] += 1
    committed[3] -= 2
    t = case_tensors(case)
    st = status_tensor()
    sta.kv_cache_append(t["k_new"], t["v_new"], t["cu"], t["seqlens_k"], t["k_cache"], t["v_cache"],
                        t["block_table"], status=st, committed_length=tensor(committed, None))
    torch.cuda.synchronize()
    kc, vc, ost = oracle.kv_cache_append(case.k_new, case.v_new, case.cu_seqlens_q, case.seqlens_k,
                                         case.k_cache, case.v_cache, case.block_table,
                                         case.block_size, committed_length=committed)
    assert int(st.item()) == ost == oracle.STATUS_CURSOR
    assert np.array_equal(t["k_cache"].cpu().numpy().view(np.uint16), kc.view(np.uint16))
    assert np.array_equal(t["v_cache"].cpu().numpy().view(np.uint16), vc.view(np.uint16))


def test_append_fp8_hand_worked_codes():
    # the hand-worked FP8 E4M3 codes through the device quantiser, eight per row
    with open(os.path.join(GOLDEN, "fp8_codes.json")) as f:
        cases = json.load(f)["cases"]
    D = 8 * ((len(cases) + 7) // 8)
    x = np.zeros((1, 1, D), dtype=np.float32)
    s = np.ones((1, D), dtype=np.float32)
    want = np.zeros(D, dtype=np.uint8)
    for i, c in enumerate(cases):
        x[0, 0, i] = np.float32(float(c["x"]))
        s[0, i] = np.float32(float(c["s"]))
        want[i] = c["code"]
    print("append fp8 hand-worked codes", flush=True)
    cu = tensor(np.array([0, 1], dtype=np.int32), None)
    sk = tensor(np.array([0], dtype=np.int32), None)
    kc = torch.zeros((1, 1, 1, D), dtype=torch.float8_e4m3fn, device="cuda")
    vc = torch.zeros_like(kc)
    xt = tensor(x, None)
    st_ = tensor(s, None)
    sta.kv_cache_append(xt, xt, cu, sk, kc, vc, None, st_, st_)
    torch.cuda.synchronize()
    got = kc.cpu().view(torch.uint8).numpy().reshape(-1)
    assert got[:len(cases)].tolist() == want[:len(cases)].tolist()


# ---- prepare_and_append: the two calls above in one launch -------------------------------

def _fused_vs_separate(case, cu=None, past=None, committed=None):
    """Run prepare_and_append and (on copies of the caches) prepare_seqlens then
    kv_cache_append; every output, every cache byte and the status must be identical."""
    t = case_tensors(case)
    cu_t = tensor(np.asarray(cu if cu is not None else case.cu_seqlens_q, dtype=np.int32))
    past_t = tensor(np.asarray(past if past is not None else case.past_seqlens, dtype=np.int32))
    cm = tensor(committed) if committed is not None else None
    B, T = int(past_t.shape[0]), case.T
    out = {}
    for mode in ("fused", "separate"):
        kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
        sq = torch.full((B,), 777, dtype=torch.int32, device="cuda")
        sk = torch.full((B,), 777, dtype=torch.int32, device="cuda")
        req = torch.full((T,), 777, dtype=torch.int32, device="cuda")
        pos = torch.full((T,), 777, dtype=torch.int32, device="cuda")
        st = status_tensor()
        if mode == "fused":
            sta.prepare_and_append(cu_t, past_t, T, sq, sk, t["k_new"], t["v_new"], kc, vc,
                                   t["block_table"], token_req=req, token_pos=pos,
                                   key_scale=t["key_scale"], value_scale=t["value_scale"],
                                   committed_length=cm, status=st)
        else:
            sta.prepare_seqlens(cu_t, past_t, T, sq, sk, req, pos, st)
            sta.kv_cache_append(t["k_new"], t["v_new"], cu_t, sk, kc, vc, t["block_table"],
                                t["key_scale"], t["value_scale"], status=st, committed_length=cm)
        torch.cuda.synchronize()
        out[mode] = (sq.cpu(), sk.cpu(), req.cpu(), pos.cpu(), _bits(kc).cpu(), _bits(vc).cpu(),
                     int(st.item()))
    for name, a, b in zip(("seqlens_q", "seqlens_k", "token_req", "token_pos", "k_cache", "v_cache"),
                          out["fused"][:6], out["separate"][:6]):
        assert torch.equal(a, b), name
    assert out["fused"][6] == out["separate"][6]
    return out["fused"]


@pytest.mark.parametrize("cache_dtype", [None, synth.I8, synth.FP8])
def test_prepare_and_append_decode_step(cache_dtype):
    print("prepare_and_append decode", cache_dtype, flush=True)
    base = synth.config_gqa_paged_decode(B=32, max_len=3000, seed=41)
    case = synth.paged_case(42, kv_lens=base.seqlens_k + 1, q_lens=np.diff(base.cu_seqlens_q), H_q=8,
                            H_kv=8, D=64, dtype=synth.F16, cache_dtype=cache_dtype, poison=True)
    sq, sk, req, pos, _, _, st = _fused_vs_separate(case)
    o = oracle.prepare_seqlens(case.cu_seqlens_q, case.past_seqlens, case.T)
    assert np.array_equal(sk.numpy(), o[1]) and np.array_equal(pos.numpy(), o[3]) and st == 0


def test_prepare_and_append_prefill_and_cursor():
    print("prepare_and_append prefill", flush=True)
    case = synth.paged_case(43, kv_lens=[300, 77, 1, 64], q_lens=[300, 20, 1, 0], H_q=4, H_kv=2, D=128,
                            dtype=synth.BF16, poison=True)
    _fused_vs_separate(case)
    committed = np.array([0, 57, 5, 64], dtype=np.int32)   # request 2 disagrees
    *_, st = _fused_vs_separate(case, committed=committed)
    assert st == sta.STATUS_CURSOR


@pytest.mark.parametrize("cu,past", [
    ([0, 3, 2, 5], [0, 0, 0]),          # decreasing boundary
    ([1, 3, 5], [4, 0]),                # cu[0] != 0
    ([0, 2, 9], [0, 0]),                # cu[B] > T
    ([0, 1, 5], [-4, 0]),               # negative past
])
def test_prepare_and_append_malformed(cu, past):
    """Malformed metadata: both paths sanitise and flag the same way, byte for byte."""
    print("prepare_and_append malformed", cu, past, flush=True)
    case = synth.paged_case(44, kv_lens=[8, 8], q_lens=[2, 3], H_q=4, H_kv=2, D=64, dtype=synth.F16,
                            num_blocks=8)
    _fused_vs_separate(case, cu=cu, past=past)


def test_prepare_and_append_many_requests_fall_back():
    """More than 255 requests: the two kernels run in order behind the same call."""
    print("prepare_and_append B=300", flush=True)
    rng = np.random.default_rng(45)
    kv = rng.integers(1, 40, size=300)
    case = synth.paged_case(46, kv_lens=kv, q_lens=np.ones(300, dtype=np.int64), H_q=4, H_kv=2, D=64,
                            dtype=synth.F16)
    _fused_vs_separate(case)
