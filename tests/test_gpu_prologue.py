"""GPU parity of qkv_prologue against the oracle.

The kernel evaluates the norm and the rotation in float32 and rounds once; the oracle
evaluates them in float64.  Bound on the kernel's float32 value before that rounding, with
u = 2^-24:

* the norm factor 1/sqrt(mean(x^2) + eps) is one number per (token, head), so its error is
  a common relative error of every output of the head.  The sum of squares is formed per
  lane over at most 4 terms, then by a 6-level butterfly across the wave: a summation tree
  of depth <= 10 over positive terms, relative error <= 10u; the mean, eps, root and
  reciprocal add <= 3u and halve the sum's share, so <= 16u relative to the output;
* the scaling by the norm and weight, the rotation's two products and its sum add <= 8u
  relative to m, the sum of the magnitudes of the terms (the oracle returns m).

So w = 16u |ref| (with the norm) + 8u m.  Rounding to the activation type and quantising
to a cache code are monotonic, so every query output and every stored key element must lie
in [round(ref - w), round(ref + w)]: bit-exact wherever ref is not within w of a rounding
boundary (a small fraction, also checked).  Value rows pass through unchanged and must be
bit-exact, as must every cache slot the step does not write (poisoned with NaN).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import oracle.prologue as pro
import selected_token_sparse_amd as sta
import synth
from synth.device import TORCH_DTYPE, tensor

from harness import assert_close, status_tensor

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _window(ref64, mag, qk_norm):
    return (16 * U * np.abs(ref64) if qk_norm else 0.0) + 8 * U * mag


def _oracle(case, **over):
    kw = dict(dtype=synth.DTYPE_NAMES[case.dtype], cu_seqlens_q=case.cu_seqlens_q,
              seqlens_k=case.seqlens_k, H_q=case.H_q, H_kv=case.H_kv, D=case.D,
              k_cache=case.k_cache, v_cache=case.v_cache, qkv=case.qkv, q=case.q, k=case.k,
              v=case.v, qk_norm=case.qk_norm, q_norm_weight=case.q_norm_weight,
              k_norm_weight=case.k_norm_weight, norm_eps=case.norm_eps, cos_table=case.cos_table,
              sin_table=case.sin_table, rotary_dim=case.rotary_dim, interleaved=case.interleaved,
              position_ids=case.position_ids, rotary_offsets=case.rotary_offsets,
              block_table=case.block_table, block_size=case.block_size, key_scale=case.key_scale,
              value_scale=case.value_scale, committed_length=case.committed_length)
    kw.update(over)
    return oracle.qkv_prologue(**kw)


def _gpu(case, position_ids=None, committed_length=None):
    dt = case.dtype
    pos = position_ids if position_ids is not None else case.position_ids
    t = dict(
        qkv=tensor(case.qkv, dt) if case.qkv is not None else None,
        q=tensor(np.ascontiguousarray(case.q), dt) if case.qkv is None else None,
        k=tensor(np.ascontiguousarray(case.k), dt) if case.qkv is None else None,
        v=tensor(np.ascontiguousarray(case.v), dt) if case.qkv is None else None,
        cu=tensor(case.cu_seqlens_q), sk=tensor(case.seqlens_k),
        kc=tensor(case.k_cache, case.cache_dtype), vc=tensor(case.v_cache, case.cache_dtype),
        bt=tensor(case.block_table), ks=tensor(case.key_scale), vs=tensor(case.value_scale),
        qw=tensor(case.q_norm_weight), kw=tensor(case.k_norm_weight),
        cos=tensor(case.cos_table), sin=tensor(case.sin_table), pos=tensor(pos),
        offs=tensor(case.rotary_offsets),
        cur=tensor(committed_length if committed_length is not None else case.committed_length))
    q_out = torch.full((case.T, case.H_q, case.D), float("nan"), dtype=TORCH_DTYPE[dt], device="cuda")
    st = status_tensor()
    sta.qkv_prologue(q_out, t["kc"], t["vc"], t["cu"], t["sk"], H_q=case.H_q, H_kv=case.H_kv,
                     qkv=t["qkv"], q=t["q"], k=t["k"], v=t["v"], qk_norm=case.qk_norm,
                     q_norm_weight=t["qw"], k_norm_weight=t["kw"], norm_eps=case.norm_eps,
                     rotary_dim=case.rotary_dim, interleaved=case.interleaved,
                     cos_table=t["cos"], sin_table=t["sin"], position_ids=t["pos"],
                     rotary_offsets=t["offs"], block_table=t["bt"], key_scale=t["ks"],
                     value_scale=t["vs"], committed_length=t["cur"], status=st)
    torch.cuda.synchronize()
    return q_out, t["kc"], t["vc"], int(st.item()), t


def _host(x: torch.Tensor):
    if x.dtype == torch.float8_e4m3fn:
        return x.cpu().view(torch.uint8).numpy()
    if x.dtype == torch.bfloat16:
        return x.cpu().float().numpy()
    return x.cpu().numpy()


def _ordered(a):
    """Values in an order-preserving float64 form (FP8 codes decoded)."""
    if a.dtype == np.uint8:
        return oracle.decode_fp8_e4m3(a)
    return a.astype(np.float64)


def _check_between(got, lo, hi, what):
    g, l, h = _ordered(got), _ordered(lo), _ordered(hi)
    nan = np.isnan(l)
    assert np.array_equal(nan, np.isnan(h)), what
    assert np.array_equal(np.isnan(g), nan), f"{what}: NaN pattern differs"
    with np.errstate(invalid="ignore"):
        bad = ~nan & ~((g >= l) & (g <= h))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        first = tuple(idx[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside the rounding interval; "
                             f"first at {idx.tolist()}: gpu {g[first]} lo {l[first]} hi {h[first]}")
    return int((l[~nan] != h[~nan]).sum())


def _check(case, name, position_ids=None, committed_length=None):
    print("prologue", name, flush=True)
    over = {}
    if position_ids is not None:
        over["position_ids"] = position_ids
    if committed_length is not None:
        over["committed_length"] = committed_length
    ref = _oracle(case, **over)
    q_out, kc, vc, st, _ = _gpu(case, position_ids=position_ids, committed_length=committed_length)
    assert st == ref["status"], (name, st, ref["status"])
    dname = synth.DTYPE_NAMES[case.dtype]
    wq = _window(ref["q64"], ref["q_mag"], case.qk_norm)
    amb_q = _check_between(_host(q_out), pro.round_to(ref["q64"] - wq, dname),
                           pro.round_to(ref["q64"] + wq, dname), f"{name}: q_out")
    wk = _window(ref["k64"], ref["k_mag"], case.qk_norm)
    kw = dict(block_table=case.block_table, block_size=case.block_size, key_scale=case.key_scale,
              value_scale=case.value_scale, skip_rows=ref["skipped"],
              committed_length=over.get("committed_length", case.committed_length))
    lo_k, _, _ = oracle.kv_cache_append(pro.round_to(ref["k64"] - wk, dname), case.v, case.cu_seqlens_q,
                                        case.seqlens_k, case.k_cache, case.v_cache, **kw)
    hi_k, _, _ = oracle.kv_cache_append(pro.round_to(ref["k64"] + wk, dname), case.v, case.cu_seqlens_q,
                                        case.seqlens_k, case.k_cache, case.v_cache, **kw)
    amb_k = _check_between(_host(kc), lo_k, hi_k, f"{name}: k_cache")
    gv = _host(vc)
    assert np.array_equal(gv, ref["v_cache"], equal_nan=gv.dtype.kind == "f"), f"{name}: v_cache differs"
    # 16-bit outputs: elements whose window holds a rounding boundary are few, so nearly
    # every element is pinned exactly (float32 outputs: the window is a few float32 ulps)
    if case.dtype != synth.F32:
        n_k = int(np.count_nonzero(ref["k_cache"] != case.k_cache)) + 1
        assert amb_q <= 8 + q_out.numel() // 50 and amb_k <= 8 + n_k // 50, (amb_q, amb_k)
    return ref, q_out, kc, vc


VARIANTS = [
    ("f16_packed_norm_rope_full", dict(kv_lens=[70, 16, 33], q_lens=[70, 3, 1], H_q=8, H_kv=2, D=64,
                                       dtype=synth.F16, packed=True, rotary_dim=64, qk_norm=True,
                                       q_scale=4.0)),
    ("f16_unpacked_interleaved_partial_d128", dict(kv_lens=[40, 90], q_lens=[8, 90], H_q=12, H_kv=1,
                                                   D=128, dtype=synth.F16, rotary_dim=32,
                                                   interleaved=True)),
    ("bf16_packed_half_partial_contig_posids", dict(kv_lens=[50, 20], q_lens=[17, 20], H_q=16, H_kv=4,
                                                    D=128, dtype=synth.BF16, packed=True,
                                                    rotary_dim=64, qk_norm=True, norm_weights=False,
                                                    contiguous=True, explicit_positions=True)),
    ("f32_interleaved_norm_offsets", dict(kv_lens=[33, 7], q_lens=[5, 7], H_q=4, H_kv=2, D=64,
                                          dtype=synth.F32, rotary_dim=64, interleaved=True,
                                          qk_norm=True, offsets=True, q_scale=0.3)),
    ("f16_int8_cache_norm_rope", dict(kv_lens=[60, 25], q_lens=[9, 25], H_q=8, H_kv=2, D=64,
                                      dtype=synth.F16, cache_dtype=synth.I8, rotary_dim=64,
                                      qk_norm=True)),
    ("bf16_fp8_cache_packed", dict(kv_lens=[45, 130], q_lens=[4, 130], H_q=8, H_kv=1, D=128,
                                   dtype=synth.BF16, cache_dtype=synth.FP8, packed=True,
                                   rotary_dim=96, qk_norm=True)),
    ("f16_fp8_cache_interleaved_bs7", dict(kv_lens=[20, 41], q_lens=[20, 6], H_q=4, H_kv=4, D=64,
                                           dtype=synth.F16, cache_dtype=synth.FP8, rotary_dim=16,
                                           interleaved=True, block_size=7)),
    ("f16_d72_partial", dict(kv_lens=[19, 5], q_lens=[19, 5], H_q=6, H_kv=3, D=72, dtype=synth.F16,
                             rotary_dim=40, qk_norm=True)),
    ("f16_d256", dict(kv_lens=[9], q_lens=[9], H_q=4, H_kv=2, D=256, dtype=synth.F16,
                      rotary_dim=128, qk_norm=True, packed=True)),
]


@pytest.mark.parametrize("name,kw", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_prologue_variants(name, kw):
    case = synth.prologue_case(seed=zlib.crc32(name.encode()) % 1000, name=name, **kw)
    _check(case, name)


def test_no_norm_no_rotation_equals_kv_cache_append():
    """With both steps off the prologue is the plain append: bit-identical caches, and the
    query rows copied unchanged."""
    for cd in (synth.F16, synth.I8, synth.FP8):
        case = synth.prologue_case(seed=21, kv_lens=[30, 64], q_lens=[6, 64], H_q=8, H_kv=2, D=64,
                                   dtype=synth.F16, cache_dtype=cd)
        q_out, kc, vc, st, t = _gpu(case)
        assert st == 0
        kc2, vc2 = tensor(case.k_cache, cd), tensor(case.v_cache, cd)
        sta.kv_cache_append(tensor(np.ascontiguousarray(case.k), case.dtype),
                            tensor(np.ascontiguousarray(case.v), case.dtype), t["cu"], t["sk"],
                            kc2, vc2, t["bt"], key_scale=t["ks"], value_scale=t["vs"])
        torch.cuda.synchronize()
        assert torch.equal(_as_bytes(kc), _as_bytes(kc2)) and torch.equal(_as_bytes(vc), _as_bytes(vc2))
        assert torch.equal(q_out.cpu(), tensor(case.q, case.dtype, "cpu"))


def _as_bytes(x):
    return x.view(torch.uint8)


def test_out_of_range_positions_and_cursor():
    case = synth.prologue_case(seed=22, kv_lens=[12, 9, 40], q_lens=[2, 3, 40], H_q=8, H_kv=2, D=64,
                               dtype=synth.F16, rotary_dim=64, qk_norm=True, max_position=64)
    pos = pro.positions(case.cu_seqlens_q, case.seqlens_k, case.T).astype(np.int32)
    pos[1] = 64
    pos[3] = -5
    pos[30] = 1 << 20
    _check(case, "bad positions", position_ids=pos)
    cur = np.array([10, 0, 0], dtype=np.int32)   # request 1 disagrees; 0 and 2 agree
    _check(case, "cursor", committed_length=cur)
    _check(case, "both", position_ids=pos, committed_length=cur)
    # the 40-row request disagrees (its waves resolve their request by the scalar path)
    _check(case, "cursor, long request", committed_length=np.array([0, 6, 5], dtype=np.int32))


def test_full_size_decode_step_shape():
    """The GQA decode workload's shape (B = 32 rows, H 64/8, D = 64, 20000-block pool):
    packed rows, norm and full rotation, every element checked."""
    base = synth.config_gqa_paged_decode(B=32, max_len=8192, seed=1002)
    kv = base.seqlens_k + 1
    ql = np.diff(base.cu_seqlens_q)
    case = synth.prologue_case(seed=23, kv_lens=kv, q_lens=ql, H_q=64, H_kv=8, D=64,
                               dtype=synth.F16, packed=True, rotary_dim=64, qk_norm=True,
                               num_blocks=base.num_blocks, poison=False, q_scale=3.0)
    _check(case, "decode shape")


def test_full_size_prefill_shape():
    """The windowed prefill workload's shape (B = 4 prompts of 1024/512/2048/1536 rows,
    H 64/8, D = 64): 5120 rows, unpacked, half-layout rotation and norm."""
    case = synth.prologue_case(seed=24, kv_lens=[1024, 512, 2048, 1536], q_lens=[1024, 512, 2048, 1536],
                               H_q=64, H_kv=8, D=64, dtype=synth.F16, rotary_dim=64, qk_norm=True,
                               num_blocks=1024, poison=False)
    _check(case, "prefill shape")


@pytest.mark.parametrize("name,kw", [
    # D = 72: 9 lanes per row (sum of squares through LDS), rotary_dim 40 (angles one by one)
    ("deep_d72_half_rd40", dict(kv_lens=[2400, 2400, 2500, 2400], q_lens=[2400, 2400, 2400, 2400],
                                H_q=8, H_kv=2, D=72, rotary_dim=40, qk_norm=True)),
    # D = 128 interleaved, INT8 cache, explicit positions
    ("deep_d128_interleaved_int8", dict(kv_lens=[1500, 1600], q_lens=[1500, 1500], H_q=16, H_kv=4,
                                        D=128, rotary_dim=96, interleaved=True, qk_norm=True,
                                        cache_dtype=synth.I8, explicit_positions=True)),
], ids=lambda v: v if isinstance(v, str) else "")
def test_many_rows_take_the_batched_launch(name, kw):
    """Enough rows (>= 65536 at D = 64, 57344 at D = 72, 32768 at D = 128) for the launch
    that gives each wave two row batches; the other shapes take one batch per wave."""
    case = synth.prologue_case(seed=26, dtype=synth.F16, poison=False, **kw)
    _check(case, name)


def test_prologue_then_attention_matches_the_oracle():
    """End to end: prologue then paged attention on the GPU against the oracle's prologue
    then attention (f16 cache, sinks, a window), the attention tolerance."""
    case = synth.prologue_case(seed=25, kv_lens=[300, 77, 1], q_lens=[1, 77, 1], H_q=16, H_kv=2, D=64,
                               dtype=synth.F16, packed=True, rotary_dim=64, qk_norm=True, q_scale=2.0)
    ref = _oracle(case)
    q_out, kc, vc, st, t = _gpu(case)
    assert st == 0
    sinks = np.random.default_rng(3).standard_normal(case.H_q).astype(np.float32)
    out = torch.empty_like(q_out)
    max_q, max_k = int(np.diff(case.cu_seqlens_q).max()), int(case.seqlens_k.max()) + 1
    sta.paged_attention_fwd(q_out, kc, vc, t["cu"], t["sk"], max_q, max_k, out,
                            block_table=t["bt"], sinks=tensor(sinks), local_window=100)
    torch.cuda.synchronize()
    want, _ = oracle.paged_attention(ref["q_out"], ref["k_cache"], ref["v_cache"], case.cu_seqlens_q,
                                     case.seqlens_k, H_kv=case.H_kv, block_table=case.block_table,
                                     block_size=case.block_size, max_seqlen_q=max_q,
                                     max_seqlen_k=max_k, local_window=100, sinks=sinks)
    assert_close(out, want, case.dtype, "prologue + attention")
