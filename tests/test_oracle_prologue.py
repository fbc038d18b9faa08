"""Pins of the oracle's QKV prologue (CPU only).

Against: the complex-number form of a planar rotation (numpy complex arithmetic), the
defining invariants of RMSNorm (unit RMS, scale invariance), the relative-position
property of rotated dot products, and the equivalences the prologue's readings state
(packed = unpacked, explicit positions = default positions, offsets = shifted positions,
fused = prologue followed by the cache append).
"""
import numpy as np
import torch
import pytest

import oracle
import oracle.prologue as pro
import synth


def _tables(max_pos, rotary_dim, base=10000.0):
    # the test's own angle tables: theta_i = base^(-2i/rotary_dim), angle = pos * theta_i
    half = rotary_dim // 2
    theta = base ** (-2.0 * np.arange(half) / rotary_dim)
    ang = np.arange(max_pos)[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang), ang


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("rotary_dim", [64, 32, 16])
def test_rotation_is_complex_multiplication(interleaved, rotary_dim):
    rng = np.random.default_rng(1)
    D = 64
    x = rng.standard_normal((7, 3, D))
    pos = rng.integers(0, 500, size=(7, 3))
    cos, sin, ang = _tables(500, rotary_dim)
    got, _ = pro.rotate(x, pos, cos, sin, rotary_dim, interleaved)
    half = rotary_dim // 2
    if interleaved:
        z = x[..., 0:rotary_dim:2] + 1j * x[..., 1:rotary_dim:2]
    else:
        z = x[..., :half] + 1j * x[..., half:rotary_dim]
    w = z * np.exp(1j * ang[pos])
    if interleaved:
        assert np.allclose(got[..., 0:rotary_dim:2], w.real, atol=1e-12)
        assert np.allclose(got[..., 1:rotary_dim:2], w.imag, atol=1e-12)
    else:
        assert np.allclose(got[..., :half], w.real, atol=1e-12)
        assert np.allclose(got[..., half:rotary_dim], w.imag, atol=1e-12)
    # channels past rotary_dim are untouched, bit for bit
    assert np.array_equal(got[..., rotary_dim:], x[..., rotary_dim:])
    # |rotated| = |x|
    assert np.allclose(np.linalg.norm(got, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotated_dot_product_depends_on_relative_position(interleaved):
    rng = np.random.default_rng(2)
    D, rd = 32, 32
    cos, sin, _ = _tables(300, rd)
    qv, kv = rng.standard_normal(D), rng.standard_normal(D)
    for m, n in [(10, 3), (120, 113), (250, 243), (7, 0)]:
        a, _ = pro.rotate(qv, np.array(m), cos, sin, rd, interleaved)
        b, _ = pro.rotate(kv, np.array(n), cos, sin, rd, interleaved)
        c, _ = pro.rotate(qv, np.array(m - n), cos, sin, rd, interleaved)
        assert abs(a @ b - c @ kv) < 1e-10


def test_position_zero_is_identity():
    cos, sin, _ = _tables(4, 16)
    x = np.random.default_rng(3).standard_normal((2, 16))
    got, _ = pro.rotate(x, np.zeros(2, dtype=int), cos, sin, 16, False)
    assert np.array_equal(got, x)


def test_rms_norm_invariants():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 4, 64)) * 3.0
    y = pro.rms_norm(x, None, 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-12)
    assert np.allclose(pro.rms_norm(7.5 * x, None, 0.0), y, rtol=1e-12)
    w = rng.uniform(0.5, 2.0, 64)
    assert np.allclose(pro.rms_norm(x, w, 0.0), y * w, rtol=1e-12)
    # eps sits under the root with the mean: a zero head stays zero, a head of RMS r is
    # scaled by 1/sqrt(r^2 + eps)
    assert np.array_equal(pro.rms_norm(np.zeros(64), None, 1e-6), np.zeros(64))
    ones = np.ones(64) * 0.01
    assert np.allclose(pro.rms_norm(ones, None, 1e-4), ones / np.sqrt(1e-4 + 1e-4), rtol=1e-12)


def test_round_to_bf16_matches_float32_then_bf16_away_from_ties():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(10000) * 10.0
    got = pro.round_to(x, "bf16")
    # bf16 keeps the top 16 bits of a float32: every result is such a value, and it is
    # the nearest one (within half a bf16 step of x)
    bits = got.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    step = np.ldexp(1.0, np.frexp(np.abs(x))[1] - 8)
    assert np.all(np.abs(got - x) <= step / 2)


def test_round_to_bf16_ties_and_subnormals_match_torch():
    """Pins round_to(.., "bf16") where a plausible mistake shows: exact ties (the low 16 bits
    of a float32 equal to 0x8000, which must go to the even bf16 neighbour, not away from
    zero and not by truncation), their neighbours 0x7FFF / 0x8001, and the subnormal range
    (spacing 2^-133 below 2^-126), against torch's float32 -> bfloat16 conversion, which
    rounds to nearest with ties to even."""
    rng = np.random.default_rng(17)
    hi = rng.integers(0, 1 << 16, size=40000).astype(np.uint32)
    hi = hi[((hi >> 7) & 0xFF) != 0xFF]                   # no inf / NaN exponents
    hi = np.concatenate([hi, np.arange(0, 1 << 8, dtype=np.uint32),            # subnormals
                         np.arange(1 << 15, (1 << 15) + (1 << 8), dtype=np.uint32)])
    for low in (0x8000, 0x7FFF, 0x8001, 0x0000, 0x3000, 0xC000):
        x = ((hi << 16) | np.uint32(low)).view(np.float32)
        got = pro.round_to(x.astype(np.float64), "bf16")
        want = torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), hex(low)
    # hand-worked ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 (even: 1);
    # 1 + 3 * 2^-8 halfway between 1 + 2^-7 and 1 + 2^-6 (even: 1 + 2^-6); same negated
    t = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), -(1 + 3 * 2.0 ** -8)])
    assert pro.round_to(t, "bf16").tolist() == [1.0, 1 + 2.0 ** -6, -1.0, -(1 + 2.0 ** -6)]


def _case(**kw):
    return synth.prologue_case(**kw)


def _run(case, **over):
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


def test_packed_equals_unpacked():
    case = _case(seed=11, kv_lens=[40, 9], q_lens=[5, 9], H_q=8, H_kv=2, D=64, dtype=synth.F16,
                 packed=True, rotary_dim=32, qk_norm=True)
    a = _run(case)
    q, k, v = pro.split_qkv(case.qkv, case.H_q, case.H_kv, case.D)
    # the packed row is [queries | keys | values]: check the split against the layout
    row = case.qkv.reshape(case.T, -1)
    assert np.array_equal(q[3, 5], row[3, 5 * 64:6 * 64])
    assert np.array_equal(k[3, 1], row[3, (8 + 1) * 64:(8 + 2) * 64])
    assert np.array_equal(v[3, 0], row[3, (8 + 2) * 64:(8 + 3) * 64])
    b = _run(case, qkv=None, q=np.ascontiguousarray(q), k=np.ascontiguousarray(k),
             v=np.ascontiguousarray(v))
    assert np.array_equal(a["q_out"], b["q_out"])
    assert np.array_equal(a["k_cache"], b["k_cache"], equal_nan=True)
    assert np.array_equal(a["v_cache"], b["v_cache"], equal_nan=True)


def test_explicit_positions_and_offsets():
    case = _case(seed=12, kv_lens=[30, 7], q_lens=[4, 7], H_q=4, H_kv=2, D=64, dtype=synth.F32,
                 rotary_dim=64, interleaved=True)
    base = _run(case)
    default = pro.positions(case.cu_seqlens_q, case.seqlens_k, case.T)
    assert default.tolist() == [26, 27, 28, 29, 0, 1, 2, 3, 4, 5, 6]
    same = _run(case, position_ids=default.astype(np.int32))
    assert np.array_equal(base["q_out"], same["q_out"])
    off = np.array([5, 11], dtype=np.int32)
    shifted = _run(case, rotary_offsets=off)
    by_ids = _run(case, position_ids=(default + np.repeat(off, [4, 7])).astype(np.int32))
    assert np.array_equal(shifted["q_out"], by_ids["q_out"])
    assert np.array_equal(shifted["k_cache"], by_ids["k_cache"], equal_nan=True)
    assert not np.array_equal(shifted["q_out"], base["q_out"])


def test_no_norm_no_rotation_is_the_plain_append():
    for cache_dtype in (synth.F16, synth.I8, synth.FP8):
        case = _case(seed=13, kv_lens=[20, 33], q_lens=[3, 8], H_q=8, H_kv=2, D=64,
                     dtype=synth.F16, cache_dtype=cache_dtype, rotary_dim=0, qk_norm=False)
        r = _run(case)
        assert np.array_equal(r["q_out"], case.q)
        kc, vc, st = oracle.kv_cache_append(case.k, case.v, case.cu_seqlens_q, case.seqlens_k,
                                            case.k_cache, case.v_cache, case.block_table,
                                            case.block_size, case.key_scale, case.value_scale)
        assert st == r["status"] == 0
        assert np.array_equal(kc, r["k_cache"], equal_nan=True)
        assert np.array_equal(vc, r["v_cache"], equal_nan=True)


def test_fused_equals_prologue_then_append():
    case = _case(seed=14, kv_lens=[50, 20], q_lens=[6, 20], H_q=8, H_kv=2, D=64,
                 dtype=synth.BF16, cache_dtype=synth.I8, rotary_dim=48, qk_norm=True)
    r = _run(case)
    k = pro.rms_norm(case.k, case.k_norm_weight, case.norm_eps)
    pos = pro.positions(case.cu_seqlens_q, case.seqlens_k, case.T)
    k, _ = pro.rotate(k, np.repeat(pos[:, None], case.H_kv, axis=1), case.cos_table,
                      case.sin_table, 48, False)
    kc, vc, _ = oracle.kv_cache_append(pro.round_to(k, "bf16"), case.v, case.cu_seqlens_q,
                                       case.seqlens_k, case.k_cache, case.v_cache, case.block_table,
                                       case.block_size, case.key_scale, case.value_scale)
    assert np.array_equal(kc, r["k_cache"])
    assert np.array_equal(vc, r["v_cache"])


def test_out_of_range_position_and_cursor():
    case = _case(seed=15, kv_lens=[12, 9], q_lens=[2, 3], H_q=4, H_kv=2, D=64, dtype=synth.F16,
                 rotary_dim=64, max_position=64)
    pos = pro.positions(case.cu_seqlens_q, case.seqlens_k, case.T).astype(np.int32)
    pos[1] = 64          # one past the table
    pos[3] = -1
    r = _run(case, position_ids=pos)
    assert r["status"] == oracle.STATUS_POSITION
    assert np.all(r["q_out"][[1, 3]] == 0) and np.any(r["q_out"][[0, 2, 4]] != 0)
    plain = _run(case)
    # rows 1 and 3 are not appended (their slots keep the old contents); the other rows
    # are exactly those of the run with in-range positions
    skip = np.zeros(case.T, dtype=bool)
    skip[[1, 3]] = True
    kc_skip, _, _ = oracle.kv_cache_append(plain["k_new"], case.v, case.cu_seqlens_q, case.seqlens_k,
                                           case.k_cache, case.v_cache, case.block_table,
                                           case.block_size, skip_rows=skip)
    ok_rows = [0, 2, 4]
    assert np.array_equal(r["q_out"][ok_rows], plain["q_out"][ok_rows])
    assert np.array_equal(r["k_cache"], kc_skip, equal_nan=True)
    bt, bs = case.block_table, case.block_size
    for t, (b, p) in {1: (0, 11), 3: (1, 7)}.items():
        blk, off = bt[b][p // bs], p % bs
        assert np.array_equal(r["k_cache"][blk, :, off], case.k_cache[blk, :, off], equal_nan=True)
        assert np.array_equal(r["v_cache"][blk, :, off], case.v_cache[blk, :, off], equal_nan=True)
    # a cursor mismatch: queries still come out, request 1 appends nothing
    cur = np.array([10, 0], dtype=np.int32)    # request 0 holds 10 keys before: right
    c = _run(case, committed_length=cur)
    assert c["status"] == oracle.STATUS_CURSOR
    assert np.array_equal(c["q_out"], plain["q_out"])
    kc1, _, _ = oracle.kv_cache_append(plain["k_new"], case.v, case.cu_seqlens_q, case.seqlens_k,
                                       case.k_cache, case.v_cache, case.block_table, case.block_size,
                                       committed_length=cur)
    assert np.array_equal(c["k_cache"], kc1, equal_nan=True)
