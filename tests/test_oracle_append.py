"""Pins of the oracle's cache append, INT8 code and FP8 E4M3 code (CPU only).

Against: hand-worked INT8 and FP8 codes (golden fixtures), the closed-form quantisation
error bounds, the library's float8_e4m3fn conversion, the cursor example of the pages'
review, and the logical key sequence the inputs were laid out from (read back through
the block table by this test's own walk).
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_int8_hand_worked_codes():
    with open(os.path.join(GOLDEN, "int8_codes.json")) as f:
        data = json.load(f)
    for case in data["cases"]:
        x = np.float32(float(case["x"]))
        s = np.float32(float(case["s"]))
        assert int(oracle.quantize_int8(x, s)) == case["code"], case["note"]


def test_int8_error_bound():
    rng = np.random.default_rng(3)
    s = rng.uniform(0.005, 0.02, size=4096).astype(np.float32)
    x = (rng.uniform(-120, 120, size=4096) * s).astype(np.float32)
    code = oracle.quantize_int8(x, s).astype(np.float64)
    # in range: |code * s - x| <= s / 2 (plus float32 rounding of the quotient)
    assert np.all(np.abs(code * s - x) <= 0.5 * s * (1 + 1e-6))


def _walk(cache, block_table, bs, b, j):
    """All KV heads of position j of request b ([nb, H_kv, bs, D] blocks)."""
    if block_table is None:
        return cache[b, :, j]
    return cache[block_table[b][j // bs], :, j % bs]


@pytest.mark.parametrize("contiguous", [False, True])
def test_append_places_rows_at_their_positions(contiguous):
    case = synth.paged_case(11, kv_lens=[5, 0, 40, 17], q_lens=[2, 0, 40, 1], H_q=4, H_kv=2,
                            D=64, block_size=16, dtype=synth.F16, contiguous=contiguous,
                            capacity=48, num_blocks=12, poison=True)
    kc, vc, st = oracle.kv_cache_append(case.k_new, case.v_new, case.cu_seqlens_q, case.seqlens_k,
                                        case.k_cache, case.v_cache, case.block_table, case.block_size)
    assert st == 0
    cu = case.cu_seqlens_q
    for b in range(case.B):
        q_len = int(cu[b + 1] - cu[b])
        kv_len = int(case.seqlens_k[b]) + 1
        for j in range(kv_len):
            got_k = _walk(kc, case.block_table, case.block_size, b, j)
            if j < kv_len - q_len:      # history untouched
                want = _walk(case.k_cache, case.block_table, case.block_size, b, j)
            else:                       # this step's rows
                want = case.k_new[cu[b] + j - (kv_len - q_len)]
            assert np.array_equal(got_k, want, equal_nan=True)
    # nothing else changed: compare everything not written
    written = np.zeros((kc.shape[0], kc.shape[2]), dtype=bool)
    for b in range(case.B):
        q_len = int(cu[b + 1] - cu[b])
        kv_len = int(case.seqlens_k[b]) + 1
        for j in range(kv_len - q_len, kv_len):
            if case.block_table is None:
                written[b, j] = True
            else:
                written[case.block_table[b][j // case.block_size], j % case.block_size] = True
    tr = (0, 2, 1, 3)
    assert np.array_equal(kc.transpose(tr)[~written], case.k_cache.transpose(tr)[~written], equal_nan=True)
    assert np.array_equal(vc.transpose(tr)[~written], case.v_cache.transpose(tr)[~written], equal_nan=True)


def test_append_int8_quantises_with_channel_scales():
    case = synth.paged_case(12, kv_lens=[9, 33], q_lens=[3, 8], H_q=8, H_kv=2, D=128,
                            block_size=16, dtype=synth.F16, cache_dtype=synth.I8)
    kc, vc, st = oracle.kv_cache_append(case.k_new, case.v_new, case.cu_seqlens_q, case.seqlens_k,
                                        case.k_cache, case.v_cache, case.block_table, case.block_size,
                                        case.key_scale, case.value_scale)
    assert st == 0
    b, j, r = 1, 32, int(case.cu_seqlens_q[2]) - 1
    code = _walk(kc, case.block_table, case.block_size, b, j).astype(np.float64)
    x = case.k_new[r].astype(np.float64)
    s = case.key_scale.astype(np.float64)
    inside = np.abs(x / s) < 126.5
    assert np.all(np.abs(code * s - x)[inside] <= 0.5 * s[inside] * (1 + 1e-6))
    assert np.all(np.abs(code[~inside]) == 127)


def test_append_skips_missing_slots():
    case = synth.paged_case(13, kv_lens=[20, 20], q_lens=[4, 4], H_q=2, H_kv=1, D=64,
                            block_size=16, dtype=synth.F32, num_blocks=4)
    bt = case.block_table.copy()
    bt[1, 1] = 99                      # block id beyond the pool
    kc, vc, st = oracle.kv_cache_append(case.k_new, case.v_new, case.cu_seqlens_q, case.seqlens_k,
                                        case.k_cache, case.v_cache, bt, case.block_size)
    assert st & oracle.STATUS_BAD_BLOCK
    sk = case.seqlens_k.copy()
    sk[0] = 40                         # beyond 2 blocks of table
    kc, vc, st = oracle.kv_cache_append(case.k_new, case.v_new, case.cu_seqlens_q, sk,
                                        case.k_cache, case.v_cache, case.block_table, case.block_size)
    assert st & oracle.STATUS_CAPACITY


def test_cursor_mismatch_page_example_appends_nothing():
    """The DynamicSparseAttention INT8 page's review finding on strict-mode cursor
    validation: batch 1, one new row, cache capacity 2, seqlens_k = {0} (the row goes to
    position 0), committed_length = {1}.  The cursor disagrees with the append position,
    so the request is flagged and the cache is left untouched."""
    rng = np.random.default_rng(21)
    kc = rng.standard_normal((1, 1, 2, 64)).astype(np.float32)   # contiguous [B, H_kv, cap, D]
    vc = rng.standard_normal((1, 1, 2, 64)).astype(np.float32)
    k_new = rng.standard_normal((1, 1, 64)).astype(np.float32)
    v_new = rng.standard_normal((1, 1, 64)).astype(np.float32)
    cu = np.array([0, 1], np.int32)
    sk = np.array([0], np.int32)
    out_k, out_v, st = oracle.kv_cache_append(k_new, v_new, cu, sk, kc, vc,
                                              committed_length=np.array([1], np.int32))
    assert st == oracle.STATUS_CURSOR
    assert np.array_equal(out_k, kc) and np.array_equal(out_v, vc)
    # the consistent cursor (0 keys before this step) appends the row at position 0
    out_k, out_v, st = oracle.kv_cache_append(k_new, v_new, cu, sk, kc, vc,
                                              committed_length=np.array([0], np.int32))
    assert st == 0
    assert np.array_equal(out_k[0, 0, 0], k_new[0, 0]) and np.array_equal(out_k[0, 0, 1], kc[0, 0, 1])


def test_cursor_check_skips_only_the_inconsistent_request():
    case = synth.paged_case(14, kv_lens=[20, 33, 7], q_lens=[3, 1, 7], H_q=2, H_kv=1, D=64,
                            block_size=16, dtype=synth.F16)
    committed = case.past_seqlens.copy()
    committed[1] += 1                    # request 1 believes it holds one key more
    kc, vc, st = oracle.kv_cache_append(case.k_new, case.v_new, case.cu_seqlens_q, case.seqlens_k,
                                        case.k_cache, case.v_cache, case.block_table,
                                        case.block_size, committed_length=committed)
    assert st == oracle.STATUS_CURSOR
    ref_k, _, st0 = oracle.kv_cache_append(case.k_new, case.v_new, case.cu_seqlens_q, case.seqlens_k,
                                           case.k_cache, case.v_cache, case.block_table,
                                           case.block_size)
    assert st0 == 0
    cu = case.cu_seqlens_q
    for b in range(case.B):
        q_len = int(cu[b + 1] - cu[b])
        kv_len = int(case.seqlens_k[b]) + 1
        for j in range(kv_len - q_len, kv_len):
            got = _walk(kc, case.block_table, case.block_size, b, j)
            want = (_walk(case.k_cache, case.block_table, case.block_size, b, j) if b == 1
                    else _walk(ref_k, case.block_table, case.block_size, b, j))
            assert np.array_equal(got, want, equal_nan=True), (b, j)


def test_fp8_hand_worked_codes():
    with open(os.path.join(GOLDEN, "fp8_codes.json")) as f:
        data = json.load(f)
    for case in data["cases"]:
        x = np.float32(float(case["x"]))
        s = np.float32(float(case["s"]))
        assert int(oracle.quantize_fp8_e4m3(x, s)) == case["code"], case["note"]


def test_fp8_decode_matches_library_type():
    """Every one of the 256 codes decodes as the library's float8_e4m3fn type does."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(oracle.decode_fp8_e4m3(codes), lib, equal_nan=True)


def test_fp8_encode_matches_library_in_range_and_round_trips():
    """Inside +-464 (where no saturation applies) the code equals the library's round-to-
    nearest-even conversion, including every exact value and every tie; each finite code
    round-trips."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    vals = oracle.decode_fp8_e4m3(finite)
    assert np.array_equal(oracle.quantize_fp8_e4m3(vals.astype(np.float32), np.float32(1)), finite)
    pos = np.unique(vals[vals > 0])
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(50000) * 100, mids, -mids, [464.0, -464.0]]).astype(np.float32)
    x = x[np.abs(x) <= 464]
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.quantize_fp8_e4m3(x, np.float32(1)), lib)


def test_fp8_error_bound_and_saturation():
    """E4M3 keeps 3 mantissa bits: for |x/s| in the normal range [2^-6, 448] the decoded
    code is within 2^-4 of x/s relatively (half a step of 2^-3), in the subnormal range
    within 2^-10 absolutely (half the 2^-9 spacing); beyond 448 the code saturates."""
    rng = np.random.default_rng(8)
    s = rng.uniform(0.005, 0.02, size=20000).astype(np.float32)
    mag = np.exp2(rng.uniform(-12, np.log2(448.0), size=20000))
    q = mag * rng.choice([-1.0, 1.0], size=20000)
    x = (q * s).astype(np.float32)
    code = oracle.quantize_fp8_e4m3(x, s)
    got = oracle.decode_fp8_e4m3(code)
    t = x.astype(np.float64) / s.astype(np.float64)
    normal = np.abs(t) >= 2.0 ** -6
    assert np.all(np.abs(got - t)[normal] <= 2.0 ** -4 * np.abs(t)[normal] * (1 + 1e-6))
    assert np.all(np.abs(got - t)[~normal] <= 2.0 ** -10 * (1 + 1e-6))
    big = np.array([449.0, 1e6, -500.0, np.inf, -np.inf], dtype=np.float32)
    assert np.array_equal(oracle.decode_fp8_e4m3(oracle.quantize_fp8_e4m3(big, np.float32(1))),
                          [448.0, 448.0, -448.0, 448.0, -448.0])


def test_append_fp8_quantises_with_channel_scales():
    case = synth.paged_case(15, kv_lens=[9, 33], q_lens=[3, 8], H_q=8, H_kv=2, D=128,
                            block_size=16, dtype=synth.F16, cache_dtype=synth.FP8, poison=True)
    kc, vc, st = oracle.kv_cache_append(case.k_new, case.v_new, case.cu_seqlens_q, case.seqlens_k,
                                        case.k_cache, case.v_cache, case.block_table, case.block_size,
                                        case.key_scale, case.value_scale)
    assert st == 0
    b, j, r = 1, 32, int(case.cu_seqlens_q[2]) - 1
    got = oracle.decode_fp8_e4m3(_walk(kc, case.block_table, case.block_size, b, j))
    x = case.k_new[r].astype(np.float64) / case.key_scale.astype(np.float64)
    inside = np.abs(x) <= 448
    # relative error of round-to-nearest with 3 mantissa bits: at most 2^-4 (normals)
    err = np.abs(got - x)
    assert np.all(err[inside] <= np.maximum(np.abs(x[inside]) * 2.0 ** -4, 2.0 ** -10))
    assert np.all(np.abs(got[~inside]) == 448)
