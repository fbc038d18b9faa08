"""Pins of the oracle's attention definition (CPU only).

Against things other than the oracle itself:

* torch.nn.functional.scaled_dot_product_attention (a library routine, float64 on the
  CPU) on dense per-request K/V that this test lays out and pages itself, with the
  bottom-right causal mask, the window mask, GQA by repeating KV heads, and the sink as
  one extra key column whose score is the sink logit and whose value row is zero;
* closed forms: one visible key gives ``v / (1 + e^(sink - s))``; zero keys with unit
  values and a zero sink give ``n / (n + 1)``, which exposes the visible-key count
  ``min(p + 1, W)`` of the window-start formula (PagedAttention metadata page, Q3);
* invariances: block-table permutation, sink = -inf equals no sink, a window at least as
  long as the sequence equals no window, replicating KV heads equals GQA, selecting every
  position equals the paged causal result, INT8 equals its dequantised float cache.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _sdpa(q, K, V, scale, sinks, mask_bool):
    """q [H, n_q, D], K/V [H, n_k, D] float64; mask_bool [n_q, n_k] (True = visible)."""
    H, nq, D = q.shape
    bias = torch.zeros(H, nq, K.shape[1] + 1, dtype=torch.float64)
    bias[:, :, :-1] = torch.where(torch.from_numpy(mask_bool), 0.0, -math.inf)
    sig = np.full(H, -np.inf) if sinks is None else sinks.astype(np.float64)
    bias[:, :, -1] = torch.from_numpy(sig)[:, None]
    Kx = torch.cat([torch.from_numpy(K), torch.zeros(H, 1, D, dtype=torch.float64)], 1)
    Vx = torch.cat([torch.from_numpy(V), torch.zeros(H, 1, D, dtype=torch.float64)], 1)
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), Kx, Vx, attn_mask=bias, scale=scale)
    return out.numpy()


def _dense_request(rng, kv_len, H_kv, D):
    return (rng.standard_normal((kv_len, H_kv, D)), rng.standard_normal((kv_len, H_kv, D)))


def _page(rng, dense_k, dense_v, bs, extra_blocks=3):
    """Lay dense per-request K/V ([L, H_kv, D]) into a shuffled paged pool with the
    library's block layout [nb, H_kv, bs, D] (this test's own layout code)."""
    B = len(dense_k)
    need = [(len(k) + bs - 1) // bs for k in dense_k]
    nb = sum(need) + extra_blocks
    H_kv, D = dense_k[0].shape[1:]
    kc = np.full((nb, H_kv, bs, D), np.nan)
    vc = np.full((nb, H_kv, bs, D), np.nan)
    perm = rng.permutation(nb)
    bt = np.full((B, max(need) + 1), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        for lb in range(need[b]):
            blk = perm[o]
            o += 1
            bt[b, lb] = blk
            seg = slice(lb * bs, min((lb + 1) * bs, len(dense_k[b])))
            n = seg.stop - seg.start
            kc[blk, :, :n] = dense_k[b][seg].transpose(1, 0, 2)
            vc[blk, :, :n] = dense_v[b][seg].transpose(1, 0, 2)
    return kc, vc, bt


@pytest.mark.parametrize("seed,W,with_sink,g", [
    (0, -1, False, 1), (1, -1, True, 4), (2, 5, True, 2), (3, 1, False, 3), (4, 64, True, 8),
    (5, 7, False, 4),
])
def test_paged_matches_library_sdpa(seed, W, with_sink, g):
    rng = np.random.default_rng(seed)
    H_kv, D, bs = 2, 16, 4
    H_q = H_kv * g
    kv_lens = [1, 13, 7, 30]
    q_lens = [1, 5, 7, 3]
    dk, dv = zip(*[_dense_request(rng, L, H_kv, D) for L in kv_lens])
    kc, vc, bt = _page(rng, dk, dv, bs)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(cu[-1])
    q = rng.standard_normal((T, H_q, D))
    sinks = rng.standard_normal(H_q) if with_sink else None
    scale = 0.3
    out, st = oracle.paged_attention(q, kc, vc, cu, np.array(kv_lens) - 1, H_kv=H_kv,
                                     block_table=bt, block_size=bs, scale=scale,
                                     local_window=W, sinks=sinks)
    assert st == 0
    for b in range(4):
        L, n = kv_lens[b], q_lens[b]
        pos = np.arange(L - n, L)[:, None]          # bottom-right aligned query positions
        j = np.arange(L)[None, :]
        mask = j <= pos
        if W > 0:
            mask &= j >= pos - W + 1
        qb = q[cu[b]:cu[b + 1]].transpose(1, 0, 2)  # [H_q, n, D]
        Kb = np.repeat(dk[b].transpose(1, 0, 2), g, axis=0)
        Vb = np.repeat(dv[b].transpose(1, 0, 2), g, axis=0)
        ref = _sdpa(qb, Kb, Vb, scale, sinks, mask).transpose(1, 0, 2)
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref, rtol=1e-12, atol=1e-12)


def test_single_visible_key_closed_form():
    rng = np.random.default_rng(7)
    D, L = 32, 9
    k = rng.standard_normal((1, 1, L, D))     # contiguous cache [B, H_kv, cap, D]
    v = rng.standard_normal((1, 1, L, D))
    q = rng.standard_normal((1, 2, D))
    sinks = np.array([0.7, -1.3])
    cu = np.array([0, 1], dtype=np.int32)
    out, _ = oracle.paged_attention(q, k, v, cu, np.array([L - 1]), H_kv=1, scale=0.25,
                                    local_window=1, sinks=sinks)
    kk, vv = k[0, 0, L - 1], v[0, 0, L - 1]
    for h in range(2):
        s = 0.25 * float(q[0, h] @ kk)
        np.testing.assert_allclose(out[0, h], vv / (1.0 + math.exp(sinks[h] - s)), rtol=1e-14)


@pytest.mark.parametrize("W", [1, 3, 16, 100, -1])
def test_visible_key_count_matches_window_formula(W):
    # K = 0 makes every score 0; V = 1 and sink 0 then give o = n / (n + 1)
    L, n_q = 40, 12
    k = np.zeros((1, 1, L, 8))
    v = np.ones((1, 1, L, 8))
    q = np.ones((n_q, 1, 8))
    cu = np.array([0, n_q], dtype=np.int32)
    out, _ = oracle.paged_attention(q, k, v, cu, np.array([L - 1]), H_kv=1, scale=1.0,
                                    local_window=W, sinks=np.zeros(1))
    for i in range(n_q):
        p = L - n_q + i
        n = min(p + 1, W) if W > 0 else p + 1
        np.testing.assert_allclose(out[i, 0], n / (n + 1.0), rtol=1e-14)


def _small_case(seed=21, **kw):
    args = dict(kv_lens=[37, 100, 1, 64], q_lens=[1, 4, 1, 8], H_q=8, H_kv=2, D=64,
                block_size=16, dtype=synth.F32, num_blocks=20, sinks=True, scale=0.125)
    args.update(kw)
    return synth.paged_case(seed, **args)


def _run_paged(case, **over):
    kw = dict(H_kv=case.H_kv, block_table=case.block_table, block_size=case.block_size,
              key_scale=case.key_scale, value_scale=case.value_scale, scale=case.scale,
              local_window=case.local_window, sinks=case.sinks)
    kw.update(over)
    return oracle.paged_attention(case.q, case.k_cache, case.v_cache, case.cu_seqlens_q,
                                  case.seqlens_k, **kw)


def test_block_table_permutation_invariance():
    case = _small_case()
    out1, _ = _run_paged(case)
    rng = np.random.default_rng(5)
    perm = rng.permutation(case.num_blocks)        # physical block i moves to perm[i]
    kc = np.empty_like(case.k_cache)
    vc = np.empty_like(case.v_cache)
    kc[perm] = case.k_cache
    vc[perm] = case.v_cache
    bt = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    out2, _ = oracle.paged_attention(case.q, kc, vc, case.cu_seqlens_q, case.seqlens_k,
                                     H_kv=case.H_kv, block_table=bt, block_size=case.block_size,
                                     scale=case.scale, sinks=case.sinks)
    assert np.array_equal(out1, out2)


def test_sink_neg_inf_equals_no_sink():
    case = _small_case()
    a, _ = _run_paged(case, sinks=np.full(case.H_q, -np.inf))
    b, _ = _run_paged(case, sinks=None)
    assert np.array_equal(a, b)


def test_long_window_equals_no_window():
    case = _small_case()
    a, _ = _run_paged(case, local_window=100)
    b, _ = _run_paged(case, local_window=-1)
    assert np.array_equal(a, b)


def test_replicated_kv_heads_equal_gqa():
    case = _small_case()
    g = case.H_q // case.H_kv
    a, _ = _run_paged(case)
    kc = np.repeat(case.k_cache, g, axis=1)
    vc = np.repeat(case.v_cache, g, axis=1)
    b, _ = oracle.paged_attention(case.q, kc, vc, case.cu_seqlens_q, case.seqlens_k, H_kv=case.H_q,
                                  block_table=case.block_table, block_size=case.block_size,
                                  scale=case.scale, sinks=case.sinks)
    # one head at a time instead of a group: only the matmul's summation order differs
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_selecting_every_position_equals_paged_causal():
    case = _small_case(seed=22)
    a, _ = _run_paged(case)
    T, H_kv = case.T, case.H_kv
    L = int(case.seqlens_k.max()) + 1
    sel = np.full((T, H_kv, L), -1, dtype=np.int32)
    req = np.searchsorted(case.cu_seqlens_q, np.arange(T), side="right") - 1
    for r in range(T):
        kv = int(case.seqlens_k[req[r]]) + 1
        sel[r, :, :kv] = np.arange(kv)
    b, st = oracle.sparse_attention(case.q, 0, case.k_cache, case.v_cache, case.cu_seqlens_q,
                                    case.seqlens_k, sel, None, L, H_kv=H_kv,
                                    block_table=case.block_table, block_size=case.block_size,
                                    scale=case.scale, sinks=case.sinks)
    assert st == 0
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("cache_dtype", [synth.I8, synth.FP8])
def test_quantised_equals_dequantised_float_cache(cache_dtype):
    case = _small_case(seed=23, dtype=synth.F16, cache_dtype=cache_dtype)
    a, _ = _run_paged(case)
    def values(codes):
        return (codes.astype(np.float64) if cache_dtype == synth.I8
                else oracle.decode_fp8_e4m3(codes))
    kf = values(case.k_cache) * case.key_scale.astype(np.float64)[None, :, None, :]
    vf = values(case.v_cache) * case.value_scale.astype(np.float64)[None, :, None, :]
    b, _ = oracle.paged_attention(case.q, kf, vf, case.cu_seqlens_q, case.seqlens_k, H_kv=case.H_kv,
                                  block_table=case.block_table, block_size=case.block_size,
                                  scale=case.scale, sinks=case.sinks)
    assert np.array_equal(a, b)


def test_scale_folding_identity():
    # folding key_scale into q and value_scale after the weighted sum is exact algebra
    rng = np.random.default_rng(8)
    q = rng.standard_normal((3, 16))
    codes_k = rng.integers(-127, 128, size=(10, 16)).astype(np.float64)
    codes_v = rng.integers(-127, 128, size=(10, 16)).astype(np.float64)
    ks = rng.uniform(0.005, 0.02, 16)
    vs = rng.uniform(0.005, 0.02, 16)
    a = oracle.attend(q, codes_k * ks, codes_v * vs, 0.2, np.array([0.1, -0.5, 2.0]))
    b = oracle.attend(q * ks, codes_k, codes_v, 0.2, np.array([0.1, -0.5, 2.0])) * vs
    np.testing.assert_allclose(a, b, rtol=1e-12)


def test_empty_sets_give_zero_rows():
    case = synth.sparse_selected_case(31, B=2, S_q=3, H_q=4, H_kv=2, D=64, capacity=50,
                                      max_selected=16, dtype=synth.F32, sinks=True,
                                      counts=np.zeros((6, 2), dtype=np.int64))
    out, st = oracle.sparse_attention(case.q, 0, case.k_cache, case.v_cache, case.cu_seqlens_q,
                                      case.seqlens_k, case.sel_idx, case.sel_count, 16,
                                      H_kv=2, scale=case.scale, sinks=case.sinks)
    assert st == 0 and np.all(out == 0)
    # all -1 with no count: zeros as well
    out, st = oracle.sparse_attention(case.q, 0, case.k_cache, case.v_cache, case.cu_seqlens_q,
                                      case.seqlens_k, np.full_like(case.sel_idx, -1), None, 16,
                                      H_kv=2, scale=case.scale, sinks=case.sinks)
    assert st == 0 and np.all(out == 0)
    # rows whose position precedes every key (fewer keys than rows) are zero and flagged
    c = _small_case(seed=24)
    sk = c.seqlens_k.copy()
    sk[3] = 2                      # 3 keys for 8 rows
    out, st = oracle.paged_attention(c.q, c.k_cache, c.v_cache, c.cu_seqlens_q, sk, H_kv=c.H_kv,
                                     block_table=c.block_table, block_size=c.block_size,
                                     scale=c.scale, sinks=c.sinks)
    assert st & oracle.STATUS_SHORT_KV
    r0 = int(c.cu_seqlens_q[3])
    assert np.all(out[r0:r0 + 5] == 0) and np.all(out[r0 + 5:r0 + 8] != 0)


def test_count_bounds_the_selection_and_guards():
    case = synth.sparse_selected_case(32, B=2, S_q=4, H_q=6, H_kv=2, D=64, capacity=300,
                                      max_selected=64, dtype=synth.F32, sinks=True, oor_frac=0.1)
    args = (case.q, 0, case.k_cache, case.v_cache, case.cu_seqlens_q, case.seqlens_k)
    kw = dict(H_kv=2, scale=case.scale, sinks=case.sinks)
    a, st = oracle.sparse_attention(*args, case.sel_idx, case.sel_count, 64, **kw)
    assert st & oracle.STATUS_BAD_INDEX
    # entries past the count do not matter
    sel = case.sel_idx.copy()
    for r in range(case.T):
        for c in range(2):
            sel[r, c, case.sel_count[r, c]:] = 5
    b, _ = oracle.sparse_attention(*args, sel, case.sel_count, 64, **kw)
    assert np.array_equal(a, b)
    # an out-of-range entry acts as padding
    sel = case.sel_idx.copy()
    bad = (sel < -1) | (sel >= 300)
    sel[bad] = -1
    c_, st2 = oracle.sparse_attention(*args, sel, case.sel_count, 64, **kw)
    assert np.array_equal(a, c_) and not (st2 & oracle.STATUS_BAD_INDEX)
    # counts outside [0, max_selected] are clamped and flagged
    cnt = case.sel_count.copy()
    cnt[0, 0] = 1000
    cnt[1, 1] = -3
    d, st3 = oracle.sparse_attention(*args, case.sel_idx, cnt, 64, **kw)
    cnt2 = cnt.copy()
    cnt2[0, 0] = 64
    cnt2[1, 1] = 0
    e, _ = oracle.sparse_attention(*args, case.sel_idx, cnt2, 64, **kw)
    assert st3 & oracle.STATUS_BAD_COUNT and np.array_equal(d, e)


def test_local_plus_aux_matches_library_sdpa():
    case = synth.sparse_local_aux_case(41, B=2, S_q=3, H_q=6, H_kv=2, D=32, capacity=40,
                                       kv_lens=[40, 25], local_window=6, aux_len=50,
                                       n_selected=9, max_selected=12, dtype=synth.F16,
                                       cache_dtype=synth.I8, sinks=True, scale=0.2, oor_frac=0.0)
    out, st = oracle.sparse_attention(case.q, 1, case.k_cache, case.v_cache, case.cu_seqlens_q,
                                      case.seqlens_k, case.sel_idx, case.sel_count, case.max_selected,
                                      H_kv=2, key_scale=case.key_scale, value_scale=case.value_scale,
                                      local_window=6, aux_k=case.aux_k, aux_v=case.aux_v,
                                      aux_len=case.aux_len, aux_batch_stride=case.aux_batch_stride,
                                      scale=case.scale, sinks=case.sinks)
    assert st == 0
    g = 3
    for r in range(case.T):
        b, i = r // 3, r % 3
        L = int(case.seqlens_k[b]) + 1
        p = L - 3 + i
        for c in range(2):
            local = list(range(max(0, p - 5), p + 1))
            Km = case.k_cache[b, c, local].astype(np.float64) * case.key_scale[c]
            Vm = case.v_cache[b, c, local].astype(np.float64) * case.value_scale[c]
            idx = case.sel_idx[r, c, :case.sel_count[r, c]]
            Ka = case.aux_k[b, idx, c].astype(np.float64)
            Va = case.aux_v[b, idx, c].astype(np.float64)
            K = np.concatenate([Km, Ka])[None].repeat(g, 0)
            V = np.concatenate([Vm, Va])[None].repeat(g, 0)
            qh = case.q[r, c * g:(c + 1) * g].astype(np.float64)[:, None, :]
            ref = _sdpa(qh, K, V, 0.2, case.sinks[c * g:(c + 1) * g],
                        np.ones((1, K.shape[1]), dtype=bool))[:, 0]
            np.testing.assert_allclose(out[r, c * g:(c + 1) * g], ref, rtol=1e-12, atol=1e-13)


def test_rows_subset_matches_full():
    case = _small_case(seed=25)
    full, _ = _run_paged(case)
    part, _ = _run_paged(case, rows=[2, 5, 9])
    assert np.array_equal(part, full[[2, 5, 9]])


def test_host_bounds_zero_rows():
    case = _small_case(seed=26)
    out, st = _run_paged(case, max_seqlen_q=4, max_seqlen_k=100)
    r0 = int(case.cu_seqlens_q[3])
    assert st & oracle.STATUS_Q_BOUND and np.all(out[r0:] == 0)
    out, st = _run_paged(case, max_seqlen_q=8, max_seqlen_k=64)
    r1, r2 = int(case.cu_seqlens_q[1]), int(case.cu_seqlens_q[2])
    assert st & oracle.STATUS_K_BOUND and np.all(out[r1:r2] == 0) and np.all(out[:r1] != 0)


def test_pool_rows_equal_the_single_call():
    """oracle.pool deals rows out to worker processes and puts them back: the result must be
    the single call's, bit for bit, status included."""
    from oracle import pool
    case = synth.paged_case(71, kv_lens=[300, 40, 129, 1], q_lens=[60, 40, 1, 1], H_q=8, H_kv=2,
                            D=64, dtype=synth.F16, sinks=True, local_window=50)
    args = (case.q, case.k_cache, case.v_cache, case.cu_seqlens_q, case.seqlens_k)
    kw = dict(H_kv=2, block_table=case.block_table, block_size=case.block_size,
              max_seqlen_q=case.max_seqlen_q, max_seqlen_k=case.max_seqlen_k, scale=case.scale,
              local_window=case.local_window, sinks=case.sinks)
    want, wst = oracle.paged_attention(*args, **kw)
    got, gst = pool.map_rows("paged_attention", args, kw, range(case.T), workers=3, chunk=7)
    assert np.array_equal(got, want) and gst == wst
    sub = [0, 5, 59, 60, 100, 101]
    got, _ = pool.map_rows("paged_attention", args, kw, sub, workers=2, chunk=2)
    assert np.array_equal(got, want[sub])
