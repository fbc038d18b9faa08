"""The C ABI library on the host (no GPU needed): it loads, exports every function the
header declares, sizes workspaces, and rejects bad arguments before touching a device.
Only calls that fail host validation are made here, so nothing is ever launched."""
import ctypes
import os
import re

import pytest

from selected_token_sparse_amd import _lib

HEADER = _lib.HEADER_PATH


def _declared():
    text = open(HEADER).read()
    return re.findall(r"SPATTN_API\s+\w+\s+(\w+)\s*\(", text)


def test_header_declares_the_abi():
    names = _declared()
    assert set(names) == {"prepare_seqlens", "kv_cache_append", "prepare_and_append",
                          "qkv_prologue", "topk_select",
                          "paged_attention_fwd", "paged_decode_step",
                          "paged_decode_step_noalloc", "sparse_attention_fwd",
                          "attention_workspace_bytes"}


def test_library_exports_every_declared_symbol():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libspattn.so not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_lib._SIGNATURES) == set(_declared())


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libspattn.so not built")
    return _lib.load()


def test_workspace_bytes(lib):
    f = lib.attention_workspace_bytes
    bad = (1 << 64) - 1
    # paged decode, 32 rows, key bound 8192, H 64/8, D 64: split partials needed
    n = f(0, 1, 32, 32, 1, 8192, 0, -1, 64, 8, 64)
    assert 0 < n < 64 << 20
    # prefill regime (max_seqlen_q > 8, fp16) needs none
    assert f(0, 1, 4, 5120, 2048, 2048, 0, 128, 64, 8, 64) == 0
    # a single short split needs none
    assert f(0, 1, 2, 2, 1, 100, 0, -1, 4, 2, 64) == 0
    # invalid arguments
    assert f(0, 1, 2, 2, 1, 100, 0, -1, 6, 4, 64) == bad      # H_q % H_kv
    assert f(0, 1, 2, 2, 1, 100, 0, -1, 4, 2, 96) == bad      # head_dim
    assert f(2, 1, 2, 2, 1, 0, 64, 0, 4, 2, 64) == bad        # local+aux without a window
    assert f(7, 1, 2, 2, 1, 100, 0, -1, 4, 2, 64) == bad      # kind
    # more keys never need less workspace
    assert f(1, 1, 16, 128, 8, 0, 4096, 0, 48, 4, 128) >= f(1, 1, 16, 128, 8, 0, 2048, 0, 48, 4, 128)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _paged(lib, **kw):
    a = dict(q=FAKE, dtype=1, k=FAKE, v=FAKE, cdt=1, bt=FAKE, mbps=4, bs=16, nb=8, ks=None, vs=None,
             cu=FAKE, sk=FAKE, B=2, T=2, mq=1, mk=64, Hq=4, Hkv=2, D=64, scale=0.0, causal=1,
             win=-1, sinks=None, out=FAKE, ws=None, wsb=0, st=None, stream=None)
    a.update(kw)
    return lib.paged_attention_fwd(*a.values())


@pytest.mark.parametrize("kw,rc", [
    (dict(causal=0), -4), (dict(D=96), -4), (dict(Hq=6, Hkv=4), -4), (dict(dtype=3), -3),
    (dict(cdt=0), -3), (dict(cdt=3), -1), (dict(q=None), -1), (dict(out=None), -1),
    (dict(k=None), -1), (dict(B=-1), -2), (dict(bs=0), -2), (dict(mbps=0), -2),
    (dict(bt=None, nb=1), -2), (dict(nb=1 << 28, bs=1 << 4), -2),
    (dict(B=0), -2), (dict(mk=-5), -2),
    (dict(T=32, mq=1, mk=8192, Hq=64, Hkv=8, ws=None), -5),
])
def test_paged_argument_errors(lib, kw, rc):
    assert _paged(lib, **kw) == rc


def test_paged_empty_batch_is_a_no_op(lib):
    assert _paged(lib, T=0) == 0


def _sparse(lib, **kw):
    a = dict(q=FAKE, dtype=1, mode=0, k=FAKE, v=FAKE, cdt=1, bt=None, mbps=0, bs=100, nb=2, ks=None,
             vs=None, cu=FAKE, sk=FAKE, B=2, T=2, mq=1, sel=FAKE, cnt=FAKE, msel=16, win=-1,
             ak=None, av=None, adt=1, alen=0, astride=0, Hq=4, Hkv=2, D=64, scale=0.0, sinks=None,
             out=FAKE, ws=None, wsb=0, st=None, stream=None)
    a.update(kw)
    return lib.sparse_attention_fwd(*a.values())


@pytest.mark.parametrize("kw,rc", [
    (dict(mode=2), -4), (dict(win=8), -4), (dict(mode=1, win=-1), -4), (dict(sel=None), -1),
    (dict(mode=1, win=8), -1), (dict(mode=1, win=8, ak=FAKE, av=FAKE, adt=2), -3),
    (dict(mode=1, win=8, ak=FAKE, av=FAKE, alen=10, astride=100), -2), (dict(D=32), -4),
    (dict(msel=-1), -2),
])
def test_sparse_argument_errors(lib, kw, rc):
    assert _sparse(lib, **kw) == rc


def test_append_argument_errors(lib):
    f = lib.kv_cache_append
    base = [FAKE, FAKE, 1, FAKE, FAKE, 2, 4, FAKE, FAKE, 1, FAKE, 4, 16, 8, None, None, 2, 64, None, None, None]
    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)
    assert call(2, 3) == -3          # int8 new rows
    assert call(9, 2) == -3          # cache dtype differs from the rows'
    assert call(9, 3) == -1          # int8 cache without scales
    assert call(0, None) == -1
    assert call(17, 60) == -2        # head_dim not a multiple of 8
    assert call(12, 0) == -2         # block size
    assert call(6, 0) == 0           # nothing to append


def test_prologue_argument_errors(lib):
    """Argument errors return before anything is enqueued (fake device pointers are never
    touched)."""
    f = lib.qkv_prologue
    # qkv, q, k, v, dtype, cu, sk, B, T, H_q, H_kv, D, qk_norm, qw, kw, eps, rd, inter, cos,
    # sin, max_pos, pos_ids, offs, q_out, kc, vc, cache_dtype, bt, mbps, bs, nb, ks, vs,
    # committed, status, stream
    base = [FAKE, None, None, None, 1, FAKE, FAKE, 2, 4, 8, 2, 64, 1, None, None, 1e-6, 32, 0,
            FAKE, FAKE, 128, None, None, FAKE, FAKE, FAKE, 1, FAKE, 4, 16, 8, None, None,
            None, None, None]
    def call(**kv):
        a = list(base)
        for i, v in kv.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a4=3) == -3                    # int8 activations
    assert call(a26=2) == -3                   # cache dtype differs from the rows'
    assert call(a26=4) == -1                   # FP8 cache without scales
    assert call(a0=None) == -1                 # neither packed rows nor q, k, v
    assert call(a0=None, a1=FAKE, a2=FAKE) == -1
    assert call(a11=60) == -2                  # head_dim not a multiple of 8
    assert call(a11=264) == -2                 # head_dim above 256
    assert call(a16=33) == -2                  # odd rotary_dim
    assert call(a16=72) == -2                  # rotary_dim above head_dim
    assert call(a18=None) == -1                # rotation without tables
    assert call(a20=0) == -2                   # empty tables
    assert call(a15=-1.0) == -2                # negative eps
    assert call(a15=float("inf")) == -2
    assert call(a23=None) == -1                # no q_out
    assert call(a29=0) == -2                   # block size
    assert call(a8=0) == 0                     # no rows: nothing to do
    assert call(a7=0) == -2                    # rows but no request


def test_prepare_and_append_argument_errors(lib):
    f = lib.prepare_and_append
    # cu, past, B, T, sq, sk, treq, tpos, k_new, v_new, new_dt, kc, vc, cache_dt, bt, mbps,
    # bs, nb, ks, vs, H_kv, D, committed, status, stream
    base = [FAKE, FAKE, 2, 4, FAKE, FAKE, None, None, FAKE, FAKE, 1, FAKE, FAKE, 1, FAKE, 4, 16,
            8, None, None, 2, 64, None, None, None]
    def call(**kv):
        a = list(base)
        for i, v in kv.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a2=8193) == -2
    assert call(a1=None) == -1
    assert call(a5=None) == -1
    assert call(a10=3) == -3           # int8 rows
    assert call(a13=3) == -1           # int8 cache without scales
    assert call(a21=60) == -2
    assert call(a16=0) == -2           # block size
    assert call(a2=0) == -2            # rows but no request
    assert call(a8=None) == -1


def test_decode_step_argument_errors(lib):
    f = lib.paged_decode_step
    # cu, past, B, T, sq, sk, q, k_new, v_new, dtype, kc, vc, cache_dt, bt, mbps, bs, nb, ks,
    # vs, max_q, max_k, H_q, H_kv, D, scale, win, sinks, out, ws, ws_bytes, committed, status,
    # stream
    base = [FAKE, FAKE, 2, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 1, FAKE, 4, 16, 8,
            None, None, 1, 64, 4, 2, 64, 0.0, -1, None, FAKE, None, 0, None, None, None]
    def call(**kv):
        a = list(base)
        for i, v in kv.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a9=0) == -4            # float32 activations: the separate calls
    assert call(a9=3) == -3            # not an activation dtype
    assert call(a2=256) == -4          # more requests than one boundary per thread
    assert call(a19=64) == -4          # a query block for the prefill kernel
    assert call(a0=None) == -1
    assert call(a1=None) == -1
    assert call(a4=None) == -1
    assert call(a7=None) == -1
    assert call(a27=None) == -1
    assert call(a12=2) == -3           # cache dtype differs from the activations
    assert call(a12=3) == -1           # INT8 cache without scales
    assert call(a23=96) == -4          # head dim
    assert call(a21=3) == -4           # H_q not a multiple of H_kv
    assert call(a2=0) == -2            # rows but no request
    assert call(a15=0) == -2           # block size
    for i in (6, 7, 8, 27):            # q, k_new, v_new, out off a 16-byte boundary
        assert call(**{f"a{i}": MIS}) == -2
    assert call(a10=MIS) == -2


def test_noalloc_decode_step_argument_errors(lib):
    """The allocation-free step validates like paged_decode_step, before it looks up its
    static scratch (so no HIP call is made here), and rejects plans whose split-K partials
    exceed the 16 MiB array."""
    f = lib.paged_decode_step_noalloc
    # paged_decode_step's arguments without workspace / workspace_bytes
    base = [FAKE, FAKE, 2, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 1, FAKE, 4, 16, 8,
            None, None, 1, 64, 4, 2, 64, 0.0, -1, None, FAKE, None, None, None]
    def call(**kv):
        a = list(base)
        for i, v in kv.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a9=0) == -4            # float32 activations
    assert call(a9=3) == -3
    assert call(a2=256) == -4
    assert call(a19=64) == -4          # a query block for the prefill kernel
    assert call(a0=None) == -1
    assert call(a27=None) == -1
    assert call(a12=2) == -3
    assert call(a23=96) == -4
    assert call(a2=0) == -2
    assert call(a6=MIS) == -2
    # 255 requests of 8 rows of H 64/8 with a 65536-key bound: about 1 GB of partials
    ws = lib.attention_workspace_bytes(0, 1, 255, 2040, 8, 65536, 0, -1, 64, 8, 64)
    assert ws > 16 << 20
    assert call(a2=255, a3=2040, a19=8, a20=65536, a21=64, a22=8) == -5


def test_topk_argument_errors(lib):
    f = lib.topk_select
    # scores, L, cu, sk, B, T, H_kv, k, tail, sel_idx, capacity, sel_count, status, stream
    base = [FAKE, 4096, FAKE, FAKE, 2, 8, 4, 512, 16, FAKE, 512, FAKE, None, None]
    def call(**kv):
        a = list(base)
        for i, v in kv.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a1=0) == -2            # no score columns
    assert call(a1=65537) == -4        # longer than one workgroup's registers hold
    assert call(a7=-1) == -2
    assert call(a8=-1) == -2
    assert call(a10=511) == -2         # capacity below k
    assert call(a0=None) == -1
    assert call(a11=None) == -1
    assert call(a9=None) == -1
    assert call(a5=0) == 0             # no rows
    assert call(a4=0) == -2            # rows but no request


def test_prepare_argument_errors(lib):
    f = lib.prepare_seqlens
    assert f(None, FAKE, 2, 4, FAKE, FAKE, None, None, None, None) == -1
    assert f(FAKE, FAKE, -1, 4, FAKE, FAKE, None, None, None, None) == -2
    assert f(FAKE, FAKE, 9000, 4, FAKE, FAKE, None, None, None, None) == -2


MIS = FAKE + 8  # an 8-byte offset: not a 16-byte boundary


@pytest.mark.parametrize("kw", [dict(q=MIS), dict(out=MIS), dict(k=MIS), dict(v=MIS)])
def test_paged_misaligned_pointers(lib, kw):
    assert _paged(lib, **kw) == -2


@pytest.mark.parametrize("kw", [dict(q=MIS), dict(out=MIS), dict(k=MIS),
                                dict(mode=1, win=8, ak=MIS, av=FAKE, alen=10, astride=0),
                                dict(mode=1, win=8, ak=FAKE, av=MIS, alen=10, astride=0)])
def test_sparse_misaligned_pointers(lib, kw):
    assert _sparse(lib, **kw) == -2


def test_append_and_prologue_misaligned_pointers(lib):
    base = [FAKE, FAKE, 1, FAKE, FAKE, 2, 4, FAKE, FAKE, 1, FAKE, 4, 16, 8, None, None, 2, 64, None, None, None]
    for i in (0, 1, 7, 8):               # k_new, v_new, k_cache, v_cache
        a = list(base)
        a[i] = MIS
        assert lib.kv_cache_append(*a) == -2, i
    pa = [FAKE, FAKE, 2, 4, FAKE, FAKE, None, None, FAKE, FAKE, 1, FAKE, FAKE, 1, FAKE, 4, 16,
          8, None, None, 2, 64, None, None, None]
    for i in (8, 9, 11):                 # k_new, v_new, k_cache
        a = list(pa)
        a[i] = MIS
        assert lib.prepare_and_append(*a) == -2, i
    pro = [FAKE, None, None, None, 1, FAKE, FAKE, 2, 4, 8, 2, 64, 1, None, None, 1e-6, 32, 0,
           FAKE, FAKE, 128, None, None, FAKE, FAKE, FAKE, 1, FAKE, 4, 16, 8, None, None,
           None, None, None]
    for i in (0, 23, 24):                # qkv, q_out, k_cache
        a = list(pro)
        a[i] = MIS
        assert lib.qkv_prologue(*a) == -2, i
