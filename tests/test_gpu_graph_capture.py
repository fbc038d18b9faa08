"""The calls need no host synchronisation: the metadata pass, the cache append, both
attention entry points, the QKV prologue and the TopK selection are recorded into HIP
graphs and replayed.  ("[WebGPU] Add
PagedAttention metadata and GPT-OSS support", Description: sequence lengths are produced
on the device so the step needs no readback and can be replayed.)

Each replay runs after unrelated eager work and a synchronisation, with the outputs
overwritten by NaN first; every replay must reproduce the eager outputs bit for bit (the
kernels are deterministic: no atomics decide any value), and the eager outputs are
checked against the oracle too."""
import numpy as np
import pytest
import torch

import oracle
import selected_token_sparse_amd as sta
import synth
from synth.device import TORCH_DTYPE, case_tensors, tensor

from harness import assert_close, oracle_paged_step, oracle_sparse, status_tensor

pytestmark = pytest.mark.gpu


def _ws(kind, case, max_sel=0):
    n = sta.attention_workspace_bytes(kind, case.dtype, case.B, case.T, case.max_seqlen_q,
                                      getattr(case, "max_seqlen_k", 0), max_sel,
                                      case.local_window, case.H_q, case.H_kv, case.D)
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")


def test_decode_prefill_sparse_step_in_one_graph():
    dec = synth.config_gqa_paged_decode(poison=True, B=8, max_len=3000, seed=91)
    pre = synth.paged_case(92, kv_lens=[130, 40], q_lens=[130, 40], H_q=16, H_kv=2, D=64,
                           dtype=synth.F16, sinks=True, local_window=64, poison=True)
    sel = synth.sparse_selected_case(93, B=3, S_q=2, H_q=24, H_kv=2, D=128, capacity=900,
                                     max_selected=256, dtype=synth.F16, sinks=True, oor_frac=0.02,
                                     poison=True)
    td, tp, ts = case_tensors(dec), case_tensors(pre), case_tensors(sel)
    sq = torch.empty(dec.B, dtype=torch.int32, device="cuda")
    sk = torch.empty(dec.B, dtype=torch.int32, device="cuda")
    st = status_tensor()
    ws_d = _ws(sta.KIND_PAGED, dec)
    ws_s = _ws(sta.KIND_SELECTED, sel, sel.max_selected)
    out_d = torch.empty((dec.T, dec.H_q, dec.D), dtype=TORCH_DTYPE[dec.dtype], device="cuda")
    out_p = torch.empty((pre.T, pre.H_q, pre.D), dtype=TORCH_DTYPE[pre.dtype], device="cuda")
    out_s = torch.empty((sel.T, sel.H_q, sel.D), dtype=TORCH_DTYPE[sel.dtype], device="cuda")

    # the prefill's prompt rows enter the cache once, before capture
    sta.kv_cache_append(tp["k_new"], tp["v_new"], tp["cu"], tp["seqlens_k"], tp["k_cache"],
                        tp["v_cache"], tp["block_table"])

    def step():
        sta.prepare_and_append(td["cu"], td["past"], dec.T, sq, sk, td["k_new"], td["v_new"],
                               td["k_cache"], td["v_cache"], td["block_table"], status=st)
        sta.paged_attention_fwd(td["q"], td["k_cache"], td["v_cache"], td["cu"], sk,
                                dec.max_seqlen_q, dec.max_seqlen_k, out_d,
                                block_table=td["block_table"], scale=dec.scale,
                                sinks=td["sinks"], workspace=ws_d, status=st)
        sta.paged_attention_fwd(tp["q"], tp["k_cache"], tp["v_cache"], tp["cu"], tp["seqlens_k"],
                                pre.max_seqlen_q, pre.max_seqlen_k, out_p,
                                block_table=tp["block_table"], scale=pre.scale,
                                local_window=pre.local_window, sinks=tp["sinks"], status=st)
        sta.sparse_attention_fwd(ts["q"], sel.mode, ts["k_cache"], ts["v_cache"], ts["cu"],
                                 ts["seqlens_k"], sel.max_seqlen_q, ts["sel_idx"], out_s,
                                 sel_count=ts["sel_count"], scale=sel.scale, sinks=ts["sinks"],
                                 workspace=ws_s, status=st)

    print("graph: eager step", flush=True)
    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in (out_d, out_p, out_s)]
    st_eager = int(st.item())
    ref_d, dst = oracle_paged_step(dec)
    assert_close(eager[0], ref_d, dec.dtype, "graph eager decode")
    ref_p, pst = oracle_paged_step(pre)       # the oracle appends the prompt rows itself
    assert_close(eager[1], ref_p, pre.dtype, "graph eager prefill")
    ref_s, sst = oracle_sparse(sel)
    assert_close(eager[2], ref_s, sel.dtype, "graph eager selected")
    assert st_eager == dst | pst | sst, (st_eager, dst, pst, sst)

    print("graph: capture", flush=True)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    noise = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        print(f"graph: replay {rep}", flush=True)
        for o in (out_d, out_p, out_s):
            o.fill_(float("nan"))
        (noise * 3.0).sum().item()  # unrelated eager work and a synchronisation
        g.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((out_d, out_p, out_s), eager, ("decode", "prefill", "selected")):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (rep, name)
    assert int(st.item()) == st_eager


def test_multi_layer_decode_step_in_one_graph():
    """One decode step of a 4-layer model as one HIP graph: the metadata pass once, then
    per layer the append into that layer's cache and the attention over it.  Every replay
    reproduces the eager outputs bit for bit, and each layer matches the oracle."""
    layers = 4
    base = synth.config_gqa_paged_decode(poison=True, B=6, max_len=2500, seed=95)
    cases = [synth.paged_case(500 + i, kv_lens=base.seqlens_k + 1, q_lens=np.diff(base.cu_seqlens_q),
                              H_q=base.H_q, H_kv=base.H_kv, D=base.D, dtype=base.dtype,
                              num_blocks=int(((base.seqlens_k + 16) // 16).sum()) + 64,
                              max_blocks_per_seq=base.max_blocks_per_seq,
                              sinks=True, scale=base.scale, poison=True,
                              max_seqlen_k=base.max_seqlen_k)
             for i in range(layers)]
    ts = [case_tensors(c) for c in cases]
    cu = ts[0]["cu"]
    past = ts[0]["past"]
    T, B = base.T, base.B
    sq = torch.empty(B, dtype=torch.int32, device="cuda")
    sk = torch.empty(B, dtype=torch.int32, device="cuda")
    st = status_tensor()
    ws = _ws(sta.KIND_PAGED, cases[0])
    outs = [torch.empty((T, base.H_q, base.D), dtype=TORCH_DTYPE[base.dtype], device="cuda")
            for _ in range(layers)]

    def step():
        sta.prepare_seqlens(cu, past, T, sq, sk, status=st)
        for t, o, c in zip(ts, outs, cases):
            sta.kv_cache_append(t["k_new"], t["v_new"], cu, sk, t["k_cache"], t["v_cache"],
                                t["block_table"], status=st)
            sta.paged_attention_fwd(t["q"], t["k_cache"], t["v_cache"], cu, sk, c.max_seqlen_q,
                                    c.max_seqlen_k, o, block_table=t["block_table"], scale=c.scale,
                                    sinks=t["sinks"], workspace=ws, status=st)

    print("multi-layer graph: eager", flush=True)
    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    assert int(st.item()) == 0
    for c, e in zip(cases, eager):
        ref, ost = oracle_paged_step(c)
        assert ost == 0
        assert_close(e, ref, c.dtype, "multi-layer eager")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"multi-layer graph: replay {rep}", flush=True)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), (rep, i)
    assert int(st.item()) == 0


def test_prologue_and_topk_in_one_graph():
    """The prologue (norm, rotation, cache append) and the TopK selection record into one
    graph too: every replay reproduces the eager query rows, cache and selection bit for
    bit, and the eager selection matches the oracle exactly."""
    pc = synth.prologue_case(97, kv_lens=[300, 41], q_lens=[4, 1], H_q=16, H_kv=2, D=128,
                             packed=True, rotary_dim=64, qk_norm=True, explicit_positions=True,
                             max_position=4096, offsets=True)
    tk = synth.topk_case(98, kv_lens=[5000, 3000], q_lens=[4, 1], H_kv=2, L=5000, k=300,
                         tail=16, capacity=320, ties=0.2, specials=0.01)
    dt = pc.dtype
    t = dict(qkv=tensor(pc.qkv, dt), cu=tensor(pc.cu_seqlens_q), sk=tensor(pc.seqlens_k),
             kc=tensor(pc.k_cache, pc.cache_dtype), vc=tensor(pc.v_cache, pc.cache_dtype),
             bt=tensor(pc.block_table), qw=tensor(pc.q_norm_weight), kw=tensor(pc.k_norm_weight),
             cos=tensor(pc.cos_table), sin=tensor(pc.sin_table), pos=tensor(pc.position_ids),
             offs=tensor(pc.rotary_offsets))
    scores, tcu, tsk = tensor(tk.scores), tensor(tk.cu_seqlens_q), tensor(tk.seqlens_k)
    q_out = torch.empty((pc.T, pc.H_q, pc.D), dtype=TORCH_DTYPE[dt], device="cuda")
    sel = torch.empty((tk.T, tk.H_kv, tk.capacity), dtype=torch.int32, device="cuda")
    cnt = torch.empty((tk.T, tk.H_kv), dtype=torch.int32, device="cuda")
    st = status_tensor()

    def step():
        sta.qkv_prologue(q_out, t["kc"], t["vc"], t["cu"], t["sk"], H_q=pc.H_q, H_kv=pc.H_kv,
                         qkv=t["qkv"], qk_norm=True, q_norm_weight=t["qw"], k_norm_weight=t["kw"],
                         norm_eps=pc.norm_eps, rotary_dim=pc.rotary_dim,
                         interleaved=pc.interleaved, cos_table=t["cos"], sin_table=t["sin"],
                         position_ids=t["pos"], rotary_offsets=t["offs"], block_table=t["bt"],
                         status=st)
        sta.topk_select(scores, tcu, tsk, tk.k, sel, cnt, tail=tk.tail, status=st)

    print("graph: eager prologue + topk", flush=True)
    step()
    torch.cuda.synchronize()
    eager = [x.clone() for x in (q_out, t["kc"], t["vc"], sel, cnt)]
    assert int(st.item()) == 0
    want_sel, want_cnt = oracle.topk_select(tk.scores, tk.cu_seqlens_q, tk.seqlens_k, k=tk.k,
                                            tail=tk.tail, capacity=tk.capacity)
    assert np.array_equal(cnt.cpu().numpy(), want_cnt)
    assert np.array_equal(sel.cpu().numpy(), want_sel)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    noise = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        print(f"graph: prologue + topk replay {rep}", flush=True)
        q_out.fill_(float("nan"))
        sel.fill_(-7)
        cnt.fill_(-7)
        (noise * 3.0).sum().item()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((q_out, t["kc"], t["vc"], sel, cnt), eager):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), rep
    assert int(st.item()) == 0
