"""GPU: paged_decode_step_noalloc (split-K partials in the library's static device array)
against paged_decode_step with a caller workspace, through the C ABI: two calls in a row,
the second with a smaller batch, each bit-identical to the allocating entry point (outputs,
lengths, every cache byte, status) and within the fp16 bound of the oracle; a call whose
partials exceed the array is rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

import selected_token_sparse_amd as sta
import synth
from synth.device import case_tensors

from harness import assert_close, oracle_paged_step, status_tensor

pytestmark = pytest.mark.gpu


def _bits(t):
    n = t.element_size()
    return t.view(torch.uint8 if n == 1 else torch.int16 if n == 2 else torch.int32)


def _call(case, t, noalloc):
    kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
    sq = torch.full((case.B,), 777, dtype=torch.int32, device="cuda")
    sk = torch.full((case.B,), 777, dtype=torch.int32, device="cuda")
    out = torch.full((case.T, case.H_q, case.D), float("nan"), dtype=torch.float16, device="cuda")
    st = status_tensor()
    kw = dict(block_table=t["block_table"], scale=case.scale, local_window=case.local_window,
              sinks=t["sinks"], status=st)
    args = (t["cu"], t["past"], case.T, sq, sk, t["q"], t["k_new"], t["v_new"], kc, vc,
            case.max_seqlen_q, case.max_seqlen_k, out)
    if noalloc:
        sta.paged_decode_step_noalloc(*args, **kw)
    else:
        need = sta.attention_workspace_bytes(sta.KIND_PAGED, case.dtype, case.B, case.T,
                                             case.max_seqlen_q, case.max_seqlen_k, 0,
                                             case.local_window, case.H_q, case.H_kv, case.D)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        sta.paged_decode_step(*args, workspace=ws, **kw)
    torch.cuda.synchronize()
    return dict(out=out, sq=sq.cpu(), sk=sk.cpu(), k=_bits(kc).cpu(), v=_bits(vc).cpu(),
                st=int(st.item()))


def test_noalloc_step_matches_the_workspace_step_twice():
    # the full GQA decode workload (about 8.4 MB of partials), then a smaller batch with a
    # window: the second call reads none of what the first left in the array
    cases = [synth.config_gqa_paged_decode(poison=True),
             synth.paged_case(902, kv_lens=[900, 1, 0, 2500, 64, 33], q_lens=[1, 1, 0, 1, 1, 1],
                              H_q=64, H_kv=8, D=64, dtype=synth.F16, sinks=True,
                              local_window=700, poison=True)]
    for n, case in enumerate(cases):
        print("noalloc call", n, case.name, "T", case.T, flush=True)
        t = case_tensors(case)
        a = _call(case, t, noalloc=True)
        b = _call(case, t, noalloc=False)
        for name in ("sq", "sk", "k", "v"):
            assert torch.equal(a[name], b[name]), (n, name)
        assert torch.equal(_bits(a["out"]).cpu(), _bits(b["out"]).cpu()), (n, "out")
        assert a["st"] == b["st"], (n, a["st"], b["st"])
        ref, ost = oracle_paged_step(case)
        assert_close(a["out"], ref, case.dtype, f"noalloc call {n}")
        assert a["st"] == ost, (n, a["st"], ost)


def test_noalloc_rejects_partials_beyond_the_array():
    # 255 requests of 8 rows of 64 heads with a key bound of 65536: about 1 GB of partials
    # (the check is on the host bounds, before any launch)
    case = synth.paged_case(903, kv_lens=[10] * 255, q_lens=[8] * 255, H_q=64, H_kv=8, D=64,
                            dtype=synth.F16, sinks=True, max_seqlen_k=65536)
    need = sta.attention_workspace_bytes(sta.KIND_PAGED, case.dtype, case.B, case.T,
                                         case.max_seqlen_q, case.max_seqlen_k, 0, -1, case.H_q,
                                         case.H_kv, case.D)
    assert need > 16 << 20
    t = case_tensors(case)
    sq = torch.full((case.B,), 777, dtype=torch.int32, device="cuda")
    sk = torch.full((case.B,), 777, dtype=torch.int32, device="cuda")
    out = torch.full((case.T, case.H_q, case.D), 3.0, dtype=torch.float16, device="cuda")
    kc = t["k_cache"].clone()
    with pytest.raises(sta.SpattnError) as e:
        sta.paged_decode_step_noalloc(t["cu"], t["past"], case.T, sq, sk, t["q"], t["k_new"],
                                      t["v_new"], kc, t["v_cache"], case.max_seqlen_q,
                                      case.max_seqlen_k, out, block_table=t["block_table"],
                                      scale=case.scale, sinks=t["sinks"])
    assert e.value.rc == -5
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((sq == 777).all())
    assert torch.equal(_bits(kc), _bits(t["k_cache"]))
