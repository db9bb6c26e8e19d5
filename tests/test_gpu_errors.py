"""Error paths and degenerate inputs on the GPU, through the C ABI.

* cu_seqlens that disagree with the host sizes: the schedule build sets the
  geometry error word, every later kernel returns without touching its
  outputs, and the index scorer writes empty rows (-1); nothing faults.
* a problem with no tokens at all: every entry point is a no-op.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_k2q_amd import binding as B
from block_sparse_attention_k2q_amd.workloads import make_workload, make_index_inputs

import msa_testlib as TL

pytestmark = pytest.mark.gpu


def test_geometry_mismatch_is_flagged_and_outputs_are_nan():
    w = make_workload("tiny", lengths=[512], num_kv_heads=1, head_dim=64, topk=4, seed=41)
    print(f"[case] geometry mismatch T={w.total_tokens}", flush=True)
    for dq_mode in (B.DQ_DS_BUFFER, B.DQ_RECOMPUTE, B.DQ_ATOMIC_POOL, B.DQ_ATOMIC_POOL_BF16):
        p = TL.problem_for(w, dq_mode=dq_mode)
        t = TL.to_dev(w)
        bad_cu = torch.tensor([0, 448], dtype=torch.int32, device=t["cu"].device)   # host says 512
        sched = B.build_schedule(p, bad_cu, t["sel"])
        torch.cuda.synchronize()
        views = TL.schedule_host(p, sched)
        assert views["err"][B.SCHED_ERR_GEOMETRY] == 1
        assert np.all(views["sel_clean"] == -1)
        # the step-by-step calls and the high-level ones: every output NaN
        out = torch.full_like(t["q"], 7.0)
        lse = torch.full((w.total_tokens, w.num_q_heads), 7.0, dtype=torch.float32, device=out.device)
        B.msa_forward(p, t["q"], t["k"], t["v"], bad_cu, sched, out, lse)
        scratch = B.alloc_scratch(p, out.device)
        dq, dk, dv = (torch.full_like(x, 7.0) for x in (t["q"], t["k"], t["v"]))
        B.msa_backward(p, t["q"], t["k"], t["v"], out, t["do"], lse, bad_cu, sched, scratch, dq, dk, dv)
        o2, l2 = B.forward(p, t["q"], t["k"], t["v"], bad_cu, sched)
        g2 = B.backward(p, t["q"], t["k"], t["v"], o2, t["do"], l2, bad_cu, sched)
        o3, l3 = B.forward_kv(p, t["q"], t["k"], t["v"], bad_cu, sched)
        torch.cuda.synchronize()
        for x in (out, lse, dq, dk, dv, o2, l2, *g2, o3, l3):
            assert torch.isnan(x).all()
    # the autograd entry point with a problem that disagrees with cu_seqlens
    from block_sparse_attention_k2q_amd.autograd import msa_attention
    qg = t["q"].clone().requires_grad_(True)
    o4 = msa_attention(qg, t["k"], t["v"], bad_cu, t["sel"], problem=p)
    o4.float().sum().backward()
    torch.cuda.synchronize()
    assert torch.isnan(o4).all() and torch.isnan(qg.grad).all()
    qi, ki = make_index_inputs(w)
    sel = B.index_select(p, qi.to(out.device), ki.to(out.device), bad_cu)
    torch.cuda.synchronize()
    assert torch.all(sel == -1)


def test_empty_problem_is_a_no_op():
    print("[case] empty problem", flush=True)
    dev = torch.device("cuda", 0)
    p = B.Problem.make([0, 0], 1, 64, 4, num_cus=B.msa_device_check(0))
    assert p.total_tokens == 0 and p.num_chunks == 0
    cu = torch.zeros(2, dtype=torch.int32, device=dev)
    sel = torch.zeros(1, 0, 4, dtype=torch.int32, device=dev)
    sched = B.build_schedule(p, cu, sel)
    q = torch.zeros(0, 16, 64, dtype=torch.bfloat16, device=dev)
    kv = torch.zeros(0, 1, 64, dtype=torch.bfloat16, device=dev)
    out, lse = B.forward(p, q, kv, kv, cu, sched)
    dq, dk, dv = B.backward(p, q, kv, kv, out, q, lse, cu, sched)
    torch.cuda.synchronize()
    assert out.shape == (0, 16, 64) and dq.shape == (0, 16, 64) and dk.shape == (0, 1, 64)
    views = TL.schedule_host(p, sched)
    assert int(views["desc"][0]) == 0 and views["err"][B.SCHED_ERR_GEOMETRY] == 0
