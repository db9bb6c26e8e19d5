"""K/V in a workspace with a start row per document (msa_build_schedule_kv;
msa_schedule page: MSABackwardSchedule.document_workspace_starts, the
128-aligned workspace row of each document; msa_backward_sm100 page:
run_backward takes k_aligned / v_aligned [W, 4, 128] and returns dk, dv in
the same rows, zero outside the documents).

Documents are placed at 128-aligned starts with gaps between them, and the
gap rows of k and v hold NaN, so a read of any row outside a document would
show.  The result must be the compact layout's: out, lse and (outside the
pool modes) dq bit for bit, dk / dv of each document's rows equal to the
compact run's within the fp32 atomic order, against the oracle within the
parity bar, and exactly 0 in every row outside the documents."""
import numpy as np
import pytest
import torch

from block_sparse_attention_k2q_amd import binding as B
from block_sparse_attention_k2q_amd.workloads import make_workload

import msa_testlib as TL
from oracle import msa_oracle as O

pytestmark = pytest.mark.gpu


def _aligned_starts(lens, align=128, gap=128):
    starts, row = [], 0
    for n in lens:
        starts.append(row)
        row = -(-(row + int(n)) // align) * align + gap
    return np.array(starts, dtype=np.int32), row


def _to_workspace(x, cu, starts, W):
    ws = torch.full((W,) + tuple(x.shape[1:]), float("nan"), dtype=x.dtype, device=x.device)
    for d in range(len(starts)):
        n = int(cu[d + 1] - cu[d])
        ws[int(starts[d]):int(starts[d]) + n] = x[int(cu[d]):int(cu[d]) + n]
    return ws


CASES = [
    (dict(lengths=[200, 77, 512, 9, 300], num_kv_heads=2, head_dim=128, topk=4, seed=51), 64, B.DQ_DS_BUFFER),
    (dict(lengths=[200, 77, 512, 9, 300], num_kv_heads=2, head_dim=128, topk=4, seed=51), 64, B.DQ_RECOMPUTE),
    (dict(lengths=[640, 130, 64], num_kv_heads=1, head_dim=64, topk=3, seed=52), 64, B.DQ_ATOMIC_POOL),
    (dict(lengths=[640, 130, 64], num_kv_heads=1, head_dim=128, topk=3, seed=52), 64, B.DQ_ATOMIC_POOL_BF16),
    (dict(lengths=[1000, 129, 300], num_kv_heads=2, head_dim=128, topk=4, seed=53), 128, B.DQ_DS_BUFFER),
]


@pytest.mark.parametrize("spec,block,dq_mode", CASES)
def test_workspace_layout_equals_compact(spec, block, dq_mode):
    w = make_workload("tiny", block=block, **spec)
    print(f"[case] workspace lens={list(w.lens)} block={block} dq_mode={dq_mode}", flush=True)
    t = TL.to_dev(w)
    p = TL.problem_for(w, dq_mode=dq_mode)
    sched = TL.run_schedule(w, p, t)
    want = TL.compare_schedule(w, p, sched)
    ref = TL.run_forward_backward(p, t, sched)

    starts, W = _aligned_starts(w.lens)
    pw = B.Problem(**{**p.__dict__, "kv_rows": W})
    kw = _to_workspace(t["k"], w.cu_seqlens, starts, W)
    vw = _to_workspace(t["v"], w.cu_seqlens, starts, W)
    sw = B.alloc_schedule(pw, kw.device)
    B.msa_build_schedule_kv(pw, t["cu"], t["sel"], torch.from_numpy(starts).to(kw.device), sw)
    torch.cuda.synchronize()
    views = TL.schedule_host(pw, sw)
    assert views["err"][B.SCHED_ERR_GEOMETRY] == 0
    np.testing.assert_array_equal(views["doc_kv_off"], starts)
    np.testing.assert_array_equal(views["task_meta"], want["task_meta"])
    out, lse = B.forward(pw, t["q"], kw, vw, t["cu"], sw)
    dq, dk, dv = B.backward(pw, t["q"], kw, vw, out, t["do"], lse, t["cu"], sw)
    torch.cuda.synchronize()

    assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])
    if dq_mode in (B.DQ_DS_BUFFER, B.DQ_RECOMPUTE):
        assert torch.equal(dq, ref[2])
    inside = np.zeros(W, dtype=bool)
    rows = np.concatenate([np.arange(int(starts[d]), int(starts[d]) + int(n)) for d, n in enumerate(w.lens)])
    inside[rows] = True
    outside = torch.from_numpy(~inside).to(dk.device)
    assert torch.all(dk[outside] == 0) and torch.all(dv[outside] == 0)
    idx = torch.from_numpy(rows).to(dk.device)
    for name, a, b in (("dk", dk, ref[3]), ("dv", dv, ref[4])):
        # the same sums in another atomic order: within a bf16 unit of the largest value
        diff = (a[idx].float() - b.float()).abs().max().item()
        assert diff <= 2.0 ** -7 * b.float().abs().max().item(), (name, diff)
    rdq, rdk, rdv, _, rout, rlse = O.backward_dense(w.q, w.k, w.v, w.do, w.cu_seqlens, want["sel_clean"],
                                                    w.block, w.scale) if w.total_tokens <= 1024 else \
        O.backward_gathered(w.q, w.k, w.v, w.do, w.cu_seqlens, want["sel_clean"], w.block, w.scale)
    TL.assert_out_lse(out, lse, rout, rlse)
    TL.assert_grads(dq, dk[idx], dv[idx], rdq, rdk, rdv)


def test_overlapping_starts_are_flagged_and_outputs_are_nan():
    w = make_workload("tiny", lengths=[300, 200], num_kv_heads=1, head_dim=64, topk=3, seed=54)
    print("[case] overlapping K/V starts", flush=True)
    t = TL.to_dev(w)
    p = B.Problem(**{**TL.problem_for(w).__dict__, "kv_rows": 1024})
    kw = torch.zeros(1024, 1, 64, dtype=torch.bfloat16, device=t["k"].device)
    for starts in ([0, 256], [512, 0], [0, 900]):        # overlap, out of order, past kv_rows
        sw = B.alloc_schedule(p, kw.device)
        B.msa_build_schedule_kv(p, t["cu"], t["sel"], torch.tensor(starts, dtype=torch.int32, device=kw.device), sw)
        out = torch.full_like(t["q"], 7.0)
        lse = torch.full((w.total_tokens, w.num_q_heads), 7.0, dtype=torch.float32, device=out.device)
        B.msa_forward(p, t["q"], kw, kw, t["cu"], sw, out, lse)
        torch.cuda.synchronize()
        assert TL.schedule_host(p, sw)["err"][B.SCHED_ERR_GEOMETRY] == 1, starts
        assert torch.isnan(out).all() and torch.isnan(lse).all()
