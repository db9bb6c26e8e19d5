"""msa_backward_noalloc (static scratch) against msa_backward (caller's
scratch) through the C ABI: every dq mode, two calls in a row with the
second problem smaller than the first (so stale contents of the shared
static array would show), element by element to the parity bar; and the
size limit refused before anything is enqueued."""
import numpy as np
import pytest
import torch

from block_sparse_attention_k2q_amd import binding as B
from block_sparse_attention_k2q_amd.workloads import make_workload

import msa_testlib as TL

pytestmark = pytest.mark.gpu

PROBLEMS = [dict(lengths=[1500, 700], num_kv_heads=2, head_dim=128, topk=6, seed=41),
            dict(lengths=[300, 77], num_kv_heads=1, head_dim=128, topk=3, seed=42)]


def _run(w, dq_mode, block=64):
    p = TL.problem_for(w, dq_mode=dq_mode)
    t = TL.to_dev(w)
    sched = TL.run_schedule(w, p, t)
    out, lse = B.forward(p, t["q"], t["k"], t["v"], t["cu"], sched)
    ref = B.backward(p, t["q"], t["k"], t["v"], out, t["do"], lse, t["cu"], sched)
    got = tuple(torch.full_like(x, float("nan")) for x in ref)
    B.msa_backward_noalloc(p, t["q"], t["k"], t["v"], out, t["do"], lse, t["cu"], sched, *got)
    torch.cuda.synchronize()
    return p, ref, got


@pytest.mark.parametrize("dq_mode", [B.DQ_RECOMPUTE, B.DQ_DS_BUFFER, B.DQ_ATOMIC_POOL, B.DQ_ATOMIC_POOL_BF16])
def test_noalloc_matches_backward_twice(dq_mode):
    for spec in PROBLEMS:                      # the second call is the smaller problem
        w = make_workload("tiny", **spec)
        print(f"[case] noalloc dq_mode={dq_mode} T={w.total_tokens} Hkv={w.num_kv_heads}", flush=True)
        p, ref, got = _run(w, dq_mode)
        assert B.msa_backward_scratch_bytes(p) <= B.NOALLOC_SCRATCH_BYTES
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.isfinite(b).all(), name
            TL.assert_grad(name, b, TL.f64(a))
        if dq_mode in (B.DQ_RECOMPUTE, B.DQ_DS_BUFFER):
            assert torch.equal(ref[0], got[0])   # dq has no atomics in these modes


def test_noalloc_refuses_problems_beyond_the_static_scratch():
    w = make_workload("single8k")
    p = TL.problem_for(w, dq_mode=B.DQ_DS_BUFFER)     # 1 GiB of dS slots
    assert B.msa_backward_scratch_bytes(p) > B.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda", 0)
    T, hq, hkv, D = p.total_tokens, p.num_q_heads, p.num_kv_heads, p.head_dim
    bf = dict(dtype=torch.bfloat16, device=dev)
    q, out, dout, dq = (torch.zeros(T, hq, D, **bf) for _ in range(4))
    k, v, dk, dv = (torch.zeros(T, hkv, D, **bf) for _ in range(4))
    lse = torch.zeros(T, hq, dtype=torch.float32, device=dev)
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    sched = B.alloc_schedule(p, dev)
    with pytest.raises(ValueError, match="static buffer"):
        B.msa_backward_noalloc(p, q, k, v, out, dout, lse, cu, sched, dq, dk, dv)
    # the same problem in recompute mode fits (34 MiB)
    p2 = TL.problem_for(w, dq_mode=B.DQ_RECOMPUTE)
    assert B.msa_backward_scratch_bytes(p2) <= B.NOALLOC_SCRATCH_BYTES
