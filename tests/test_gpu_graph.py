"""The whole step (schedule build, forward, backward) captured in a HIP
graph through torch.cuda.graph and replayed: every replay, with eager work
and synchronisations in between, must reproduce the eager results (the
kernels clear their own counters and accumulators, so no memset node is
recorded).  out, lse and dq are deterministic (bit-equal); dk and dv sum
fp32 atomics in a run-dependent order before their bf16 cast, so they may
differ by one bf16 ulp at their largest magnitude (2^-8 of the max), far
below what a replay bug (accumulators not cleared: doubled values) gives."""
import pytest
import torch

from block_sparse_attention_k2q_amd import binding as B
from block_sparse_attention_k2q_amd.workloads import make_workload

import msa_testlib as TL

pytestmark = pytest.mark.gpu


def test_step_in_a_graph_matches_eager_on_every_replay():
    w = make_workload("tiny", lengths=[700, 300], num_kv_heads=2, head_dim=128, topk=4, seed=51)
    print(f"[case] graph capture T={w.total_tokens}", flush=True)
    p = TL.problem_for(w, dq_mode=B.DQ_DS_BUFFER)
    t = TL.to_dev(w)

    def step():
        sched = B.build_schedule(p, t["cu"], t["sel"])
        out, lse = B.forward(p, t["q"], t["k"], t["v"], t["cu"], sched)
        dq, dk, dv = B.backward(p, t["q"], t["k"], t["v"], out, t["do"], lse, t["cu"], sched)
        return out, lse, dq, dk, dv

    ref = [x.clone() for x in step()]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    for rep in range(3):
        step()                           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        out, lse, dq, dk, dv = outs
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]) and torch.equal(dq, ref[2]), rep
        for got, want in ((dk, ref[3]), (dv, ref[4])):
            tol = 2.0 ** -8 * float(want.float().abs().max())
            assert float((got.float() - want.float()).abs().max()) <= tol, rep
