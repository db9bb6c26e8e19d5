"""The planner-driven forward (msa_forward_kv: KV-parallel over the task
table, exact cross-workgroup softmax merge) against the oracle, through the
C ABI: the small edge cases element by element (ragged and empty documents,
junk slots, both head dims, chunks selecting nothing, scores growing far past
the first block's max, both walk regimes and tail walks), and the full-size
uniform and long-context workloads on sampled chunks.  Its out / lse must
also agree with the query-parallel msa_forward to the parity bar."""
import numpy as np
import pytest
import torch

from block_sparse_attention_k2q_amd import binding as B
from block_sparse_attention_k2q_amd.workloads import make_workload
from oracle import msa_oracle as O

import msa_testlib as TL
from test_gpu_parity import SMALL, _oracle_full, _stack_rows, _gpu_rows

pytestmark = pytest.mark.gpu

CASES = ["tiny", "ragged_docs_junk", "d64_two_heads", "large_walk", "zipf_small", "empty_chunks",
         "growing_max", "overflowing_max"]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("num_cus", [None, 7])
def test_forward_kv_small_cases(case, num_cus):
    w = SMALL[case]()
    print(f"[case] forward_kv {case} num_cus={num_cus} T={w.total_tokens}", flush=True)
    p = TL.problem_for(w, num_cus, B.DQ_DS_BUFFER)
    t = TL.to_dev(w)
    sched = TL.run_schedule(w, p, t)
    want = TL.compare_schedule(w, p, sched)
    out, lse = B.forward_kv(p, t["q"], t["k"], t["v"], t["cu"], sched)
    ref_out, ref_lse = B.forward(p, t["q"], t["k"], t["v"], t["cu"], sched)
    torch.cuda.synchronize()
    _, _, _, rout, rlse = _oracle_full(w, want["sel_clean"])
    TL.assert_out_lse(out, lse, rout, rlse)
    # both forwards against each other: out within two bf16 units; lse within
    # 2^-8 (the query-parallel forward sums its bf16-rounded probabilities,
    # each off by at most 2^-9 relative, this one sums them in fp32)
    fin = torch.isfinite(ref_lse)
    assert torch.equal(torch.isfinite(lse), fin)
    assert (lse[fin] - ref_lse[fin]).abs().max().item() <= 2.0 ** -8
    assert (out.float() - ref_out.float()).abs().max().item() <= 2.0 ** -6 * max(1.0, ref_out.float().abs().max().item())


@pytest.mark.parametrize("name", ["single8k", "long64k"])
def test_forward_kv_full_size_sampled(name):
    w = make_workload(name)
    print(f"[case] forward_kv full-size {name}", flush=True)
    p = TL.problem_for(w, dq_mode=B.DQ_DS_BUFFER)
    t = TL.to_dev(w)
    sched = TL.run_schedule(w, p, t)
    want = TL.compare_schedule(w, p, sched)
    out, lse = B.forward_kv(p, t["q"], t["k"], t["v"], t["cu"], sched)
    torch.cuda.synchronize()
    lay = want["layout"]
    chunks = sorted({(j % w.num_kv_heads, int(g)) for j, g in
                     enumerate(np.linspace(0, lay.C - 1, 256).round().astype(int))})
    res = O.chunk_rows(w.q, w.k, w.v, w.do, w.cu_seqlens, want["sel_clean"], w.block, w.scale, chunks)
    toks, heads, rout, rlse, _ = _stack_rows(res)
    TL.assert_out_lse(_gpu_rows(out, toks, heads), _gpu_rows(lse, toks, heads), rout, rlse)
    assert torch.isfinite(out).all()
