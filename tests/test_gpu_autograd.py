"""The torch.autograd entry point on the GPU: out/lse and the gradients that
autograd delivers to q, k, v match the fp64 oracle (same bars as the parity
tests), at key block 64 and 128."""
import pytest
import torch

from block_sparse_attention_k2q_amd.autograd import msa_attention
from block_sparse_attention_k2q_amd.workloads import make_workload
from oracle import msa_oracle as O

import msa_testlib as TL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("block", [64, 128])
def test_autograd_matches_oracle(block):
    w = make_workload("tiny", lengths=[300, 129], num_kv_heads=2, head_dim=128, block=block, topk=3,
                      seed=31)
    print(f"[case] autograd block={block} T={w.total_tokens}", flush=True)
    t = TL.to_dev(w)
    q, k, v = (t[n].clone().requires_grad_() for n in ("q", "k", "v"))
    out, lse = msa_attention(q, k, v, t["cu"], t["sel"], block_size=block, softmax_scale=w.scale,
                             return_lse=True)
    assert not lse.requires_grad
    (out.float() * t["do"].float()).sum().backward()
    torch.cuda.synchronize()
    lay = O.DocLayout(w.cu_seqlens, w.block)
    sel_clean, _ = O.clean_selection(w.sel, lay)
    rdq, rdk, rdv, _, rout, rlse = O.backward_dense(w.q, w.k, w.v, w.do, w.cu_seqlens, sel_clean,
                                                    w.block, w.scale)
    TL.assert_out_lse(out, lse, rout, rlse)
    TL.assert_grads(q.grad, k.grad, v.grad, rdq, rdk, rdv)


def test_autograd_with_host_lengths_matches_device_lengths():
    """cu_seqlens given on the host (no device-to-host copy in the call) gives
    the same result as the device tensor."""
    w = make_workload("tiny", lengths=[200, 77, 300], num_kv_heads=1, head_dim=64, topk=3, seed=33)
    print(f"[case] autograd host cu_seqlens T={w.total_tokens}", flush=True)
    t = TL.to_dev(w)
    outs = []
    for cu in (t["cu"], w.cu_seqlens):
        q = t["q"].clone().requires_grad_()
        out = msa_attention(q, t["k"], t["v"], cu, t["sel"], softmax_scale=w.scale)
        (out.float() * t["do"].float()).sum().backward()
        outs.append((out.detach(), q.grad))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
