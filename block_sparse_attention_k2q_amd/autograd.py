"""torch.autograd entry point of the sparse attention.

The forward builds the schedule (selection ingest, k2q CSR, task table) and
runs the sparse forward; it saves q, k, v, out, lse and the schedule, as the
msa_schedule page's MSABackwardSchedule is kept for the backward; the
backward runs the KV-parallel backward on them (msa_backward_sm100 page:
`run_backward` takes the forward's out and lse and returns bf16 dq, dk, dv).
Argument marshalling only: every step runs in libmsa's kernels, on torch's
current stream.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as B


class MSAAttentionFunction(torch.autograd.Function):
    """out, lse = f(q, k, v); lse is returned but not differentiable."""

    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens, sel, problem: B.Problem):
        sched = B.build_schedule(problem, cu_seqlens, sel)
        out, lse = B.forward(problem, q, k, v, cu_seqlens, sched)
        ctx.save_for_backward(q, k, v, out, lse, cu_seqlens, sched)
        ctx.problem = problem
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, out, lse, cu_seqlens, sched = ctx.saved_tensors
        dq, dk, dv = B.backward(ctx.problem, q, k, v, out, dout.contiguous(), lse, cu_seqlens, sched)
        return dq, dk, dv, None, None, None


def msa_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                  sel: torch.Tensor, problem: Optional[B.Problem] = None, *,
                  block_size: int = 64, softmax_scale: Optional[float] = None,
                  dq_mode: int = B.DQ_DS_BUFFER, return_lse: bool = False):
    """Sparse attention over THD tensors: q [T, 16*Hkv, D], k / v [T, Hkv, D]
    (bf16, on one GPU), cu_seqlens int32 [docs + 1], sel int32 [Hkv, C, topk]
    of document-local key-block ids (-1 = empty slot).

    The host-side sizes (the Problem) come from `problem` when given; else
    from cu_seqlens: on the host (a CPU tensor or an array) it is read there
    and copied to the device, on the device it is copied to the host first,
    which waits for the device.  Pass `problem` (built once from the host
    lengths) or host cu_seqlens to keep the call free of that wait."""
    dev = q.device
    if problem is None:
        if q.dim() != 3 or k.dim() != 3 or sel.dim() != 3:
            raise ValueError("q, k must be [T, H, D] and sel [Hkv, C, topk]")
        on_device = isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda
        cu_host = (cu_seqlens.detach().to("cpu") if on_device else torch.as_tensor(cu_seqlens)).numpy()
        problem = B.Problem.make(cu_host, k.shape[1], q.shape[2], sel.shape[2],
                                 num_cus=B.msa_device_check(dev.index or 0),
                                 softmax_scale=softmax_scale, block_size=block_size, dq_mode=dq_mode)
    if not (isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda):
        cu_seqlens = torch.as_tensor(cu_seqlens, dtype=torch.int32).to(dev)
    out, lse = MSAAttentionFunction.apply(q, k, v, cu_seqlens, sel, problem)
    return (out, lse) if return_lse else out
