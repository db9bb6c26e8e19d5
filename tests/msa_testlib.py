"""Shared helpers for the parity tests: run the HIP path through the C-ABI
binding and the fp64 oracle on the same seeded workload, and compare."""
from __future__ import annotations

import numpy as np
import torch

from block_sparse_attention_k2q_amd import binding as B
from oracle import msa_oracle as O

O_TOL = 1e-2       # max abs error of out and lse (see out_tolerance for out)
GRAD_TOL = 2e-2    # max abs error of dq/dk/dv divided by the tensor's max abs


def device_cus() -> int:
    return B.msa_device_check(0)


def problem_for(w, num_cus=None, dq_mode=B.DQ_RECOMPUTE) -> B.Problem:
    return B.Problem.make(w.cu_seqlens, w.num_kv_heads, w.head_dim, w.topk,
                          num_cus=num_cus if num_cus is not None else device_cus(),
                          softmax_scale=w.scale, block_size=w.block, dq_mode=dq_mode)


def to_dev(w):
    dev = torch.device("cuda", 0)
    return dict(q=w.q.to(dev), k=w.k.to(dev), v=w.v.to(dev), do=w.do.to(dev),
                cu=torch.from_numpy(w.cu_seqlens).to(dev), sel=torch.from_numpy(w.sel).to(dev))


def run_schedule(w, p, t):
    sched = B.build_schedule(p, t["cu"], t["sel"])
    torch.cuda.synchronize()
    return sched


def schedule_host(p, sched) -> dict:
    v = B.schedule_views(p, sched)
    return {k: x.cpu().numpy() for k, x in v.items()}


def compare_schedule(w, p, sched) -> None:
    got = schedule_host(p, sched)
    want = O.build_schedule(w.sel, w.cu_seqlens, w.block, p.num_cus)
    assert got["err"][B.SCHED_ERR_GEOMETRY] == 0
    np.testing.assert_array_equal(got["sel_clean"], want["sel_clean"])
    assert int(got["err"][B.SCHED_ERR_DROPPED]) == want["dropped"]
    np.testing.assert_array_equal(got["row_ptr"], want["row_ptr"])
    np.testing.assert_array_equal(got["q_idx"], want["q_idx"])
    np.testing.assert_array_equal(got["task_meta"], want["task_meta"])
    np.testing.assert_array_equal(got["desc"], want["desc"])
    return want


def run_forward_backward(p, t, sched):
    out, lse = B.forward(p, t["q"], t["k"], t["v"], t["cu"], sched)
    dq, dk, dv = B.backward(p, t["q"], t["k"], t["v"], out, t["do"], lse, t["cu"], sched)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def f64(x) -> np.ndarray:
    return x.detach().to("cpu", torch.float64).numpy()


def bf16_ulp(x) -> np.ndarray:
    """Spacing of the bf16 numbers (8 significant bits) at |x|: 2^(floor(log2|x|) - 7)."""
    e = np.floor(np.log2(np.maximum(np.abs(np.asarray(x, dtype=np.float64)), np.finfo(np.float64).tiny)))
    return np.exp2(e - 7)


def out_tolerance(out_ref) -> np.ndarray:
    """Per-element bar for the bf16 output: 1e-2 absolute below |out| = 4,
    one bf16 unit of the exact value from |out| = 4 on.  Below 4 a correctly
    rounded bf16 number is within half a unit (at most 2^-7 < 1e-2 on
    [2, 4)), so the plain bar is attainable there and is kept.  From 4 on
    the spacing is 2^-5 and more: no bf16 number lies within 1e-2 of every
    real there, so the bar becomes one unit (faithful rounding)."""
    x = np.abs(np.asarray(out_ref, dtype=np.float64))
    return np.where(x >= 4.0, np.maximum(O_TOL, bf16_ulp(x)), O_TOL)


def assert_out_lse(out_gpu, lse_gpu, out_ref, lse_ref, rows=None) -> None:
    og, lg = f64(out_gpu), f64(lse_gpu)
    if rows is not None:
        og, lg, out_ref, lse_ref = og[rows], lg[rows], out_ref[rows], lse_ref[rows]
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(lg), np.isneginf(lse_ref)), "empty-row pattern differs"
    assert np.all(og[~fin] == 0)
    diff = np.abs(og - out_ref)
    ratio = diff / out_tolerance(out_ref)
    err_l = float(np.abs(lg[fin] - lse_ref[fin]).max(initial=0.0))
    if ratio.size and float(ratio.max()) > 1.0:
        at = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"out error {float(diff[at])} at {tuple(int(x) for x in at)} "
                             f"(exact {float(out_ref[at])}, bar {float(out_tolerance(out_ref[at]))})")
    assert err_l <= O_TOL, f"lse max abs error {err_l}"


def rel_err(got, ref) -> float:
    den = float(np.abs(ref).max(initial=0.0))
    num = float(np.abs(got - ref).max(initial=0.0))
    if den == 0.0:
        return num
    return num / den


def assert_grad(name, got, ref, rows=None) -> None:
    g = f64(got)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    e = rel_err(g, ref)
    assert e <= GRAD_TOL, f"{name} relative max abs error {e}"


def assert_grads(dq, dk, dv, ref_dq, ref_dk, ref_dv) -> None:
    assert_grad("dq", dq, ref_dq)
    assert_grad("dk", dk, ref_dk)
    assert_grad("dv", dv, ref_dv)


def inject_junk(w, seed):
    """Replace some slots by repeats, out-of-range, non-causal and negative ids."""
    rng = np.random.default_rng(seed)
    sel = w.sel.copy()
    H, C, K = sel.shape
    layout = O.DocLayout(w.cu_seqlens, w.block)
    for _ in range(max(4, C // 8)):
        i, g = int(rng.integers(H)), int(rng.integers(C))
        d, c = layout.chunk_local(g)
        s = int(rng.integers(K))
        kind = int(rng.integers(4))
        if kind == 0:
            sel[i, g, s] = sel[i, g, 0]                          # repeat
        elif kind == 1:
            sel[i, g, s] = int(layout.nblocks[d]) + int(rng.integers(3))   # past the document
        elif kind == 2:
            sel[i, g, s] = min(int(layout.nblocks[d]) - 1, (8 * c) // w.block + 1)  # maybe non-causal
        else:
            sel[i, g, s] = -2 - int(rng.integers(5))              # negative, not the empty marker
    w.sel = sel
    return w
