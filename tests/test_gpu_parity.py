"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Small cases (the oracle finishes in seconds; several tiles, ragged tails,
empty documents, junk selection slots, both head dims, both walk regimes and
the tail walks) are compared element by element.  The five workloads at full
size are run in the same launch configuration as bench.py: the schedule
tables are compared bit-exactly, and out/lse/dq/dk/dv on sampled chunks and
key blocks that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_k2q_amd import binding as B
from block_sparse_attention_k2q_amd.workloads import make_workload, draw_selection
from oracle import msa_oracle as O

import msa_testlib as TL

pytestmark = pytest.mark.gpu


SMALL = {
    "tiny": lambda: make_workload("tiny"),
    "ragged_docs_junk": lambda: TL.inject_junk(make_workload(
        "tiny", lengths=[200, 0, 77, 512, 9], num_kv_heads=2, head_dim=128, topk=5, seed=11), 3),
    "d64_two_heads": lambda: make_workload("tiny", lengths=[300, 129], num_kv_heads=2, head_dim=64,
                                           topk=3, seed=12),
    "large_walk": lambda: make_workload("tiny", lengths=[2048], num_kv_heads=2, head_dim=128, topk=8,
                                        seed=13),
    "zipf_small": lambda: make_workload("tiny", lengths=[4096], num_kv_heads=1, head_dim=128, topk=6,
                                        selection="zipf", seed=14),
    "uniform_first_small": lambda: make_workload("tiny", lengths=[1024, 960], num_kv_heads=1,
                                                 head_dim=128, topk=5, selection="uniform_first",
                                                 do_std=0.1, seed=15),
}


def _empty_rows_workload():
    w = make_workload("tiny", lengths=[256, 64], num_kv_heads=1, head_dim=128, topk=3, seed=16)
    w.sel[0, 5:9] = -1          # four chunks select nothing
    w.sel[0, 12, :] = -1        # one chunk keeps only an earlier block, not its diagonal
    w.sel[0, 12, 1] = 0
    return w


SMALL["empty_chunks"] = _empty_rows_workload


def _scaled_late_keys(factor):
    """Keys of the blocks from 4 on scaled by `factor` (exact in bf16: a
    power of two), so chunks whose first selected block is an early one meet
    scores far above its max later: the forward's running max must move and
    rescale what it has summed (by about 2^35 at factor 8; at factor 64 an
    unrescaled sum would overflow fp32), and the backward runs with LSE up
    to about 330."""
    def make():
        w = make_workload("tiny", lengths=[1024], num_kv_heads=1, head_dim=128, topk=6, seed=31)
        k = w.k.float().clone()
        k[4 * w.block:] *= factor
        w.k = k.to(torch.bfloat16)
        return w
    return make


SMALL["growing_max"] = _scaled_late_keys(8.0)
SMALL["overflowing_max"] = _scaled_late_keys(64.0)
# Hot buckets checked element by element: block 0 forced for every chunk
# (1024 tasks in one CSR row, 16 walks of 64), and Zipf-skewed selection.
SMALL["hot_row_first"] = lambda: make_workload("tiny", lengths=[8192], num_kv_heads=1, head_dim=128, topk=8,
                                               selection="uniform_first", seed=17)
SMALL["hot_rows_zipf"] = lambda: make_workload("tiny", lengths=[8192], num_kv_heads=1, head_dim=128, topk=8,
                                               selection="zipf", seed=18)


def _oracle_full(w, sel_clean):
    """(dq, dk, dv, out, lse) of the whole problem: literal dense masks up to
    1024 tokens, the batched gathered evaluation above."""
    if w.total_tokens <= 1024:
        dq, dk, dv, _, out, lse = O.backward_dense(w.q, w.k, w.v, w.do, w.cu_seqlens, sel_clean, w.block,
                                                   w.scale)
        return dq, dk, dv, out, lse
    return O.backward_batched(w.q, w.k, w.v, w.do, w.cu_seqlens, sel_clean, w.block, w.scale)


@pytest.mark.parametrize("case", list(SMALL))
@pytest.mark.parametrize("num_cus,dq_mode", [(None, B.DQ_RECOMPUTE), (7, B.DQ_RECOMPUTE),
                                             (None, B.DQ_ATOMIC_POOL), (7, B.DQ_ATOMIC_POOL),
                                             (None, B.DQ_DS_BUFFER), (7, B.DQ_DS_BUFFER),
                                             (None, B.DQ_ATOMIC_POOL_BF16), (7, B.DQ_ATOMIC_POOL_BF16)])
def test_small_cases_full_parity(case, num_cus, dq_mode):
    w = SMALL[case]()
    print(f"[case] {case} num_cus={num_cus} dq_mode={dq_mode} T={w.total_tokens} "
          f"Hkv={w.num_kv_heads} D={w.head_dim} k={w.topk}", flush=True)
    p = TL.problem_for(w, num_cus, dq_mode)
    t = TL.to_dev(w)
    sched = TL.run_schedule(w, p, t)
    want = TL.compare_schedule(w, p, sched)
    out, lse, dq, dk, dv = TL.run_forward_backward(p, t, sched)
    sel_clean = want["sel_clean"]
    rdq, rdk, rdv, rout, rlse = _oracle_full(w, sel_clean)
    TL.assert_out_lse(out, lse, rout, rlse)
    TL.assert_grads(dq, dk, dv, rdq, rdk, rdv)
    # keys no query attends get exactly zero gradient
    attended = np.zeros(w.total_tokens * w.num_kv_heads, dtype=bool).reshape(w.total_tokens, -1)
    lay = want["layout"]
    for i in range(w.num_kv_heads):
        for g in range(lay.C):
            d, _, keys = O.chunk_keys(lay, sel_clean, i, g)
            attended[int(lay.cu[d]) + keys, i] = True
    assert torch.all(dk.cpu()[torch.from_numpy(~attended)] == 0)
    assert torch.all(dv.cpu()[torch.from_numpy(~attended)] == 0)


# Key block 128 (the pages' production block size): documents that end
# inside the first or the second 64-key half of a block, diagonal blocks
# whose second half lies after the chunk, junk slots, both head dims and
# both walk regimes.
SMALL128 = {
    "tiny_b128": lambda: make_workload("tiny", block=128, topk=3),
    "ragged_b128_junk": lambda: TL.inject_junk(make_workload(
        "tiny", lengths=[200, 0, 77, 512, 9, 300], num_kv_heads=2, head_dim=128, block=128, topk=4,
        seed=21), 5),
    "d64_b128": lambda: make_workload("tiny", lengths=[1000, 129], num_kv_heads=2, head_dim=64,
                                      block=128, topk=5, seed=22),
    "large_walk_b128": lambda: make_workload("tiny", lengths=[4096], num_kv_heads=2, head_dim=128,
                                             block=128, topk=8, seed=23),
}


@pytest.mark.parametrize("case", list(SMALL128))
@pytest.mark.parametrize("num_cus,dq_mode", [(None, B.DQ_DS_BUFFER), (7, B.DQ_DS_BUFFER),
                                             (1, B.DQ_DS_BUFFER),   # 1: the grid has no spare walk
                                             (None, B.DQ_RECOMPUTE), (7, B.DQ_RECOMPUTE),
                                             (None, B.DQ_ATOMIC_POOL), (7, B.DQ_ATOMIC_POOL),
                                             (None, B.DQ_ATOMIC_POOL_BF16), (1, B.DQ_ATOMIC_POOL_BF16)])
def test_small_cases_block128_full_parity(case, num_cus, dq_mode):
    w = SMALL128[case]()
    print(f"[case] {case} num_cus={num_cus} dq_mode={dq_mode} T={w.total_tokens} Hkv={w.num_kv_heads} "
          f"D={w.head_dim} k={w.topk} block={w.block}", flush=True)
    p = TL.problem_for(w, num_cus, dq_mode)
    t = TL.to_dev(w)
    sched = TL.run_schedule(w, p, t)
    want = TL.compare_schedule(w, p, sched)
    out, lse, dq, dk, dv = TL.run_forward_backward(p, t, sched)
    rdq, rdk, rdv, rout, rlse = _oracle_full(w, want["sel_clean"])
    TL.assert_out_lse(out, lse, rout, rlse)
    TL.assert_grads(dq, dk, dv, rdq, rdk, rdv)


FULL = ["single8k", "varlen8", "long64k", "zipf16k"]
SPREAD_CHUNKS = 256        # evenly spread (index head, chunk) pairs checked at full size
HOT_CHUNK_CAP = 2100       # the hot row whose every chunk is checked has at most this many entries


def _stack_rows(results):
    """(token index, head index) of every checked row, and the oracle's
    out [n, D], lse [n] and dq [n, D] of those rows."""
    toks, heads, outs, lses, dqs = [], [], [], [], []
    for tq, hs, o_, l_, q_ in results:
        tt, hh = np.meshgrid(tq, hs, indexing="ij")
        toks.append(tt.ravel())
        heads.append(hh.ravel())
        outs.append(o_.reshape(-1, o_.shape[-1]))
        lses.append(l_.ravel())
        dqs.append(q_.reshape(-1, q_.shape[-1]))
    return (np.concatenate(toks), np.concatenate(heads), np.concatenate(outs), np.concatenate(lses),
            np.concatenate(dqs))


def _gpu_rows(x, toks, heads):
    return x[torch.as_tensor(toks, device=x.device), torch.as_tensor(heads, device=x.device)].cpu()


@pytest.mark.parametrize("name,dq_mode", [(n, B.DQ_RECOMPUTE) for n in FULL] +
                         [(n, B.DQ_DS_BUFFER) for n in FULL] + [("single8k", B.DQ_ATOMIC_POOL),
                                                                ("single8k", B.DQ_ATOMIC_POOL_BF16),
                                                                ("single8k_b128", B.DQ_DS_BUFFER),
                                                                ("single8k_b128", B.DQ_RECOMPUTE),
                                                                ("single8k_b128", B.DQ_ATOMIC_POOL),
                                                                ("varlen8_b128", B.DQ_RECOMPUTE),
                                                                ("zipf16k_b128", B.DQ_ATOMIC_POOL_BF16),
                                                                ("long64k_b128", B.DQ_RECOMPUTE),
                                                                ("varlen8_b128", B.DQ_DS_BUFFER),
                                                                ("long64k_b128", B.DQ_DS_BUFFER)])
def test_full_size_configs_sampled(name, dq_mode):
    """Full size, in the bench's launch configuration.  out / lse / dq on 256
    evenly spread (index head, chunk) pairs plus every chunk of one hot CSR
    row (the hottest of head 0 with at most 2100 entries); dk / dv on the
    hottest CSR row of the workload (long64k: the forced block 0, selected by
    all 8192 chunks of a head; zipf16k: block 0, about 2047 chunks) and on
    two random rows, each complete (every selecting chunk evaluated)."""
    print(f"[case] full-size {name} dq_mode={dq_mode}", flush=True)
    if name.endswith("_b128"):   # the same workload at key block 128
        w = make_workload(name[:-len("_b128")], block=128)
    else:
        w = make_workload(name)
    p = TL.problem_for(w, dq_mode=dq_mode)
    t = TL.to_dev(w)
    sched = TL.run_schedule(w, p, t)
    want = TL.compare_schedule(w, p, sched)
    print(f"[case] {name}: schedule bit-exact, N={int(want['desc'][0])}", flush=True)
    out, lse, dq, dk, dv = TL.run_forward_backward(p, t, sched)
    del t
    lay = want["layout"]
    sel_clean = want["sel_clean"]
    counts = np.diff(want["row_ptr"], axis=1)
    # out / lse / dq
    spread = [(j % w.num_kv_heads, int(g))
              for j, g in enumerate(np.linspace(0, lay.C - 1, SPREAD_CHUNKS).round().astype(int))]
    capped = np.where(counts[0] <= HOT_CHUNK_CAP, counts[0], -1)
    hot = int(np.argmax(capped))
    hot_chunks = O.chunks_selecting_block(want, 0, hot)
    chunks = sorted(set(spread) | set(hot_chunks))
    res = O.chunk_rows(w.q, w.k, w.v, w.do, w.cu_seqlens, sel_clean, w.block, w.scale, chunks)
    toks, heads, rout, rlse, rdq = _stack_rows(res)
    print(f"[case] {name}: {len(chunks)} chunks ({len(hot_chunks)} of row {hot}), {len(toks)} rows",
          flush=True)
    TL.assert_out_lse(_gpu_rows(out, toks, heads), _gpu_rows(lse, toks, heads), rout, rlse)
    TL.assert_grad("dq", _gpu_rows(dq, toks, heads), rdq)
    # dk / dv on the hottest row and two random rows
    i_hot, r_hot = np.unravel_index(int(np.argmax(counts)), counts.shape)
    rng = np.random.default_rng(7)
    picks = [(int(i_hot), int(r_hot))] + [(int(rng.integers(w.num_kv_heads)), int(rng.integers(lay.R)))
                                          for _ in range(2)]
    for i, r in picks:
        toks, gk, gv = O.key_block_grads(w.q, w.k, w.v, w.do, w.cu_seqlens, sel_clean, w.block, w.scale, i, r)
        print(f"[case] {name}: dk/dv of head {i} row {r} ({int(counts[i, r])} chunks)", flush=True)
        hk = np.full(len(toks), i)
        TL.assert_grad("dk", _gpu_rows(dk, toks, hk), gk)
        TL.assert_grad("dv", _gpu_rows(dv, toks, hk), gv)
    # properties at full size
    assert torch.isfinite(out).all() and torch.isfinite(dq).all()
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()
