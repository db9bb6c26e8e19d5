"""Randomised small problems (fixed seeds), compared element by element with
the fp64 oracle: document lengths from 0 to 1500 tokens (empty, ragged,
partial chunks and blocks), 1 to 4 index heads, head dim 64 or 128, top-k
1..12, key block 64 or 128, the three selection generators, every dQ mode,
several compute-unit counts (walk regimes and tail
walks), junk selection slots.  Small top-k leaves rows that attend to a few
keys, whose outputs reach |out| > 4 (the bf16 bar of out_tolerance)."""
import numpy as np
import pytest

from block_sparse_attention_k2q_amd import binding as B
from block_sparse_attention_k2q_amd.workloads import make_workload
from oracle import msa_oracle as O

import msa_testlib as TL

pytestmark = pytest.mark.gpu

MODES = [B.DQ_RECOMPUTE, B.DQ_ATOMIC_POOL, B.DQ_DS_BUFFER, B.DQ_ATOMIC_POOL_BF16]


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    ndocs = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(0, 1501, size=ndocs)]
    if sum(lens) == 0:
        lens[0] = 9
    block = int(rng.choice([64, 128]))
    w = make_workload("tiny", lengths=lens, num_kv_heads=int(rng.integers(1, 5)),
                      head_dim=int(rng.choice([64, 128])), block=block, topk=int(rng.integers(1, 13)),
                      selection=str(rng.choice(["uniform", "zipf", "uniform_first"])), seed=2000 + seed)
    if rng.random() < 0.5:
        w = TL.inject_junk(w, 3000 + seed)
    mode = MODES[int(rng.integers(len(MODES)))]
    num_cus = [None, 7, 1, 3][int(rng.integers(4))]
    return w, mode, num_cus


@pytest.mark.parametrize("seed", range(48))
def test_random_small_problem(seed):
    w, mode, num_cus = _case(seed)
    print(f"[case] random seed={seed} lens={list(w.lens)} Hkv={w.num_kv_heads} D={w.head_dim} "
          f"k={w.topk} block={w.block} dq_mode={mode} num_cus={num_cus}", flush=True)
    p = TL.problem_for(w, num_cus, mode)
    t = TL.to_dev(w)
    sched = TL.run_schedule(w, p, t)
    want = TL.compare_schedule(w, p, sched)
    out, lse, dq, dk, dv = TL.run_forward_backward(p, t, sched)
    rdq, rdk, rdv, _, rout, rlse = O.backward_gathered(w.q, w.k, w.v, w.do, w.cu_seqlens, want["sel_clean"],
                                                       w.block, w.scale)
    TL.assert_out_lse(out, lse, rout, rlse)
    TL.assert_grads(dq, dk, dv, rdq, rdk, rdv)
