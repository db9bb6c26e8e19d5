"""Seeded synthetic workloads for MSA main attention.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle: it draws inputs and holds none of the attention arithmetic.  Every
array comes from ``numpy.random.Generator(PCG64(seed))`` in a fixed order:
document lengths, then block selections, then q, k, v, dO as float32 normals
rounded to bfloat16 (round-to-nearest-even, done by torch's CPU cast).

Topology follows the MSA schedule contract page (msa_schedule, module data):
an 8-query chunk (QUERY_CHUNK), 16 query heads per index/KV head
(NUM_Q_HEADS / NUM_INDEX_HEADS), softmax scale HEAD_DIM ** -0.5.  The key
block size, head dim, head count and top-k are parameters so the five
workloads below can differ from the page's compiled-in topology.

Selection recipe (one set per (index head, chunk), document-local block ids):
the chunk's own diagonal block is always present; the remaining slots are
drawn without replacement from the earlier blocks of the same document
(uniformly, or Zipf-weighted), fewer if not enough exist; unused slots hold
-1.  Each row is sorted ascending, so the diagonal block comes last.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

QUERY_CHUNK = 8           # msa_schedule page, QUERY_CHUNK
Q_HEADS_PER_KV = 16       # msa_backward_sm100 page, MAIN_HEADS_PER_INDEX = 64 // 4
_GEN_TOKENS_PER_DRAW = 2048  # fixed draw granularity, so streams do not depend on memory


@dataclasses.dataclass
class Workload:
    name: str
    cu_seqlens: np.ndarray        # int32 [docs + 1]
    num_kv_heads: int             # index heads == KV heads
    q_per_kv: int                 # 16
    head_dim: int
    block: int                    # key block size
    chunk: int                    # query chunk (8)
    topk: int
    scale: float
    sel: np.ndarray               # int32 [Hkv, C, topk], document-local block ids, -1 = empty
    q: torch.Tensor               # bf16 [T, Hq, D]
    k: torch.Tensor               # bf16 [T, Hkv, D]
    v: torch.Tensor               # bf16 [T, Hkv, D]
    do: torch.Tensor              # bf16 [T, Hq, D]

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens.astype(np.int64))

    @property
    def num_q_heads(self) -> int:
        return self.num_kv_heads * self.q_per_kv

    @property
    def num_docs(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def num_chunks(self) -> int:
        return int(sum(-(-int(n) // self.chunk) for n in self.lens))

    @property
    def num_kblocks(self) -> int:
        return int(sum(-(-int(n) // self.block) for n in self.lens))


# name -> recipe.  "lengths" is either a list of document lengths or a
# (count, lo, hi, multiple) tuple drawn uniformly then rounded to the multiple.
CONFIGS = {
    "tiny": dict(lengths=[512], num_kv_heads=1, head_dim=64, block=64, topk=4,
                 selection="uniform", do_std=1.0, seed=1000),
    "single8k": dict(lengths=[8192], num_kv_heads=4, head_dim=128, block=64, topk=16,
                     selection="uniform", do_std=1.0, seed=1001),
    "varlen8": dict(lengths=(8, 512, 8192, 64), num_kv_heads=4, head_dim=128, block=64, topk=16,
                    selection="uniform", do_std=1.0, seed=1002),
    "long64k": dict(lengths=[65536], num_kv_heads=4, head_dim=128, block=64, topk=32,
                    selection="uniform_first", do_std=0.1, seed=1003),
    "zipf16k": dict(lengths=[16384], num_kv_heads=4, head_dim=128, block=64, topk=16,
                    selection="zipf", zipf_s=1.2, do_std=1.0, seed=1004),
}
CONFIG_ORDER = ["tiny", "single8k", "varlen8", "long64k", "zipf16k"]


def _draw_lengths(rng: np.random.Generator, spec) -> list[int]:
    if isinstance(spec, tuple):
        count, lo, hi, mult = spec
        raw = rng.integers(lo, hi + 1, size=count)
        return [int(max(mult, mult * round(int(x) / mult))) for x in raw]
    return [int(x) for x in spec]


def draw_selection(rng: np.random.Generator, lens: Sequence[int], num_kv_heads: int,
                   block: int, topk: int, kind: str = "uniform", zipf_s: float = 1.2,
                   chunk: int = QUERY_CHUNK) -> np.ndarray:
    """Draw sel[Hkv, C, topk] (document-local block ids, -1 = empty slot).

    For a chunk whose first query sits in block ``diag`` the set is
    {diag} + (up to topk-1 distinct earlier blocks).  ``uniform_first`` also
    forces block 0.  Sampling without replacement uses exponential keys
    (the Efraimidis-Spirakis method): each candidate j gets key u_j ** (1/w_j)
    with u uniform, and the largest keys win; with all w equal this is a
    uniform draw without replacement.
    """
    assert block % chunk == 0, "a chunk must not straddle key blocks"
    per_block = block // chunk
    nchunks = [-(-int(n) // chunk) for n in lens]
    sel = np.full((num_kv_heads, sum(nchunks), topk), -1, dtype=np.int32)
    goff = 0
    for n, nc in zip(lens, nchunks):
        nblocks = -(-int(n) // block)
        for b in range(nblocks):
            c0, c1 = b * per_block, min((b + 1) * per_block, nc)
            if c1 <= c0:
                continue
            m = c1 - c0
            forced = [b]
            cand = np.arange(b, dtype=np.int64)
            if kind == "uniform_first" and b > 0:
                forced = [0, b]
                cand = np.arange(1, b, dtype=np.int64)
            n_extra = max(0, min(topk - len(forced), len(cand)))
            rows = np.full((num_kv_heads, m, topk), -1, dtype=np.int32)
            if n_extra > 0:
                u = rng.random((num_kv_heads, m, len(cand)))
                if kind == "zipf":
                    w = (cand + 1.0) ** (-zipf_s)
                    keys = np.log(u) / w          # monotone in u ** (1/w)
                else:
                    keys = u
                top = np.argpartition(-keys, n_extra - 1, axis=-1)[..., :n_extra]
                picked = cand[top]
            else:
                picked = np.zeros((num_kv_heads, m, 0), dtype=np.int64)
            forced_arr = np.broadcast_to(np.array(forced, dtype=np.int64), (num_kv_heads, m, len(forced)))
            allb = np.sort(np.concatenate([picked, forced_arr], axis=-1), axis=-1)
            rows[..., : allb.shape[-1]] = allb[..., :topk]
            sel[:, goff + c0: goff + c1, :] = rows
        goff += nc
    return sel


def _bf16_normals(rng: np.random.Generator, shape, std: float) -> torch.Tensor:
    out = torch.empty(shape, dtype=torch.bfloat16)
    flat = out.view(shape[0], -1)
    for t0 in range(0, shape[0], _GEN_TOKENS_PER_DRAW):
        t1 = min(shape[0], t0 + _GEN_TOKENS_PER_DRAW)
        x = rng.standard_normal((t1 - t0, flat.shape[1]), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        flat[t0:t1] = torch.from_numpy(x).to(torch.bfloat16)
    return out


def make_workload(name: str = "tiny", *, lengths=None, num_kv_heads=None, head_dim=None,
                  block=None, topk=None, selection=None, seed: Optional[int] = None,
                  do_std=None, zipf_s=None, sel: Optional[np.ndarray] = None) -> Workload:
    """Build a seeded workload; keyword overrides make the small edge cases."""
    base = dict(CONFIGS[name]) if name in CONFIGS else dict(CONFIGS["tiny"])
    for key, val in dict(lengths=lengths, num_kv_heads=num_kv_heads, head_dim=head_dim,
                         block=block, topk=topk, selection=selection, seed=seed,
                         do_std=do_std, zipf_s=zipf_s).items():
        if val is not None:
            base[key] = val
    rng = np.random.Generator(np.random.PCG64(base["seed"]))
    lens = _draw_lengths(rng, base["lengths"])
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    hkv, d, blk, k = base["num_kv_heads"], base["head_dim"], base["block"], base["topk"]
    if sel is None:
        sel = draw_selection(rng, lens, hkv, blk, k, base["selection"], base.get("zipf_s", 1.2))
    t = int(cu[-1])
    hq = hkv * Q_HEADS_PER_KV
    q = _bf16_normals(rng, (t, hq, d), 1.0)
    kk = _bf16_normals(rng, (t, hkv, d), 1.0)
    v = _bf16_normals(rng, (t, hkv, d), 1.0)
    do = _bf16_normals(rng, (t, hq, d), base["do_std"])
    return Workload(name=name, cu_seqlens=cu, num_kv_heads=hkv, q_per_kv=Q_HEADS_PER_KV,
                    head_dim=d, block=blk, chunk=QUERY_CHUNK, topk=k,
                    scale=1.0 / math.sqrt(d), sel=np.ascontiguousarray(sel, dtype=np.int32),
                    q=q, k=kk, v=v, do=do)


INDEX_DIM = 128           # msa_schedule page, INDEX_DIM


def make_index_inputs(w: Workload, seed: int = 0) -> tuple[torch.Tensor, torch.Tensor]:
    """Synthetic index projections for the index scorer: qi, ki bf16
    [T, Hkv, INDEX_DIM], N(0, 1), from a generator of their own
    (PCG64(10000 + seed)), so the attention inputs of ``w`` are unchanged.
    With such inputs the selection is close to uniform over earlier blocks,
    like the workloads' own selections."""
    rng = np.random.Generator(np.random.PCG64(10000 + seed))
    t = w.total_tokens
    qi = _bf16_normals(rng, (t, w.num_kv_heads, INDEX_DIM), 1.0)
    ki = _bf16_normals(rng, (t, w.num_kv_heads, INDEX_DIM), 1.0)
    return qi, ki
