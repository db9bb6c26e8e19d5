"""Host-side checks of the C-ABI library (no GPU needed): the library loads,
exports every entry point include/msa.h declares, rejects bad problems before
touching the device, and the binding fails loudly when the library is absent."""
import ctypes
import os
import re

import numpy as np
import pytest

from block_sparse_attention_k2q_amd import binding as B
from oracle import msa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "msa.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(msa_\w+)\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 10
    h = B.lib()
    for n in names:
        assert hasattr(h, n), n
    assert set(names) == set(B.EXPORTED)


def test_grid_launch_bound_matches_walk_rule():
    for cap in (0, 1, 7, 2399, 2400, 61696, 65536, 1 << 20):
        for s in (1, 7, 256):
            assert B.msa_grid_launch_bound(cap, s) == O.grid_launch_bound(cap, s)


def test_schedule_layout_is_host_only_and_sized():
    p = B.Problem.make([0, 8192], 4, 128, 16, dq_mode=B.DQ_RECOMPUTE)
    L = B.msa_schedule_layout_of(p)
    cap = 4 * 1024 * 16
    assert L.task_meta + 6 * cap <= L.total
    offs = [L.desc, L.err, L.doc_chunk_off, L.doc_blk_off, L.chunk_doc, L.sel_clean, L.row_cursor,
            L.row_ptr, L.head_off, L.q_idx, L.task_meta, L.total]
    assert offs == sorted(offs)
    base = 4 * 8192 * 64 + 2 * 4 * 8192 * 4 * 128            # Delta, dK, dV (fp32)
    assert base <= B.msa_backward_scratch_bytes(p) < base + 4096
    pa = B.Problem(**{**p.__dict__, "dq_mode": B.DQ_ATOMIC_POOL})
    assert B.msa_backward_scratch_bytes(pa) >= base + 4 * 8192 * 64 * 128   # plus the fp32 dQ pool
    pb = B.Problem(**{**p.__dict__, "dq_mode": B.DQ_ATOMIC_POOL_BF16})
    assert base + 2 * 8192 * 64 * 128 <= B.msa_backward_scratch_bytes(pb) < base + 2 * 8192 * 64 * 128 + 4096
    pd = B.Problem(**{**p.__dict__, "dq_mode": B.DQ_DS_BUFFER})
    slots = 4 * 1024 * 16
    assert base + slots * 128 * 64 * 2 <= B.msa_backward_scratch_bytes(pd) < base + slots * 128 * 64 * 2 + 4096


@pytest.mark.parametrize("field,value,exc", [
    ("head_dim", 96, NotImplementedError),
    ("q_per_kv", 8, NotImplementedError),
    ("block_size", 96, NotImplementedError),
    ("topk", 65, NotImplementedError),
    ("num_chunks", 5, ValueError),
    ("num_docs", 0, ValueError),
    ("softmax_scale", 0.0, ValueError),
    ("dq_mode", 4, ValueError),
])
def test_bad_problems_are_rejected_on_the_host(field, value, exc):
    good = B.Problem.make([0, 512], 1, 64, 4)
    bad = B.Problem(**{**good.__dict__, field: value})
    with pytest.raises(exc):
        B.msa_schedule_layout_of(bad)


def test_key_block_128_rules():
    """Key block 128 runs as two 64-key tiles: topk <= 32 in every dQ mode,
    and twice the dS slots of key block 64 at the same topk."""
    p = B.Problem.make([0, 8192], 4, 128, 16, block_size=128, dq_mode=B.DQ_DS_BUFFER)
    assert p.num_kblocks == 64
    L = B.msa_schedule_layout_of(p)
    assert L.task_meta + 6 * 4 * 1024 * 16 <= L.total
    base = 4 * 8192 * 64 + 2 * 4 * 8192 * 4 * 128
    slots = 4 * 1024 * 16 * 2
    assert base + slots * 128 * 64 * 2 <= B.msa_backward_scratch_bytes(p) < base + slots * 128 * 64 * 2 + 4096
    for mode in (B.DQ_DS_BUFFER, B.DQ_RECOMPUTE, B.DQ_ATOMIC_POOL, B.DQ_ATOMIC_POOL_BF16):
        q = B.Problem(**{**p.__dict__, "dq_mode": mode})
        assert B.msa_schedule_layout_of(q).total == L.total
        assert B.msa_backward_scratch_bytes(q) >= base
        with pytest.raises(NotImplementedError):
            B.msa_schedule_layout_of(B.Problem(**{**q.__dict__, "topk": 33}))
    # without the dS slots the recompute mode needs only Delta and dK/dV
    rq = B.Problem(**{**p.__dict__, "dq_mode": B.DQ_RECOMPUTE})
    assert base <= B.msa_backward_scratch_bytes(rq) < base + 4096
    with pytest.raises(ValueError):   # 63 blocks of 128 cannot hold 8192 tokens
        B.msa_schedule_layout_of(B.Problem(**{**p.__dict__, "num_kblocks": 63}))


def test_missing_library_raises_unavailable(monkeypatch):
    monkeypatch.setattr(B, "LIB_PATH", os.path.join(ROOT, "no_such_libmsa.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(B.UnavailableError):
        B.lib()
    monkeypatch.setattr(B, "_lib", None)   # a failed bind is not cached


def test_binding_type_checks():
    import torch
    p = B.Problem.make([0, 64], 1, 64, 2)
    with pytest.raises(TypeError):
        B._expect(torch.zeros(2, dtype=torch.int64), "cu_seqlens", torch.int32, (2,))
    with pytest.raises(ValueError):
        B._expect(torch.zeros(3, dtype=torch.int32), "cu_seqlens", torch.int32, (2,))


def test_autograd_entry_refuses_host_tensors():
    """The autograd entry point only marshals: host tensors are refused before
    anything runs (there is no CPU path)."""
    import torch
    from block_sparse_attention_k2q_amd.autograd import msa_attention
    p = B.Problem.make([0, 64], 1, 64, 1)
    q = torch.zeros(64, 16, 64, dtype=torch.bfloat16)
    kv = torch.zeros(64, 1, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 64], dtype=torch.int32)
    sel = torch.zeros(1, 8, 1, dtype=torch.int32)
    with pytest.raises(ValueError):
        msa_attention(q, kv, kv, cu, sel, p)


def test_index_scorer_limits():
    p = B.Problem.make([0, 8192], 4, 128, 16)
    base = 4 * 1024 * 128 * 4 + 4 * 128 * 128 * 4     # chunk query sums + block key means (fp32)
    assert base <= B.msa_index_scratch_bytes(p) < base + 1024
    long_doc = B.Problem.make([0, 300000], 1, 128, 16)   # 4688 key blocks in one document
    with pytest.raises(NotImplementedError):
        B.msa_index_scratch_bytes(long_doc)
    assert B.msa_index_scratch_bytes(B.Problem.make([0, 262144], 1, 128, 16)) > 0   # 4096 blocks


def test_tensors_on_different_devices_are_refused():
    import torch
    with pytest.raises(ValueError):
        B._on_device(torch.zeros(1), torch.zeros(1, device="meta"))


def test_kv_rows_fewer_than_tokens_is_a_shape_error():
    p = B.Problem.make(np.array([0, 100, 300], dtype=np.int32), 1, 64, 2)
    B.msa_schedule_layout_of(B.Problem(**{**p.__dict__, "kv_rows": 300}))
    B.msa_schedule_layout_of(B.Problem(**{**p.__dict__, "kv_rows": 4096}))
    with pytest.raises(ValueError):
        B.msa_schedule_layout_of(B.Problem(**{**p.__dict__, "kv_rows": 299}))
    with pytest.raises(ValueError):
        B.msa_schedule_layout_of(B.Problem(**{**p.__dict__, "kv_rows": -1}))
    # the backward scratch grows with the K/V rows (fp32 dK / dV accumulators)
    grow = (B.msa_backward_scratch_bytes(B.Problem(**{**p.__dict__, "kv_rows": 4096}))
            - B.msa_backward_scratch_bytes(p))
    assert grow >= 2 * 4 * (4096 - 300) * 64
