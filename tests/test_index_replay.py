"""CPU replay of the index arithmetic the kernels derive from the schedule
(no GPU): for every task of the walk, and for every (index head, chunk) of
the query-parallel kernels, the rows and byte offsets each kernel reads or
writes are recomputed in int64 from the schedule tables (the oracle's, which
the GPU tables equal bit for bit) and checked against the tensor sizes the
caller allocates; every value a kernel keeps in a 32-bit integer is checked
to fit in one.  Covers the five workloads at full size, both key block
sizes, ragged and empty documents, and a K/V workspace with gaps."""
import numpy as np
import pytest

from block_sparse_attention_k2q_amd.workloads import make_workload
from oracle import msa_oracle as O

I32 = 2 ** 31
TILE_M = 128                      # 8 queries x 16 heads


def _replay(w, num_sms=256, kv_starts=None, kv_rows=None):
    s = O.build_schedule(w.sel, w.cu_seqlens, w.block, num_sms)
    lay = s["layout"]
    Hkv, D, B, K = w.num_kv_heads, w.head_dim, w.block, w.topk
    Hq = 16 * Hkv
    T = w.total_tokens
    sub = B // 64
    kv0_doc = np.asarray(w.cu_seqlens[:-1] if kv_starts is None else kv_starts, dtype=np.int64)
    W = T if kv_rows is None else kv_rows
    cap = Hkv * lay.C * K
    assert cap < I32 // 6                       # the host's size check

    # --- walk: every task row exactly once, bounds inside the table ---------
    n, rpc, full, tail, tail_walks, grid, capd, _ = (int(x) for x in s["desc"])
    assert capd == cap and grid <= O.grid_launch_bound(cap, num_sms)
    covered = np.zeros(n, dtype=np.int64)
    for wg in range(grid):
        lo, hi = O.walk_bounds(n, rpc, num_sms, wg)
        assert 0 <= lo <= hi <= n and hi - lo <= 64    # a walk's meta fits its 64 LDS rows
        covered[lo:hi] += 1
    assert np.all(covered == 1)

    tm = s["task_meta"][:n].astype(np.int64)
    i, r, qb, qc, d, b = (tm[:, x] for x in range(6))
    tok0 = lay.cu[d]
    ln = lay.lens[d]
    kv0 = kv0_doc[d]
    assert np.all((qc >= 1) & (qc <= 8) & (qb >= 0) & (qb + qc <= ln))
    assert np.all((b >= 0) & (b * B <= qb + qc - 1) & (b * B < ln))

    # --- KV-parallel backward (and the planner-driven forward's walk) -------
    # Q / dO rows of a half tile: token tok0 + qb + min(j, qc - 1), 16 heads of head i
    for half in (0, 1):
        j = np.minimum(4 * half + np.arange(4)[None, :], qc[:, None] - 1)
        row = (tok0 + qb)[:, None] + j
        assert np.all((row >= tok0[:, None]) & (row < (tok0 + ln)[:, None]))
        first = (row * Hq + 16 * i[:, None]) * D       # 64-bit element offset of the piece
        assert first.max() + 16 * D <= T * Hq * D
        # LSE / Delta of each lane's row
        assert ((row * Hq + 16 * i[:, None] + 15).max() < T * Hq)
    # K / V rows of each 64-key tile (keys past the end read the last key) and
    # the dK / dV rows the flush adds into (keys past the end go to the tile's first key)
    for t in range(sub):
        tile = sub * b + t
        live = tile * 64 <= qb + qc - 1
        keys = np.minimum(tile[:, None] * 64 + np.arange(64)[None, :], ln[:, None] - 1)
        krow = kv0[:, None] + keys
        assert np.all(krow[live] >= 0) and krow[live].max(initial=0) < W
        elem = (krow * Hkv + i[:, None]) * D + D - 1
        assert elem[live].max(initial=0) < W * Hkv * D
        # 32-bit: the flush's per-register offset (key within the tile) * Hkv * D
        assert 63 * Hkv * D < I32
        # dS slot of the tile: (row * K + slot) * sub + t, row = i * C + global chunk
        g = lay.chunk_off[d] + qb // 8
        sel = s["sel_clean"][i, g]                      # [n, K]
        slot = np.argmax(sel == b[:, None], axis=1)
        assert np.all(sel[np.arange(n), slot] == b)
        slot_idx = ((i * lay.C + g) * K + slot) * sub + t
        assert slot_idx.max(initial=0) < cap * sub and slot_idx.max(initial=0) < I32
        # its byte offset in the scratch (16 KiB per slot) is formed in 64 bits
        assert (slot_idx.max(initial=0) + 1) * 16384 <= cap * sub * 16384

    # --- atomic-pool backward: every tile of every task, live or not ---------
    # (a tile after the chunk's last query computes zeros; its K / V rows are
    # read only below the document end, and it flushes only when it starts
    # inside the document, each key past the end going to the tile's first key)
    for t in range(sub):
        tile = sub * b + t
        flushes = tile * 64 < ln
        key = tile[:, None] * 64 + np.arange(64)[None, :]
        kpos = np.where(key < ln[:, None], key, tile[:, None] * 64)
        frow = kv0[:, None] + kpos
        assert np.all(frow[flushes] >= 0) and frow[flushes].max(initial=0) < W
        loaded = key < ln[:, None]
        assert (kv0[:, None] + key)[loaded].max(initial=0) < W
    # dQ pool rows: the chunk's tokens, rows past the document end sent to the tile's first row
    assert ((tok0 + qb + qc - 1) * Hq + 16 * i + 15).max() < T * Hq

    # --- query-parallel forward and dQ kernels, per (index head, chunk) -----
    sc = s["sel_clean"].astype(np.int64)                # [Hkv, C, K]
    g = np.arange(lay.C)
    dg = lay.chunk_doc
    c = g - lay.chunk_off[dg]
    qcount = np.minimum(8, lay.lens[dg] - 8 * c)
    assert np.all(qcount >= 1)
    last_q = 8 * c + qcount - 1
    for t in range(sub):
        tile = sub * sc + t                             # 64-key tile of each slot
        kept = (sc >= 0) & (tile * 64 <= last_q[None, :, None])
        keys_hi = np.minimum(tile * 64 + 63, (lay.lens[dg] - 1)[None, :, None])
        krow = kv0_doc[dg][None, :, None] + keys_hi
        lens_b = np.broadcast_to(lay.lens[dg][None, :, None], sc.shape)
        assert np.all(krow[kept] < W) and np.all(tile[kept] * 64 < lens_b[kept])
        # the tile copy's 32-bit byte offset from the block's first row
        assert 64 * Hkv * D * 2 < I32
    qrow = (lay.cu[dg] + 8 * c + qcount - 1)[None, :] * Hq + 16 * np.arange(Hkv)[:, None] + 15
    assert qrow.max() < T * Hq
    # dS slots the dQ kernel reads: row_base * sub + lane position, row_base = (i*C + g) * K
    row_base = (np.arange(Hkv)[:, None] * lay.C + g[None, :]) * K
    assert (row_base.max() * sub + sub * K - 1) < cap * sub
    return n


@pytest.mark.parametrize("name", ["tiny", "single8k", "varlen8", "long64k", "zipf16k"])
@pytest.mark.parametrize("block", [64, 128])
def test_replay_full_size_workloads(name, block):
    w = make_workload(name, block=block)
    n = _replay(w)
    assert n > 0


@pytest.mark.parametrize("seed", range(6))
def test_replay_ragged_and_workspace(seed):
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(0, 900, size=5)]
    w = make_workload("tiny", lengths=lens, num_kv_heads=int(rng.integers(1, 4)), head_dim=128,
                      block=int(rng.choice([64, 128])), topk=int(rng.integers(1, 9)), seed=seed)
    for sms in (1, 7, 256):
        _replay(w, num_sms=sms)
    # documents at 128-aligned starts with gaps (the K/V workspace layout)
    starts, row = [], 0
    for x in lens:
        starts.append(row)
        row = -(-(row + x) // 128) * 128 + 128
    _replay(w, kv_starts=np.array(starts), kv_rows=row)
