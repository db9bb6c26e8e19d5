"""Pins of the oracle's CSR inversion, walk rule and task table.

* a hand-derived golden example (tests/golden/csr_tiny.json);
* brute force: for every key-block row, scan every (head, chunk, slot);
* exhaustive walk enumeration (the msa_schedule page says its CPU tests
  exhaust the walk rule): every row walked exactly once, and
  chunk_map(n, r, s)[2] <= n // r + s <= grid_launch_bound(cap, s).
"""
import json
import os

import numpy as np
import pytest

from oracle import msa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_csr_example():
    with open(os.path.join(GOLDEN, "csr_tiny.json")) as f:
        g = json.load(f)
    s = O.build_schedule(np.array(g["sel"], dtype=np.int32), g["cu_seqlens"], g["block"], g["num_sms"])
    np.testing.assert_array_equal(s["sel_clean"], g["sel_clean"])
    assert s["dropped"] == g["dropped"]
    np.testing.assert_array_equal(s["row_ptr"], g["row_ptr"])
    np.testing.assert_array_equal(s["q_idx"], g["q_idx"])
    np.testing.assert_array_equal(s["task_meta"][: len(g["task_meta"])], g["task_meta"])
    assert np.all(s["task_meta"][len(g["task_meta"]):] == -1)
    np.testing.assert_array_equal(s["desc"], g["desc"])


def _brute_csr(sel, layout):
    hkv, C, k = sel.shape
    rows = []
    for i in range(hkv):
        per_row = []
        for d in range(layout.docs):
            for b in range(int(layout.nblocks[d])):
                ents = []
                for c in range(int(layout.nchunks[d])):
                    g = int(layout.chunk_off[d]) + c
                    last = min(8 * c + 7, int(layout.lens[d]) - 1)
                    if b * layout.block <= last and any(int(x) == b for x in sel[i, g]):
                        ents.append(8 * c)
                per_row.append(ents)
        rows.append(per_row)
    return rows


@pytest.mark.parametrize("seed", range(6))
def test_csr_matches_brute_force(seed):
    _csr_brute_force_case(seed, None)


@pytest.mark.parametrize("seed", range(3))
def test_csr_matches_brute_force_block128(seed):
    _csr_brute_force_case(100 + seed, 128)


def _csr_brute_force_case(seed, block):
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(0, 120 if block is None else 500, size=rng.integers(1, 5))]
    block = int(rng.choice([8, 16, 32, 64])) if block is None else block
    hkv, k = int(rng.integers(1, 4)), int(rng.integers(1, 6))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    layout = O.DocLayout(cu, block)
    sel = rng.integers(-2, max(2, int(layout.nblocks.max(initial=1)) + 2),
                       size=(hkv, layout.C, k)).astype(np.int32)
    s = O.build_schedule(sel, cu, block, num_sms=7)
    want = _brute_csr(sel, layout)
    for i in range(hkv):
        rp = s["row_ptr"][i]
        assert rp[0] == 0 and np.all(np.diff(rp) >= 0)
        got = [list(s["q_idx"][i, rp[r]:rp[r + 1]]) for r in range(layout.R)]
        assert got == want[i]
        assert np.all(s["q_idx"][i, rp[-1]:] == -1)
    # every kept slot appears exactly once; row_ptr[-1] = number of kept slots
    assert sum(int(s["row_ptr"][i, -1]) for i in range(hkv)) == int((s["sel_clean"] >= 0).sum())
    n_nonempty = int((sel != -1).sum())
    assert s["dropped"] == n_nonempty - int((s["sel_clean"] >= 0).sum())


@pytest.mark.parametrize("seed", range(4))
def test_task_table_columns(seed):
    rng = np.random.default_rng(100 + seed)
    lens = [int(x) for x in rng.integers(1, 300, size=3)]
    block = 64
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    layout = O.DocLayout(cu, block)
    sel = rng.integers(-1, 6, size=(2, layout.C, 4)).astype(np.int32)
    s = O.build_schedule(sel, cu, block, num_sms=256)
    meta, desc = s["task_meta"], s["desc"]
    n = int(desc[0])
    seen = set()
    for t in range(n):
        i, r, qb, qc, d, b = (int(x) for x in meta[t])
        assert r == layout.blk_off[d] + b and 0 <= b < layout.nblocks[d]
        assert qb % 8 == 0 and qc == min(8, int(layout.lens[d]) - qb) and qc > 0
        g = int(layout.chunk_off[d]) + qb // 8
        assert b in set(int(x) for x in s["sel_clean"][i, g])
        assert (i, g, b) not in seen
        seen.add((i, g, b))
    assert len(seen) == int((s["sel_clean"] >= 0).sum())
    # CSR order: (head, row, q_begin) strictly increasing
    keys = [tuple(int(x) for x in meta[t, [0, 1, 2]]) for t in range(n)]
    assert keys == sorted(keys) and len(set(keys)) == n
    assert np.all(meta[n:] == -1)


@pytest.mark.parametrize("num_sms", [1, 2, 7, 256])
def test_walk_rule_exhaustive(num_sms):
    cap = 5000
    bound = O.grid_launch_bound(cap, num_sms)
    for n in range(cap + 1):
        r = O.rows_per_cta(n)
        assert r == (4 if n < 2400 else 64)
        full, tail, grid = O.chunk_map(n, r, num_sms)
        assert full * r + tail == n and 0 <= tail < r
        assert grid <= n // r + num_sms
        assert grid <= bound
        if n in (0, 1, 3, 4, 5, 2399, 2400, 2401, 2463, 2464, cap) or n % 97 == 0:
            covered = np.zeros(n, dtype=np.int32)
            prev_hi = 0
            for cta in range(grid):
                lo, hi = O.walk_bounds(n, r, num_sms, cta)
                assert lo == prev_hi and hi > lo and hi - lo <= r
                covered[lo:hi] += 1
                prev_hi = hi
            assert prev_hi == n and np.all(covered == 1)
    # the bound is also a bound for every smaller capacity
    for c2 in (0, 1, 100, 2399, 2400, 4999):
        assert O.grid_launch_bound(c2, num_sms) <= bound


def test_golden_walks_with_tail():
    """The tail split (tests/golden/walk_tail.json, hand-derived): walk
    bounds of every case, and the page's bound n // r + s reached when the
    tail has at least s rows (which only a tail spread over s walks does)."""
    with open(os.path.join(GOLDEN, "walk_tail.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        n, s, r = case["n"], case["s"], case["r"]
        assert O.rows_per_cta(n) == r
        assert O.chunk_map(n, r, s) == tuple(case["chunk_map"])
        full, tail, grid = case["chunk_map"]
        walks = [O.walk_bounds(n, r, s, cta) for cta in range(grid)]
        if "walks" in case:
            assert walks == [tuple(x) for x in case["walks"]]
        else:
            assert walks[full:] == [tuple(x) for x in case["walks_tail"]]
            assert walks[:full] == [(x * r, (x + 1) * r) for x in range(full)]
        if tail >= s:
            assert grid == n // r + s
