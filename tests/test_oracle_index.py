"""Pins of the oracle's index scorer and top-k block selection (CPU).

The pages name the scorer (msa_bindings page: MSAKernels, ``fmha_sm100``) and
its sizes (msa_schedule page: INDEX_DIM, NUM_INDEX_HEADS, TOPK_BLOCKS) but
not its scoring function; the oracle states its reading (chunk query sum .
block key mean, diagonal forced, top-(k-1) earlier blocks, ties to the
smaller id).  These tests pin that reading by routes other than the
oracle's own formula:

* planted structure: every key of block b equals v_b e_0 and every query
  e_0 (or -e_0), so the ranking is the ranking of v (or of -v), found by
  sorting v directly;
* brute force: each score as the token-level double sum
  sum_{t in c} sum_{j in b} q_t . k_j / |b| in explicit loops;
* the kept set maximises the sum of scores over all subsets of the allowed
  size (enumerated);
* structure and invariances (diagonal kept, ids ascending and distinct,
  shuffling tokens inside a key block, positive scaling of the queries).
"""
import itertools

import numpy as np
import pytest

from oracle import msa_oracle as O


def _planted(lens, block, heads, dim, seed, sign=1.0):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    qi = np.zeros((T, heads, dim))
    ki = np.zeros((T, heads, dim))
    qi[:, :, 0] = sign
    v = {}
    for d, n in enumerate(lens):
        nb = -(-n // block)
        for h in range(heads):
            vals = rng.permutation(nb).astype(float) + 0.5      # distinct magnitudes
            v[d, h] = vals
            for b in range(nb):
                ki[cu[d] + b * block: cu[d] + min((b + 1) * block, n), h, 0] = vals[b]
    return cu, qi, ki, v


@pytest.mark.parametrize("block,sign", [(64, 1.0), (64, -1.0), (128, 1.0)])
def test_planted_block_magnitudes(block, sign):
    lens, heads, topk = [1000, 77, 640], 2, 5
    cu, qi, ki, v = _planted(lens, block, heads, 8, seed=3, sign=sign)
    sel = O.index_select(qi, ki, cu, block, topk)
    layout = O.DocLayout(cu, block)
    for d, n in enumerate(lens):
        for h in range(heads):
            for c in range(int(layout.nchunks[d])):
                diag = (8 * c) // block
                rank = np.argsort(-sign * v[d, h][:diag], kind="stable")[:topk - 1]
                want = sorted([diag] + [int(b) for b in rank])
                got = sel[h, layout.chunk_off[d] + c]
                assert list(got[:len(want)]) == want and np.all(got[len(want):] == -1)


def test_ties_go_to_the_smaller_block():
    lens, block, topk = [512], 64, 3
    cu, qi, ki, _ = _planted(lens, block, 1, 4, seed=5)
    ki[:, 0, 0] = 1.0
    ki[block * 2: block * 3, 0, 0] = 2.0          # block 2 best, blocks 0, 1, 3, ... tie
    ki[block * 5: block * 6, 0, 0] = 2.0          # block 5 ties with block 2
    sel = O.index_select(qi, ki, cu, block, topk)
    g = 63                                         # chunk 63: diagonal block 7
    assert list(sel[0, g]) == [2, 5, 7]
    sel2 = O.index_select(qi, ki, cu, block, 4)
    assert list(sel2[0, g]) == [0, 2, 5, 7]        # the next tie among 0, 1, 3, 4, 6 -> 0


def test_scores_match_token_double_sum():
    rng = np.random.default_rng(7)
    lens, block, H, X = [70, 45], 16, 2, 3
    cu = np.concatenate([[0], np.cumsum(lens)])
    qi = rng.standard_normal((sum(lens), H, X))
    ki = rng.standard_normal((sum(lens), H, X))
    layout, scores = O.index_scores(qi, ki, cu, block)
    for d, n in enumerate(lens):
        S, M = scores[d]
        for h in range(H):
            for c in range(int(layout.nchunks[d])):
                for b in range(int(layout.nblocks[d])):
                    ts = [t for t in range(n) if t // 8 == c]
                    js = [j for j in range(n) if j // block == b]
                    tot = 0.0
                    mag = 0.0
                    for x in range(X):
                        qx = sum(qi[cu[d] + t, h, x] for t in ts)
                        qa = sum(abs(qi[cu[d] + t, h, x]) for t in ts)
                        kx = sum(ki[cu[d] + j, h, x] for j in js) / len(js)
                        ka = sum(abs(ki[cu[d] + j, h, x]) for j in js) / len(js)
                        tot += qx * kx
                        mag += qa * ka
                    brute = sum(float(np.dot(qi[cu[d] + t, h], ki[cu[d] + j, h])) for t in ts for j in js) / len(js)
                    assert abs(S[h, c, b] - brute) < 1e-12 and abs(S[h, c, b] - tot) < 1e-12
                    assert abs(M[h, c, b] - mag) < 1e-12


def test_kept_set_maximises_the_score_sum():
    rng = np.random.default_rng(11)
    lens, block, H, X, topk = [96, 40], 8, 2, 5, 4
    cu = np.concatenate([[0], np.cumsum(lens)])
    qi = rng.standard_normal((sum(lens), H, X))
    ki = rng.standard_normal((sum(lens), H, X))
    sel = O.index_select(qi, ki, cu, block, topk)
    layout, scores = O.index_scores(qi, ki, cu, block)
    for d in range(len(lens)):
        S = scores[d][0]
        for h in range(H):
            for c in range(int(layout.nchunks[d])):
                diag = (8 * c) // block
                m = min(topk - 1, diag)
                best = max((sum(S[h, c, list(s)]) for s in itertools.combinations(range(diag), m)),
                           default=0.0)
                row = [b for b in sel[h, layout.chunk_off[d] + c] if b >= 0 and b != diag]
                assert len(row) == m
                assert abs(sum(S[h, c, row]) - best) < 1e-9


def test_structure_and_invariances():
    rng = np.random.default_rng(13)
    lens, block, H, X, topk = [900, 130, 8], 64, 2, 16, 6
    cu = np.concatenate([[0], np.cumsum(lens)])
    qi = rng.standard_normal((sum(lens), H, X))
    ki = rng.standard_normal((sum(lens), H, X))
    sel = O.index_select(qi, ki, cu, block, topk)
    layout = O.DocLayout(cu, block)
    for h in range(H):
        for g in range(layout.C):
            d, c = layout.chunk_local(g)
            diag = (8 * c) // block
            row = [int(b) for b in sel[h, g] if b >= 0]
            assert diag in row and row == sorted(set(row)) and max(row) == diag
            assert len(row) == min(topk, diag + 1)
            assert np.all(sel[h, g, len(row):] == -1)
    # shuffle the tokens inside every key block: block means are unchanged
    ki2 = ki.copy()
    for d, n in enumerate(lens):
        for b in range(int(layout.nblocks[d])):
            lo, hi = cu[d] + b * block, cu[d] + min((b + 1) * block, n)
            ki2[lo:hi] = ki[lo:hi][rng.permutation(hi - lo)]
    np.testing.assert_array_equal(O.index_select(qi, ki2, cu, block, topk), sel)
    np.testing.assert_array_equal(O.index_select(3.5 * qi, ki, cu, block, topk), sel)
