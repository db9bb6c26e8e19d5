"""Pins of the oracle's batched evaluations (chunk_rows, backward_batched,
key_block_grads), which the full-size parity tests use for the hot key
blocks: against torch's own scaled_dot_product_attention (fp64, CPU) and its
autograd under the brute-force mask of the definition, with ragged
documents, junk selection slots, chunks that select nothing, both key block
sizes and batches that split every group (CPU)."""
import numpy as np
import pytest

from oracle import msa_oracle as O
from test_oracle_pins import _brute_mask, _rand_problem, _random_sel, _sdpa_reference


CASES = [([96, 37, 64], 16, 16, 2, 3, True), ([200, 9, 131], 64, 32, 1, 2, False),
         ([300, 77], 128, 16, 2, 2, True)]


@pytest.mark.parametrize("lens,block,d,hkv,topk,junk", CASES)
def test_batched_evaluations_are_masked_sdpa(lens, block, d, hkv, topk, junk):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    layout = O.DocLayout(cu, block)
    q, k, v, do = _rand_problem(lens, hkv, d, block, seed=29)
    sel = _random_sel(layout, hkv, topk, seed=8, with_junk=junk)
    sel[:, 3, :] = -1                                   # a chunk that selects nothing
    sel_clean, _ = O.clean_selection(sel, layout)
    scale = d ** -0.5

    def mask_fn(doc):
        return np.repeat(np.stack([_brute_mask(layout, sel, i, doc) for i in range(hkv)]), 16, axis=0)

    out, lse, dq, dk, dv = _sdpa_reference(q, k, v, do, layout, scale, mask_fn)
    # rows that see no key: SDPA under an all-false mask gives NaN; the
    # definition gives O = 0 and LSE = -inf there
    empty = ~np.isfinite(lse)
    out[empty] = 0.0
    dq[empty] = 0.0
    for batch in (1, 3, 32):
        bq, bk, bv, bo, bl = O.backward_batched(q, k, v, do, cu, sel_clean, block, scale, batch=batch)
        np.testing.assert_allclose(bo, out, atol=1e-12, rtol=0)
        np.testing.assert_array_equal(np.isneginf(bl), empty)
        np.testing.assert_allclose(bl[~empty], lse[~empty], atol=1e-12, rtol=0)
        np.testing.assert_allclose(bq, dq, atol=1e-11, rtol=0)
        np.testing.assert_allclose(bk, dk, atol=1e-11, rtol=0)
        np.testing.assert_allclose(bv, dv, atol=1e-11, rtol=0)
    chunks = [(i, g) for g in range(layout.C - 1, -1, -2) for i in range(hkv)]
    for tq, heads, o_, l_, q_ in O.chunk_rows(q, k, v, do, cu, sel_clean, block, scale, chunks, batch=4):
        np.testing.assert_allclose(o_, out[np.ix_(tq, heads)], atol=1e-12, rtol=0)
        np.testing.assert_allclose(q_, dq[np.ix_(tq, heads)], atol=1e-11, rtol=0)
        np.testing.assert_array_equal(np.isneginf(l_), empty[np.ix_(tq, heads)])
    for i in range(hkv):
        for r in range(layout.R):
            toks, gk, gv = O.key_block_grads(q, k, v, do, cu, sel_clean, block, scale, i, r, batch=2)
            np.testing.assert_allclose(gk, dk[toks, i], atol=1e-11, rtol=0)
            np.testing.assert_allclose(gv, dv[toks, i], atol=1e-11, rtol=0)
