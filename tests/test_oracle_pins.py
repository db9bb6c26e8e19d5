"""Pins of the fp64 oracle against things other than itself.

* torch's own scaled_dot_product_attention (fp64, CPU) and its autograd:
  with every causal block selected the method is dense causal attention
  (msa_backward_sm100 page: each query sees its chunk's selected key blocks,
  causally); with a sparse selection it is SDPA under the boolean mask that a
  brute-force loop builds from the definition.
* central finite differences of L = sum(O * dO) for the analytic backward.
* closed forms: the first query of a document sees only key 0, so O = v_0
  and LSE = scale q_0.k_0; v = 1 gives O = 1; equal keys give dQ = 0.
* the selection set semantics (duplicates / out-of-range / non-causal ids).
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(lens, hkv, d, block, seed, bf16=True):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    hq = 16 * hkv
    mk = (lambda *s: torch.from_numpy(rng.standard_normal(s)).to(torch.bfloat16)) if bf16 else \
        (lambda *s: rng.standard_normal(s))
    return mk(T, hq, d), mk(T, hkv, d), mk(T, hkv, d), mk(T, hq, d)


def _all_causal_sel(layout, hkv):
    k = int(layout.nblocks.max())
    sel = np.full((hkv, layout.C, k), -1, dtype=np.int32)
    for g in range(layout.C):
        d, c = layout.chunk_local(g)
        last = min(c * layout.chunk + layout.chunk - 1, int(layout.lens[d]) - 1)
        nb = last // layout.block + 1
        sel[:, g, :nb] = np.arange(nb)
    return sel


def _random_sel(layout, hkv, k, seed, with_junk=False):
    """Random causal selection, diagonal included; optionally junk slots."""
    rng = np.random.default_rng(seed)
    sel = np.full((hkv, layout.C, k), -1, dtype=np.int32)
    for i in range(hkv):
        for g in range(layout.C):
            d, c = layout.chunk_local(g)
            diag = (c * layout.chunk) // layout.block
            extra = rng.permutation(diag)[: max(0, k - 1)]
            row = list(extra) + [diag]
            if with_junk and k >= 3:
                row = row[: k - 2] + [diag, int(layout.nblocks[d]) + 3]  # dup + out of range
            sel[i, g, : len(row)] = row
            rng.shuffle(sel[i, g])
    return sel


def _brute_mask(layout, sel, i, d):
    """M[p, j] straight from the definition, one (p, j) at a time."""
    n = int(layout.lens[d])
    g0 = int(layout.chunk_off[d])
    M = np.zeros((n, n), dtype=bool)
    for p in range(n):
        chosen = set(int(b) for b in sel[i, g0 + p // layout.chunk]
                     if 0 <= b < layout.nblocks[d] and b * layout.block <= p)
        for j in range(p + 1):
            M[p, j] = (j // layout.block) in chosen
    return M


def _sdpa_reference(q, k, v, do, layout, scale, mask_fn):
    """torch SDPA (fp64) per document with GQA by repeat; autograd backward."""
    q64, k64, v64, do64 = (torch.from_numpy(O.f64(x)) for x in (q, k, v, do))
    T, hq, D = q64.shape
    hkv = k64.shape[1]
    out = torch.zeros_like(q64)
    lse = torch.full((T, hq), float("nan"), dtype=torch.float64)
    dq = torch.zeros_like(q64)
    dk = torch.zeros_like(k64)
    dv = torch.zeros_like(v64)
    for d in range(layout.docs):
        a, b = int(layout.cu[d]), int(layout.cu[d + 1])
        qd = q64[a:b].transpose(0, 1).clone().requires_grad_(True)          # [Hq, n, D]
        kd = k64[a:b].transpose(0, 1).clone().requires_grad_(True)          # [Hkv, n, D]
        vd = v64[a:b].transpose(0, 1).clone().requires_grad_(True)
        kr = kd.repeat_interleave(16, dim=0)
        vr = vd.repeat_interleave(16, dim=0)
        mask = mask_fn(d)                                                   # [Hq, n, n] bool or None
        if mask is None:
            o = torch.nn.functional.scaled_dot_product_attention(
                qd[None], kr[None], vr[None], is_causal=True, scale=scale)[0]
            m = torch.ones(b - a, b - a, dtype=torch.bool).tril()[None].expand(hq, -1, -1)
        else:
            m = torch.from_numpy(mask)
            o = torch.nn.functional.scaled_dot_product_attention(
                qd[None], kr[None], vr[None], attn_mask=m[None], scale=scale)[0]
        s = scale * (qd.detach() @ kr.detach().transpose(1, 2))
        lse[a:b] = torch.logsumexp(s.masked_fill(~m, float("-inf")), dim=-1).transpose(0, 1)
        o.backward(do64[a:b].transpose(0, 1))
        out[a:b] = o.detach().transpose(0, 1)
        dq[a:b] = qd.grad.transpose(0, 1)
        dk[a:b] = kd.grad.transpose(0, 1)
        dv[a:b] = vd.grad.transpose(0, 1)
    return out.numpy(), lse.numpy(), dq.numpy(), dk.numpy(), dv.numpy()


@pytest.mark.parametrize("lens,block,d", [([64], 16, 16), ([40, 16, 72], 16, 8), ([128], 64, 32),
                                          ([200, 77], 128, 16)])
def test_all_blocks_selected_is_dense_causal_attention(lens, block, d):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    layout = O.DocLayout(cu, block)
    hkv = 2
    q, k, v, do = _rand_problem(lens, hkv, d, block, seed=7)
    sel = _all_causal_sel(layout, hkv)
    sel_clean, dropped = O.clean_selection(sel, layout)
    assert dropped == 0
    scale = d ** -0.5
    ref = _sdpa_reference(q, k, v, do, layout, scale, lambda doc: None)
    for mode in ("dense", "gathered"):
        bw = O.backward_dense if mode == "dense" else O.backward_gathered
        dq, dk, dv, delta, out, lse = bw(q, k, v, do, cu, sel_clean, block, scale)
        np.testing.assert_allclose(out, ref[0], atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse, ref[1], atol=1e-12, rtol=0)
        np.testing.assert_allclose(dq, ref[2], atol=1e-11, rtol=0)
        np.testing.assert_allclose(dk, ref[3], atol=1e-11, rtol=0)
        np.testing.assert_allclose(dv, ref[4], atol=1e-11, rtol=0)
        fo, fl = (O.forward_dense if mode == "dense" else O.forward_gathered)(
            q, k, v, cu, sel_clean, block, scale)
        np.testing.assert_allclose(fo, ref[0], atol=1e-12, rtol=0)
        np.testing.assert_allclose(fl, ref[1], atol=1e-12, rtol=0)


@pytest.mark.parametrize("junk", [False, True])
def test_sparse_selection_is_masked_sdpa(junk):
    lens, block, d, hkv, topk = [96, 37, 64], 16, 16, 2, 3
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    layout = O.DocLayout(cu, block)
    q, k, v, do = _rand_problem(lens, hkv, d, block, seed=11)
    sel = _random_sel(layout, hkv, topk, seed=5, with_junk=junk)
    sel_clean, dropped = O.clean_selection(sel, layout)
    assert (dropped > 0) == junk
    scale = d ** -0.5

    def mask_fn(doc):
        per_kv = [_brute_mask(layout, sel, i, doc) for i in range(hkv)]
        return np.repeat(np.stack(per_kv), 16, axis=0)

    ref = _sdpa_reference(q, k, v, do, layout, scale, mask_fn)
    for bw in (O.backward_dense, O.backward_gathered):
        dq, dk, dv, delta, out, lse = bw(q, k, v, do, cu, sel_clean, block, scale)
        np.testing.assert_allclose(out, ref[0], atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse, ref[1], atol=1e-12, rtol=0)
        np.testing.assert_allclose(dq, ref[2], atol=1e-11, rtol=0)
        np.testing.assert_allclose(dk, ref[3], atol=1e-11, rtol=0)
        np.testing.assert_allclose(dv, ref[4], atol=1e-11, rtol=0)
    # the raw selection (junk included) gives exactly the clean selection's result
    raw = O.forward_gathered(q, k, v, cu, O.clean_selection(sel, layout)[0], block, scale)
    np.testing.assert_array_equal(raw[0], O.forward_gathered(q, k, v, cu, sel_clean, block, scale)[0])


def test_mask_matches_brute_force():
    lens, block = [50, 8, 64], 16
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    layout = O.DocLayout(cu, block)
    sel = _random_sel(layout, 2, 3, seed=3, with_junk=True)
    sel_clean, _ = O.clean_selection(sel, layout)
    for i in range(2):
        for d in range(layout.docs):
            np.testing.assert_array_equal(O.visibility_mask(layout, sel_clean, i, d),
                                          _brute_mask(layout, sel, i, d))


def test_backward_matches_finite_differences():
    lens, block, d, hkv, topk = [24, 17], 8, 4, 1, 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    layout = O.DocLayout(cu, block)
    q, k, v, do = _rand_problem(lens, hkv, d, block, seed=19, bf16=False)
    sel_clean, _ = O.clean_selection(_random_sel(layout, hkv, topk, seed=2), layout)
    scale = 0.37
    dq, dk, dv, *_ = O.backward_gathered(q, k, v, do, cu, sel_clean, block, scale)

    def loss(qq, kk, vv):
        out, _ = O.forward_dense(qq, kk, vv, cu, sel_clean, block, scale)
        return float((out * do).sum())

    rng = np.random.default_rng(0)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        idx = [tuple(rng.integers(0, s) for s in x.shape) for _ in range(12)]
        for ix in idx:
            xp, xm = x.copy(), x.copy()
            xp[ix] += h
            xm[ix] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (loss(**{"qq": args_p["q"], "kk": args_p["k"], "vv": args_p["v"]})
                  - loss(**{"qq": args_m["q"], "kk": args_m["k"], "vv": args_m["v"]})) / (2 * h)
            assert abs(fd - g[ix]) <= 1e-6 * max(1.0, abs(g[ix])), (name, ix, fd, g[ix])


def test_closed_forms():
    lens, block, d, hkv = [64, 40], 16, 16, 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    layout = O.DocLayout(cu, block)
    q, k, v, do = _rand_problem(lens, hkv, d, block, seed=23)
    sel_clean, _ = O.clean_selection(_random_sel(layout, hkv, 2, seed=1), layout)
    scale = d ** -0.5
    out, lse = O.forward_gathered(q, k, v, cu, sel_clean, block, scale)
    q64, k64, v64 = O.f64(q), O.f64(k), O.f64(v)
    for doc in range(layout.docs):
        t0 = int(cu[doc])
        for h in range(16 * hkv):
            np.testing.assert_array_equal(out[t0, h], v64[t0, h // 16])
            assert lse[t0, h] == pytest.approx(scale * q64[t0, h] @ k64[t0, h // 16], abs=1e-13)
    # v = 1 everywhere -> every output row is exactly the all-ones vector (rows of P sum to 1)
    ones = np.ones_like(v64)
    out1, _ = O.forward_gathered(q64, k64, ones, cu, sel_clean, block, scale)
    np.testing.assert_allclose(out1, 1.0, atol=1e-13)
    # LSE is at least the largest visible score (log of a sum of positive terms)
    s_max = np.full(lse.shape, -np.inf)
    for doc in range(layout.docs):
        a, b = int(cu[doc]), int(cu[doc + 1])
        for i in range(hkv):
            M = O.visibility_mask(layout, sel_clean, i, doc)
            for h in range(16 * i, 16 * i + 16):
                S = np.where(M, scale * q64[a:b, h] @ k64[a:b, i].T, -np.inf)
                s_max[a:b, h] = S.max(axis=1)
    assert np.all(lse >= s_max - 1e-12)
    # identical keys -> softmax is flat in q, so dQ = scale * sum_j dS_pj k = 0
    kc = np.broadcast_to(k64[:1], k64.shape).copy()
    dq, *_ = O.backward_gathered(q64, kc, v64, O.f64(do), cu, sel_clean, block, scale)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)


def test_empty_selection_gives_zero_output_and_neg_inf_lse():
    lens, block, d = [32], 16, 8
    cu = np.array([0, 32], dtype=np.int32)
    layout = O.DocLayout(cu, block)
    q, k, v, do = _rand_problem(lens, 1, d, block, seed=3)
    sel = np.full((1, layout.C, 2), -1, dtype=np.int32)
    sel[0, 0, 0] = 0                               # only chunk 0 selects anything
    sel_clean, _ = O.clean_selection(sel, layout)
    for bw in (O.backward_dense, O.backward_gathered):
        dq, dk, dv, delta, out, lse = bw(q, k, v, do, cu, sel_clean, block, 0.5)
        assert np.all(np.isneginf(lse[8:])) and np.all(out[8:] == 0) and np.all(dq[8:] == 0)
        assert np.all(np.isfinite(lse[:8]))
        assert np.all(dk[8:] == 0) and np.all(dv[8:] == 0)


def test_golden_constants_match_oracle_defaults():
    with open(os.path.join(GOLDEN, "schedule_constants.json")) as f:
        g = json.load(f)
    assert O.QUERY_CHUNK == g["QUERY_CHUNK"]
    assert O.ROWS_PER_CTA_SMALL == g["ROWS_PER_CTA_SMALL"]
    assert O.ROWS_PER_CTA_LARGE == g["ROWS_PER_CTA_LARGE"]
    assert O.ROWS_PER_CTA_SWITCH == g["ROWS_PER_CTA_SWITCH"]
    assert O.Q_HEADS_PER_INDEX == g["NUM_Q_HEADS"] // g["NUM_INDEX_HEADS"]
    assert g["TILE_M"] == O.QUERY_CHUNK * O.Q_HEADS_PER_INDEX
