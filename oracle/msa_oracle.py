"""fp64 CPU oracle for MSA main attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never calls it and shares no code with it.

What it computes (sources are the four NeMo AutoModel API pages on the
MiniMax-M3 MSA kernels):

* Attention (msa_backward_sm100 page, module description and ``run_backward``;
  msa_schedule page, ``QUERY_CHUNK`` and ``SOFTMAX_SCALE``).  Query head h of
  a document belongs to index/KV head i = h // 16.  A query at
  document-local position p lies in chunk c = p // 8 and sees the keys
        A(p) = { j : j <= p, j < len_d, j // B in Sel[i, c] }.
  With s_j = scale * q_p . k_j it outputs LSE_p = ln sum_{j in A} exp(s_j),
  P_pj = exp(s_j - LSE_p) and O_p = sum_j P_pj v_j.  The backward takes dO
  and returns dV_j = sum_{p,h} P_pj dO_p, dK_j = scale sum_{p,h} dS_pj q_p,
  dQ_p = scale sum_j dS_pj k_j with dS_pj = P_pj (dO_p . v_j - D_p) and
  D_p = dO_p . O_p (the backward preprocess, kernels page submodule list).
  This is the exact result the method reaches; only the summation order of
  an implementation differs.
* Selection semantics: Sel[i, c] is a *set* of document-local block ids.
  Slots holding -1 are empty; ids outside the document, ids of blocks that
  start after the chunk's last query, and repeated ids add no key to A(p),
  so they are dropped and counted (``clean_selection``).
* k2q CSR (msa_schedule page, ``MSABackwardSchedule.row_ptr`` and
  ``q_indices``): per index head one CSR row per key block, rows ordered by
  (document, block); the entries of a row are the document-local first query
  positions (8 c) of the chunks that selected the block, ascending.
* Walk rule and task table (msa_schedule page, ``rows_per_cta``,
  ``chunk_map``, ``grid_launch_bound``, ``ROWS_PER_CTA_*``, and the
  ``scheduler_metadata`` column order).
* Index scorer and top-k block selection (``index_select``).  The pages name
  the scorer (msa_bindings page: MSAKernels lists ``fmha_sm100``, the
  scorer, beside the planner) and its sizes (msa_schedule page, module data:
  ``INDEX_DIM``, ``NUM_INDEX_HEADS``, ``TOPK_BLOCKS``) but not its scoring
  function; the reading taken here is the plainest one that produces the
  selection the attention consumes: per index head, the score of key block
  b for chunk c is  (sum of the chunk's index queries) . (mean of the
  block's index keys); the chunk keeps its own (diagonal) block plus the
  topk - 1 highest-scoring earlier blocks of its document, ties to the
  smaller block id, fewer when fewer exist; ids ascending, -1 padding.

Evaluation modes of the attention: literal dense (T x T masks per document
and head), gathered (each chunk over its selected keys only; masked terms are
exactly 0, so the result is the same), and the batched gathered functions
(``chunk_rows``, ``backward_batched``, ``key_block_grads``), which evaluate
the same per-chunk formulas several chunks per library call so that the
full-size workloads' hot key blocks can be checked in seconds.

Floating point is fp64 throughout; bf16 inputs are widened exactly.
"""
from __future__ import annotations

import numpy as np

# msa_schedule page, module data.
QUERY_CHUNK = 8
ROWS_PER_CTA_SMALL = 4
ROWS_PER_CTA_LARGE = 64
ROWS_PER_CTA_SWITCH = 2400
Q_HEADS_PER_INDEX = 16          # msa_backward_sm100 page, MAIN_HEADS_PER_INDEX = 64 // 4
TASK_COLUMNS = ("index_head", "row_linear", "q_begin", "q_count",
                "document_ordinal", "document_local_kblock")


def f64(x) -> np.ndarray:
    """Widen a bf16/fp32 torch tensor or array to fp64 numpy (exact)."""
    if isinstance(x, np.ndarray):   # numpy input: no torch import needed
        return np.asarray(x, dtype=np.float64)
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


class DocLayout:
    """Document geometry from cu_seqlens (msa_schedule page, ``cu_seqlens``)."""

    def __init__(self, cu_seqlens, block: int, chunk: int = QUERY_CHUNK):
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        self.cu = cu
        self.lens = np.diff(cu)
        self.docs = len(self.lens)
        self.block = int(block)
        self.chunk = int(chunk)
        self.nchunks = -(-self.lens // self.chunk)
        self.nblocks = -(-self.lens // self.block)
        self.chunk_off = np.concatenate([[0], np.cumsum(self.nchunks)]).astype(np.int64)
        self.blk_off = np.concatenate([[0], np.cumsum(self.nblocks)]).astype(np.int64)
        self.C = int(self.chunk_off[-1])
        self.R = int(self.blk_off[-1])
        # document of every global chunk / every global key-block row
        self.chunk_doc = np.repeat(np.arange(self.docs), self.nchunks)
        self.row_doc = np.repeat(np.arange(self.docs), self.nblocks)

    def chunk_local(self, g: int) -> tuple[int, int]:
        d = int(self.chunk_doc[g])
        return d, int(g - self.chunk_off[d])


# ---------------------------------------------------------------------------
# Selection, CSR, walk, tasks
# ---------------------------------------------------------------------------

def clean_selection(sel: np.ndarray, layout: DocLayout) -> tuple[np.ndarray, int]:
    """Keep each id that adds keys to A(p), once, in its slot; -1 elsewhere.

    Returns (sel_clean [Hkv, C, k] int32, number of dropped non-empty slots).
    An id b is kept for chunk c of document d when 0 <= b < ceil(len_d / B),
    b * B <= the chunk's last query position, and no earlier slot of the same
    chunk kept b.
    """
    sel = np.asarray(sel, dtype=np.int64)
    hkv, C, k = sel.shape
    assert C == layout.C
    d = layout.chunk_doc
    c_local = np.arange(C) - layout.chunk_off[d]
    last_q = np.minimum(c_local * layout.chunk + layout.chunk - 1, layout.lens[d] - 1)
    nb = layout.nblocks[d]
    valid = (sel >= 0) & (sel < nb[None, :, None]) & (sel * layout.block <= last_q[None, :, None])
    out = np.where(valid, sel, -1)
    for s in range(1, k):              # drop repeats of an id kept in an earlier slot
        dup = np.zeros((hkv, C), dtype=bool)
        for s2 in range(s):
            dup |= (out[:, :, s2] == out[:, :, s]) & (out[:, :, s] >= 0)
        out[:, :, s] = np.where(dup, -1, out[:, :, s])
    dropped = int(np.count_nonzero((sel != -1) & (out == -1)))
    return out.astype(np.int32), dropped


def build_k2q_csr(sel_clean: np.ndarray, layout: DocLayout):
    """Invert the per-chunk selection into key-block -> query buckets.

    Returns (row_ptr [Hkv, R+1] int32, q_idx [Hkv, C*k] int32, padded with -1).
    Row r = blk_off[d] + b; entries are 8*c (document-local chunk start),
    ascending within a row.  A stable sort by (row, chunk) is the only step.
    """
    hkv, C, k = sel_clean.shape
    R = layout.R
    row_ptr = np.zeros((hkv, R + 1), dtype=np.int32)
    q_idx = np.full((hkv, C * k), -1, dtype=np.int32)
    d = layout.chunk_doc
    c_local = np.arange(C) - layout.chunk_off[d]
    for i in range(hkv):
        g, s = np.nonzero(sel_clean[i] >= 0)
        rows = layout.blk_off[d[g]] + sel_clean[i, g, s]
        order = np.lexsort((g, rows))          # by row, then by chunk
        counts = np.bincount(rows, minlength=R)
        row_ptr[i, 1:] = np.cumsum(counts)
        q_idx[i, : len(order)] = (c_local[g] * layout.chunk)[order]
    return row_ptr, q_idx


def rows_per_cta(num_rows: int) -> int:
    """Walk length (msa_schedule page, ``rows_per_cta``): the small walk below
    ROWS_PER_CTA_SWITCH rows, the large one from there on."""
    return ROWS_PER_CTA_SMALL if num_rows < ROWS_PER_CTA_SWITCH else ROWS_PER_CTA_LARGE


def chunk_map(num_rows: int, rpc: int, num_sms: int) -> tuple[int, int, int]:
    """(num_full_ctas, tail_rows, grid_ctas) (msa_schedule page, ``chunk_map``).

    Full walks take ``rpc`` rows each; the tail rows left over are spread over
    at most one extra walk per SM (min(tail_rows, num_sms) walks), so that
    grid_ctas <= num_rows // rpc + num_sms as the page states.
    """
    full = num_rows // rpc
    tail = num_rows - full * rpc
    return full, tail, full + min(tail, num_sms)


def walk_bounds(num_rows: int, rpc: int, num_sms: int, cta: int) -> tuple[int, int]:
    """Rows [lo, hi) walked by workgroup ``cta``: full walks first, then the
    tail split as evenly as possible, earlier tail walks taking one more row."""
    full, tail, grid = chunk_map(num_rows, rpc, num_sms)
    if cta < full:
        return cta * rpc, (cta + 1) * rpc
    t = cta - full
    nt = grid - full
    assert 0 <= t < nt
    base, extra = divmod(tail, nt)
    lo = full * rpc + t * base + min(t, extra)
    return lo, lo + base + (1 if t < extra else 0)


def grid_launch_bound(capacity: int, num_sms: int) -> int:
    """Grid size that covers every count in [0, capacity] (msa_schedule page,
    ``grid_launch_bound``): full walks plus at most one tail walk per SM, the
    larger of the small-walk and the large-walk regime."""
    small = min(capacity, ROWS_PER_CTA_SWITCH - 1) // ROWS_PER_CTA_SMALL
    large = capacity // ROWS_PER_CTA_LARGE if capacity >= ROWS_PER_CTA_SWITCH else 0
    return max(small, large) + num_sms


def build_tasks(row_ptr: np.ndarray, q_idx: np.ndarray, layout: DocLayout, num_sms: int):
    """Task table in CSR order, heads first (msa_schedule page,
    ``scheduler_metadata`` columns), and the walk descriptor.

    Returns (task_meta [Hkv*C*k, 6] int32 padded with -1, desc int32 [8]) with
    desc = (N, rows_per_cta, num_full, tail_rows, tail_ctas, grid_ctas, capacity, 0).
    """
    hkv = row_ptr.shape[0]
    cap = q_idx.shape[1] * hkv
    meta = np.full((cap, 6), -1, dtype=np.int32)
    t = 0
    for i in range(hkv):
        n_i = int(row_ptr[i, -1])
        counts = np.diff(row_ptr[i].astype(np.int64))
        rows = np.repeat(np.arange(layout.R), counts)
        docs = layout.row_doc[rows]
        qb = q_idx[i, :n_i].astype(np.int64)
        meta[t:t + n_i, 0] = i
        meta[t:t + n_i, 1] = rows
        meta[t:t + n_i, 2] = qb
        meta[t:t + n_i, 3] = np.minimum(layout.chunk, layout.lens[docs] - qb)
        meta[t:t + n_i, 4] = docs
        meta[t:t + n_i, 5] = rows - layout.blk_off[docs]
        t += n_i
    n = t
    rpc = rows_per_cta(n)
    full, tail, grid = chunk_map(n, rpc, num_sms)
    desc = np.array([n, rpc, full, tail, grid - full, grid, cap, 0], dtype=np.int32)
    return meta, desc


def build_schedule(sel: np.ndarray, cu_seqlens, block: int, num_sms: int):
    """Everything the schedule build produces, as a dict of int arrays."""
    layout = DocLayout(cu_seqlens, block)
    sel_clean, dropped = clean_selection(sel, layout)
    row_ptr, q_idx = build_k2q_csr(sel_clean, layout)
    meta, desc = build_tasks(row_ptr, q_idx, layout, num_sms)
    return dict(layout=layout, sel_clean=sel_clean, dropped=dropped, row_ptr=row_ptr,
                q_idx=q_idx, task_meta=meta, desc=desc)


# ---------------------------------------------------------------------------
# Attention, literal dense mode (T x T masks per document and head)
# ---------------------------------------------------------------------------

def visibility_mask(layout: DocLayout, sel_clean: np.ndarray, i: int, d: int) -> np.ndarray:
    """M[p, j] = (j <= p) and (j // B in Sel[i, p // 8]) for one document."""
    n = int(layout.lens[d])
    chosen = np.zeros((int(layout.nchunks[d]), max(int(layout.nblocks[d]), 1)), dtype=bool)
    g0 = int(layout.chunk_off[d])
    for c in range(int(layout.nchunks[d])):
        for b in sel_clean[i, g0 + c]:
            if b >= 0:
                chosen[c, b] = True
    p = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return (j <= p) & chosen[p // layout.chunk, j // layout.block]


def forward_dense(q, k, v, cu_seqlens, sel_clean, block: int, scale: float):
    """O [T, Hq, D] and LSE [T, Hq] (natural log; -inf and O = 0 for an empty A(p))."""
    q, k, v = f64(q), f64(k), f64(v)
    layout = DocLayout(cu_seqlens, block)
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    out = np.zeros_like(q)
    lse = np.full((T, Hq), -np.inf)
    for d in range(layout.docs):
        a, b_ = int(layout.cu[d]), int(layout.cu[d + 1])
        if b_ == a:
            continue
        for i in range(k.shape[1]):
            M = visibility_mask(layout, sel_clean, i, d)
            any_row = M.any(axis=1)
            K, V = k[a:b_, i], v[a:b_, i]
            for h in range(G * i, G * (i + 1)):
                S = scale * (q[a:b_, h] @ K.T)
                S = np.where(M, S, -np.inf)
                m = np.where(any_row, S.max(axis=1), 0.0)
                with np.errstate(divide="ignore"):
                    l_ = np.log(np.exp(S - m[:, None]).sum(axis=1)) + m
                l_ = np.where(any_row, l_, -np.inf)
                P = np.where(M, np.exp(S - np.where(any_row, l_, 0.0)[:, None]), 0.0)
                out[a:b_, h] = P @ V
                lse[a:b_, h] = l_
    return out, lse


def backward_dense(q, k, v, do, cu_seqlens, sel_clean, block: int, scale: float):
    """(dq, dk, dv, delta, out, lse) by the analytic backward, dense masks."""
    q, k, v, do = f64(q), f64(k), f64(v), f64(do)
    out, lse = forward_dense(q, k, v, cu_seqlens, sel_clean, block, scale)
    layout = DocLayout(cu_seqlens, block)
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    delta = (do * out).sum(axis=-1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for d in range(layout.docs):
        a, b_ = int(layout.cu[d]), int(layout.cu[d + 1])
        if b_ == a:
            continue
        for i in range(k.shape[1]):
            M = visibility_mask(layout, sel_clean, i, d)
            K, V = k[a:b_, i], v[a:b_, i]
            for h in range(G * i, G * (i + 1)):
                S = scale * (q[a:b_, h] @ K.T)
                L = lse[a:b_, h]
                P = np.where(M, np.exp(S - np.where(np.isfinite(L), L, 0.0)[:, None]), 0.0)
                dP = do[a:b_, h] @ V.T
                dS = P * (dP - delta[a:b_, h][:, None])
                dq[a:b_, h] = scale * (dS @ K)
                dk[a:b_, i] += scale * (dS.T @ q[a:b_, h])
                dv[a:b_, i] += P.T @ do[a:b_, h]
    return dq, dk, dv, delta, out, lse


# ---------------------------------------------------------------------------
# Attention, block-gathered mode (only the selected keys of each chunk)
# ---------------------------------------------------------------------------

def chunk_keys(layout: DocLayout, sel_clean: np.ndarray, i: int, g: int):
    """(doc, doc-local query positions, doc-local key positions) of chunk g."""
    d, c = layout.chunk_local(g)
    n = int(layout.lens[d])
    blocks = sorted({int(b) for b in sel_clean[i, g] if b >= 0})
    keys = [np.arange(b * layout.block, min((b + 1) * layout.block, n)) for b in blocks]
    keys = np.concatenate(keys) if keys else np.zeros(0, dtype=np.int64)
    qpos = np.arange(c * layout.chunk, min((c + 1) * layout.chunk, n))
    return d, qpos, keys


def _take(x, tokens, heads) -> np.ndarray:
    """x[tokens][:, heads] as fp64 numpy, for numpy arrays or torch tensors."""
    if isinstance(x, np.ndarray):
        return np.asarray(x[np.asarray(tokens)][:, np.asarray(heads)], dtype=np.float64)
    import torch
    t = torch.as_tensor(np.asarray(tokens, dtype=np.int64))
    h = torch.as_tensor(np.asarray(heads, dtype=np.int64))
    return f64(x.index_select(0, t).index_select(1, h))


def _chunk_probs(qh, K, qpos, keys, scale):
    """S [nq, G, nk] -> (P, LSE) for one chunk and one head group."""
    nq, G, D = qh.shape
    S = scale * (qh.reshape(nq * G, D) @ K.T).reshape(nq, G, -1)
    M = (keys[None, :] <= qpos[:, None])[:, None, :]
    S = np.where(M, S, -np.inf)
    any_row = M.any(axis=2)
    m = np.where(any_row, S.max(axis=2, initial=-np.inf), 0.0)
    with np.errstate(divide="ignore"):
        lse = np.log(np.exp(S - m[..., None]).sum(axis=2)) + m
    lse = np.where(any_row, lse, -np.inf)
    P = np.where(M, np.exp(S - np.where(any_row, lse, 0.0)[..., None]), 0.0)
    return P, lse


def forward_chunk(q, k, v, layout, sel_clean, i, g, scale):
    """Oracle rows of one (index head, chunk): (tokens, heads, O, LSE)."""
    d, qpos, keys = chunk_keys(layout, sel_clean, i, g)
    G = q.shape[1] // k.shape[1]
    tq = int(layout.cu[d]) + qpos
    tk = int(layout.cu[d]) + keys
    heads = np.arange(G * i, G * (i + 1))
    qh = _take(q, tq, heads)
    K = _take(k, tk, [i])[:, 0]
    V = _take(v, tk, [i])[:, 0]
    P, lse = _chunk_probs(qh, K, qpos, keys, scale)
    nq = len(qpos)
    O = (P.reshape(nq * G, -1) @ V).reshape(nq, G, -1)
    return tq, heads, O, lse


def forward_gathered(q, k, v, cu_seqlens, sel_clean, block: int, scale: float,
                     chunks=None):
    """O and LSE over the selected keys only; ``chunks`` = iterable of (i, g)
    restricts the work (rows outside stay O = 0, LSE = nan)."""
    q, k, v = f64(q), f64(k), f64(v)
    layout = DocLayout(cu_seqlens, block)
    T, Hq, D = q.shape
    out = np.zeros_like(q)
    lse = np.full((T, Hq), np.nan)
    if chunks is None:
        chunks = [(i, g) for i in range(k.shape[1]) for g in range(layout.C)]
    for i, g in chunks:
        tq, heads, O, L = forward_chunk(q, k, v, layout, sel_clean, i, g, scale)
        out[np.ix_(tq, heads)] = O
        lse[np.ix_(tq, heads)] = L
    return out, lse


def backward_gathered(q, k, v, do, cu_seqlens, sel_clean, block: int, scale: float,
                      chunks=None):
    """(dq, dk, dv, delta, out, lse) over the selected keys only.  With
    ``chunks`` given, only those (i, g) contribute: dq rows of those chunks
    are complete, and dk/dv rows are complete for key blocks whose every
    selecting chunk is listed."""
    q, k, v, do = f64(q), f64(k), f64(v), f64(do)
    layout = DocLayout(cu_seqlens, block)
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    out = np.zeros_like(q)
    lse = np.full((T, Hq), np.nan)
    delta = np.full((T, Hq), np.nan)
    if chunks is None:
        chunks = [(i, g) for i in range(k.shape[1]) for g in range(layout.C)]
    for i, g in chunks:
        d, qpos, keys = chunk_keys(layout, sel_clean, i, g)
        tq = int(layout.cu[d]) + qpos
        tk = int(layout.cu[d]) + keys
        heads = np.arange(G * i, G * (i + 1))
        qh, doh = q[tq][:, heads], do[tq][:, heads]
        K, V = k[tk, i], v[tk, i]
        P, L = _chunk_probs(qh, K, qpos, keys, scale)
        nq = len(qpos)
        O = (P.reshape(nq * G, -1) @ V).reshape(nq, G, D)
        Dl = (doh * O).sum(axis=-1)
        dP = (doh.reshape(nq * G, D) @ V.T).reshape(nq, G, -1)
        dS = P * (dP - Dl[..., None])
        dq[np.ix_(tq, heads)] = scale * (dS.reshape(nq * G, -1) @ K).reshape(nq, G, D)
        if len(tk):
            dk[tk, i] += scale * (dS.reshape(nq * G, -1).T @ qh.reshape(nq * G, D))
            dv[tk, i] += P.reshape(nq * G, -1).T @ doh.reshape(nq * G, D)
        out[np.ix_(tq, heads)] = O
        lse[np.ix_(tq, heads)] = L
        delta[np.ix_(tq, heads)] = Dl
    return dq, dk, dv, delta, out, lse


def _chunk_batches(q, k, v, do, layout: DocLayout, sel_clean, chunks, batch: int):
    """Group the listed (index head, chunk) pairs by (index head, number of
    queries, number of selected keys) and yield, per group of at most
    ``batch`` chunks, fp64 torch tensors of their rows stacked along a batch
    axis: (members, i, Q [nb, nq*16, D], dO, K [nb, nk, D], V, ktok [nb, nk],
    vis [nb, nq*16, nk]); members are (position in ``chunks``, token indices
    of the queries).  vis is the causal visibility (key position <= query
    position) of each chunk's selected keys; row r = query r // 16, head
    r % 16 of the index head's group."""
    import torch
    G = Q_HEADS_PER_INDEX
    Dh = q.shape[2]
    qt, kt, vt, dot = (torch.as_tensor(x) for x in (q, k, v, do))
    groups: dict = {}
    for n, (i, g) in enumerate(chunks):
        d, qpos, keys = chunk_keys(layout, sel_clean, i, g)
        groups.setdefault((i, len(qpos), len(keys)), []).append((n, int(layout.cu[d]), qpos, keys))
    for (i, nq, nk), members in groups.items():
        for s0 in range(0, len(members), batch):
            part = members[s0:s0 + batch]
            nb = len(part)
            qtok = torch.as_tensor(np.stack([t0 + qp for _, t0, qp, _ in part]))
            ktok = torch.as_tensor(np.stack([t0 + ks for _, t0, _, ks in part]).reshape(nb, nk))
            Q = qt[qtok.reshape(-1), G * i:G * (i + 1)].double().reshape(nb, nq * G, Dh)
            dO = dot[qtok.reshape(-1), G * i:G * (i + 1)].double().reshape(nb, nq * G, Dh)
            K = kt[ktok.reshape(-1), i].double().reshape(nb, nk, Dh)
            V = vt[ktok.reshape(-1), i].double().reshape(nb, nk, Dh)
            qpos = torch.as_tensor(np.stack([qp for _, _, qp, _ in part]))
            kpos = torch.as_tensor(np.stack([ks for _, _, _, ks in part]).reshape(nb, nk))
            vis = (kpos[:, None, :] <= qpos[:, :, None])
            vis = vis[:, :, None, :].expand(nb, nq, G, nk).reshape(nb, nq * G, nk)
            yield [(n, t0 + qp) for n, t0, qp, _ in part], i, Q, dO, K, V, ktok, vis


def _softmax_rows(Q, K, V, vis, scale):
    """Per stacked chunk: s = scale Q K^T over the visible keys, LSE (-inf for
    a row that sees no key), P = exp(s - LSE) (0 off the visible set), O = P V."""
    import torch
    neg = torch.tensor(-np.inf, dtype=torch.float64)
    zero = torch.zeros((), dtype=torch.float64)
    any_row = vis.any(dim=2, keepdim=True)
    S = torch.where(vis, scale * torch.bmm(Q, K.transpose(1, 2)), neg)
    lse = torch.where(any_row, torch.logsumexp(S, dim=2, keepdim=True), neg)
    P = torch.where(vis, torch.exp(S - torch.where(any_row, lse, zero)), zero)
    return lse, P, torch.bmm(P, V)


def chunk_rows(q, k, v, do, cu_seqlens, sel_clean, block: int, scale: float, chunks, batch: int = 32):
    """O, LSE and dQ of the rows of the listed (index head, chunk) pairs, by
    the same formulas as ``backward_gathered`` (each chunk over all of its
    selected keys): LSE = ln sum exp(s), P = exp(s - LSE), O = P V,
    D = rowsum(dO * O), dS = P (dO V^T - D), dQ = scale dS K; chunks are
    evaluated several at a time (``_chunk_batches``), only their rows read.

    Returns a list of (token indices [nq], head indices [16], O [nq, 16, D],
    LSE [nq, 16], dQ [nq, 16, D]) in the order of ``chunks``; a row with no
    visible key gets O = dQ = 0 and LSE = -inf."""
    import torch
    layout = DocLayout(cu_seqlens, block)
    G = Q_HEADS_PER_INDEX
    result = [None] * len(chunks)
    for members, i, Q, dO, K, V, _, vis in _chunk_batches(q, k, v, do, layout, sel_clean, chunks, batch):
        lse, P, O = _softmax_rows(Q, K, V, vis, scale)
        Dl = (dO * O).sum(dim=2, keepdim=True)
        dQ = scale * torch.bmm(P * (torch.bmm(dO, V.transpose(1, 2)) - Dl), K)
        heads = np.arange(G * i, G * (i + 1))
        for x, (n, tq) in enumerate(members):
            nq = len(tq)
            result[n] = (tq, heads, O[x].reshape(nq, G, -1).numpy(), lse[x, :, 0].reshape(nq, G).numpy(),
                         dQ[x].reshape(nq, G, -1).numpy())
    return result


def backward_batched(q, k, v, do, cu_seqlens, sel_clean, block: int, scale: float, batch: int = 32):
    """(dq, dk, dv, out, lse) of the whole problem by the formulas of
    ``chunk_rows``, with every chunk's dK_j = scale sum dS_pj q_p and
    dV_j = sum P_pj dO_p added into the rows of its keys."""
    import torch
    layout = DocLayout(cu_seqlens, block)
    T, Hq, Dh = q.shape
    Hkv = k.shape[1]
    G = Q_HEADS_PER_INDEX
    dq = np.zeros((T, Hq, Dh))
    out = np.zeros((T, Hq, Dh))
    lse = np.full((T, Hq), -np.inf)
    dk = torch.zeros(T, Hkv, Dh, dtype=torch.float64)
    dv = torch.zeros(T, Hkv, Dh, dtype=torch.float64)
    chunks = [(i, g) for i in range(Hkv) for g in range(layout.C)]
    for members, i, Q, dO, K, V, ktok, vis in _chunk_batches(q, k, v, do, layout, sel_clean, chunks, batch):
        lse_b, P, O = _softmax_rows(Q, K, V, vis, scale)
        Dl = (dO * O).sum(dim=2, keepdim=True)
        dS = P * (torch.bmm(dO, V.transpose(1, 2)) - Dl)
        dQ = scale * torch.bmm(dS, K)
        dk[:, i].index_add_(0, ktok.reshape(-1), (scale * torch.bmm(dS.transpose(1, 2), Q)).reshape(-1, Dh))
        dv[:, i].index_add_(0, ktok.reshape(-1), torch.bmm(P.transpose(1, 2), dO).reshape(-1, Dh))
        heads = np.arange(G * i, G * (i + 1))
        for x, (n, tq) in enumerate(members):
            nq = len(tq)
            out[np.ix_(tq, heads)] = O[x].reshape(nq, G, -1).numpy()
            dq[np.ix_(tq, heads)] = dQ[x].reshape(nq, G, -1).numpy()
            lse[np.ix_(tq, heads)] = lse_b[x, :, 0].reshape(nq, G).numpy()
    return dq, dk.numpy(), dv.numpy(), out, lse


def key_block_grads(q, k, v, do, cu_seqlens, sel_clean, block: int, scale: float, i: int, row: int,
                    batch: int = 32):
    """dK and dV of the keys of one k2q CSR row (key block ``row`` of index
    head ``i``), complete: the sum over every chunk that selects the block.

    Each selecting chunk is evaluated over all of its selected keys, as in
    ``backward_gathered``: LSE, P and O = P V from the chunk's scores, the
    preprocess D = rowsum(dO * O); the block's own columns then give
    dV_j = sum_{p,h} P_pj dO_p and dK_j = scale sum_{p,h} dS_pj q_p with
    dS_pj = P_pj (dO_p . v_j - D_p).  Chunks are evaluated several at a time
    (``_chunk_batches``) and only their rows are read, so a row that
    thousands of chunks select stays within time and memory.

    Returns (token indices of the block's keys, dk [n, D], dv [n, D])."""
    import torch
    layout = DocLayout(cu_seqlens, block)
    d = int(layout.row_doc[row])
    b = row - int(layout.blk_off[d])
    t0, n = int(layout.cu[d]), int(layout.lens[d])
    bkeys = np.arange(b * layout.block, min((b + 1) * layout.block, n))
    Dh = q.shape[2]
    dk = torch.zeros(len(bkeys), Dh, dtype=torch.float64)
    dv = torch.zeros(len(bkeys), Dh, dtype=torch.float64)
    g0 = int(layout.chunk_off[d])
    chunks = [(i, g0 + c) for c in range(int(layout.nchunks[d])) if np.any(sel_clean[i, g0 + c] == b)]
    for _, _, Q, dO, K, V, ktok, vis in _chunk_batches(q, k, v, do, layout, sel_clean, chunks, batch):
        nb = Q.shape[0]
        _, P, O = _softmax_rows(Q, K, V, vis, scale)
        Dl = (dO * O).sum(dim=2, keepdim=True)
        # the block's keys inside each chunk's key list
        cols = torch.searchsorted(ktok, torch.as_tensor(t0 + bkeys)[None, :].expand(nb, -1).contiguous())
        Pb = torch.gather(P, 2, cols[:, None, :].expand(nb, P.shape[1], len(bkeys)))
        Vb = torch.gather(V, 1, cols[:, :, None].expand(nb, len(bkeys), Dh))
        dSb = Pb * (torch.bmm(dO, Vb.transpose(1, 2)) - Dl)
        dv += torch.bmm(Pb.transpose(1, 2), dO).sum(dim=0)
        dk += scale * torch.bmm(dSb.transpose(1, 2), Q).sum(dim=0)
    return t0 + bkeys, dk.numpy(), dv.numpy()


def chunks_selecting_block(sched: dict, i: int, row: int) -> list[tuple[int, int]]:
    """(i, g) of every chunk whose clean selection holds key-block row ``row``
    (read from the oracle's own CSR)."""
    layout = sched["layout"]
    rp, qi = sched["row_ptr"][i], sched["q_idx"][i]
    d = int(layout.row_doc[row])
    return [(i, int(layout.chunk_off[d]) + int(x) // layout.chunk)
            for x in qi[rp[row]:rp[row + 1]]]


# ---------------------------------------------------------------------------
# Index scorer and top-k block selection (reading stated in the module header)
# ---------------------------------------------------------------------------

def index_scores(qi, ki, cu_seqlens, block: int):
    """Per document d: S[d] of shape [H, C_d, nb_d] with S[h, c, b] =
    (sum of the index queries of chunk c) . (mean of the index keys of block
    b), over the tokens of the document (a chunk or block cut by the
    document end uses the tokens it has), and the matching magnitude
    M[h, c, b] = sum_x |qsum_x| * mean_j |k_jx| (the scale of the score's
    rounding error in a float32 evaluation)."""
    layout = DocLayout(cu_seqlens, block)
    q, k = f64(qi), f64(ki)
    out = []
    for d in range(layout.docs):
        t0, n = int(layout.cu[d]), int(layout.lens[d])
        nc, nb = int(layout.nchunks[d]), int(layout.nblocks[d])
        H, X = q.shape[1], q.shape[2]
        qsum = np.zeros((H, nc, X))
        qabs = np.zeros((H, nc, X))
        for c in range(nc):
            rows = q[t0 + QUERY_CHUNK * c: t0 + min(QUERY_CHUNK * (c + 1), n)]
            qsum[:, c] = rows.sum(axis=0)
            qabs[:, c] = np.abs(rows).sum(axis=0)
        kbar = np.zeros((H, nb, X))
        kabs = np.zeros((H, nb, X))
        for b in range(nb):
            rows = k[t0 + block * b: t0 + min(block * (b + 1), n)]
            kbar[:, b] = rows.mean(axis=0)
            kabs[:, b] = np.abs(rows).mean(axis=0)
        out.append((qsum @ kbar.transpose(0, 2, 1), qabs @ kabs.transpose(0, 2, 1)))
    return layout, out


def index_select(qi, ki, cu_seqlens, block: int, topk: int) -> np.ndarray:
    """sel int32 [H, C, topk]: the diagonal block of each chunk plus its
    topk - 1 best-scoring earlier blocks (ties to the smaller id), ascending,
    -1 padding."""
    layout, scores = index_scores(qi, ki, cu_seqlens, block)
    H = f64(qi).shape[1]
    sel = np.full((H, layout.C, topk), -1, dtype=np.int32)
    for d, (S, _) in enumerate(scores):
        for h in range(H):
            for c in range(int(layout.nchunks[d])):
                diag = (QUERY_CHUNK * c) // block
                cand = np.arange(diag)
                order = np.lexsort((cand, -S[h, c, :diag]))    # score descending, then id
                keep = sorted([diag] + [int(b) for b in cand[order[:topk - 1]]])
                sel[h, int(layout.chunk_off[d]) + c, :len(keep)] = keep
    return sel
