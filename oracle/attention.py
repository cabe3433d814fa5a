"""Oracle: chunk attention forward and backward (TEST INFRASTRUCTURE ONLY; see package docstring).

Source: web summaries of "Out of the Memory Barrier: A Highly Memory Efficient Training System
for LLMs with Million-Token Contexts" (gist.science pt / es / it).

* pt 2.A / es 2.A / it 2.A: the sequence is cut into chunks processed one after another; each
  chunk attends to the keys of every earlier chunk plus its own. Backward recomputes what the
  forward dropped.
* pt 2.B / es 2.B / it 2.B: keys, values and their gradients live in pages; backward adds the
  key/value gradients in place.
* pt 2.C / es 2.B / it 2.D: page-level sparse attention attends only to selected key pages.
  pt 2.C picks the pages for each query page: a selection may hold one page list per KV head
  (shared by the whole chunk) or one per (KV head, query page of ``page`` chunk tokens).

The pages never write the attention formula. The reading used here is standard scaled
dot-product softmax attention with grouped query heads:

    query head h reads KV head g = h // G, G = H_q / H_kv;
    query token t of the chunk sits at position q0 + t, key token j at position j;
    key j is visible to query t iff j <= q0 + t and j belongs to the visible key set
    (all earlier tokens when dense; selected pages plus the chunk's own block when sparse);
    S_tj = scale * q_t . k_j,  LSE_t = log sum_j exp S_tj,  P_tj = exp(S_tj - LSE_t),
    O_t = sum_j P_tj v_j.

Backward (analytic): D_t = dO_t . O_t, dS_tj = P_tj (dO_t . v_j - D_t),
dQ_t = scale * sum_j dS_tj k_j, dK_j = scale * sum_{h in g, t} dS_tj q_t,
dV_j = sum_{h in g, t} P_tj dO_t.

Arithmetic: float64 by default; ``dtype=np.float32`` gives the float32-from-bf16 mode used at
sizes where float64 is too slow. Query rows are processed in blocks only to bound memory; each
row is independent, and key/value gradients are the sum over blocks.
"""
from __future__ import annotations

import numpy as np


def widen_bf16(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact. Float arrays pass through unchanged."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (np.ascontiguousarray(x).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return x


def visible_keys(q0: int, chunk: int, page: int, sel_pages=None) -> np.ndarray:
    """Logical key tokens the chunk may attend to for one KV head.

    Dense: every token before the end of the chunk, [0, q0 + chunk). Sparse (pt 2.C, es 2.B):
    the tokens of the selected prior pages (ascending) followed by the chunk's own block
    [q0, q0 + chunk), which is always attended causally. Causality is applied per query row.
    """
    if sel_pages is None:
        return np.arange(q0 + chunk, dtype=np.int64)
    sel = np.asarray(sel_pages, dtype=np.int64).reshape(-1)
    toks = (sel[:, None] * page + np.arange(page, dtype=np.int64)[None, :]).reshape(-1)
    return np.concatenate([toks, np.arange(q0, q0 + chunk, dtype=np.int64)])


def group_forward(qrows, qpos, keys, vals, kpos, scale):
    """Softmax attention of query rows against one KV head's visible keys.

    qrows [M][d], qpos [M]; keys, vals [N][d], kpos [N]. Key j is visible to row i iff
    kpos[j] <= qpos[i]; every row must see at least one key. Returns O [M][d], LSE [M] and the
    probabilities P [M][N] (rows sum to one).
    """
    s = scale * (qrows @ keys.T)
    masked = kpos[None, :] > qpos[:, None]
    s = np.where(masked, -np.inf, s)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    p = e / l[:, None]
    o = p @ vals
    lse = m + np.log(l)
    return o, lse, p


def group_backward(qrows, qpos, dorows, keys, vals, kpos, scale):
    """Analytic backward of ``group_forward`` for loss gradients dO = dorows.

    Returns dQ [M][d], dK [N][d], dV [N][d], O [M][d], LSE [M]. P is recomputed from scratch,
    mirroring the forward's dropped activations being recomputed (pt 2.A).
    """
    o, lse, p = group_forward(qrows, qpos, keys, vals, kpos, scale)
    dd = (dorows * o).sum(axis=1)
    dp = dorows @ vals.T
    ds = p * (dp - dd[:, None])
    dq = scale * (ds @ keys)
    dk = scale * (ds.T @ qrows)
    dv = p.T @ dorows
    return dq, dk, dv, o, lse


def _prep(q, kseq, vseq, dtype):
    q = widen_bf16(q).astype(dtype, copy=False)
    k = widen_bf16(kseq).astype(dtype, copy=False)
    v = widen_bf16(vseq).astype(dtype, copy=False)
    return q, k, v


def _key_sets(q0, C, page, sel, g, rows):
    """(visible key tokens, positions into ``rows``) for KV head g.

    sel None or sel[g] one-dimensional: one key set for every row. sel[g] two-dimensional
    ([C/page][n_sel], pt 2.C): the rows of query page i (chunk tokens [i*page, (i+1)*page)) see
    the pages sel[g][i] plus the own block."""
    if sel is None or np.ndim(sel[g]) == 1:
        yield visible_keys(q0, C, page if page else 1, None if sel is None else sel[g]), np.arange(len(rows))
        return
    lists = np.asarray(sel[g])
    assert page and lists.shape[0] * page == C, "one page list per query page"
    qpage = rows // page
    for i in range(lists.shape[0]):
        pos = np.nonzero(qpage == i)[0]
        if len(pos):
            yield visible_keys(q0, C, page, lists[i]), pos


def _row_blocks(rows, block):
    for i in range(0, len(rows), block):
        yield rows[i:i + block]


def chunk_forward(q, kseq, vseq, q0, scale, sel=None, page=None, rows=None,
                  dtype=np.float64, block=512):
    """Forward of one query chunk.

    q: [C][H_q][d]; kseq, vseq: [L][H_kv][d] logical key/value tokens with L >= q0 + C (bf16 bits
    or floats). sel: None for dense, else [H_kv][n_sel] selected logical prior pages (page size
    ``page``), or [H_kv][C/page][n_sel] with one list per query page. rows: optional chunk token
    indices to evaluate (default: all C).

    Returns O [R][H_q][d] and LSE [H_q][R] (natural log, including the scale), R = len(rows).
    """
    q, k, v = _prep(q, kseq, vseq, dtype)
    C, H_q, d = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    rows = np.arange(C) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), H_q, d), dtype=dtype)
    lse = np.zeros((H_q, len(rows)), dtype=dtype)
    for g in range(H_kv):
        for kidx, pos in _key_sets(q0, C, page, sel, g, rows):
            kg, vg = k[kidx, g, :], v[kidx, g, :]
            for hh in range(G):
                h = g * G + hh
                for i0 in range(0, len(pos), block):
                    pb = pos[i0:i0 + block]
                    r = rows[pb]
                    o, l_, _ = group_forward(q[r, h, :], q0 + r, kg, vg, kidx, scale)
                    out[pb, h, :] = o
                    lse[h, pb] = l_
    return out, lse


def chunk_backward(q, kseq, vseq, do, q0, scale, sel=None, page=None, rows=None,
                   dtype=np.float64, block=512):
    """Backward of one query chunk.

    Same arguments as ``chunk_forward`` plus do [C][H_q][d]. Returns a dict with
      dq:   [R][H_q][d] for the evaluated rows,
      keys: list over KV heads of the visible logical key tokens (with one page list per query
            page: the ascending union over the lists),
      dk, dv: lists over KV heads of [N_g][d] gradients of those keys from this chunk,
      o, lse: the forward outputs of the evaluated rows.
    When ``rows`` is a subset, dk/dv hold only those rows' contributions.
    """
    q, k, v = _prep(q, kseq, vseq, dtype)
    do = widen_bf16(do).astype(dtype, copy=False)
    C, H_q, d = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    rows = np.arange(C) if rows is None else np.asarray(rows, dtype=np.int64)
    dq = np.zeros((len(rows), H_q, d), dtype=dtype)
    o_all = np.zeros((len(rows), H_q, d), dtype=dtype)
    lse_all = np.zeros((H_q, len(rows)), dtype=dtype)
    keys, dks, dvs = [], [], []
    for g in range(H_kv):
        sets = list(_key_sets(q0, C, page, sel, g, rows))
        allk = sets[0][0] if len(sets) == 1 else np.unique(np.concatenate([ks for ks, _ in sets]))
        dkg = np.zeros((len(allk), d), dtype=dtype)
        dvg = np.zeros((len(allk), d), dtype=dtype)
        for kidx, pos in sets:
            at = np.searchsorted(allk, kidx) if len(sets) > 1 else np.arange(len(kidx))
            kg, vg = k[kidx, g, :], v[kidx, g, :]
            for hh in range(G):
                h = g * G + hh
                for i0 in range(0, len(pos), block):
                    pb = pos[i0:i0 + block]
                    r = rows[pb]
                    dq_, dk_, dv_, o_, l_ = group_backward(q[r, h, :], q0 + r, do[r, h, :], kg, vg, kidx, scale)
                    dq[pb, h, :] = dq_
                    o_all[pb, h, :] = o_
                    lse_all[h, pb] = l_
                    dkg[at] += dk_
                    dvg[at] += dv_
        keys.append(allk)
        dks.append(dkg)
        dvs.append(dvg)
    return {"dq": dq, "keys": keys, "dk": dks, "dv": dvs, "o": o_all, "lse": lse_all}


def key_gradients(q, kseq, vseq, do, q0, scale, keys, lse, dd, dtype=np.float64, block=512):
    """dK and dV of chosen keys from the row statistics of a finished forward (pt 2.B / it 2.B: the
    backward adds these into the keys' gradient pages).

    For each KV head g in ``keys`` (a dict g -> logical key tokens, each a subset of the keys every
    chunk row of that head may see; causality is applied here) and each of its query heads h, every
    chunk row t contributes, with P_tj = exp(scale q_t.k_j - LSE_t) for key j <= q0 + t (else 0) and
    dS_tj = P_tj (dO_t.v_j - D_t):
        dK_j += scale dS_tj q_t,    dV_j += P_tj dO_t.
    lse [H_q][C] and dd [H_q][C] (D_t = dO_t.O_t) come from the forward; q, do [C][H_q][d];
    kseq, vseq [L][H_kv][d]. Returns {g: (dK [n_g][d], dV [n_g][d])}. This is the backward of
    ``group_backward`` written per key from the stored statistics, so that a few keys' gradients can
    be evaluated without recomputing every key's."""
    q, k, v = _prep(q, kseq, vseq, dtype)
    do = widen_bf16(do).astype(dtype, copy=False)
    lse = np.asarray(lse, dtype=dtype)
    dd = np.asarray(dd, dtype=dtype)
    C, H_q, d = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    out = {}
    for g, kidx in keys.items():
        kidx = np.asarray(kidx, dtype=np.int64)
        kg, vg = k[kidx, g, :], v[kidx, g, :]
        dk = np.zeros((len(kidx), d), dtype=dtype)
        dv = np.zeros((len(kidx), d), dtype=dtype)
        for hh in range(G):
            h = g * G + hh
            for t0 in range(0, C, block):
                t = np.arange(t0, min(t0 + block, C))
                visible = kidx[None, :] <= (q0 + t)[:, None]
                p = np.where(visible, np.exp(scale * (q[t, h, :] @ kg.T) - lse[h, t][:, None]), 0.0)
                ds = p * (do[t, h, :] @ vg.T - dd[h, t][:, None])
                dk += scale * (ds.T @ q[t, h, :])
                dv += p.T @ do[t, h, :]
        out[g] = (dk, dv)
    return out
