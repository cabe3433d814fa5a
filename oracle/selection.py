"""Oracle: page representatives, page scores and top-K page selection (TEST INFRASTRUCTURE ONLY).

Source: web summaries of "Out of the Memory Barrier: A Highly Memory Efficient Training System
for LLMs with Million-Token Contexts" (gist.science pt / es / it).

* es 2.B "Page-level sparse attention": one mean representative vector per key page; the most
  relevant pages for the current queries are kept (top-K retrieval).
* pt 2.C: top-K retrieval of the most relevant key pages approximates dense attention.
* it 2.D: for natively sparse models only the most recent pages (or selected ones) are kept.

Readings where the pages are silent:
* One selection per (query chunk, KV head), shared by the KV head's query heads; the chunk's
  query summary is the sum of its queries over tokens and the group's heads; a page's
  representative is its mean key; score = plain dot product. Positive scale factors do not change
  the ranking, so sums are used where means would only rescale.
* pt 2.C instead picks pages for each query page: ``topk_pages_per_query_page`` applies the same
  summary and ranking to every page of queries on its own, giving one list per (KV head, query
  page), still shared by the KV head's query heads.
* The n_local most recent prior pages are always kept and take no part in the ranking; top-K is
  taken over the remaining older pages; ties go to the lower logical page id; a NaN score ranks
  below every other score; the result is sorted ascending.
* Selected indices must be reproduced exactly, so every sum below is evaluated in float32 in one
  fixed order with no fused multiply-add:
    ksum[p,g,j] = sequential over t = 0..P-1 of K[pP+t, g, j], starting from +0.0;
    rep = ksum * (1/P)  (exact: P is a power of two);
    part[h,b,j] = sequential over t = 0..63 of Q[64b+t, h, j];
    hsum[h,j]   = sequential over b = 0..C/64-1 of part[h,b,j];
    qsum[g,j]   = sequential over hh = 0..G-1 of hsum[gG+hh, j];
    score[g,p]  = sequential over j = 0..d-1 of acc = fl(acc + fl(qsum[g,j] * rep[p,g,j])).
NumPy float32 element-wise add/multiply are single IEEE operations, so the vectorised loops below
perform exactly these operations.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import widen_bf16


def page_key_sums(kseq, page: int) -> np.ndarray:
    """Per-page float32 key sums, sequential over the page's tokens. kseq: [n*page][H_kv][d]."""
    k = widen_bf16(kseq).astype(np.float32, copy=False)
    n = k.shape[0] // page
    k = k[: n * page].reshape(n, page, k.shape[1], k.shape[2])
    acc = np.zeros((n, k.shape[2], k.shape[3]), dtype=np.float32)
    for t in range(page):
        acc = np.add(acc, k[:, t], dtype=np.float32)
    return acc


def page_reps(ksum: np.ndarray, page: int) -> np.ndarray:
    """Mean key per page per KV head: ksum * (1/page), exact for power-of-two page sizes."""
    assert page & (page - 1) == 0
    return np.multiply(ksum, np.float32(1.0 / page), dtype=np.float32)


def query_sum(q, h_kv: int) -> np.ndarray:
    """Float32 query summary per KV head [H_kv][d] in the fixed order of the module docstring."""
    x = widen_bf16(q).astype(np.float32, copy=False)
    C, H_q, d = x.shape
    assert C % 64 == 0
    G = H_q // h_kv
    nb = C // 64
    xb = x.reshape(nb, 64, H_q, d)
    part = np.zeros((nb, H_q, d), dtype=np.float32)
    for t in range(64):
        part = np.add(part, xb[:, t], dtype=np.float32)
    hsum = np.zeros((H_q, d), dtype=np.float32)
    for b in range(nb):
        hsum = np.add(hsum, part[b], dtype=np.float32)
    qsum = np.zeros((h_kv, d), dtype=np.float32)
    for hh in range(G):
        qsum = np.add(qsum, hsum[np.arange(h_kv) * G + hh], dtype=np.float32)
    return qsum


def page_scores(qsum: np.ndarray, reps: np.ndarray) -> np.ndarray:
    """score[g, p] = sequential float32 dot of qsum[g] and reps[p, g] (no FMA). reps: [n][H_kv][d]."""
    qsum = np.asarray(qsum, dtype=np.float32)
    reps = np.asarray(reps, dtype=np.float32)
    n, h_kv, d = reps.shape
    acc = np.zeros((h_kv, n), dtype=np.float32)
    for j in range(d):
        prod = np.multiply(qsum[:, j][:, None], reps[:, :, j].T, dtype=np.float32)
        acc = np.add(acc, prod, dtype=np.float32)
    return acc


def n_selected(n_prior: int, top_k: int, n_local: int) -> int:
    """Number of selected prior pages: min(top_k, candidates) + the local pages."""
    n_cand = max(n_prior - n_local, 0)
    return min(top_k, n_cand) + (n_prior - n_cand)


def select_pages(scores: np.ndarray, n_prior: int, top_k: int, n_local: int) -> np.ndarray:
    """Top-K over candidates [0, n_prior - n_local) by (score desc, id asc), NaN lowest, plus the
    n_local most recent prior pages; each row sorted ascending. scores: [H_kv][>= n_cand]."""
    n_cand = max(n_prior - n_local, 0)
    kk = min(top_k, n_cand)
    out = []
    for g in range(scores.shape[0]):
        s = scores[g]
        order = sorted(range(n_cand),
                       key=lambda p: (math.isnan(s[p]), 0.0 if math.isnan(s[p]) else -float(s[p]), p))
        chosen = sorted(order[:kk]) + list(range(n_cand, n_prior))
        out.append(chosen)
    return np.asarray(out, dtype=np.int32).reshape(scores.shape[0], kk + (n_prior - n_cand))


def topk_pages(q, kseq_prior, page: int, h_kv: int, n_prior: int, top_k: int, n_local: int):
    """Whole selection for one chunk: reps from the prior keys, query summary, scores, choice.

    Returns (sel [H_kv][n_sel] int32, scores [H_kv][n_cand] float32, reps [n_prior][H_kv][d])."""
    reps = page_reps(page_key_sums(kseq_prior, page), page)[:n_prior]
    qs = query_sum(q, h_kv)
    n_cand = max(n_prior - n_local, 0)
    sc = page_scores(qs, reps[:n_cand])
    return select_pages(sc, n_prior, top_k, n_local), sc, reps


def topk_pages_per_query_page(q, kseq_prior, page: int, h_kv: int, n_prior: int, top_k: int, n_local: int):
    """Selection per query page (pt 2.C: the most relevant key pages for each page of queries).

    The chunk's queries are cut into query pages of ``page`` tokens. Each query page is summarised
    and ranks the candidates exactly as a whole chunk does in ``topk_pages``, over its own tokens
    only (same fixed float32 order; page is a multiple of 64).
    Returns (sel [H_kv][C/page][n_sel] int32, scores [H_kv][C/page][n_cand] float32, reps)."""
    x = np.asarray(q)
    C = x.shape[0]
    assert C % page == 0 and page % 64 == 0
    reps = page_reps(page_key_sums(kseq_prior, page), page)[:n_prior]
    n_cand = max(n_prior - n_local, 0)
    sels, scs = [], []
    for i in range(C // page):
        sc = page_scores(query_sum(x[i * page:(i + 1) * page], h_kv), reps[:n_cand])
        sels.append(select_pages(sc, n_prior, top_k, n_local))
        scs.append(sc)
    return np.stack(sels, axis=1), np.stack(scs, axis=1), reps
