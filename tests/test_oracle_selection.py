"""Pins for the page-selection oracle: exact integer sums, hand-derived order-sensitive cases,
error bounds against exact (fsum / float64) arithmetic, and the selection rule on hand-built
score vectors. The selection rule (mean key per page, dot-product score, top-K plus the most
recent pages, lower page id on ties) is the reading of the "Page-level sparse attention" parts
of the OOMB summaries (es 2.B, pt 2.C, it 2.D)."""
import math

import numpy as np
import pytest

import oracle
import synth


def _bits(x):
    return synth.bf16_round(np.asarray(x, dtype=np.float32))


def test_key_sums_exact_for_small_integers():
    rng = np.random.default_rng(0)
    ints = rng.integers(-200, 200, size=(4 * 64, 2, 16))
    ks = oracle.page_key_sums(_bits(ints), 64)
    assert np.array_equal(ks.astype(np.int64), ints.reshape(4, 64, 2, 16).sum(axis=1))
    reps = oracle.page_reps(ks, 64)
    assert np.array_equal(reps, (ints.reshape(4, 64, 2, 16).sum(axis=1) / 64.0).astype(np.float32))


def test_key_sum_order_is_sequential_from_token_zero():
    # Column 0: tokens 0,1,2 = 2^24, 1, -2^24. Sequential float32: 2^24 + 1 ties to even -> 2^24,
    # then - 2^24 -> 0. Any order adding the 1 last would give 1.
    k = np.zeros((64, 1, 2), dtype=np.float32)
    k[0, 0, 0], k[1, 0, 0], k[2, 0, 0] = 2.0 ** 24, 1.0, -(2.0 ** 24)
    k[:, 0, 1] = 0.5
    ks = oracle.page_key_sums(_bits(k), 64)
    assert ks[0, 0, 0] == 0.0 and ks[0, 0, 1] == 32.0
    assert oracle.page_reps(ks, 64)[0, 0, 1] == 0.5


def test_key_sum_error_bound():
    rng = np.random.default_rng(1)
    x = _bits(rng.standard_normal((128 * 8, 1, 4)).astype(np.float32) * 3)
    ks = oracle.page_key_sums(x, 128)
    xf = synth.bf16_widen(x).reshape(8, 128, 1, 4).astype(np.float64)
    for p in range(8):
        for j in range(4):
            exact = math.fsum(xf[p, :, 0, j])
            bound = 127 * 2.0 ** -24 * np.abs(xf[p, :, 0, j]).sum() * 1.01
            assert abs(float(ks[p, 0, j]) - exact) <= bound


def test_query_sum_order_and_exactness():
    # Order (block-sequential per head, then blocks, then heads) pinned by a cancelling case:
    # head 0: block 0 sums to 2^24, block 1 to 1 -> 2^24 (tie to even); head 1: -2^24 -> total 0.
    q = np.zeros((128, 2, 1), dtype=np.float32)
    q[0, 0, 0] = 2.0 ** 24
    q[64, 0, 0] = 1.0
    q[0, 1, 0] = -(2.0 ** 24)
    assert oracle.query_sum(_bits(q), 1)[0, 0] == 0.0
    # Integers: exact, and heads map to KV heads in contiguous groups.
    rng = np.random.default_rng(2)
    ints = rng.integers(-100, 100, size=(256, 6, 8))
    qs = oracle.query_sum(_bits(ints), 3)
    expect = ints.sum(axis=0).reshape(3, 2, 8).sum(axis=1)
    assert np.array_equal(qs.astype(np.int64), expect)


def test_query_sum_error_bound():
    rng = np.random.default_rng(3)
    x = _bits(rng.standard_normal((512, 4, 16)))
    qs = oracle.query_sum(x, 2).astype(np.float64)
    xf = synth.bf16_widen(x).astype(np.float64)
    exact = xf.sum(axis=0).reshape(2, 2, 16).sum(axis=1)
    bound = (63 + 8 + 2) * 2.0 ** -24 * np.abs(xf).sum(axis=0).reshape(2, 2, 16).sum(axis=1) * 1.01
    assert np.all(np.abs(qs - exact) <= bound)


def test_score_uses_no_fused_multiply_add():
    # Products: -(1+2^-11) exactly, and (1+2^-12)^2 = 1 + 2^-11 + 2^-24 which rounds (tie to
    # even) to 1 + 2^-11. Separate rounding gives exactly 0; a fused multiply-add gives 2^-24.
    qs = np.array([[-1.0, 1.0 + 2.0 ** -12]], dtype=np.float32)
    reps = np.array([[[1.0 + 2.0 ** -11, 1.0 + 2.0 ** -12]]], dtype=np.float32)
    assert oracle.page_scores(qs, reps)[0, 0] == 0.0


def test_scores_match_float64_within_bound():
    rng = np.random.default_rng(4)
    qs = rng.standard_normal((2, 128)).astype(np.float32) * 50
    reps = rng.standard_normal((300, 2, 128)).astype(np.float32)
    sc = oracle.page_scores(qs, reps).astype(np.float64)
    exact = np.einsum("gj,pgj->gp", qs.astype(np.float64), reps.astype(np.float64))
    mag = np.einsum("gj,pgj->gp", np.abs(qs.astype(np.float64)), np.abs(reps.astype(np.float64)))
    assert np.all(np.abs(sc - exact) <= 129 * 2.0 ** -24 * mag * 1.01)


def test_selection_rule_hand_example():
    # 8 prior pages, 2 local (pages 6, 7) always kept, candidates 0..5, top-3.
    # Scores 5, 7, 5, 1, 7, NaN: ranking 7(id1), 7(id4), 5(id0), 5(id2), 1(id3), NaN(id5).
    s = np.array([[5.0, 7.0, 5.0, 1.0, 7.0, np.nan]], dtype=np.float32)
    assert oracle.select_pages(s, 8, 3, 2).tolist() == [[0, 1, 4, 6, 7]]
    assert oracle.n_selected(8, 3, 2) == 5
    # -0.0 and +0.0 tie; the lower id wins.
    s = np.array([[-1.0, -0.0, 0.0]], dtype=np.float32)
    assert oracle.select_pages(s, 3, 1, 0).tolist() == [[1]]
    s = np.array([[0.0, -0.0, -1.0]], dtype=np.float32)
    assert oracle.select_pages(s, 3, 1, 0).tolist() == [[0]]
    # Fewer prior pages than local pages: everything is local, nothing competes.
    assert oracle.select_pages(np.zeros((2, 0), np.float32), 3, 5, 4).tolist() == [[0, 1, 2], [0, 1, 2]]
    assert oracle.n_selected(3, 5, 4) == 3
    assert oracle.n_selected(0, 64, 4) == 0


def test_local_only_selection():
    """top_k = 0 keeps exactly the n_local most recent prior pages whatever the scores (local
    sliding-window layers); n_local = 0 as well leaves no prior page (own block only)."""
    rng = np.random.default_rng(9)
    s = rng.standard_normal((2, 10)).astype(np.float32)
    assert oracle.select_pages(s, 12, 0, 2).tolist() == [[10, 11], [10, 11]]
    assert oracle.n_selected(12, 0, 2) == 2
    assert oracle.select_pages(s, 10, 0, 0).shape == (2, 0)
    assert oracle.n_selected(10, 0, 0) == 0
    assert oracle.select_pages(np.zeros((2, 0), np.float32), 1, 0, 3).tolist() == [[0], [0]]


def test_selection_all_when_k_covers_candidates_and_nesting():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((3, 40)).astype(np.float32)
    allsel = oracle.select_pages(s, 44, 64, 4)
    assert allsel.tolist() == [list(range(44))] * 3
    prev = None
    for k in range(0, 41):
        cur = oracle.select_pages(s, 44, k, 4)
        for g in range(3):
            assert len(cur[g]) == k + 4 and list(cur[g]) == sorted(cur[g])
            if prev is not None:
                assert set(prev[g]) <= set(cur[g])
        prev = cur


def test_selection_against_float64_bruteforce():
    wl = synth.WORKLOADS["topk256k"]
    n_prior = 96
    kk, _ = synth.kv_tokens(wl, 0, n_prior)
    q = synth.q_chunk(wl, 63)
    sel, sc, reps = oracle.topk_pages(q, kk, wl.page, wl.h_kv, n_prior, 16, 4)
    kf = synth.bf16_widen(kk).astype(np.float64).reshape(n_prior, wl.page, wl.h_kv, wl.d).mean(axis=1)
    qf = synth.bf16_widen(q).astype(np.float64).sum(axis=0).reshape(wl.h_kv, wl.group, wl.d).sum(axis=1)
    checked = 0
    for g in range(wl.h_kv):
        s64 = kf[: n_prior - 4, g, :] @ qf[g]
        order = sorted(range(n_prior - 4), key=lambda p: (-s64[p], p))
        gap = s64[order[15]] - s64[order[16]]
        if gap > 1e-6 * np.max(np.abs(s64)):
            assert sorted(order[:16]) + list(range(n_prior - 4, n_prior)) == sel[g].tolist()
            checked += 1
    assert checked >= 3


def test_duplicate_pages_tie_to_lower_id():
    wl = synth.WORKLOADS["topk256k"]
    kk, _ = synth.kv_tokens(wl, 0, 12)
    kk = kk.reshape(12, wl.page, wl.h_kv, wl.d)
    kk[9] = kk[2]            # page 9 duplicates page 2: identical scores
    q = synth.q_chunk(wl, 63)
    sel, sc, _ = oracle.topk_pages(q, kk.reshape(-1, wl.h_kv, wl.d), wl.page, wl.h_kv, 12, 1, 0)
    for g in range(wl.h_kv):
        assert sc[g, 2] == sc[g, 9]
        best = sel[g, 0]
        assert best != 9


def test_per_query_page_single_page_equals_chunk_selection():
    """A chunk of one query page selects exactly what the whole-chunk rule selects."""
    wl = synth.WORKLOADS["topk256k"]
    n_prior = 40
    kk, _ = synth.kv_tokens(wl, 0, n_prior)
    q = synth.q_chunk(wl, 63)[: wl.page]
    want, sc, _ = oracle.topk_pages(q, kk, wl.page, wl.h_kv, n_prior, 8, 2)
    got, sc3, _ = oracle.topk_pages_per_query_page(q, kk, wl.page, wl.h_kv, n_prior, 8, 2)
    assert got.shape == (wl.h_kv, 1, 10)
    assert np.array_equal(got[:, 0], want)
    assert np.array_equal(sc3[:, 0], sc)


def test_per_query_page_hand_built():
    """Query page i points at key page 2 + 2i: each query page picks its own page (pt 2.C)."""
    P, d, n_prior = 64, 8, 6
    k = np.zeros((n_prior * P, 1, d), np.float32)
    for p in range(n_prior):
        k[p * P:(p + 1) * P, 0, p] = 1.0          # every key of page p is e_p: rep = e_p
    q = np.zeros((2 * P, 1, d), np.float32)
    q[:P, 0, 2] = 1.0                              # query page 0 -> e_2
    q[P:, 0, 4] = 1.0                              # query page 1 -> e_4
    sel, sc, _ = oracle.topk_pages_per_query_page(q, k, P, 1, n_prior, 1, 0)
    assert sel.tolist() == [[[2], [4]]]
    assert sc[0, 0, 2] == 64.0 and sc[0, 1, 4] == 64.0
    sel, _, _ = oracle.topk_pages_per_query_page(q, k, P, 1, n_prior, 1, 1)
    assert sel.tolist() == [[[2, 5], [4, 5]]]
    # The whole-chunk rule sees 64 e_2 + 64 e_4: a tie between pages 2 and 4, lower id wins.
    whole, _, _ = oracle.topk_pages(q, k, P, 1, n_prior, 1, 0)
    assert whole.tolist() == [[2]]


def test_per_query_page_against_float64_bruteforce():
    wl = synth.WORKLOADS["topk256k"]
    n_prior, K, n_local = 96, 16, 4
    kk, _ = synth.kv_tokens(wl, 0, n_prior)
    q = synth.q_chunk(wl, 63)[: 4 * wl.page]
    sel, _, _ = oracle.topk_pages_per_query_page(q, kk, wl.page, wl.h_kv, n_prior, K, n_local)
    assert sel.shape == (wl.h_kv, 4, K + n_local)
    kf = synth.bf16_widen(kk).astype(np.float64).reshape(n_prior, wl.page, wl.h_kv, wl.d).mean(axis=1)
    qf = synth.bf16_widen(q).astype(np.float64).reshape(4, wl.page, wl.h_kv, wl.group, wl.d).sum(axis=(1, 3))
    checked = 0
    for g in range(wl.h_kv):
        for i in range(4):
            s64 = kf[: n_prior - n_local, g, :] @ qf[i, g]
            order = sorted(range(n_prior - n_local), key=lambda p: (-s64[p], p))
            gap = s64[order[K - 1]] - s64[order[K]]
            if gap > 1e-6 * np.max(np.abs(s64)):
                assert sorted(order[:K]) + list(range(n_prior - n_local, n_prior)) == sel[g, i].tolist()
                checked += 1
    assert checked >= 10
    # Different query pages do pick different pages on this data.
    assert any(not np.array_equal(sel[g, 0], sel[g, i]) for g in range(wl.h_kv) for i in range(1, 4))
