"""GPU parity for page selection per query page (pt 2.C: each page of queries picks its own key
pages): bit-exact selection lists, attention forward/backward with one page list per (KV head,
query page) against the oracle, row blocks that end inside a query page, and agreement with the
shared-list path when every query page holds the same list."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import ATOL_GRAD, ATOL_LSE, ATOL_O, compare, fill_pool, host, i32, say, scatter_grads, t16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_fwd_amd as m
    m.load()
    return m


def _run(pkv, wl, sel_for_chunk):
    """Fill the pool, run forward + backward of every chunk with its per-query-page selection."""
    bt_np = synth.page_permutation(wl)
    pool, bt = fill_pool(pkv, wl, wl.n_pages, bt_np)
    outs = []
    for c in wl.chunks:
        n_prior = wl.n_prior(c)
        q, do = synth.q_chunk(wl, c), synth.do_chunk(wl, c)
        sel = sel_for_chunk(pool, bt, c, n_prior, q)
        o, lse = pkv.chunk_attn_fwd(pool, bt, n_prior, t16(q), wl.scale, sel=sel)
        dq = pkv.chunk_attn_bwd(pool, bt, n_prior, t16(q), o, t16(do), lse, wl.scale, sel=sel)
        outs.append((c, sel.cpu().numpy(), host(o), lse.cpu().numpy(), host(dq)))
    dk = pool.export(pkv.PKV_DK, bt, 0, wl.n_pages).cpu().numpy()
    dv = pool.export(pkv.PKV_DV, bt, 0, wl.n_pages).cpu().numpy()
    torch.cuda.synchronize()
    pool.check()
    pool.free()
    return outs, dk, dv


def _check(wl, outs, dk, dv):
    k, v = synth.kv_tokens(wl, 0, wl.n_pages)
    dk_ref = np.zeros((wl.context, wl.h_kv, wl.d))
    dv_ref = np.zeros_like(dk_ref)
    for c, sel, o, lse, dq in outs:
        q, do = synth.q_chunk(wl, c), synth.do_chunk(wl, c)
        say(f"chunk {c}: selection {sel.shape}")
        ref = oracle.chunk_backward(q, k, v, do, wl.q0(c), wl.scale, sel=sel, page=wl.page)
        compare("O", o, ref["o"], ATOL_O)
        compare("LSE", lse, ref["lse"], ATOL_LSE, rel=1e-5)
        compare("dQ", dq, ref["dq"], ATOL_GRAD)
        a, b = scatter_grads(ref, wl.context, wl.h_kv, wl.d)
        dk_ref += a
        dv_ref += b
    say("accumulated over chunks:")
    compare("dK", dk, dk_ref, ATOL_GRAD)
    compare("dV", dv, dv_ref, ATOL_GRAD)
    # Keys no query page selected (and no own block covers) receive nothing.
    assert np.all(dk[np.all(dk_ref == 0, axis=2)] == 0)


def _random_lists(wl, c, n_prior, k):
    """Distinct sorted page lists per (KV head, query page)."""
    n_q = wl.chunk // wl.page
    if n_prior == 0:
        return np.zeros((wl.h_kv, n_q, 0), np.int32)
    rng = np.random.default_rng(500 + c)
    k = min(k, n_prior)
    return np.array([[np.sort(rng.choice(n_prior, k, replace=False)) for _ in range(n_q)] for _ in range(wl.h_kv)],
                    dtype=np.int32)


def test_qpage_selection_bit_exact(pkv):
    wl = synth.Workload("qsel", 28, 4, 128, 128, 128 * 200, 4096, (0,), offset_std=0.5, seed=19)
    n_prior = 168
    pool, bt = fill_pool(pkv, wl, n_prior, synth.page_permutation(wl))
    q = synth.q_chunk(wl, 5)
    kk, _ = synth.kv_tokens(wl, 0, n_prior)
    say("per-query-page selection: 32 query pages x 4 KV heads over 168 prior pages")
    for top_k, n_local in ((16, 4), (64, 4), (0, 3), (200, 4), (1, 0)):
        got = pkv.page_topk_select(pool, bt, n_prior, t16(q), top_k, n_local, per_query_page=True).cpu().numpy()
        want, _, _ = oracle.topk_pages_per_query_page(q, kk, wl.page, wl.h_kv, n_prior, top_k, n_local)
        say(f"  top_k={top_k} n_local={n_local}: {got.shape}")
        assert got.shape == want.shape and np.array_equal(got, want), (top_k, n_local)
    # The shared-list call still returns the whole-chunk rule.
    got = pkv.page_topk_select(pool, bt, n_prior, t16(q), 16, 4).cpu().numpy()
    assert np.array_equal(got, oracle.topk_pages(q, kk, wl.page, wl.h_kv, n_prior, 16, 4)[0])
    torch.cuda.synchronize()
    pool.free()


def test_qpage_selection_page64(pkv):
    wl = synth.Workload("qsel64", 8, 2, 64, 64, 64 * 40, 256, (0,), offset_std=0.5, seed=20)
    n_prior = 36
    pool, bt = fill_pool(pkv, wl, n_prior, synth.page_permutation(wl))
    q = synth.q_chunk(wl, 2)
    kk, _ = synth.kv_tokens(wl, 0, n_prior)
    got = pkv.page_topk_select(pool, bt, n_prior, t16(q), 5, 2, per_query_page=True).cpu().numpy()
    want, _, _ = oracle.topk_pages_per_query_page(q, kk, wl.page, wl.h_kv, n_prior, 5, 2)
    assert got.shape == (2, 4, 7) and np.array_equal(got, want)
    torch.cuda.synchronize()
    pool.free()


def test_qpage_mid_end_to_end(pkv):
    """Selection on the GPU (checked bit for bit), then attention with it: 14/2 heads, d=128, page
    128, chunks of 3 query pages (896 rows each, 7 row blocks)."""
    wl = synth.Workload("qmid", 14, 2, 128, 128, 384 * 4, 384, (0, 1, 2, 3), offset_std=0.5, seed=23)
    say("case qmid: per-query-page top-2 + 1 local, 4 chunks")
    k_all, _ = synth.kv_tokens(wl, 0, wl.n_pages)

    def sel_fn(pool, bt, c, n_prior, q):
        sel = pkv.page_topk_select(pool, bt, n_prior, t16(q), 2, 1, per_query_page=True)
        want, _, _ = oracle.topk_pages_per_query_page(q, k_all[: n_prior * wl.page], wl.page, wl.h_kv, n_prior, 2, 1)
        assert np.array_equal(sel.cpu().numpy(), want)
        return sel

    outs, dk, dv = _run(pkv, wl, sel_fn)
    assert any(not np.array_equal(s[:, 0], s[:, 1]) for _, s, *_ in outs if s.shape[2] > 0)
    _check(wl, outs, dk, dv)


def test_qpage_page64_rows_end_inside_blocks(pkv):
    """3 query heads per KV head and 64-token pages: 192 rows per query page, so each query page
    ends inside a 128-row block of the forward and dQ passes."""
    wl = synth.Workload("qp64", 6, 2, 64, 64, 256 * 4, 256, (0, 1, 2, 3), offset_std=0.5, seed=24)
    say("case qp64: 6/2 heads d=64 page 64 C=256, random lists per query page")
    outs, dk, dv = _run(pkv, wl, lambda pool, bt, c, n_prior, q: i32(_random_lists(wl, c, n_prior, 5)))
    _check(wl, outs, dk, dv)


def test_qpage_identical_lists_match_shared_list(pkv):
    wl = synth.Workload("qsame", 14, 2, 128, 128, 384 * 3, 384, (0, 1, 2), offset_std=0.5, seed=25)
    c = 2
    n_prior = wl.n_prior(c)
    bt_np = synth.page_permutation(wl)
    q, do = t16(synth.q_chunk(wl, c)), t16(synth.do_chunk(wl, c))
    rng = np.random.default_rng(3)
    sel2 = np.stack([np.sort(rng.choice(n_prior, 3, replace=False)) for _ in range(wl.h_kv)]).astype(np.int32)
    sel3 = np.repeat(sel2[:, None, :], wl.chunk // wl.page, axis=1)
    res = []
    for sel in (sel2, sel3):
        pool, bt = fill_pool(pkv, wl, wl.n_pages, bt_np)
        o, lse = pkv.chunk_attn_fwd(pool, bt, n_prior, q, wl.scale, sel=i32(sel))
        dq = pkv.chunk_attn_bwd(pool, bt, n_prior, q, o, do, lse, wl.scale, sel=i32(sel))
        dk = pool.export(pkv.PKV_DK, bt, 0, wl.n_pages).cpu().numpy()
        torch.cuda.synchronize()
        res.append((o, lse, dq, dk))
        pool.free()
    # Same keys for every row; the two calls may cut rows and key ranges differently (896 rows per
    # query page take 128-row blocks, the shared list 256-row blocks), so compare to rounding.
    compare("O shared vs per query page", host(res[1][0]), host(res[0][0]), 4e-3, rel=2e-3)
    compare("LSE shared vs per query page", res[1][1].cpu().numpy(), res[0][1].cpu().numpy(), 1e-5, rel=1e-6)
    compare("dQ shared vs per query page", host(res[1][2]), host(res[0][2]), 4e-3, rel=2e-3)
    compare("dK shared vs per query page", res[1][3], res[0][3], 4e-3, rel=2e-3)  # via O's rounding in D


def test_qpage_rejects_bad_list_counts(pkv):
    wl = synth.Workload("qbad", 4, 2, 64, 64, 256 * 2, 256, (0, 1), seed=26)
    pool, bt = fill_pool(pkv, wl, wl.n_pages, synth.page_permutation(wl))
    n_prior = wl.n_prior(1)
    q = t16(synth.q_chunk(wl, 1))
    bad = i32(np.zeros((wl.h_kv, 2, 1), np.int32))   # 2 lists for 4 query pages
    with pytest.raises(pkv.PkvError):
        pkv.chunk_attn_fwd(pool, bt, n_prior, q, wl.scale, sel=bad)
    torch.cuda.synchronize()
    pool.free()
