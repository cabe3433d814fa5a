"""GPU parity at full size (256K context and the 32K chunk loop, 28/4 heads, d=128, page 128), in
the launch configuration the benchmark times: sampled rows against the oracle computed row by row
in float32, the complete sparse step against the oracle, gradient-sum invariants that hold at any
size, and bit-exact page selection."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import ATOL_GRAD, ATOL_LSE, ATOL_O, compare, fill_pool, host, i32, say, t16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_fwd_amd as m
    m.load()
    return m


@pytest.fixture(scope="module")
def big(pkv):
    wl = synth.WORKLOADS["dense256k"]
    c = wl.chunks[0]
    say("setup dense256k pool (2048 pages)")
    bt_np = synth.page_permutation(wl)
    pool, bt = fill_pool(pkv, wl, wl.n_pages, bt_np)
    k, v = synth.kv_tokens(wl, 0, wl.n_pages)
    q, do = synth.q_chunk(wl, c), synth.do_chunk(wl, c)
    yield wl, c, pool, bt, k, v, q, do
    pool.free()


def _sample_rows(C):
    rng = np.random.default_rng(1234)
    return np.unique(np.concatenate([[0, 1, 127, 128, C - 1], rng.choice(C, 19, replace=False)]))


def test_dense256k_sampled_rows_and_invariants(pkv, big):
    wl, c, pool, bt, k, v, q, do = big
    n_prior = wl.n_prior(c)
    pool.zero_grad()
    qt, dot = t16(q), t16(do)
    o, lse = pkv.chunk_attn_fwd(pool, bt, n_prior, qt, wl.scale)
    dq = pkv.chunk_attn_bwd(pool, bt, n_prior, qt, o, dot, lse, wl.scale)
    dk = pool.export(pkv.PKV_DK, bt, 0, wl.n_pages).cpu().numpy().astype(np.float64)
    dv = pool.export(pkv.PKV_DV, bt, 0, wl.n_pages).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    pool.check()
    rows = _sample_rows(wl.chunk)
    say(f"dense256k: oracle on {len(rows)} sampled tokens x {wl.h_q} heads (float32)")
    ref = oracle.chunk_backward(q, k, v, do, wl.q0(c), wl.scale, page=wl.page, rows=rows, dtype=np.float32)
    compare("O rows", host(o)[rows], ref["o"], ATOL_O)
    compare("LSE rows", lse.cpu().numpy()[:, rows], ref["lse"], ATOL_LSE, rel=1e-5)
    compare("dQ rows", host(dq)[rows], ref["dq"], ATOL_GRAD)
    # Invariants per KV head: sum_j dV_j = sum of dO over the group's rows; sum_j dK_j = 0.
    dof = synth.bf16_widen(do).astype(np.float64)
    G = wl.group
    for g in range(wl.h_kv):
        want = dof[:, g * G:(g + 1) * G].sum(axis=(0, 1))
        got = dv[:, g].sum(axis=0)
        err = np.linalg.norm(got - want) / np.linalg.norm(want)
        skew = np.linalg.norm(dk[:, g].sum(axis=0)) / np.abs(dk[:, g]).sum(axis=0).mean()
        say(f"  head {g}: |sum dV - sum dO|/|sum dO| = {err:.2e}; |sum dK| / mean sum|dK| = {skew:.2e}")
        assert err < 1e-2 and skew < 1e-2
    # Keys after the chunk's end were never attended: their gradients stay zero; all attended
    # pages received gradient.
    assert np.all(np.abs(dk).reshape(wl.n_pages, -1).max(axis=1) > 0)


def _row_stats(q, k, v, do, q0, scale, page, g, G):
    """The oracle's float32 forward over every chunk row of KV head g (its G query heads against all
    keys the rows see): LSE [G][C] and D = dO.O [G][C]."""
    qg, dog = q[:, g * G:(g + 1) * G], do[:, g * G:(g + 1) * G]
    o, lse = oracle.chunk_forward(qg, k[:, g:g + 1], v[:, g:g + 1], q0, scale, page=page, dtype=np.float32)
    dd = np.einsum("thd,thd->ht", synth.bf16_widen(dog).astype(np.float32), o)
    return qg, dog, lse, dd


def test_dense256k_sampled_pages_dkdv_over_all_rows(pkv, big):
    """The dense 256K backward's accumulated dK/dV element by element for sampled pages (four prior
    pages spread over the context and the first and last own pages) of two KV heads, each against
    the oracle's sum over all 28,672 rows of the head's query heads (the oracle's own float32 forward
    statistics of every row, then the key gradients from them)."""
    wl, c, pool, bt, k, v, q, do = big
    n_prior, P, G, q0 = wl.n_prior(c), wl.page, wl.group, wl.q0(c)
    pool.zero_grad()
    qt, dot = t16(q), t16(do)
    o, lse = pkv.chunk_attn_fwd(pool, bt, n_prior, qt, wl.scale)
    pkv.chunk_attn_bwd(pool, bt, n_prior, qt, o, dot, lse, wl.scale)
    dk = pool.export(pkv.PKV_DK, bt, 0, wl.n_pages).cpu().numpy().astype(np.float64)
    dv = pool.export(pkv.PKV_DV, bt, 0, wl.n_pages).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    pool.check()
    pages = [0, 517, 1333, n_prior - 1, n_prior, wl.n_pages - 1]
    toks = np.concatenate([np.arange(p * P, (p + 1) * P) for p in pages])
    for g in (0, 3):
        say(f"dense256k: oracle forward statistics of all {wl.chunk * G} rows of KV head {g} (float32)")
        qg, dog, lse_g, dd_g = _row_stats(q, k, v, do, q0, wl.scale, P, g, G)
        compare(f"LSE head {g} all rows", lse.cpu().numpy()[g * G:(g + 1) * G], lse_g, ATOL_LSE, rel=1e-5)
        ref = oracle.key_gradients(qg, k[:, g:g + 1], v[:, g:g + 1], dog, q0, wl.scale, {0: toks}, lse_g, dd_g,
                                   dtype=np.float32)[0]
        compare(f"dK pages {pages} head {g}", dk[toks, g], ref[0], ATOL_GRAD)
        compare(f"dV pages {pages} head {g}", dv[toks, g], ref[1], ATOL_GRAD)


def test_topk256k_selection_and_full_sparse_step(pkv, big):
    wl, c, pool, bt, k, v, q, do = big
    wk = synth.WORKLOADS["topk256k"]
    n_prior = wl.n_prior(c)
    pool.zero_grad()
    qt, dot = t16(q), t16(do)
    sel = pkv.page_topk_select(pool, bt, n_prior, qt, wk.top_k, wk.n_local)
    o, lse = pkv.chunk_attn_fwd(pool, bt, n_prior, qt, wl.scale, sel=sel)
    dq = pkv.chunk_attn_bwd(pool, bt, n_prior, qt, o, dot, lse, wl.scale, sel=sel)
    dk = pool.export(pkv.PKV_DK, bt, 0, wl.n_pages).cpu().numpy()
    dv = pool.export(pkv.PKV_DV, bt, 0, wl.n_pages).cpu().numpy()
    torch.cuda.synchronize()
    pool.check()
    sel_np = sel.cpu().numpy()
    say("topk256k: oracle selection over 2012 candidates")
    want, scores, _ = oracle.topk_pages(q, k[: n_prior * wl.page], wl.page, wl.h_kv, n_prior, wk.top_k, wk.n_local)
    assert sel_np.shape == (wl.h_kv, 68)
    assert np.array_equal(sel_np, want)
    # Gap between the K-th and (K+1)-th candidate score, for the record.
    for g in range(wl.h_kv):
        s = np.sort(scores[g])[::-1]
        say(f"  head {g}: score gap at K: {s[wk.top_k - 1] - s[wk.top_k]:.3e}")
    say("topk256k: full sparse oracle (float32), all rows and selected keys")
    ref = oracle.chunk_backward(q, k, v, do, wl.q0(c), wl.scale, sel=want, page=wl.page, dtype=np.float32)
    compare("O", host(o), ref["o"], ATOL_O)
    compare("LSE", lse.cpu().numpy(), ref["lse"], ATOL_LSE, rel=1e-5)
    compare("dQ", host(dq), ref["dq"], ATOL_GRAD)
    for g in range(wl.h_kv):
        keys = ref["keys"][g]
        compare(f"dK head {g}", dk[keys, g], ref["dk"][g], ATOL_GRAD)
        compare(f"dV head {g}", dv[keys, g], ref["dv"][g], ATOL_GRAD)
        untouched = np.setdiff1d(np.arange(wl.context), keys)
        assert np.all(dk[untouched, g] == 0) and np.all(dv[untouched, g] == 0)


def test_qpage256k_selection_and_full_sparse_step(pkv, big):
    """Top-64 + 4 local pages chosen per query page (32 query pages x 4 KV heads), full size."""
    wl, c, pool, bt, k, v, q, do = big
    wk = synth.WORKLOADS["topk256k"]
    n_prior = wl.n_prior(c)
    pool.zero_grad()
    qt, dot = t16(q), t16(do)
    sel = pkv.page_topk_select(pool, bt, n_prior, qt, wk.top_k, wk.n_local, per_query_page=True)
    o, lse = pkv.chunk_attn_fwd(pool, bt, n_prior, qt, wl.scale, sel=sel)
    dq = pkv.chunk_attn_bwd(pool, bt, n_prior, qt, o, dot, lse, wl.scale, sel=sel)
    dk = pool.export(pkv.PKV_DK, bt, 0, wl.n_pages).cpu().numpy()
    dv = pool.export(pkv.PKV_DV, bt, 0, wl.n_pages).cpu().numpy()
    torch.cuda.synchronize()
    pool.check()
    sel_np = sel.cpu().numpy()
    say("qpage256k: oracle selection per query page")
    want, _, _ = oracle.topk_pages_per_query_page(q, k[: n_prior * wl.page], wl.page, wl.h_kv, n_prior, wk.top_k,
                                                  wk.n_local)
    assert sel_np.shape == (wl.h_kv, wl.chunk // wl.page, 68)
    assert np.array_equal(sel_np, want)
    union = [len(np.unique(want[g])) for g in range(wl.h_kv)]
    say(f"  distinct prior pages selected per KV head: {union}")
    say("qpage256k: full sparse oracle (float32)")
    ref = oracle.chunk_backward(q, k, v, do, wl.q0(c), wl.scale, sel=want, page=wl.page, dtype=np.float32)
    compare("O", host(o), ref["o"], ATOL_O)
    compare("LSE", lse.cpu().numpy(), ref["lse"], ATOL_LSE, rel=1e-5)
    compare("dQ", host(dq), ref["dq"], ATOL_GRAD)
    for g in range(wl.h_kv):
        keys = ref["keys"][g]
        compare(f"dK head {g}", dk[keys, g], ref["dk"][g], ATOL_GRAD)
        compare(f"dV head {g}", dv[keys, g], ref["dv"][g], ATOL_GRAD)
        untouched = np.setdiff1d(np.arange(wl.context), keys)
        assert np.all(dk[untouched, g] == 0) and np.all(dv[untouched, g] == 0)


def test_qwen32k_all_chunks_sampled_rows_last_page_and_invariants(pkv):
    """The 32K dense workload at full size (28/4 heads, d=128, 8 chunks of 4096, page 128, shuffled
    table), run as the chunk loop runs it: each chunk appended, then its forward and backward, dK/dV
    accumulated in the gradient pages over all chunks. Sampled rows of every chunk against the
    oracle; the last page's accumulated dK/dV element by element (only the last chunk's final
    128 rows see its keys); gradient-sum invariants over all chunks."""
    wl = synth.WORKLOADS["qwen32k"]
    C, P, G = wl.chunk, wl.page, wl.group
    bt_np = synth.page_permutation(wl)
    pool = pkv.Pool(wl.n_pages, P, wl.h_kv, wl.d, grads=True)
    bt = i32(bt_np)
    k, v = synth.kv_tokens(wl, 0, wl.n_pages)
    rows = _sample_rows(C)
    do_sum = np.zeros((wl.h_kv, wl.d))
    for c in wl.chunks:
        q0, n_prior = wl.q0(c), wl.n_prior(c)
        pool.append(bt, q0, t16(k[q0:q0 + C]), t16(v[q0:q0 + C]))
        q, do = synth.q_chunk(wl, c), synth.do_chunk(wl, c)
        qt, dot = t16(q), t16(do)
        o, lse = pkv.chunk_attn_fwd(pool, bt, n_prior, qt, wl.scale)
        dq = pkv.chunk_attn_bwd(pool, bt, n_prior, qt, o, dot, lse, wl.scale)
        say(f"qwen32k chunk {c} (q0 = {q0}): oracle on {len(rows)} sampled tokens x {wl.h_q} heads (float32)")
        ref = oracle.chunk_backward(q, k, v, do, q0, wl.scale, page=P, rows=rows, dtype=np.float32)
        compare("O rows", host(o)[rows], ref["o"], ATOL_O)
        compare("LSE rows", lse.cpu().numpy()[:, rows], ref["lse"], ATOL_LSE, rel=1e-5)
        compare("dQ rows", host(dq)[rows], ref["dq"], ATOL_GRAD)
        dof = synth.bf16_widen(do).astype(np.float64)
        for g in range(wl.h_kv):
            do_sum[g] += dof[:, g * G:(g + 1) * G].sum(axis=(0, 1))
    dk = pool.export(pkv.PKV_DK, bt, 0, wl.n_pages).cpu().numpy().astype(np.float64)
    dv = pool.export(pkv.PKV_DV, bt, 0, wl.n_pages).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    pool.check()
    c = wl.chunks[-1]
    q, do = synth.q_chunk(wl, c), synth.do_chunk(wl, c)
    say("qwen32k: last page's accumulated gradients from the oracle over the last 128 rows")
    ref = oracle.chunk_backward(q, k, v, do, wl.q0(c), wl.scale, page=P, rows=np.arange(C - P, C),
                                dtype=np.float32)
    first_last = wl.context - P
    for g in range(wl.h_kv):
        keys = ref["keys"][g]
        last = keys >= first_last
        assert int(last.sum()) == P
        compare(f"dK last page, head {g}", dk[keys[last], g], ref["dk"][g][last], ATOL_GRAD)
        compare(f"dV last page, head {g}", dv[keys[last], g], ref["dv"][g][last], ATOL_GRAD)
    for g in range(wl.h_kv):
        err = np.linalg.norm(dv[:, g].sum(axis=0) - do_sum[g]) / np.linalg.norm(do_sum[g])
        skew = np.linalg.norm(dk[:, g].sum(axis=0)) / np.abs(dk[:, g]).sum(axis=0).mean()
        say(f"  head {g}: |sum dV - sum dO|/|sum dO| = {err:.2e}; |sum dK| / mean sum|dK| = {skew:.2e}")
        assert err < 1e-2 and skew < 1e-2
    # A mid-sequence page (logical page 100, in chunk 3) after all 8 chunks: its gradient pages hold
    # the sum of chunks 3..7's contributions, each from all of that chunk's rows.
    mid, g = 100, 2
    toks = np.arange(mid * P, (mid + 1) * P)
    ref_dk = np.zeros((P, wl.d))
    ref_dv = np.zeros((P, wl.d))
    for c in wl.chunks:
        q0 = wl.q0(c)
        if q0 + C <= mid * P:
            continue
        say(f"qwen32k: page {mid} head {g}: oracle statistics of chunk {c}'s {C * G} rows")
        q, do = synth.q_chunk(wl, c), synth.do_chunk(wl, c)
        qg, dog = q[:, g * G:(g + 1) * G], do[:, g * G:(g + 1) * G]
        L = q0 + C
        o_g, lse_g = oracle.chunk_forward(qg, k[:L, g:g + 1], v[:L, g:g + 1], q0, wl.scale, page=P, dtype=np.float32)
        dd_g = np.einsum("thd,thd->ht", synth.bf16_widen(dog).astype(np.float32), o_g)
        r = oracle.key_gradients(qg, k[:L, g:g + 1], v[:L, g:g + 1], dog, q0, wl.scale, {0: toks}, lse_g, dd_g,
                                 dtype=np.float32)[0]
        ref_dk += r[0]
        ref_dv += r[1]
    compare(f"dK page {mid} head {g} over all chunks", dk[toks, g], ref_dk, ATOL_GRAD)
    compare(f"dV page {mid} head {g} over all chunks", dv[toks, g], ref_dv, ATOL_GRAD)
    pool.free()
