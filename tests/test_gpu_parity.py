"""GPU parity: HIP path (through the C ABI) against the CPU oracle on the same seeded inputs."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (ATOL_GRAD, ATOL_LSE, ATOL_O, compare, fill_pool, host, i32, say, scatter_grads, t16)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_fwd_amd as m
    m.load()
    return m


def _run_chunks(pkv, wl, bt_np, sel_fn=None, chunks=None):
    """Append everything, run fwd+bwd for the chunks in order; return per-chunk outputs and grads."""
    L = wl.context
    pool, bt = fill_pool(pkv, wl, wl.n_pages, bt_np)
    outs = []
    for c in (chunks or wl.chunks):
        n_prior = wl.n_prior(c)
        q, do = synth.q_chunk(wl, c), synth.do_chunk(wl, c)
        sel = sel_fn(c, n_prior) if sel_fn else None
        sel_t = i32(sel) if sel is not None else None
        o, lse = pkv.chunk_attn_fwd(pool, bt, n_prior, t16(q), wl.scale, sel=sel_t)
        dq = pkv.chunk_attn_bwd(pool, bt, n_prior, t16(q), o, t16(do), lse, wl.scale, sel=sel_t)
        outs.append((c, sel, host(o), lse.cpu().numpy(), host(dq)))
    dk = pool.export(pkv.PKV_DK, bt, 0, wl.n_pages).cpu().numpy()
    dv = pool.export(pkv.PKV_DV, bt, 0, wl.n_pages).cpu().numpy()
    torch.cuda.synchronize()
    pool.check()
    pool.free()
    return outs, dk, dv


def _check_against_oracle(wl, outs, dk, dv, page):
    k, v = synth.kv_tokens(wl, 0, wl.n_pages)
    dk_ref = np.zeros((wl.context, wl.h_kv, wl.d))
    dv_ref = np.zeros_like(dk_ref)
    for c, sel, o, lse, dq in outs:
        q, do = synth.q_chunk(wl, c), synth.do_chunk(wl, c)
        say(f"chunk {c}:")
        ref = oracle.chunk_backward(q, k, v, do, wl.q0(c), wl.scale, sel=sel, page=page)
        compare("O", o, ref["o"], ATOL_O)
        compare("LSE", lse, ref["lse"], ATOL_LSE, rel=1e-5)
        compare("dQ", dq, ref["dq"], ATOL_GRAD)
        a, b = scatter_grads(ref, wl.context, wl.h_kv, wl.d)
        dk_ref += a
        dv_ref += b
    say("accumulated over chunks:")
    compare("dK", dk, dk_ref, ATOL_GRAD)
    compare("dV", dv, dv_ref, ATOL_GRAD)


def test_tiny_all_chunks_dense(pkv):
    """4/1 heads, d=64, 2048 tokens as 4x512, page 64, seeded page permutation, dense."""
    wl = synth.WORKLOADS["tiny"]
    say("case tiny dense seed 0")
    outs, dk, dv = _run_chunks(pkv, wl, synth.page_permutation(wl))
    _check_against_oracle(wl, outs, dk, dv, wl.page)


@pytest.mark.parametrize("seed", [1, 2])
def test_tiny_other_seeds(pkv, seed):
    wl = synth.WORKLOADS["tiny"].with_seed(seed)
    say(f"case tiny dense seed {seed}")
    outs, dk, dv = _run_chunks(pkv, wl, synth.page_permutation(wl))
    _check_against_oracle(wl, outs, dk, dv, wl.page)


def _mid(seed=0, G=7, h_kv=2, C=384, chunks=(0, 1, 2), d=128, page=128, offset=0.5):
    # 2688 rows per KV head (10.5 blocks of 256): spans several tiles and a ragged tail.
    return synth.Workload("mid", G * h_kv, h_kv, d, page, C * len(chunks), C, tuple(chunks), offset_std=offset,
                          seed=seed)


def test_mid_gqa7_ragged_dense(pkv):
    wl = _mid()
    say("case mid 14/2 heads d=128 page 128 C=384 dense")
    outs, dk, dv = _run_chunks(pkv, wl, synth.page_permutation(wl))
    _check_against_oracle(wl, outs, dk, dv, wl.page)


def test_mid_sparse_selection(pkv):
    wl = _mid(seed=3, chunks=(0, 1, 2, 3))
    say("case mid sparse (fixed selections)")

    def sel_fn(c, n_prior):
        if n_prior == 0:
            return np.zeros((wl.h_kv, 0), np.int32)
        rng = np.random.default_rng(100 + c)
        k = max(1, n_prior // 2)
        return np.stack([np.sort(rng.choice(n_prior, k, replace=False)) for _ in range(wl.h_kv)]).astype(np.int32)

    outs, dk, dv = _run_chunks(pkv, wl, synth.page_permutation(wl), sel_fn=sel_fn)
    _check_against_oracle(wl, outs, dk, dv, wl.page)


def test_mid_page64_d64(pkv):
    wl = _mid(seed=4, G=3, h_kv=2, C=256, chunks=(0, 1, 2), d=64, page=64, offset=0.0)
    say("case mid 6/2 heads d=64 page 64 C=256")
    outs, dk, dv = _run_chunks(pkv, wl, synth.page_permutation(wl))
    _check_against_oracle(wl, outs, dk, dv, wl.page)


@pytest.mark.parametrize("name,G,h_kv,C,n_chunks,d,page", [
    ("no GQA (G=1), 128-row chunks in 256-row blocks", 1, 2, 128, 3, 128, 128),
    ("one-page chunks (C = page = 64), six chunks", 4, 1, 64, 6, 64, 64),
    ("one-page chunks (C = page = 128)", 2, 2, 128, 4, 128, 128),
    ("wide group (G=16, one KV head)", 16, 1, 128, 3, 128, 128),
])
def test_degenerate_shapes_dense(pkv, name, G, h_kv, C, n_chunks, d, page):
    """Chunk sizes and group sizes at the edges of the tiling, every chunk checked against the
    oracle and the gradient pages accumulated over all chunks."""
    wl = _mid(seed=11, G=G, h_kv=h_kv, C=C, chunks=tuple(range(n_chunks)), d=d, page=page)
    say(f"case {name}")
    outs, dk, dv = _run_chunks(pkv, wl, synth.page_permutation(wl))
    _check_against_oracle(wl, outs, dk, dv, wl.page)


def test_head_subsets_match_full_call(pkv):
    """Running KV heads one at a time (kvh0/n_kvh) gives the same bits as one call over all heads."""
    wl = _mid(seed=5, chunks=(0, 1))
    c = 1
    bt_np = synth.page_permutation(wl)
    pool, bt = fill_pool(pkv, wl, wl.n_pages, bt_np)
    q = t16(synth.q_chunk(wl, c))
    n_prior = wl.n_prior(c)
    o_all, lse_all = pkv.chunk_attn_fwd(pool, bt, n_prior, q, wl.scale)
    o_h = torch.zeros_like(o_all)
    lse_h = torch.zeros_like(lse_all)
    for g in range(wl.h_kv):
        pkv.chunk_attn_fwd(pool, bt, n_prior, q, wl.scale, kvh0=g, n_kvh=1, o=o_h, lse=lse_h)
    torch.cuda.synchronize()
    # Split counts may differ between the calls, so compare to tolerance, not bits.
    compare("O heads", host(o_h), host(o_all), 1e-2)
    compare("LSE heads", lse_h.cpu().numpy(), lse_all.cpu().numpy(), 1e-4, rel=1e-5)
    pool.free()


def test_permutation_invariance_bitwise(pkv):
    """Two page permutations of the same data: identical O/LSE/dQ bits (the kernels walk logical
    pages in the same order); dK/dV equal up to the order of the atomic adds of row splits."""
    wl = _mid(seed=6, chunks=(0, 1, 2))
    res = []
    for perm_seed in (11, 12):
        bt_np = np.random.default_rng(perm_seed).permutation(wl.n_pages).astype(np.int32)
        outs, dk, dv = _run_chunks(pkv, wl, bt_np)
        res.append((outs, dk, dv))
    for (c, _, o1, l1, q1), (_, _, o2, l2, q2) in zip(res[0][0], res[1][0]):
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2) and np.array_equal(q1, q2), c
    for a, b in ((res[0][1], res[1][1]), (res[0][2], res[1][2])):
        assert np.max(np.abs(a - b)) <= 1e-5 * max(1.0, float(np.max(np.abs(a))))


def test_sparse_all_pages_equals_dense_bitwise(pkv):
    wl = _mid(seed=7, chunks=(0, 1, 2))
    c = 2
    bt_np = synth.page_permutation(wl)
    pool, bt = fill_pool(pkv, wl, wl.n_pages, bt_np)
    n_prior = wl.n_prior(c)
    q = t16(synth.q_chunk(wl, c))
    sel = i32(np.tile(np.arange(n_prior, dtype=np.int32), (wl.h_kv, 1)))
    o1, l1 = pkv.chunk_attn_fwd(pool, bt, n_prior, q, wl.scale)
    o2, l2 = pkv.chunk_attn_fwd(pool, bt, n_prior, q, wl.scale, sel=sel)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    pool.free()


def test_sparse_backward_leaves_unselected_pages(pkv):
    wl = _mid(seed=8, chunks=(0, 1, 2, 3))
    c = 3
    bt_np = synth.page_permutation(wl)
    pool, bt = fill_pool(pkv, wl, wl.n_pages, bt_np)
    n_prior = wl.n_prior(c)
    sel_np = np.array([[0, 3, 5], [1, 2, 6]], dtype=np.int32)
    sel = i32(sel_np)
    q, do = t16(synth.q_chunk(wl, c)), t16(synth.do_chunk(wl, c))
    # Put known non-zero values in every gradient page first: run a dense backward of chunk 1.
    q1, do1 = t16(synth.q_chunk(wl, 1)), t16(synth.do_chunk(wl, 1))
    o1, l1 = pkv.chunk_attn_fwd(pool, bt, wl.n_prior(1), q1, wl.scale)
    pkv.chunk_attn_bwd(pool, bt, wl.n_prior(1), q1, o1, do1, l1, wl.scale)
    before = pool.export(pkv.PKV_DK, bt, 0, wl.n_pages).cpu().numpy()
    o, lse = pkv.chunk_attn_fwd(pool, bt, n_prior, q, wl.scale, sel=sel)
    pkv.chunk_attn_bwd(pool, bt, n_prior, q, o, do, lse, wl.scale, sel=sel)
    after = pool.export(pkv.PKV_DK, bt, 0, wl.n_pages).cpu().numpy()
    torch.cuda.synchronize()
    P = wl.page
    for g in range(wl.h_kv):
        for lp in range(n_prior):
            same = np.array_equal(before[lp * P:(lp + 1) * P, g], after[lp * P:(lp + 1) * P, g])
            assert same == (lp not in sel_np[g]), (g, lp)
    pool.free()


def test_topk_selection_bit_exact(pkv):
    wl = synth.Workload("sel", 28, 4, 128, 128, 128 * 200, 4096, (0,), offset_std=0.5, seed=9)
    n_prior = 168
    bt_np = synth.page_permutation(wl)
    pool, bt = fill_pool(pkv, wl, n_prior, bt_np)
    q_np = synth.q_chunk(wl, 5)
    kk, _ = synth.kv_tokens(wl, 0, n_prior)
    for top_k, n_local in ((16, 4), (64, 4), (0, 3), (200, 4), (5, 0)):
        sel = pkv.page_topk_select(pool, bt, n_prior, t16(q_np), top_k, n_local)
        want, sc, reps = oracle.topk_pages(q_np, kk, wl.page, wl.h_kv, n_prior, top_k, n_local)
        got = sel.cpu().numpy()
        say(f"  top_k={top_k} n_local={n_local}: n_sel={got.shape[1]}")
        assert np.array_equal(got, want), (top_k, n_local)
    rep_g = pool.export(pkv.PKV_REP, bt, 0, n_prior).cpu().numpy()
    assert np.array_equal(rep_g, oracle.page_reps(oracle.page_key_sums(kk, wl.page), wl.page))
    torch.cuda.synchronize()
    pool.free()


def test_topk_no_fma_and_ties(pkv):
    """Constructed keys: the score of page 1 is exactly 0 only without FMA; duplicated pages tie and
    the lower id wins."""
    wl = synth.Workload("fma", 1, 1, 64, 64, 64 * 6, 64, (0,), seed=0)
    P, d = 64, 64
    K = np.zeros((6 * P, 1, d), np.float32)
    # page 1: dims 0,1 mean to 1 + 2^-11 and 1 + 2^-12 (one token each a bit above 1).
    K[P:2 * P, 0, 0] = 1.0
    K[P:2 * P, 0, 1] = 1.0
    K[P, 0, 0] = 1.0 + 2.0 ** -5     # sum = 64 + 2^-5 -> mean 1 + 2^-11
    K[P, 0, 1] = 1.0 + 2.0 ** -6     # mean 1 + 2^-12
    K[2 * P:3 * P, 0, 2] = 0.5       # page 2 score = 0.5 * qsum[2]
    K[3 * P:4 * P] = K[2 * P:3 * P]  # page 3 duplicates page 2
    Kb = synth.bf16_round(K)
    Vb = synth.bf16_round(np.zeros_like(K))
    # Queries: qsum = (-1, 1 + 2^-12, 1, 0, ...): token 0 carries (-1, 1, 1), token 1 carries 2^-12 on dim 1.
    Q = np.zeros((64, 1, d), np.float32)
    Q[0, 0, 0], Q[0, 0, 1], Q[0, 0, 2] = -1.0, 1.0, 1.0
    Q[1, 0, 1] = 2.0 ** -12
    Qb = synth.bf16_round(Q)
    pool = pkv.Pool(6, P, 1, d)
    bt = i32(np.arange(6))
    pool.append(bt, 0, t16(Kb), t16(Vb))
    # Scores: pages 0, 1, 4, 5 -> exactly 0 (page 1 only without FMA), pages 2, 3 -> 0.5.
    for top_k, expect in ((1, [2]), (3, [0, 2, 3]), (4, [0, 1, 2, 3])):
        want, sc, _ = oracle.topk_pages(Qb, Kb, P, 1, 6, top_k, 0)
        assert sc[0, 1] == 0.0 and sc[0, 2] == sc[0, 3] == 0.5
        assert want.tolist() == [expect]
        got = pkv.page_topk_select(pool, bt, 6, t16(Qb), top_k, 0).cpu().numpy()
        assert got.tolist() == [expect], (top_k, got)
    torch.cuda.synchronize()
    pool.free()


def _tied_pool(pkv, n_pages, h_kv, seed):
    """Pages whose keys are one constant per (page, head) on dimension 0, drawn from five
    bf16-exact values, so scores take five values and ties fill whole id ranges."""
    P, d = 64, 64
    rng = np.random.default_rng(seed)
    vals = np.array([-0.5, 0.25, 0.5, 0.75, 1.0], np.float32)
    pick = vals[rng.integers(0, len(vals), (n_pages, h_kv))]
    K = np.zeros((n_pages * P, h_kv, d), np.float32)
    K[:, :, 0] = np.repeat(pick, P, axis=0)
    K = synth.bf16_round(K)
    Q = np.zeros((64, h_kv, d), np.float32)
    Q[0, :, 0] = 1.0
    Q = synth.bf16_round(Q)
    perm = rng.permutation(n_pages).astype(np.int32)
    pool = pkv.Pool(n_pages, P, h_kv, d, grads=False)
    bt = i32(perm)
    per = 4096
    for p0 in range(0, n_pages, per):
        n = min(per, n_pages - p0)
        kk = K[p0 * P:(p0 + n) * P]
        pool.append(bt, p0 * P, t16(kk), t16(np.zeros_like(kk)))
    return pool, bt, K, Q, P


@pytest.mark.parametrize("n_pages", [2600, 16400])
def test_topk_ties_across_chunks(pkv, n_pages):
    """Five distinct scores over thousands of candidates: the K-th page's score is tied with
    hundreds of others spread over several 1024-id compaction chunks; the lowest ids must win.
    16400 candidates exceed what the selection kernel stages on chip."""
    pool, bt, K, Q, P = _tied_pool(pkv, n_pages, 2, seed=n_pages)
    for top_k, n_local in ((1000, 4), (1500, 0), (7, 0), (n_pages - 5, 4), (n_pages // 2, 16)):
        say(f"  n_pages={n_pages} top_k={top_k} n_local={n_local}")
        want, sc, _ = oracle.topk_pages(Q, K, P, 2, n_pages, top_k, n_local)
        assert len(np.unique(sc)) <= 5
        got = pkv.page_topk_select(pool, bt, n_pages, t16(Q), top_k, n_local).cpu().numpy()
        assert np.array_equal(got, want), (top_k, n_local)
    pool.check()
    torch.cuda.synchronize()
    pool.free()


def test_binding_rejects_mis_shaped_tensors(pkv):
    """The library sees only pointers; the binding refuses tensors whose shape does not match the
    pool or the call before anything is launched (a float32 array passed as bf16 bits doubles d)."""
    pool = pkv.Pool(4, 64, 2, 64)
    bt = i32(np.arange(4))
    good_q = torch.zeros((64, 4, 64), dtype=torch.bfloat16, device="cuda")
    bad_q = torch.zeros((64, 4, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((128, 2, 64), dtype=torch.bfloat16, device="cuda")
    pool.append(bt, 0, kv, kv)
    with pytest.raises(ValueError):
        pool.append(bt, 128, torch.zeros((64, 2, 128), dtype=torch.bfloat16, device="cuda"), kv[:64])
    with pytest.raises(ValueError):
        pkv.page_topk_select(pool, bt, 1, bad_q, 1, 0)
    with pytest.raises(ValueError):
        pkv.chunk_attn_fwd(pool, bt, 1, bad_q, 0.125)
    with pytest.raises(ValueError):
        pkv.chunk_attn_fwd(pool, bt, 1, good_q, 0.125, sel=torch.zeros((1, 1), dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        pkv.chunk_attn_fwd(pool, bt, 1, good_q, 0.125, lse=torch.zeros((4, 32), dtype=torch.float32, device="cuda"))
    o, lse = pkv.chunk_attn_fwd(pool, bt, 1, good_q, 0.125)
    with pytest.raises(ValueError):
        pkv.chunk_attn_bwd(pool, bt, 1, good_q, o, good_q[:32].contiguous(), lse, 0.125)
    with pytest.raises(ValueError):
        pkv.chunk_attn_bwd(pool, bt, 1, good_q, o, good_q, lse.t().contiguous(), 0.125)
    torch.cuda.synchronize()
    pool.free()


@pytest.mark.parametrize("page,d", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_page_reps_ragged_appends(pkv, page, d):
    """Representatives written by appends that start and end inside pages, with 3 KV heads (so the
    last workgroup of four (page, head) blocks is partly empty), equal the oracle's fixed-order
    float32 key sums times 1/page, bit for bit; pages not yet full have no representative."""
    wl = synth.Workload("reps", 6, 3, d, page, page * 11, page, (0,), offset_std=0.5, seed=4)
    bt_np = synth.page_permutation(wl)
    pool = pkv.Pool(wl.n_pages, page, wl.h_kv, d, grads=True)
    bt = i32(bt_np)
    k, v = synth.kv_tokens(wl, 0, wl.n_pages)
    cuts = [0, page // 2 + 3, 3 * page + 1, 3 * page + 5, 9 * page + page // 4]
    for a, b in zip(cuts[:-1], cuts[1:]):
        pool.append(bt, a, t16(k[a:b]), t16(v[a:b]))
    full = cuts[-1] // page
    got = pool.export(pkv.PKV_REP, bt, 0, full).cpu().numpy()
    torch.cuda.synchronize()
    pool.check()
    want = oracle.page_reps(oracle.page_key_sums(k[:full * page], page), page)
    assert got.shape == want.shape
    assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32))
    pool.free()


@pytest.mark.parametrize("page,d", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_page_reps_bulk_append(pkv, page, d):
    """An append that completes over a thousand (page, head) blocks at once, starting inside a
    page and ending inside another, with 3 KV heads so the last workgroup is partly filled:
    representatives equal the oracle's bit for bit."""
    n_pages = 352
    wl = synth.Workload("reps_bulk", 6, 3, d, page, page * n_pages, page, (0,), offset_std=0.5, seed=6)
    bt_np = synth.page_permutation(wl)
    pool = pkv.Pool(n_pages, page, wl.h_kv, d, grads=True)
    bt = i32(bt_np)
    k, v = synth.kv_tokens(wl, 0, n_pages)
    a, b = page // 3, (n_pages - 1) * page + page // 2
    pool.append(bt, 0, t16(k[:a]), t16(v[:a]))
    pool.append(bt, a, t16(k[a:b]), t16(v[a:b]))
    assert (b // page - 1) * wl.h_kv >= 1024
    full = b // page
    got = pool.export(pkv.PKV_REP, bt, 0, full).cpu().numpy()
    torch.cuda.synchronize()
    pool.check()
    want = oracle.page_reps(oracle.page_key_sums(k[:full * page], page), page)
    assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32))
    pool.free()


def test_mfma_probe_runs_and_counts(pkv):
    """The sustained-MFMA diagnostic: finite outputs, the FLOP count it reports, a rate below the
    datasheet peak."""
    n_wg, iters = 8, 2000
    out = torch.empty(n_wg * 512, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flop = pkv.mfma_probe(n_wg, iters, out)
    e1.record()
    torch.cuda.synchronize()
    assert flop == n_wg * 8 * iters * 4 * 32 * 32 * 16 * 2
    assert bool(torch.isfinite(out).all())
    tflops = flop / (e0.elapsed_time(e1) * 1e-3) / 1e12
    say(f"  mfma probe on {n_wg} CUs: {tflops:.1f} TFLOP/s")
    assert 0 < tflops < 2600.0 * n_wg / 256


def test_atomic_probe_adds_exactly(pkv):
    """The fp32 atomic-add diagnostic: every float of region r ends at the number of workgroups that
    add into it (counts below 2^24 are exact in fp32), with and without contention, and the byte
    count it reports."""
    region = 3000  # not a multiple of the 256 threads: the strided tail is covered too
    for n_wg, n_regions in ((64, 64), (70, 8)):
        buf = torch.zeros(n_regions * region, dtype=torch.float32, device="cuda")
        nbytes = pkv.atomic_probe(n_wg, n_regions, region, buf)
        torch.cuda.synchronize()
        assert nbytes == n_wg * region * 4
        want = torch.tensor([sum(1 for w in range(n_wg) if w % n_regions == r) for r in range(n_regions)],
                            dtype=torch.float32).repeat_interleave(region)
        assert torch.equal(buf.cpu(), want)
    with pytest.raises(pkv.PkvError):
        pkv.atomic_probe(4, 8, region, torch.zeros(8 * region, dtype=torch.float32, device="cuda"))


def test_bad_table_and_selection_entries_are_skipped_and_reported(pkv):
    """Device-side validation: a block-table entry outside the pool and a selection id outside
    [0, n_prior) are skipped by every kernel (the page acts as absent) and reported once through
    paged_kv_check (PKV_E_DEVICE). Results equal the oracle's with that page left out."""
    wl = synth.Workload("bad", 4, 1, 64, 64, 64 * 12, 256, (2,), offset_std=0.5, seed=41)
    c = wl.chunks[0]
    q0, C, P, n_prior = wl.q0(c), wl.chunk, wl.page, wl.n_prior(c)  # 8 prior pages
    bt_np = synth.page_permutation(wl).copy()
    bad_lp = 5
    bt_np[bad_lp] = wl.n_pages + 3  # outside the pool
    pool = pkv.Pool(wl.n_pages, P, wl.h_kv, wl.d, grads=True)
    bt = i32(bt_np)
    k, v = synth.kv_tokens(wl, 0, wl.n_pages)
    pool.append(bt, 0, t16(k), t16(v))
    torch.cuda.synchronize()
    with pytest.raises(pkv.PkvError) as ei:
        pool.check()
    assert ei.value.code == pkv.PKV_E_DEVICE
    pool.check()  # the error word was cleared by the read
    q, do = synth.q_chunk(wl, c), synth.do_chunk(wl, c)
    keep = np.array([[p for p in range(n_prior) if p != bad_lp]], np.int32)
    cases = (("dense pass over a bad table entry", None, keep),
             ("selection with an id past n_prior", np.array([[0, 2, 7, n_prior + 91]], np.int32),
              np.array([[0, 2, 7]], np.int32)))
    for name, sel_gpu, sel_ref in cases:
        say(f"case {name}")
        pool.zero_grad()
        sel_t = None if sel_gpu is None else i32(sel_gpu)
        o, lse = pkv.chunk_attn_fwd(pool, bt, n_prior, t16(q), wl.scale, sel=sel_t)
        dq = pkv.chunk_attn_bwd(pool, bt, n_prior, t16(q), o, t16(do), lse, wl.scale, sel=sel_t)
        dk = pool.export(pkv.PKV_DK, bt, 0, wl.n_pages).cpu().numpy()
        torch.cuda.synchronize()
        with pytest.raises(pkv.PkvError) as ei:
            pool.check()
        assert ei.value.code == pkv.PKV_E_DEVICE
        ref = oracle.chunk_backward(q, k, v, do, q0, wl.scale, sel=sel_ref, page=P)
        compare("O", host(o), ref["o"], ATOL_O)
        compare("LSE", lse.cpu().numpy(), ref["lse"], ATOL_LSE, rel=1e-5)
        compare("dQ", host(dq), ref["dq"], ATOL_GRAD)
        keys = ref["keys"][0]
        compare("dK", dk[keys, 0], ref["dk"][0], ATOL_GRAD)
        assert np.all(dk[bad_lp * P:(bad_lp + 1) * P] == 0)
    pool.free()
