"""GPU parity for the pinned-host page tier: selection on the host-tier pool, per-head H2D gathers on
a side stream overlapped with compute, sparse forward/backward from the gathered device slots and
gradients accumulated into the host-tier pool's device gradient pages."""
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


def _run_host_tier(pkv, wl, c, top_k, n_local):
    from paged_kv_cache_fwd_amd.host_tier import HostTierStep
    n_prior = wl.n_prior(c)
    q0, C, P = wl.q0(c), wl.chunk, wl.page
    bt_np = synth.page_permutation(wl)
    hpool, hbt = fill_pool(pkv, wl, wl.n_pages, bt_np, host_tier=True)
    step = HostTierStep(hpool, hbt, n_prior, C, wl.h_q, top_k, n_local, torch.device("cuda:0"))
    k_own, v_own = synth.kv_tokens(wl, n_prior, C // P)
    step.append_own(t16(k_own), t16(v_own))
    q, do = t16(synth.q_chunk(wl, c)), t16(synth.do_chunk(wl, c))
    o, dq = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((wl.h_q, C), dtype=torch.float32, device=q.device)
    hpool.zero_grad()
    sel = step.run(q, do, wl.scale, o, lse, dq)
    torch.cuda.synchronize()
    hpool.check()
    step.dev.check()
    res = dict(sel=sel.cpu().numpy(), o=o.clone(), lse=lse.clone(), dq=dq.clone(),
               dk=hpool.export(pkv.PKV_DK, hbt, 0, wl.n_pages).cpu().numpy(),
               dv=hpool.export(pkv.PKV_DV, hbt, 0, wl.n_pages).cpu().numpy())
    # The same selection over a device-resident pool, all heads in one call.
    dpool, dbt = fill_pool(pkv, wl, wl.n_pages, bt_np)
    o2, lse2 = pkv.chunk_attn_fwd(dpool, dbt, n_prior, q, wl.scale, sel=sel)
    dq2 = pkv.chunk_attn_bwd(dpool, dbt, n_prior, q, o2, do, lse2, wl.scale, sel=sel)
    torch.cuda.synchronize()
    res.update(o_res=o2, lse_res=lse2, dq_res=dq2,
               dk_res=dpool.export(pkv.PKV_DK, dbt, 0, wl.n_pages).cpu().numpy())
    step.free()
    dpool.free()
    hpool.free()
    return res


def test_host_tier_small_full_parity(pkv):
    wl = synth.Workload("host-small", 14, 2, 128, 128, 128 * 24, 384, (7,), offset_std=0.5, seed=21)
    c = 7  # q0 = 2688 = 21 pages
    top_k, n_local = 6, 2
    say("host tier small: 24 pages, 21 prior, top-6 + 2 local")
    res = _run_host_tier(pkv, wl, c, top_k, n_local)
    n_prior = wl.n_prior(c)
    k, v = synth.kv_tokens(wl, 0, wl.n_pages)
    q, do = synth.q_chunk(wl, c), synth.do_chunk(wl, c)
    want, _, _ = oracle.topk_pages(q, k[: n_prior * wl.page], wl.page, wl.h_kv, n_prior, top_k, n_local)
    assert np.array_equal(res["sel"], want)
    ref = oracle.chunk_backward(q, k, v, do, wl.q0(c), wl.scale, sel=want, page=wl.page)
    compare("O", host(res["o"]), ref["o"], ATOL_O)
    compare("LSE", res["lse"].cpu().numpy(), ref["lse"], ATOL_LSE, rel=1e-5)
    compare("dQ", host(res["dq"]), ref["dq"], ATOL_GRAD)
    for g in range(wl.h_kv):
        keys = ref["keys"][g]
        compare(f"dK head {g}", res["dk"][keys, g], ref["dk"][g], ATOL_GRAD)
        compare(f"dV head {g}", res["dv"][keys, g], ref["dv"][g], ATOL_GRAD)
    compare("O host tier vs resident", host(res["o"]), host(res["o_res"]), 1e-2, rel=1e-2)


def test_host_grads_small_parity_and_accumulation(pkv):
    """Gradient pages in host memory: after one step they hold the oracle's dK/dV (selected and own
    pages, added from the device slots by paged_kv_grad_offload); a second identical step doubles
    them; the device slots end cleared."""
    from paged_kv_cache_fwd_amd.host_tier import HostTierStep
    wl = synth.Workload("host-small", 14, 2, 128, 128, 128 * 24, 384, (7,), offset_std=0.5, seed=22)
    c, top_k, n_local = 7, 6, 2
    n_prior, C, P = wl.n_prior(c), wl.chunk, wl.page
    say("host gradient pages: 24 pages, 21 prior, top-6 + 2 local, two steps")
    bt_np = synth.page_permutation(wl)
    hpool, hbt = fill_pool(pkv, wl, wl.n_pages, bt_np, host_tier=True, host_grads=True)
    step = HostTierStep(hpool, hbt, n_prior, C, wl.h_q, top_k, n_local, torch.device("cuda:0"))
    assert step.host_grads
    k_own, v_own = synth.kv_tokens(wl, n_prior, C // P)
    step.append_own(t16(k_own), t16(v_own))
    q, do = t16(synth.q_chunk(wl, c)), t16(synth.do_chunk(wl, c))
    o, dq = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((wl.h_q, C), dtype=torch.float32, device=q.device)
    hpool.zero_grad()
    sel = step.run(q, do, wl.scale, o, lse, dq)
    torch.cuda.synchronize()
    dk1 = hpool.export(pkv.PKV_DK, hbt, 0, wl.n_pages).cpu().numpy()
    dv1 = hpool.export(pkv.PKV_DV, hbt, 0, wl.n_pages).cpu().numpy()
    step.run(q, do, wl.scale, o, lse, dq)
    torch.cuda.synchronize()
    dk2 = hpool.export(pkv.PKV_DK, hbt, 0, wl.n_pages).cpu().numpy()
    # Two more steps back to back, each re-appending the own block (which clears its device gradient
    # blocks) while the previous step's offload may still be running.
    for _ in range(2):
        step.append_own(t16(k_own), t16(v_own))
        step.run(q, do, wl.scale, o, lse, dq)
    torch.cuda.synchronize()
    dk4 = hpool.export(pkv.PKV_DK, hbt, 0, wl.n_pages).cpu().numpy()
    slots = step.dev.export(pkv.PKV_DK, torch.arange(step.dev.n_pages, dtype=torch.int32, device=q.device), 0,
                            step.dev.n_pages).cpu().numpy()
    hpool.check()
    step.dev.check()
    k, v = synth.kv_tokens(wl, 0, wl.n_pages)
    qn, don = synth.q_chunk(wl, c), synth.do_chunk(wl, c)
    want, _, _ = oracle.topk_pages(qn, k[: n_prior * P], P, wl.h_kv, n_prior, top_k, n_local)
    assert np.array_equal(sel.cpu().numpy(), want)
    ref = oracle.chunk_backward(qn, k, v, don, wl.q0(c), wl.scale, sel=want, page=P)
    for g in range(wl.h_kv):
        keys = ref["keys"][g]
        compare(f"host dK head {g}", dk1[keys, g], ref["dk"][g], ATOL_GRAD)
        compare(f"host dV head {g}", dv1[keys, g], ref["dv"][g], ATOL_GRAD)
        untouched = np.setdiff1d(np.arange(wl.context), keys)
        assert not np.any(dk1[untouched, g]) and not np.any(dv1[untouched, g])
    compare("second step doubles dK", dk2, 2.0 * dk1, 1e-5, rel=1e-5)
    compare("four steps quadruple dK", dk4, 4.0 * dk1, 1e-5, rel=1e-5)
    assert not np.any(slots)
    step.free()
    hpool.free()


@pytest.mark.parametrize("offload", ["staged", "kernel"])
def test_host_grads_back_to_back_steps_with_different_selections(pkv, offload):
    """Gradient pages in host memory over two steps enqueued back to back whose queries, and so page
    selections, differ. The second step selects and gathers while the first step's gradient offload
    may still be running, so the offload must keep reading its own step's selection and device block
    tables: the host pages must hold the sum of the oracle's two results, pages selected by neither
    step none, and every device gradient slot must end cleared."""
    from paged_kv_cache_fwd_amd.host_tier import HostTierStep
    wl = synth.Workload("host-small", 14, 2, 128, 128, 128 * 24, 384, (7,), offset_std=0.5, seed=23)
    wl2 = wl.with_seed(24)  # the second step's queries and output gradients
    c, top_k, n_local = 7, 6, 2
    n_prior, C, P = wl.n_prior(c), wl.chunk, wl.page
    say(f"host gradient pages ({offload} offload): two back-to-back steps with different selections")
    bt_np = synth.page_permutation(wl)
    hpool, hbt = fill_pool(pkv, wl, wl.n_pages, bt_np, host_tier=True, host_grads=True)
    step = HostTierStep(hpool, hbt, n_prior, C, wl.h_q, top_k, n_local, torch.device("cuda:0"), grad_offload=offload)
    k, v = synth.kv_tokens(wl, 0, wl.n_pages)
    step.append_own(t16(k[n_prior * P:]), t16(v[n_prior * P:]))
    hpool.zero_grad()
    qs = [synth.q_chunk(wl, c), synth.q_chunk(wl2, c)]
    dos = [synth.do_chunk(wl, c), synth.do_chunk(wl2, c)]
    outs = []
    for qn, don in zip(qs, dos):
        q, do = t16(qn), t16(don)
        o, dq = torch.empty_like(q), torch.empty_like(q)
        lse = torch.empty((wl.h_q, C), dtype=torch.float32, device=q.device)
        sel = step.run(q, do, wl.scale, o, lse, dq)
        outs.append((sel, q, do, o, dq, lse))  # keep every buffer alive until the end
    torch.cuda.synchronize()
    sels = [o[0].cpu().numpy() for o in outs]
    dk = hpool.export(pkv.PKV_DK, hbt, 0, wl.n_pages).cpu().numpy().astype(np.float64)
    dv = hpool.export(pkv.PKV_DV, hbt, 0, wl.n_pages).cpu().numpy().astype(np.float64)
    slots = step.dev.export(pkv.PKV_DK, torch.arange(step.dev.n_pages, dtype=torch.int32, device="cuda"), 0,
                            step.dev.n_pages).cpu().numpy()
    slots_v = step.dev.export(pkv.PKV_DV, torch.arange(step.dev.n_pages, dtype=torch.int32, device="cuda"), 0,
                              step.dev.n_pages).cpu().numpy()
    hpool.check()
    step.dev.check()
    want_dk = np.zeros_like(dk)
    want_dv = np.zeros_like(dv)
    wants = []
    for qn, don, got in zip(qs, dos, sels):
        want, _, _ = oracle.topk_pages(qn, k[: n_prior * P], P, wl.h_kv, n_prior, top_k, n_local)
        assert np.array_equal(got, want)
        wants.append(want)
        ref = oracle.chunk_backward(qn, k, v, don, wl.q0(c), wl.scale, sel=want, page=P)
        for g in range(wl.h_kv):
            np.add.at(want_dk[:, g], ref["keys"][g], ref["dk"][g])
            np.add.at(want_dv[:, g], ref["keys"][g], ref["dv"][g])
    assert not np.array_equal(wants[0], wants[1]), "the two steps must select different pages"
    for g in range(wl.h_kv):
        compare(f"host dK (two steps) head {g}", dk[:, g], want_dk[:, g], ATOL_GRAD)
        compare(f"host dV (two steps) head {g}", dv[:, g], want_dv[:, g], ATOL_GRAD)
    assert not np.any(dk[want_dk == 0]) and not np.any(dv[want_dv == 0])
    assert not np.any(slots) and not np.any(slots_v)
    step.free()
    hpool.free()


def test_host_tier_lookahead_matches_plain_steps(pkv):
    """Three steps with different queries, each looking ahead to the next one's selection and first
    gather (run(..., next_q=...)), against the same steps run plainly: selections, O, LSE and dQ equal
    bit for bit, and the host gradient pages (staged offload) equal to fp32 atomic-order rounding."""
    from paged_kv_cache_fwd_amd.host_tier import HostTierStep
    wl = synth.Workload("host-small", 14, 2, 128, 128, 128 * 24, 384, (7,), offset_std=0.5, seed=25)
    c, top_k, n_local = 7, 6, 2
    n_prior, C, P = wl.n_prior(c), wl.chunk, wl.page
    say("host tier lookahead: 3 steps with next-step selection and first gather overlapped")
    bt_np = synth.page_permutation(wl)
    k, v = synth.kv_tokens(wl, 0, wl.n_pages)
    qs = [t16(synth.q_chunk(wl.with_seed(s), c)) for s in (25, 26, 27)]
    dos = [t16(synth.do_chunk(wl.with_seed(s), c)) for s in (25, 26, 27)]
    runs = []
    for lookahead in (False, True):
        hpool, hbt = fill_pool(pkv, wl, wl.n_pages, bt_np, host_tier=True, host_grads=True)
        step = HostTierStep(hpool, hbt, n_prior, C, wl.h_q, top_k, n_local, torch.device("cuda:0"))
        step.append_own(t16(k[n_prior * P:]), t16(v[n_prior * P:]))
        hpool.zero_grad()
        outs = []
        for i, (q, do) in enumerate(zip(qs, dos)):
            o, dq = torch.empty_like(q), torch.empty_like(q)
            lse = torch.empty((wl.h_q, C), dtype=torch.float32, device=q.device)
            nxt = qs[i + 1] if lookahead and i + 1 < len(qs) else None
            sel = step.run(q, do, wl.scale, o, lse, dq, next_q=nxt)
            outs.append((sel.clone(), o, lse, dq))
        torch.cuda.synchronize()
        dk = hpool.export(pkv.PKV_DK, hbt, 0, wl.n_pages).cpu().numpy()
        hpool.check()
        step.dev.check()
        runs.append((outs, dk))
        step.free()
        hpool.free()
    (plain, dk0), (ahead, dk1) = runs
    for i, (a, b) in enumerate(zip(plain, ahead)):
        for name, x, y in zip(("selection", "O", "LSE", "dQ"), a, b):
            assert torch.equal(x, y), f"step {i}: {name} differs with the lookahead"
    compare("host dK, lookahead vs plain", dk1, dk0, 1e-5, rel=1e-5)


def test_dense_layer_prefetch_matches_resident(pkv):
    """Two layers whose KV and gradient pages live in pinned host memory, run dense with the next
    layer's pages copied in (and the last one's gradients copied home) beside each step. O, LSE and
    dQ must equal the device-resident results bit for bit (the same kernels read the same bytes at
    the same physical pages); the host gradient pages must hold the oracle's dK/dV after one step
    per layer and twice that after two."""
    from paged_kv_cache_fwd_amd.host_tier import DenseLayerPrefetch
    c = 7
    wls = [synth.Workload("dense-host", 14, 2, 128, 128, 128 * 24, 384, (c,), offset_std=0.5, seed=s)
           for s in (31, 32)]
    say("dense layer prefetch: 2 layers x 24 pages (21 prior + 3 own) in pinned host memory, 4 steps")
    n_prior, C, P = wls[0].n_prior(c), wls[0].chunk, wls[0].page
    dev = torch.device("cuda:0")
    res, hosts, bts, inputs = [], [], [], []
    for wl in wls:
        bt_np = synth.page_permutation(wl)
        dpool, dbt = fill_pool(pkv, wl, wl.n_pages, bt_np)
        q, do = t16(synth.q_chunk(wl, c)), t16(synth.do_chunk(wl, c))
        o, lse = pkv.chunk_attn_fwd(dpool, dbt, n_prior, q, wl.scale)
        dq = pkv.chunk_attn_bwd(dpool, dbt, n_prior, q, o, do, lse, wl.scale)
        hp = pkv.Pool(wl.n_pages, P, wl.h_kv, wl.d, grads=True, host_tier=True, host_grads=True)
        pkv.paged_kv_copy(dpool, hp, pkv.PKV_COPY_KV)
        torch.cuda.synchronize()
        res.append(dict(o=o, lse=lse, dq=dq, dk=dpool.export(pkv.PKV_DK, dbt, 0, wl.n_pages).cpu().numpy()))
        dpool.free()
        hosts.append(hp)
        bts.append(dbt)
        inputs.append((q, do))
    run = DenseLayerPrefetch(hosts, dev)
    outs = []

    def step(layer, nxt):
        wl = wls[layer]
        q, do = inputs[layer]
        o, dq = torch.empty_like(q), torch.empty_like(q)
        lse = torch.empty((wl.h_q, C), dtype=torch.float32, device=dev)
        run.run(layer, nxt, bts[layer], n_prior, q, do, wl.scale, o, lse, dq)
        outs.append((layer, o, lse, dq))

    step(0, 1)
    step(1, 0)
    torch.cuda.synchronize()
    once = [(h.export(pkv.PKV_DK, bt, 0, h.n_pages).cpu().numpy(), h.export(pkv.PKV_DV, bt, 0, h.n_pages).cpu().numpy())
            for h, bt in zip(hosts, bts)]
    step(0, 1)
    step(1, None)
    torch.cuda.synchronize()
    twice = [h.export(pkv.PKV_DK, bt, 0, h.n_pages).cpu().numpy() for h, bt in zip(hosts, bts)]
    for h in hosts:
        h.check()
    for i, (layer, o, lse, dq) in enumerate(outs):
        r = res[layer]
        assert torch.equal(o, r["o"]), f"step {i}: O differs from the resident result"
        assert torch.equal(lse, r["lse"]), f"step {i}: LSE differs"
        assert torch.equal(dq, r["dq"]), f"step {i}: dQ differs"
    for layer, wl in enumerate(wls):
        k, v = synth.kv_tokens(wl, 0, wl.n_pages)
        ref = oracle.chunk_backward(synth.q_chunk(wl, c), k, v, synth.do_chunk(wl, c), wl.q0(c), wl.scale)
        dk1, dv1 = once[layer]
        for g in range(wl.h_kv):
            keys = ref["keys"][g]
            compare(f"layer {layer} host dK head {g}", dk1[keys, g], ref["dk"][g], ATOL_GRAD)
            compare(f"layer {layer} host dV head {g}", dv1[keys, g], ref["dv"][g], ATOL_GRAD)
        compare(f"layer {layer} host dK vs resident", dk1, res[layer]["dk"], 1e-5, rel=1e-5)
        compare(f"layer {layer} second step doubles dK", twice[layer], 2.0 * dk1, 1e-5, rel=1e-5)
    run.free()
    for h in hosts:
        h.free()


def test_host_tier_1m_matches_resident(pkv):
    """1M tokens: 8192 pages (8160 prior) in pinned host memory, top-128 + 8 local."""
    wl = synth.WORKLOADS["host1m"]
    c = wl.chunks[0]
    say("host tier 1M: generating and filling 8192 pages (host tier and device-resident)")
    res = _run_host_tier(pkv, wl, c, wl.top_k, wl.n_local)
    assert res["sel"].shape == (wl.h_kv, 136)
    # Bit-exact selection against the oracle, reps computed page batch by page batch.
    n_prior = wl.n_prior(c)
    reps = []
    for p0 in range(0, n_prior, 1024):
        kk, _ = synth.kv_tokens(wl, p0, min(1024, n_prior - p0))
        reps.append(oracle.page_reps(oracle.page_key_sums(kk, wl.page), wl.page))
    reps = np.concatenate(reps)
    q = synth.q_chunk(wl, c)
    n_cand = n_prior - wl.n_local
    sc = oracle.page_scores(oracle.query_sum(q, wl.h_kv), reps[:n_cand])
    want = oracle.select_pages(sc, n_prior, wl.top_k, wl.n_local)
    assert np.array_equal(res["sel"], want)
    # Gathered slots compute exactly what resident pages compute (same kernels, same bytes); the
    # per-head calls may split key ranges differently, so compare to tolerance.
    compare("O host tier vs resident", host(res["o"]), host(res["o_res"]), 1e-2, rel=1e-2)
    compare("LSE host tier vs resident", res["lse"].cpu().numpy(), res["lse_res"].cpu().numpy(), 1e-4, rel=1e-5)
    compare("dQ host tier vs resident", host(res["dq"]), host(res["dq_res"]), 1e-2, rel=1e-2)
    compare("dK host tier vs resident", res["dk"], res["dk_res"], 1e-3, rel=1e-3)
    # Sampled rows against the oracle.
    rows = np.array([0, 1, 1000, 2047, 4095])
    sel_pages = want
    pages_needed = sorted(set(sel_pages.reshape(-1).tolist()) | set(range(n_prior, wl.n_pages)))
    # Build a compacted sequence: selected prior pages (per head they differ) are handled by the oracle
    # on the full logical index space, so materialise only the pages it reads.
    k_full = np.zeros((wl.context, wl.h_kv, wl.d), np.uint16)
    v_full = np.zeros_like(k_full)
    for p in pages_needed:
        k_full[p * wl.page:(p + 1) * wl.page] = synth.k_page(wl, p)
        v_full[p * wl.page:(p + 1) * wl.page] = synth.v_page(wl, p)
    ref = oracle.chunk_backward(q, k_full, v_full, synth.do_chunk(wl, c), wl.q0(c), wl.scale, sel=sel_pages,
                                page=wl.page, rows=rows, dtype=np.float32)
    compare("O rows", host(res["o"])[rows], ref["o"], ATOL_O)
    compare("dQ rows", host(res["dq"])[rows], ref["dq"], ATOL_GRAD)
    # LSE of every row and dK/dV of sampled selected pages and the last own page over all rows, for
    # two KV heads, against the oracle (its float32 statistics of every row of the head).
    do = synth.do_chunk(wl, c)
    G, P, q0 = wl.group, wl.page, wl.q0(c)
    for g in (0, 3):
        say(f"host tier 1M: oracle statistics of all rows of KV head {g} over its {len(sel_pages[g])} pages")
        qg, dog = q[:, g * G:(g + 1) * G], do[:, g * G:(g + 1) * G]
        o_g, lse_g = oracle.chunk_forward(qg, k_full[:, g:g + 1], v_full[:, g:g + 1], q0, wl.scale, sel=[sel_pages[g]],
                                          page=P, dtype=np.float32)
        compare(f"LSE head {g} all rows", res["lse"].cpu().numpy()[g * G:(g + 1) * G], lse_g, ATOL_LSE, rel=1e-5)
        dd_g = np.einsum("thd,thd->ht", synth.bf16_widen(dog).astype(np.float32), o_g)
        picked = [sel_pages[g][i] for i in (0, 40, 90, len(sel_pages[g]) - 1)] + [wl.n_pages - 1]
        toks = np.concatenate([np.arange(p * P, (p + 1) * P) for p in picked])
        r = oracle.key_gradients(qg, k_full[:, g:g + 1], v_full[:, g:g + 1], dog, q0, wl.scale, {0: toks}, lse_g, dd_g,
                                 dtype=np.float32)[0]
        compare(f"dK pages {picked} head {g}", res["dk"][toks, g], r[0], ATOL_GRAD)
        compare(f"dV pages {picked} head {g}", res["dv"][toks, g], r[1], ATOL_GRAD)


def test_paged_kv_copy_rejects_bad_arguments(pkv):
    """Copies between pools are refused before anything is enqueued when shapes, ranges or the
    gradient pages do not fit, and a valid copy moves exactly the requested physical pages."""
    a = pkv.Pool(6, 64, 2, 64, grads=True)
    b = pkv.Pool(6, 64, 2, 64, grads=False)
    c = pkv.Pool(6, 64, 1, 64, grads=True)
    h = pkv.Pool(6, 64, 2, 64, grads=True, host_tier=True, host_grads=True)
    bt = i32(np.arange(6))
    k = torch.randn(6 * 64, 2, 64, device="cuda").to(torch.bfloat16)
    a.append(bt, 0, k, k)
    with pytest.raises(pkv.PkvError):
        pkv.paged_kv_copy(a, c, pkv.PKV_COPY_KV)           # head count differs
    with pytest.raises(pkv.PkvError):
        pkv.paged_kv_copy(a, b, pkv.PKV_COPY_GRAD)         # destination has no gradient pages
    with pytest.raises(pkv.PkvError):
        pkv.paged_kv_copy(a, h, pkv.PKV_COPY_KV, 4, 3)     # pages [4, 7) outside both pools
    with pytest.raises(pkv.PkvError):
        pkv.paged_kv_copy(a, a, pkv.PKV_COPY_KV)           # same pool
    with pytest.raises(pkv.PkvError):
        pkv.paged_kv_copy(a, h, 8)                         # unknown bit
    pkv.paged_kv_copy(a, h, pkv.PKV_COPY_KV, 2, 3)         # physical pages 2..4 only
    torch.cuda.synchronize()
    got = h.export(pkv.PKV_K, bt, 0, 6).cpu()
    want = a.export(pkv.PKV_K, bt, 0, 6).cpu()
    assert torch.equal(got[2 * 64:5 * 64], want[2 * 64:5 * 64])
    assert not torch.any(got[:2 * 64].float()) and not torch.any(got[5 * 64:].float())
    with pytest.raises(ValueError):
        pkv.chunk_attn_fwd(a, bt, 2, k[:128].contiguous(), 0.1, sel=i32(np.zeros((2, 1, 1, 1))))
    for p in (a, b, c, h):
        p.free()


@pytest.mark.parametrize("n_wg", [1, 2, 3, 0, 64])
def test_gather_workgroup_counts(pkv, n_wg):
    """paged_kv_gather moves the same blocks and writes the same device block table whatever number of
    workgroups copies them (0: the default, 8); the blocks match the appended K/V bit for bit."""
    wl = synth.Workload("gather-wg", 14, 2, 128, 128, 128 * 24, 384, (7,), offset_std=0.5, seed=22)
    n, P, kvh = wl.n_pages, wl.page, 1
    say(f"gather: 10 of {n} host pages, head {kvh}, n_workgroups={n_wg}")
    hpool, hbt = fill_pool(pkv, wl, n, synth.page_permutation(wl), host_tier=True)
    rng = np.random.default_rng(5)
    sel_np = np.sort(rng.choice(n, 10, replace=False)).astype(np.int32)
    dst_np = rng.permutation(14)[:10].astype(np.int32)  # device pages 14 and 15 stay unused
    dpool = pkv.Pool(16, P, wl.h_kv, wl.d, grads=False)
    dev_bt = torch.full((n,), 15, dtype=torch.int32, device="cuda:0")
    pkv.paged_kv_gather(hpool, dpool, hbt, i32(sel_np), kvh, i32(dst_np), dev_bt_out=dev_bt, n_workgroups=n_wg)
    torch.cuda.synchronize()
    hpool.check()
    dpool.check()
    want_bt = np.full(n, 15, np.int32)
    want_bt[sel_np] = dst_np
    assert np.array_equal(dev_bt.cpu().numpy(), want_bt)
    k, v = synth.kv_tokens(wl, 0, n)
    rows = (sel_np[:, None] * P + np.arange(P)[None, :]).reshape(-1)
    for what, ref in ((pkv.PKV_K, k), (pkv.PKV_V, v)):
        got = dpool.export(what, dev_bt, 0, n).view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got[rows, kvh], np.ascontiguousarray(ref).view(np.uint16)[rows, kvh])
    with pytest.raises(RuntimeError):
        pkv.paged_kv_gather(hpool, dpool, hbt, i32(sel_np), kvh, i32(dst_np), n_workgroups=65)
    dpool.free()
    hpool.free()
