"""GPU parity for local-only and mixed layer policies (it 2.D: natively sparse models keep recent
pages; pt 2.C: top-K pages approximate dense attention). A local layer selects no top-K page, only
the n_local most recent prior pages (plus the causal own block); the other layers use top-K. The
selection runs through page_topk_select on the device and is compared bit for bit with the oracle,
then forward and backward over it are compared with the oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import ATOL_GRAD, ATOL_LSE, ATOL_O, compare, fill_pool, host, say, scatter_grads, t16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_fwd_amd as m
    m.load()
    return m


def _wl(seed, G=7, h_kv=2, C=384, chunks=(0, 1, 2, 3), d=128, page=128):
    return synth.Workload("layers", G * h_kv, h_kv, d, page, C * len(chunks), C, tuple(chunks), offset_std=0.5,
                          seed=seed)


def _layer(pkv, wl, top_k, n_local):
    """All chunks of one layer in order: device selection, forward, backward."""
    pool, bt = fill_pool(pkv, wl, wl.n_pages, synth.page_permutation(wl))
    outs = []
    for c in wl.chunks:
        n_prior = wl.n_prior(c)
        q = t16(synth.q_chunk(wl, c))
        sel = pkv.page_topk_select(pool, bt, n_prior, q, top_k, n_local)
        o, lse = pkv.chunk_attn_fwd(pool, bt, n_prior, q, wl.scale, sel=sel)
        dq = pkv.chunk_attn_bwd(pool, bt, n_prior, q, o, t16(synth.do_chunk(wl, c)), lse, wl.scale, sel=sel)
        outs.append((c, sel.cpu().numpy(), host(o), lse.cpu().numpy(), host(dq)))
    dk = pool.export(pkv.PKV_DK, bt, 0, wl.n_pages).cpu().numpy()
    dv = pool.export(pkv.PKV_DV, bt, 0, wl.n_pages).cpu().numpy()
    torch.cuda.synchronize()
    pool.check()
    pool.free()
    return outs, dk, dv


def _check(wl, outs, dk, dv, top_k, n_local):
    k, v = synth.kv_tokens(wl, 0, wl.n_pages)
    dk_ref = np.zeros((wl.context, wl.h_kv, wl.d))
    dv_ref = np.zeros_like(dk_ref)
    for c, sel, o, lse, dq in outs:
        n_prior = wl.n_prior(c)
        q, do = synth.q_chunk(wl, c), synth.do_chunk(wl, c)
        if n_prior > 0:
            want, _, _ = oracle.topk_pages(q, k[: n_prior * wl.page], wl.page, wl.h_kv, n_prior, top_k, n_local)
        else:
            want = np.zeros((wl.h_kv, 0), np.int32)
        say(f"chunk {c}: selection {want.tolist()}")
        assert np.array_equal(sel, want)
        ref = oracle.chunk_backward(q, k, v, do, wl.q0(c), wl.scale, sel=want, page=wl.page)
        compare("O", o, ref["o"], ATOL_O)
        compare("LSE", lse, ref["lse"], ATOL_LSE, rel=1e-5)
        compare("dQ", dq, ref["dq"], ATOL_GRAD)
        a, b = scatter_grads(ref, wl.context, wl.h_kv, wl.d)
        dk_ref += a
        dv_ref += b
    compare("dK", dk, dk_ref, ATOL_GRAD)
    compare("dV", dv, dv_ref, ATOL_GRAD)


def test_local_window_layer(pkv):
    """top_k = 0, n_local = 2: each chunk sees the 2 most recent prior pages and its own block."""
    wl = _wl(seed=30)
    say("local layer: 14/2 heads, C=384, window 2 pages + own block")
    outs, dk, dv = _layer(pkv, wl, top_k=0, n_local=2)
    for c, sel, *_ in outs:
        n_prior = wl.n_prior(c)
        assert sel.tolist() == [list(range(max(n_prior - 2, 0), n_prior))] * wl.h_kv
    _check(wl, outs, dk, dv, 0, 2)


def test_own_block_only_layer(pkv):
    """top_k = 0, n_local = 0: no prior page at all, only the causal own block."""
    wl = _wl(seed=31, chunks=(0, 1, 2))
    say("own-block-only layer")
    outs, dk, dv = _layer(pkv, wl, top_k=0, n_local=0)
    assert all(sel.shape == (wl.h_kv, 0) for _, sel, *_ in outs)
    _check(wl, outs, dk, dv, 0, 0)


def test_mixed_layer_pair(pkv):
    """A local layer (window 1) and a top-K layer (K = 2 plus 1 recent page) over their own caches."""
    say("mixed pair: local window 1, then top-2 + 1 local")
    wa = _wl(seed=32)
    outs, dk, dv = _layer(pkv, wa, top_k=0, n_local=1)
    _check(wa, outs, dk, dv, 0, 1)
    wb = _wl(seed=33)
    outs, dk, dv = _layer(pkv, wb, top_k=2, n_local=1)
    _check(wb, outs, dk, dv, 2, 1)
