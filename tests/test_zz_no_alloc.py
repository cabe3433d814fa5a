"""page_topk_select_noalloc (static scratch, no allocation) against page_topk_select (caller's
workspace) through the C ABI: bit-identical selections on two calls in a row, the second with a
smaller input (fewer prior pages, a shorter chunk, a smaller K), for one list per KV head and one
per query page, and a request beyond the static scratch refused with nothing written."""
import ctypes

import numpy as np
import pytest

import synth
from gpu_util import i32, say, t16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_fwd_amd as m
    m.load()
    return m


def _noalloc(pkv, pool, bt, n_prior, q, top_k, n_local, n_lists, sel):
    """Direct C-ABI call of page_topk_select_noalloc on the current stream; returns (status, n_sel)."""
    lib = pkv.load()
    n_out = ctypes.c_int32(-1)
    rc = lib.page_topk_select_noalloc(pool.handle, ctypes.c_void_p(bt.data_ptr()), bt.numel(), n_prior,
                                      ctypes.c_void_p(q.data_ptr()), q.shape[0], q.shape[1], top_k, n_local, n_lists,
                                      ctypes.c_void_p(sel.data_ptr()), ctypes.byref(n_out),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc, n_out.value


def test_noalloc_selection_matches_workspace_selection(pkv):
    wl = synth.Workload("noalloc", 28, 4, 128, 128, 128 * 1032, 4096, (250,), offset_std=0.5, seed=41)
    n_pages = wl.n_pages
    say(f"noalloc selection: pool of {n_pages} pages (28/4 heads, d=128, page 128)")
    bt_np = synth.page_permutation(wl)
    pool = pkv.Pool(n_pages, wl.page, wl.h_kv, wl.d, grads=False)
    bt = i32(bt_np)
    for p0 in range(0, n_pages, 512):
        n = min(512, n_pages - p0)
        k, v = synth.kv_tokens(wl, p0, n)
        pool.append(bt, p0 * wl.page, t16(k), t16(v))
    q_full = t16(synth.q_chunk(wl, 250))
    # (n_prior, chunk tokens, top_k, n_local): a large call, then a smaller one right after it.
    cases = [(1000, 4096, 64, 4), (300, 2048, 16, 2)]
    for per_query_page in (False, True):
        for n_prior, C, top_k, n_local in cases:
            q = q_full[:C].contiguous()
            n_lists = C // wl.page if per_query_page else 1
            n_cand = max(n_prior - n_local, 0)
            n_sel = min(top_k, n_cand) + (n_prior - n_cand)
            shape = (wl.h_kv, n_lists, n_sel) if per_query_page else (wl.h_kv, n_sel)
            say(f"  n_prior {n_prior}, C {C}, top-{top_k} + {n_local}, lists {n_lists}")
            ref = pkv.page_topk_select(pool, bt, n_prior, q, top_k, n_local, per_query_page=per_query_page,
                                       ws=torch.empty(pkv.page_topk_ws_bytes(pool, n_prior, C, wl.h_q, n_lists),
                                                      dtype=torch.uint8, device="cuda"))
            got = torch.full(shape, -7, dtype=torch.int32, device="cuda")
            rc, n_out = _noalloc(pkv, pool, bt, n_prior, q, top_k, n_local, n_lists, got)
            assert rc == 0, pkv.load().pkv_last_error()
            assert n_out == n_sel
            torch.cuda.synchronize()
            assert torch.equal(got.cpu(), ref.cpu()), "static-scratch selection differs from the workspace one"
            # The same call again through the binding (the scratch now holds the previous contents).
            got2 = pkv.page_topk_select_noalloc(pool, bt, n_prior, q, top_k, n_local,
                                                torch.zeros(shape, dtype=torch.int32, device="cuda"),
                                                per_query_page=per_query_page)
            torch.cuda.synchronize()
            assert torch.equal(got2.cpu(), ref.cpu())
    # Beyond the static scratch (the query partial sums of a 2^17-token chunk of 28 heads alone take
    # 29 MB): refused before anything is enqueued, the output untouched.
    lib = pkv.load()
    need = lib.page_topk_ws_bytes(pool.handle, 1000, 1 << 17, wl.h_q, 1)
    assert need > (16 << 20)
    big_q = torch.zeros((1 << 17, wl.h_q, wl.d), dtype=torch.bfloat16, device="cuda")
    sel = torch.full((wl.h_kv, 68), -7, dtype=torch.int32, device="cuda")
    rc, _ = _noalloc(pkv, pool, bt, 1000, big_q, 64, 4, 1, sel)
    assert rc == pkv.PKV_E_NOMEM and b"scratch" in lib.pkv_last_error()
    torch.cuda.synchronize()
    assert torch.all(sel == -7)
    pool.check()
    pool.free()
