"""Library calls captured in a HIP graph (through torch.cuda.CUDAGraph): one whole sparse training
step (gradient zeroing, append, page selection, forward, backward) recorded once and replayed. Every
replay, with eager work and synchronisations between replays, must reproduce the eager step: O, LSE,
dQ and the selection bit for bit (their kernels have a fixed summation order), the gradient pages to
float32 rounding (they are summed with atomics in any order)."""
import numpy as np
import pytest

import synth
from gpu_util import fill_pool, say, t16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_fwd_amd as m
    m.load()
    return m


@pytest.mark.parametrize("top_k,n_local", [(6, 2), (None, 0)])
def test_graph_replayed_step_matches_eager(pkv, top_k, n_local):
    wl = synth.Workload("graph", 14, 2, 128, 128, 384 * 8, 384, (7,), offset_std=0.5, seed=31)
    c = wl.chunks[0]
    C, P, q0, n_prior = wl.chunk, wl.page, wl.q0(c), wl.n_prior(c)
    bt_np = synth.page_permutation(wl)
    pool, bt = fill_pool(pkv, wl, n_prior, bt_np)
    k, v = synth.kv_tokens(wl, n_prior, C // P)
    k_own, v_own = t16(k), t16(v)
    q, do = t16(synth.q_chunk(wl, c)), t16(synth.do_chunk(wl, c))
    dev = q.device
    o, dq = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((wl.h_q, C), dtype=torch.float32, device=dev)
    sparse = top_k is not None
    n_sel = min(top_k, n_prior - n_local) + n_local if sparse else n_prior
    sel = torch.empty((wl.h_kv, n_sel), dtype=torch.int32, device=dev)
    lib = pkv.load()
    ws_f = torch.empty(max(pkv.chunk_attn_fwd_ws_bytes(pool, n_prior, n_sel if sparse else -1, wl.h_kv, C, wl.h_q),
                           1), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(pkv.chunk_attn_bwd_ws_bytes(pool, n_prior, n_sel if sparse else -1, wl.h_kv, C, wl.h_q),
                           1), dtype=torch.uint8, device=dev)
    ws_t = torch.empty(max(lib.page_topk_ws_bytes(pool.handle, n_prior, C, wl.h_q, 1), 1), dtype=torch.uint8,
                       device=dev)

    def step():
        pool.zero_grad()
        pool.append(bt, q0, k_own, v_own)
        s = pkv.page_topk_select(pool, bt, n_prior, q, top_k, n_local, sel=sel, ws=ws_t) if sparse else None
        pkv.chunk_attn_fwd(pool, bt, n_prior, q, wl.scale, sel=s, o=o, lse=lse, ws=ws_f)
        pkv.chunk_attn_bwd(pool, bt, n_prior, q, o, do, lse, wl.scale, sel=s, dq=dq, ws=ws_b)

    def snapshot():
        dk = pool.export(pkv.PKV_DK, bt, 0, wl.n_pages)
        dv = pool.export(pkv.PKV_DV, bt, 0, wl.n_pages)
        torch.cuda.synchronize()
        return {"o": o.clone(), "lse": lse.clone(), "dq": dq.clone(), "sel": sel.clone(), "dk": dk, "dv": dv}

    say(f"case graph step: {'top-%d + %d local' % (top_k, n_local) if sparse else 'dense'}, 14/2 heads, "
        f"{n_prior} prior pages")
    step()
    want = snapshot()
    pool.check()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        o.zero_()
        dq.zero_()
        lse.fill_(float("nan"))
        sel.fill_(-1)
        g.replay()
        got = snapshot()
        pool.check()
        for name in ("o", "lse", "dq") + (("sel",) if sparse else ()):
            assert torch.equal(got[name], want[name]), (r, name)
        for name in ("dk", "dv"):
            a, b = got[name].double(), want[name].double()
            rel = float((a - b).norm() / b.norm())
            say(f"  replay {r}: {name} relative difference to eager {rel:.2e}")
            assert rel < 1e-5, (r, name, rel)
        # Eager work between replays.
        torch.cuda.synchronize()
        _ = (o.float() * 2).sum().item()
    pool.free()
