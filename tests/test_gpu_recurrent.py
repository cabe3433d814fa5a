"""GPU test of the chunk-recurrent driver: one attention layer trained chunk by chunk (forward in
order, backward in reverse with recomputation, K/V and their gradients in pages outside autograd)
against the same layer run over the whole sequence with ordinary autograd in float64 on the CPU.

The reference rounds q, k, v and O to bf16 exactly where the driver does (straight-through in
backward), so the remaining differences are the kernels' bf16 probabilities and bf16 dQ/dK/dV."""
import math

import numpy as np
import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def rec():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_fwd_amd as m
    m.load()
    from paged_kv_cache_fwd_amd import recurrent
    return recurrent


def _bf16(t):
    """Round to bf16 in the forward, identity in the backward."""
    return t + (t.to(torch.bfloat16).to(t.dtype) - t).detach()


def _reference(layer, xs, rs, sels):
    """Whole-sequence loss and gradients (float64, CPU) with the driver's page selections."""
    W = {n: getattr(layer, n).detach().cpu().double().requires_grad_(True) for n in ("wq", "wk", "wv", "wo")}
    x = torch.cat([xi.cpu().double() for xi in xs]).requires_grad_(True)
    L, C, P, G = x.shape[0], layer.chunk, layer.page, layer.h_q // layer.h_kv
    q = _bf16(x @ W["wq"]).view(L, layer.h_q, layer.d)
    k = _bf16(x @ W["wk"]).view(L, layer.h_kv, layer.d)
    v = _bf16(x @ W["wv"]).view(L, layer.h_kv, layer.d)
    pos = torch.arange(L)
    allowed = pos[None, :] <= pos[:, None]  # [query][key] causal
    masks = []
    for g in range(layer.h_kv):
        m = allowed.clone()
        for i, sel in enumerate(sels):
            if sel is None:
                continue
            rows = slice(i * C, (i + 1) * C)
            prior_ok = torch.zeros(L, dtype=torch.bool)
            for p in sel[g].tolist():
                prior_ok[p * P:(p + 1) * P] = True
            own = (pos >= i * C) & (pos < (i + 1) * C)
            m[rows] &= (prior_ok | own)[None, :]
        masks.append(m)
    outs = []
    for h in range(layer.h_q):
        g = h // G
        s = (q[:, h] @ k[:, g].T) * layer.scale
        s = s.masked_fill(~masks[g], float("-inf"))
        outs.append(torch.softmax(s, dim=-1) @ v[:, g])
    o = _bf16(torch.stack(outs, dim=1))
    y = o.reshape(L, -1) @ W["wo"]
    terms = [y[i * C:(i + 1) * C] * rs[i].cpu().double() for i in range(len(xs))]
    loss = sum(t.sum() for t in terms)
    magnitude = sum(t.abs().sum().item() for t in terms)
    loss.backward()
    return loss.item(), magnitude, {n: w.grad for n, w in W.items()}, x.grad


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)


def _run(rec, top_k=None, n_local=0, seed=0):
    d_model, h_q, h_kv, d, page, chunk, n_chunks = 96, 4, 2, 64, 64, 128, 4
    layer = rec.ChunkRecurrentAttention(d_model, h_q, h_kv, d, page, chunk, chunk * n_chunks, top_k=top_k,
                                        n_local=n_local, seed=seed)
    g = torch.Generator().manual_seed(100 + seed)
    xs = [torch.randn(chunk, d_model, generator=g).cuda() for _ in range(n_chunks)]
    rs = [torch.randn(chunk, d_model, generator=g).cuda() / math.sqrt(chunk) for _ in range(n_chunks)]
    loss, dxs = layer.train_step(xs, lambda y, i: (y * rs[i]).sum())
    torch.cuda.synchronize()
    layer.pool.check()
    sels = [None if s is None else s.cpu() for s in layer.last_selection]
    ref_loss, magnitude, ref_grads, ref_dx = _reference(layer, xs, rs, sels)
    say(f"loss {loss.item():.6f} vs reference {ref_loss:.6f} (sum of |terms| {magnitude:.1f})")
    # The loss is a sum of ~5e4 terms of either sign; bound its error by the terms' total size.
    assert abs(loss.item() - ref_loss) <= 1e-3 * magnitude
    for n, rg in ref_grads.items():
        e = _rel(getattr(layer, n).grad.cpu(), rg)
        say(f"  d{n}: rel-fro {e:.2e}")
        assert e < 2e-2
    e = _rel(torch.cat(dxs).cpu(), ref_dx)
    say(f"  dx: rel-fro {e:.2e}")
    assert e < 2e-2
    layer.free()


def test_recurrent_dense(rec):
    say("chunk-recurrent layer, 4 chunks of 128 tokens, dense")
    _run(rec)


def test_recurrent_topk(rec):
    say("chunk-recurrent layer, 4 chunks, top-1 page + 1 local page per KV head")
    _run(rec, top_k=1, n_local=1, seed=1)
