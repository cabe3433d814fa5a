"""Chunk-recurrent training of one attention layer over the paged KV cache.

"Out of the Memory Barrier" summaries: pt 2.A / es 2.A / it 2.A (the sequence is split into chunks;
a chunk's activations are dropped after its forward and recomputed on demand in backward, so only
the KV cache grows with the context), pt 2.B / es 2.B / it 2.B (the KV cache and its gradients live
in pages outside autograd; custom kernels add the gradients in place).

Forward: the chunks run in order with no autograd graph. Each projects its queries, keys and
values, appends K/V to its pages and attends to the cache (library forward); its loss is summed and
everything but the paged cache (and the chunk's page selection, if sparse) is dropped.

Backward: the chunks run in reverse order. Each recomputes its projections under autograd and
calls PagedChunkAttention, whose forward is the library forward again and whose backward is the
library backward: it returns dQ and adds dK/dV to every page the chunk attended to. All later
chunks have run by then, so the chunk's own pages hold its complete dK/dV; they are read back and
returned as the gradients of the chunk's keys and values, which autograd carries into the
projection weights and the chunk's input.

Torch supplies the projections (matrix products) and the autograd plumbing around the attention;
every attention step runs in the library.
"""
from __future__ import annotations

import math
from typing import Callable, List, Optional, Sequence

import torch

from . import (PKV_DK, PKV_DV, Pool, chunk_attn_bwd, chunk_attn_bwd_ws_bytes, chunk_attn_fwd, chunk_attn_fwd_ws_bytes,
               page_topk_select, page_topk_ws_bytes)


class PagedChunkAttention(torch.autograd.Function):
    """Attention of one chunk over the paged cache; its own K/V must already be in the pages.

    Inputs q [C][H_q][d], k and v [C][H_kv][d] (bf16). k and v only route gradients: the kernels
    read the pages. The backward must run after every later chunk's backward (reverse order)."""

    @staticmethod
    def forward(ctx, q, k, v, layer, n_prior, sel):
        o, lse = chunk_attn_fwd(layer.pool, layer.bt, n_prior, q, layer.scale, sel=sel, ws=layer.ws_f)
        ctx.save_for_backward(q, o, lse)
        ctx.layer, ctx.n_prior, ctx.sel = layer, n_prior, sel
        return o

    @staticmethod
    def backward(ctx, do):
        q, o, lse = ctx.saved_tensors
        layer, n_prior, sel = ctx.layer, ctx.n_prior, ctx.sel
        dq = chunk_attn_bwd(layer.pool, layer.bt, n_prior, q, o, do.to(torch.bfloat16).contiguous(), lse,
                            layer.scale, sel=sel, ws=layer.ws_b)
        C = q.shape[0]
        n_own = C // layer.page
        shape = (C, layer.h_kv, layer.d)
        dk = layer.pool.export(PKV_DK, layer.bt, n_prior, n_own).view(shape)
        dv = layer.pool.export(PKV_DV, layer.bt, n_prior, n_own).view(shape)
        return dq, dk.to(torch.bfloat16), dv.to(torch.bfloat16), None, None, None


class ChunkRecurrentAttention(torch.nn.Module):
    """One attention layer (GQA, head size d) trained chunk by chunk over a paged KV cache.

    Projections: q = x Wq, k = x Wk, v = x Wv (float32 weights, results rounded to bf16), then
    y = O Wo. top_k None = dense attention over all earlier keys; otherwise each chunk attends to
    its top-K prior pages plus the n_local most recent ones and its own block."""

    def __init__(self, d_model: int, h_q: int, h_kv: int, d: int, page: int, chunk: int, context: int,
                 top_k: Optional[int] = None, n_local: int = 0, device=None, seed: int = 0):
        super().__init__()
        assert chunk % page == 0 and context % chunk == 0 and h_q % h_kv == 0
        self.d_model, self.h_q, self.h_kv, self.d = d_model, h_q, h_kv, d
        self.page, self.chunk, self.context = page, chunk, context
        self.top_k, self.n_local = top_k, n_local
        self.scale = 1.0 / math.sqrt(d)
        device = torch.device(device or "cuda:0")
        g = torch.Generator().manual_seed(seed)

        def w(rows, cols):
            return torch.nn.Parameter((torch.randn(rows, cols, generator=g) / math.sqrt(rows)).to(device))

        self.wq, self.wk, self.wv = w(d_model, h_q * d), w(d_model, h_kv * d), w(d_model, h_kv * d)
        self.wo = w(h_q * d, d_model)
        self.n_pages = context // page
        self.pool = Pool(self.n_pages, page, h_kv, d, grads=True)
        self.bt = torch.arange(self.n_pages, dtype=torch.int32, device=device)
        # Workspaces sized once for the largest call of any chunk position, so the steps allocate
        # nothing in the library calls.
        per_chunk = chunk // page
        fb = bb = tb = 1
        for n_prior in range(0, self.n_pages - per_chunk + 1, per_chunk):
            n_sel = -1
            if top_k is not None:
                n_cand = max(n_prior - n_local, 0)
                n_sel = min(top_k, n_cand) + (n_prior - n_cand)
                tb = max(tb, page_topk_ws_bytes(self.pool, n_prior, chunk, h_q))
            fb = max(fb, chunk_attn_fwd_ws_bytes(self.pool, n_prior, n_sel, h_kv, chunk, h_q))
            bb = max(bb, chunk_attn_bwd_ws_bytes(self.pool, n_prior, n_sel, h_kv, chunk, h_q))
        self.ws_f = torch.empty(fb, dtype=torch.uint8, device=device)
        self.ws_b = torch.empty(bb, dtype=torch.uint8, device=device)
        self.ws_t = torch.empty(tb, dtype=torch.uint8, device=device)

    def qkv(self, x: torch.Tensor):
        C = x.shape[0]
        q = (x @ self.wq).view(C, self.h_q, self.d).to(torch.bfloat16)
        k = (x @ self.wk).view(C, self.h_kv, self.d).to(torch.bfloat16)
        v = (x @ self.wv).view(C, self.h_kv, self.d).to(torch.bfloat16)
        return q, k, v

    def out(self, o: torch.Tensor) -> torch.Tensor:
        return o.float().reshape(o.shape[0], -1) @ self.wo

    def _select(self, q: torch.Tensor, n_prior: int):
        if self.top_k is None:
            return None
        return page_topk_select(self.pool, self.bt, n_prior, q, self.top_k, self.n_local, ws=self.ws_t)

    def train_step(self, xs: Sequence[torch.Tensor],
                   loss_fn: Callable[[torch.Tensor, int], torch.Tensor]) -> tuple:
        """One pass over the chunks xs[i] ([chunk][d_model] float32, i-th chunk of the sequence).

        Adds the weight gradients to .grad and returns (total loss, [dx_i]). loss_fn(y_i, i) gives
        chunk i's scalar loss. The chunks' page selections stay in .last_selection."""
        assert len(xs) * self.chunk <= self.context
        per_chunk = self.chunk // self.page
        sels: List[Optional[torch.Tensor]] = []
        total = torch.zeros((), device=self.wq.device)
        with torch.no_grad():
            for i, x in enumerate(xs):
                n_prior = i * per_chunk
                q, k, v = self.qkv(x)
                self.pool.append(self.bt, n_prior * self.page, k.contiguous(), v.contiguous())
                sel = self._select(q, n_prior)
                sels.append(sel)
                o, _ = chunk_attn_fwd(self.pool, self.bt, n_prior, q, self.scale, sel=sel, ws=self.ws_f)
                total += loss_fn(self.out(o), i)
        self.last_selection = sels
        self.pool.zero_grad()
        dxs: List[Optional[torch.Tensor]] = [None] * len(xs)
        for i in reversed(range(len(xs))):
            x = xs[i].detach().requires_grad_(True)
            with torch.enable_grad():
                q, k, v = self.qkv(x)
                o = PagedChunkAttention.apply(q, k, v, self, i * per_chunk, sels[i])
                loss = loss_fn(self.out(o), i)
            loss.backward()
            dxs[i] = x.grad
        return total, dxs

    def free(self):
        self.pool.free()
