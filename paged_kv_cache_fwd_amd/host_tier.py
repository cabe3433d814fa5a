"""Sparse chunk step over a pinned-host page tier (stream orchestration of library calls only).

"Out of the Memory Barrier" summaries, pt 2.D / es 2.B / it 2.C: the KV cache lives in pinned CPU
memory and moves to the GPU on dedicated streams, overlapped with compute; with sparse attention
only the selected pages move (pt 2.C, it 2.D).

Per chunk: page_topk_select on the host-tier pool (its representatives are on the device), then for
each KV head g a side stream gathers g's selected (page, head) blocks into g's device slots
(paged_kv_gather also writes g's device block table) while the compute stream runs the backward
of head g-1. Gradients go to the host-tier pool's device-resident gradient pages through
its own block table, or, when the host pool keeps its gradient pages in host memory, into device
slots that the side stream then adds to the host pages (pt 2.D: the gradients of the KV cache
move to CPU memory too). Every computation is a library kernel; this module only orders them.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from . import (PKV_COPY_GRAD, PKV_COPY_KV, Pool, chunk_attn_bwd, chunk_attn_bwd_ws_bytes, chunk_attn_fwd,
               chunk_attn_fwd_ws_bytes, grad_staging_bytes, load, page_topk_select, paged_kv_copy, paged_kv_gather,
               paged_kv_grad_accumulate, paged_kv_grad_offload, paged_kv_grad_stage)


_COPY_STREAMS = {}

# Workgroups of a gather that the compute stream waits for (8 reach the host link's rate) and of one
# that runs beside a backward (each keeps a CU to itself; 2 move about 22 GB/s, which finishes a
# head's pages well within the previous head's backward).
GATHER_WG_WAITED = 8
GATHER_WG_BESIDE = 2


def copy_streams(device) -> list:
    """The process's three copy streams on `device` (default priority), shared by every host-tier
    driver: HIP spreads a process's streams over a few hardware queues, and a copy stream that
    lands on the compute stream's queue runs its copies behind the kernels instead of beside
    them. Reusing one small set keeps the copy streams on queues of their own however many
    drivers a process builds."""
    key = torch.device(device).index if torch.device(device).index is not None else torch.cuda.current_device()
    if key not in _COPY_STREAMS:
        _COPY_STREAMS[key] = [torch.cuda.Stream(device=key) for _ in range(3)]
    return _COPY_STREAMS[key]


class HostTierStep:
    """Reusable buffers and streams for the sparse step of one chunk shape over a host-tier pool."""

    def __init__(self, host: Pool, host_bt: torch.Tensor, n_prior: int, C: int, H_q: int, top_k: int,
                 n_local: int, device: torch.device, grad_offload: str = "staged"):
        """grad_offload (gradient pages in host memory only): "staged" copies each head's device
        gradient slots to pinned staging with the copy engines and adds them into the host pages on
        host threads (paged_kv_grad_stage / paged_kv_grad_accumulate); "kernel" adds them with a
        kernel that reads and writes the host pages over the host link (paged_kv_grad_offload)."""
        assert host.host_tier
        assert grad_offload in ("staged", "kernel")
        self.grad_offload = grad_offload
        self.host, self.host_bt = host, host_bt
        self.n_prior, self.C, self.H_q = n_prior, C, H_q
        self.top_k, self.n_local = top_k, n_local
        P, H = host.page, host.h_kv
        self.n_own = C // P
        n_cand = max(n_prior - n_local, 0)
        self.n_sel = min(top_k, n_cand) + (n_prior - n_cand)
        n_dev = self.n_own + H * self.n_sel
        # Device pool: the chunk's own pages first, then n_sel slots per KV head. With gradient pages
        # in host memory the device pool carries gradient slots that the backward accumulates into.
        self.host_grads = host.host_grads
        self.dev = Pool(n_dev, P, H, host.d, grads=self.host_grads)
        n_bt = host_bt.numel()
        base = torch.zeros(n_bt, dtype=torch.int32, device=device)
        base[n_prior:n_prior + self.n_own] = torch.arange(self.n_own, dtype=torch.int32, device=device)
        self.own_bt = base.clone()
        # The selection and the per-head device block tables are double-buffered by step parity: the
        # gradient offload of step s still reads them while step s + 1 selects and gathers.
        self.bt: List[List[torch.Tensor]] = [[base.clone() for _ in range(H)] for _ in range(2)]
        self.slots = [torch.arange(self.n_own + g * self.n_sel, self.n_own + (g + 1) * self.n_sel, dtype=torch.int32,
                                   device=device) for g in range(H)]
        self.sel = [torch.empty((H, self.n_sel), dtype=torch.int32, device=device) for _ in range(2)]
        self.parity = 0
        self._pre: Optional[torch.Tensor] = None  # queries whose selection a lookahead enqueued
        self.own_lps = torch.arange(n_prior, n_prior + self.n_own, dtype=torch.int32, device=device)
        lib = load()
        self.ws_t = torch.empty(max(lib.page_topk_ws_bytes(host.handle, n_prior, C, H_q, 1), 1), dtype=torch.uint8,
                                device=device)
        self.ws_f = torch.empty(max(chunk_attn_fwd_ws_bytes(self.dev, n_prior, self.n_sel, 1, C, H_q), 1),
                                dtype=torch.uint8, device=device)
        self.ws_b = torch.empty(max(chunk_attn_bwd_ws_bytes(self.dev, n_prior, self.n_sel, 1, C, H_q), 1),
                                dtype=torch.uint8, device=device)
        streams = copy_streams(device)
        self.side = streams[0]
        self.ready = [torch.cuda.Event() for _ in range(H)]
        self.done = [torch.cuda.Event() for _ in range(H)]
        # Gradient offloads run on a stream of their own, so the next step's gathers need not queue
        # behind them; the next backward of head g waits for head g's offload.
        self.off = streams[1] if self.host_grads else None
        # off_done[b][g]: the offload of head g by the last step that used buffer b (it reads
        # sel[b][g] and bt[b][g] and clears head g's device gradient slots).
        self.off_done = [[torch.cuda.Event() for _ in range(H)] for _ in range(2)]
        self.own_done = torch.cuda.Event()  # the last head's own-page offload
        # Staged offload: pinned staging per (buffer, head) for the own pages and the selected slots,
        # the host copy of the host pool's block table, and a stream that runs the host-side adds.
        # added[b][g]: the adds that last read staging[b][g] have run.
        self.staged = self.host_grads and grad_offload == "staged"
        self.added = [[torch.cuda.Event() for _ in range(H)] for _ in range(2)]
        if self.staged:
            self.acc = streams[2]
            self.host_bt_host = host_bt.to("cpu").contiguous()
            nb_own = grad_staging_bytes(host, self.n_own)
            nb_sel = grad_staging_bytes(host, self.n_sel)
            self.stg_own = [[torch.empty(nb_own, dtype=torch.uint8, pin_memory=True) for _ in range(H)]
                            for _ in range(2)]
            self.stg_sel = [[torch.empty(max(nb_sel, 1), dtype=torch.uint8, pin_memory=True) for _ in range(H)]
                            for _ in range(2)]
        for ev in self.done + self.off_done[0] + self.off_done[1] + self.added[0] + self.added[1] + [self.own_done]:
            ev.record(torch.cuda.current_stream(device))

    @property
    def last_sel(self) -> torch.Tensor:
        """The selection of the last step that gathered."""
        return self.sel[self.parity ^ 1]

    @property
    def last_bt(self) -> List[torch.Tensor]:
        """The per-head device block tables of the last step that gathered."""
        return self.bt[self.parity ^ 1]

    def append_own(self, k: torch.Tensor, v: torch.Tensor):
        """Append the chunk's own K/V ([C][H_kv][d] bf16) into its device pages.

        The append also clears the pages' device gradient blocks, so with gradient pages in host
        memory it first waits for the last head's offload of them (the offload stream runs in
        order, so every earlier head's has finished too)."""
        if self.host_grads:
            torch.cuda.current_stream(k.device).wait_event(self.own_done)
        self.dev.append(self.own_bt, self.n_prior * self.dev.page, k, v)

    def cancel_lookahead(self):
        """Drop the selection and first gather that the last run() enqueued for next_q: the next run()
        then selects and gathers anew (after that gather has finished reading its selection)."""
        if self._pre is not None:
            torch.cuda.current_stream(self._pre.device).wait_event(self.ready[0])
            self._pre = None

    def _lookahead(self, next_q: torch.Tensor, compute):
        """Enqueue on the side stream the next step's selection (into the next step's buffers) and its
        first head's gather, behind this step's gathers and the last head's forward, so that they
        run beside the last head's backward instead of at the start of the next step."""
        H = self.host.h_kv
        nb = self.parity  # the next step's buffers
        after = torch.cuda.Event()
        after.record(compute)  # next_q is ready, and head 0's slots are no longer read
        with torch.cuda.stream(self.side):
            self.side.wait_event(after)
            if self.host_grads:
                self.side.wait_event(self.off_done[nb][H - 1])  # sel[nb] no longer read by an offload
            page_topk_select(self.host, self.host_bt, self.n_prior, next_q, self.top_k, self.n_local,
                             sel=self.sel[nb], ws=self.ws_t, stream=self.side)
            if self.host_grads:
                self.side.wait_event(self.off_done[nb][0])  # bt[nb][0] no longer read by an offload
            paged_kv_gather(self.host, self.dev, self.host_bt, self.sel[nb][0], 0, self.slots[0],
                            dev_bt_out=self.bt[nb][0], n_workgroups=GATHER_WG_BESIDE, stream=self.side)
            self.ready[0].record(self.side)
        self._pre = next_q

    def run(self, q: torch.Tensor, dout: torch.Tensor, scale: float, o: torch.Tensor, lse: torch.Tensor,
            dq: torch.Tensor, gather: bool = True, next_q: Optional[torch.Tensor] = None):
        """One sparse step. With gather=False the slots are assumed filled already (for timing the
        same selection without host traffic; not with gradient pages in host memory).

        Head g's gather (g >= 1) is enqueued behind head g-1's forward, so that it runs beside head
        g-1's backward on few CUs; head 0's, which the step waits for, runs on more.

        next_q (the next step's queries, already written on the current stream): the next step's page
        selection and its first head's gather are enqueued on the side stream beside this step's
        last backward, so that the next step starts with head 0's pages in place. The next run() must
        then take that same tensor as q (or cancel_lookahead() must come first).

        Gradient pages in host memory: head g's backward accumulates into its device slots. An
        offload stream then copies them, and head g's blocks of the chunk's own pages, to pinned
        staging and clears them (paged_kv_grad_stage), and a second stream has the library's host
        threads add the staging into the host pages (paged_kv_grad_accumulate); with
        grad_offload="kernel" one kernel adds the device blocks into the host pages over the host
        link and clears them (paged_kv_grad_offload). The next step's backward of head g waits for
        the clearing, so a slot is cleared before it is reused. Host gradient pages are complete
        once the accumulation stream has passed the step (torch.cuda.synchronize())."""
        assert gather or not self.host_grads
        assert next_q is None or gather
        compute = torch.cuda.current_stream(q.device)
        H = self.host.h_kv
        pre = self._pre is not None
        if pre:
            if self._pre is not q or not gather:
                raise ValueError("the last step looked ahead to other queries: pass them as q, or cancel_lookahead()")
            self._pre = None
        if gather:
            b = self.parity
            self.parity ^= 1
        else:
            b = self.parity ^ 1  # the buffers the last gathering step filled
        prev = b ^ 1
        bts = self.bt[b]
        if pre:
            sel = self.sel[b]  # selected, and head 0 gathered, by the last step's lookahead
        else:
            if self.host_grads:
                # sel[b] was last read by the offloads of the step before the previous one; the offload
                # stream runs in order, so its last head's event covers them all.
                compute.wait_event(self.off_done[b][H - 1])
            sel = page_topk_select(self.host, self.host_bt, self.n_prior, q, self.top_k, self.n_local,
                                   sel=self.sel[b], ws=self.ws_t)

        def enqueue_gather(g, n_wg):
            # Events are waited on at their latest record: `after` is this step's selection or head
            # g-1's forward, done[g] the previous step's backward of head g (recorded again only
            # later in this step).
            after = torch.cuda.Event()
            after.record(compute)
            with torch.cuda.stream(self.side):
                self.side.wait_event(self.done[g])  # slots of g are free once its last backward ended
                if self.host_grads:
                    self.side.wait_event(self.off_done[b][g])  # bt[b][g] is no longer read by an offload
                self.side.wait_event(after)
                paged_kv_gather(self.host, self.dev, self.host_bt, sel[g], g, self.slots[g], dev_bt_out=bts[g],
                                n_workgroups=n_wg, stream=self.side)
                self.ready[g].record(self.side)

        if gather and not pre:
            enqueue_gather(0, GATHER_WG_WAITED)
        for g in range(H):
            if gather:
                compute.wait_event(self.ready[g])
            chunk_attn_fwd(self.dev, bts[g], self.n_prior, q, scale, sel=sel, kvh0=g, n_kvh=1, o=o, lse=lse,
                           ws=self.ws_f)
            if gather and g + 1 < H:
                enqueue_gather(g + 1, GATHER_WG_BESIDE)  # behind the selection too, after a lookahead
            if g == H - 1 and next_q is not None:
                self._lookahead(next_q, compute)
            if self.host_grads:
                # Head g's gradient slots are cleared by the previous step's offload of head g.
                compute.wait_event(self.off_done[prev][g])
                chunk_attn_bwd(self.dev, bts[g], self.n_prior, q, o, dout, lse, scale, sel=sel, kvh0=g, n_kvh=1,
                               gpool=self.dev, gbt=bts[g], dq=dq, ws=self.ws_b)
            else:
                chunk_attn_bwd(self.dev, bts[g], self.n_prior, q, o, dout, lse, scale, sel=sel, kvh0=g, n_kvh=1,
                               gpool=self.host, gbt=self.host_bt, dq=dq, ws=self.ws_b)
            self.done[g].record(compute)
            if self.staged:
                with torch.cuda.stream(self.off):
                    self.off.wait_event(self.done[g])
                    self.off.wait_event(self.added[b][g])  # staging[b][g] read by the adds of two steps ago
                    # Own pages first: the next chunk's append waits for them, not for the slots.
                    paged_kv_grad_stage(self.dev, 0, self.n_own, g, self.own_lps, self.stg_own[b][g], stream=self.off)
                    self.own_done.record(self.off)
                    paged_kv_grad_stage(self.dev, self.n_own + g * self.n_sel, self.n_sel, g, sel[g],
                                        self.stg_sel[b][g], stream=self.off)
                    self.off_done[b][g].record(self.off)
                with torch.cuda.stream(self.acc):
                    self.acc.wait_event(self.off_done[b][g])
                    paged_kv_grad_accumulate(self.host, self.host_bt_host, self.n_own, g, self.stg_own[b][g],
                                             stream=self.acc)
                    paged_kv_grad_accumulate(self.host, self.host_bt_host, self.n_sel, g, self.stg_sel[b][g],
                                             stream=self.acc)
                    self.added[b][g].record(self.acc)
            elif self.host_grads:
                with torch.cuda.stream(self.off):
                    self.off.wait_event(self.done[g])
                    # Only head g's backward writes head g's blocks of the own pages. They go first:
                    # the next chunk's append waits for them, not for the selected pages.
                    paged_kv_grad_offload(self.host, self.host_bt, self.dev, self.own_bt, self.own_lps, kvh0=g,
                                          n_kvh=1, stream=self.off)
                    self.own_done.record(self.off)
                    paged_kv_grad_offload(self.host, self.host_bt, self.dev, bts[g], sel[g], kvh0=g, n_kvh=1,
                                          stream=self.off)
                    self.off_done[b][g].record(self.off)
        return sel

    def free(self):
        self.dev.free()


class DenseLayerPrefetch:
    """Dense chunk steps over a stack of layers whose KV and gradient pages live in pinned host memory.

    pt 2.D: with dense (or local) attention the next block is fetched while the current one is
    computed; es 2.B: the transfers overlap the next layer's computation. Here a block is one layer's
    whole page pool. Two device pools alternate: while layer l's forward and backward run on one,
    a load stream fills the other with the next layer's KV and gradient pages (paged_kv_copy, a copy
    engine), and a write-back stream copies layer l's gradient pages home once its backward is done.
    Physical page numbers are the same on host and device, so the layer's block table serves both.

    A step is the chunk's forward and backward with its own K/V already in the pages, as in the
    reverse pass of the chunk-recurrent loop; gradients add to the host pages' running sums."""

    def __init__(self, hosts: Sequence[Pool], device: torch.device):
        h0 = hosts[0]
        for h in hosts:
            assert h.host_tier and h.host_grads, "layers need KV and gradient pages in host memory"
            assert (h.n_pages, h.page, h.h_kv, h.d) == (h0.n_pages, h0.page, h0.h_kv, h0.d)
        self.hosts = list(hosts)
        self.dev = [Pool(h0.n_pages, h0.page, h0.h_kv, h0.d, grads=True) for _ in range(2)]
        self.load_s, self.wb_s = copy_streams(device)[:2]
        self.loaded = [torch.cuda.Event() for _ in range(2)]
        self.written = [torch.cuda.Event() for _ in range(2)]
        self.computed = [torch.cuda.Event() for _ in range(2)]
        for ev in self.written:
            ev.record(torch.cuda.current_stream(device))
        self.layer_written = [torch.cuda.Event() for _ in hosts]  # last write-back of each layer
        self.buf_layer = [None, None]  # layer whose pages a device pool holds (or is receiving)
        self.cur = 0                   # device pool of the next step
        self.ws_f = self.ws_b = None

    def prefetch(self, layer: int, buf: Optional[int] = None):
        """Enqueue the copy of layer's KV and gradient pages into device pool buf (default: the pool
        after the current one), once that pool's previous gradients and the layer's own latest
        gradients have been written back (a layer run twice in a row is then not overlapped)."""
        j = (self.cur ^ 1) if buf is None else buf
        with torch.cuda.stream(self.load_s):
            self.load_s.wait_event(self.written[j])
            self.load_s.wait_event(self.layer_written[layer])
            paged_kv_copy(self.hosts[layer], self.dev[j], PKV_COPY_KV | PKV_COPY_GRAD, stream=self.load_s)
            self.loaded[j].record(self.load_s)
        self.buf_layer[j] = layer

    def run(self, layer: int, next_layer: Optional[int], bt: torch.Tensor, n_prior: int, q: torch.Tensor,
            dout: torch.Tensor, scale: float, o: torch.Tensor, lse: torch.Tensor, dq: torch.Tensor):
        """Forward + backward of one chunk of `layer` (bt: its logical-to-physical block table). The
        pages of next_layer (if given) are fetched meanwhile into the other device pool."""
        compute = torch.cuda.current_stream(q.device)
        j = self.cur
        if self.buf_layer[j] != layer:
            self.prefetch(layer, j)
        if next_layer is not None:
            self.prefetch(next_layer, j ^ 1)
        dev = self.dev[j]
        C, H_q = q.shape[0], q.shape[1]
        if self.ws_f is None:
            self.ws_f = torch.empty(max(chunk_attn_fwd_ws_bytes(dev, n_prior, -1, dev.h_kv, C, H_q), 1),
                                    dtype=torch.uint8, device=q.device)
            self.ws_b = torch.empty(max(chunk_attn_bwd_ws_bytes(dev, n_prior, -1, dev.h_kv, C, H_q), 1),
                                    dtype=torch.uint8, device=q.device)
        compute.wait_event(self.loaded[j])
        chunk_attn_fwd(dev, bt, n_prior, q, scale, o=o, lse=lse, ws=self.ws_f)
        chunk_attn_bwd(dev, bt, n_prior, q, o, dout, lse, scale, dq=dq, ws=self.ws_b)
        self.computed[j].record(compute)
        with torch.cuda.stream(self.wb_s):
            self.wb_s.wait_event(self.computed[j])
            paged_kv_copy(dev, self.hosts[layer], PKV_COPY_GRAD, stream=self.wb_s)
            self.written[j].record(self.wb_s)
            self.layer_written[layer].record(self.wb_s)
        self.cur = j ^ 1
        if next_layer is None:
            self.buf_layer[j ^ 1] = None

    def free(self):
        for d in self.dev:
            d.free()
