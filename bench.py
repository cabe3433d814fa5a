#!/usr/bin/env python
"""Benchmark: paged chunk attention forward + backward at a 256K context on one MI355X.

Workload (one step = the whole hot path over one synthetic batch, inputs resident in HBM):
  dense256k  append the final 4096-token chunk's K/V into its pages, forward, backward
             (28 query / 4 KV heads, d=128, page 128, 2016 prior pages + the causal own block);
  topk256k   the same plus page selection (top-64 by mean-key score + 4 most recent pages), with
             forward and backward over the selected pages only;
  local256k  a local layer: the most recent prior page and the causal own block (top_k = 0).
The headline value is the dense step's algorithmic TFLOP/s (forward 4*d*H_q*pairs, backward
10*d*H_q*pairs); the top-K step is reported beside it.

Prints one JSON line on stdout. Progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "chunk attn fwd+bwd TFLOP/s (and % bf16 peak) at 256K ctx, dense and top-K paged"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak
HBM_PEAK_GBS = 8000.0
LOCAL_WINDOW = 1  # pages kept by a local (sliding-window) layer


# HBM bytes per launch of the dense 256K step's attention kernels, from one FETCH_SIZE and one
# WRITE_SIZE rocprofv3 pass each, scaled by what those counters read for a plain 1 GiB streaming
# kernel (x2.0 fetch, x1.0 write). Valid only for the kernel sources they were taken on.
TRAFFIC_SOURCES = ("paged_kv_cache_fwd_amd/csrc/k_attn_fwd.hip", "paged_kv_cache_fwd_amd/csrc/k_attn_fwd64.hip",
                   "paged_kv_cache_fwd_amd/csrc/k_attn_dq64.hip",
                   "paged_kv_cache_fwd_amd/csrc/k_attn_bwd.hip",
                   "paged_kv_cache_fwd_amd/csrc/k_attn_dkdv.hip", "paged_kv_cache_fwd_amd/csrc/pkv_device.h", "paged_kv_cache_fwd_amd/csrc/pkv_internal.h",
                   "paged_kv_cache_fwd_amd/csrc/pkv_abi.cpp", "paged_kv_cache_fwd_amd/build.py")
TRAFFIC_SHA = "bc62b71d223e1f31"
TRAFFIC_BYTES = {"k_attn_fwd64": (2.0 * 1206855 * 1024, 231168 * 1024),
                 "k_bwd_dq64": (2.0 * 1176240 * 1024, 229376 * 1024),
                 "k_bwd_dkdv": (2.0 * 1386450 * 1024, 1048576 * 1024)}


def traffic_bytes(kernel):
    """(fetch, write) bytes per launch if the attention sources are those the counters were taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != TRAFFIC_SHA or kernel not in TRAFFIC_BYTES:
        return None
    return TRAFFIC_BYTES[kernel]


def mfma_loop_peak(pkv, dev, ms_target=30.0):
    """Sustained bf16 MFMA rate of this GPU (the library's diagnostic loop, one 8-wave workgroup per
    CU, about 30 ms per launch, best of three), in TFLOP/s."""
    import torch
    n_wg = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(n_wg * 512, dtype=torch.float32, device=dev)
    iters = 1000
    flop = pkv.mfma_probe(n_wg, iters, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    pkv.mfma_probe(n_wg, iters, out)
    e1.record()
    torch.cuda.synchronize()
    iters = max(1000, int(iters * ms_target / max(e0.elapsed_time(e1), 1e-3)))
    best = 0.0
    for _ in range(3):
        e0.record()
        flop = pkv.mfma_probe(n_wg, iters, out)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, flop / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    assert torch.isfinite(out).all()
    return best


def atomic_probe_rates(pkv, dev, wl):
    """fp32 atomic-add rates of this GPU (the library's diagnostic) in the two patterns that decide how
    the backward is split: one add per element (the key-major dK/dV pass flushes each gradient
    element once) and one add per 256-row block into each 64 KB region (dK/dV of a 64-key tile), as a
    query-major one-pass backward would flush them. The one-pass estimate prices that backward's
    partials (row blocks x keys x 2 d floats per KV head) at the contended rate."""
    import torch
    region = 64 * 2 * wl.d  # floats: dK and dV of 64 keys
    row_blocks = wl.chunk * wl.group // 256
    out = {}
    for name, n_wg, n_regions in (("one_add_per_element", 4096, 4096),
                                  (f"{row_blocks}_adds_per_element", 64 * row_blocks, 64)):
        buf = torch.zeros(n_regions * region, dtype=torch.float32, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nbytes = pkv.atomic_probe(n_wg, n_regions, region, buf)
        best = 0.0
        for _ in range(3):
            e0.record()
            pkv.atomic_probe(n_wg, n_regions, region, buf)
            e1.record()
            torch.cuda.synchronize()
            best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        assert torch.all(buf == 4.0 * (n_wg // n_regions)).item(), "atomic probe lost adds"
        out[name] = {"GBps": round(best, 1), "bytes_per_launch": int(nbytes)}
        del buf
    partial_bytes = float(row_blocks) * wl.context * 2 * wl.d * 4 * wl.h_kv
    rate = out[f"{row_blocks}_adds_per_element"]["GBps"]
    out["one_pass_backward_partials_GB"] = round(partial_bytes / 1e9, 1)
    out["one_pass_backward_atomic_ms_at_contended_rate"] = round(partial_bytes / (rate * 1e9) * 1e3, 1)
    return out


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pairs_dense(C, q0):
    return C * q0 + C * (C + 1) // 2


def pairs_sparse(C, n_sel, P):
    return C * n_sel * P + C * (C + 1) // 2


def cpu_baseline(wl, k_np, v_np, q_np, do_np, c, tokens):
    """The oracle, untuned, in float32 on the host cores: KV head 0 and its query heads, the last
    `tokens` chunk tokens against every visible key (forward + backward)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    G = wl.group
    q0 = wl.q0(c)
    L = q0 + wl.chunk
    q = oracle.widen_bf16(q_np[:, :G, :])
    do = oracle.widen_bf16(do_np[:, :G, :])
    k = oracle.widen_bf16(k_np[:L, :1, :])
    v = oracle.widen_bf16(v_np[:L, :1, :])
    rows = np.arange(wl.chunk - tokens, wl.chunk)
    t0 = time.perf_counter()
    oracle.chunk_forward(q, k, v, q0, wl.scale, page=wl.page, rows=rows, dtype=np.float32)
    oracle.chunk_backward(q, k, v, do, q0, wl.scale, page=wl.page, rows=rows, dtype=np.float32)
    dt = time.perf_counter() - t0
    pairs = int(sum(q0 + t + 1 for t in rows)) * G
    flop = 14.0 * wl.d * pairs
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": model, "host_cpus": os.cpu_count(),
            "sample": f"KV head 0 with its {G} query heads, last {tokens} of {wl.chunk} chunk tokens against all "
                      f"{L} visible keys, forward+backward, float32; {flop:.3e} FLOP in {dt:.2f} s"}


def bench_host1m(args, pkv, synth, dev, t16):
    """1M-token sparse step with the prior pages in pinned host memory: selection, per-KV-head H2D
    gathers on a side stream overlapped with the previous head's backward."""
    import torch
    from paged_kv_cache_fwd_amd.host_tier import HostTierStep

    wl = synth.WORKLOADS["host1m"]
    c = wl.chunks[0]
    C, P, H_q, H_kv, d = wl.chunk, wl.page, wl.h_q, wl.h_kv, wl.d
    n_prior = wl.n_prior(c)
    log(f"[bench] host1m: generating and appending {wl.n_pages} pages into pinned host memory")
    hpool = pkv.Pool(wl.n_pages, P, H_kv, d, grads=True, host_tier=True)
    hbt = torch.from_numpy(synth.page_permutation(wl)).to(dev)
    for p0 in range(0, n_prior, 512):
        n = min(512, n_prior - p0)
        k, v = synth.kv_tokens(wl, p0, n)
        hpool.append(hbt, p0 * P, t16(k), t16(v))
    step = HostTierStep(hpool, hbt, n_prior, C, H_q, wl.top_k, wl.n_local, dev)
    k_own, v_own = synth.kv_tokens(wl, n_prior, C // P)
    k_own, v_own = t16(k_own), t16(v_own)
    q, do = t16(synth.q_chunk(wl, c)), t16(synth.do_chunk(wl, c))
    o, dq = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((H_q, C), dtype=torch.float32, device=dev)

    def timed(gather, lookahead=False):
        # With lookahead each step also enqueues the next step's selection and first gather (the
        # same queries here) beside its last heads, as a chunk loop that knows the next chunk's
        # queries would.
        nxt = q if lookahead else None
        for _ in range(args.warmup):
            step.append_own(k_own, v_own)
            step.run(q, do, wl.scale, o, lse, dq, gather=gather, next_q=nxt)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step.append_own(k_own, v_own)
            step.run(q, do, wl.scale, o, lse, dq, gather=gather, next_q=nxt)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / args.steps * 1e3
        step.cancel_lookahead()
        return ms

    log("[bench] host1m: steps with H2D gathers on a side stream")
    ms_host = timed(True)
    log("[bench] host1m: the same steps, each looking ahead to the next one's selection and first gather")
    ms_host_ahead = timed(True, lookahead=True)
    log("[bench] host1m: the same steps with the selected pages already on the device")
    ms_res = timed(False)
    # H2D gathers alone.
    sel, sel_bt = step.last_sel, step.last_bt
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for g in range(H_kv):
            pkv.paged_kv_gather(hpool, step.dev, hbt, sel[g], g, step.slots[g], dev_bt_out=sel_bt[g])
    torch.cuda.synchronize()
    ms_gather = (time.perf_counter() - t0) / args.steps * 1e3
    # Pinned host -> device copy of the same byte count, for the link's practical peak.
    h2d_bytes_all = H_kv * step.n_sel * 2 * P * d * 2
    src = torch.empty(h2d_bytes_all, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(h2d_bytes_all, dtype=torch.uint8, device=dev)
    for _ in range(2):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    ms_memcpy = (time.perf_counter() - t0) / args.steps * 1e3
    del src, dst
    hpool.check()
    step.dev.check()
    h2d_bytes = H_kv * step.n_sel * 2 * P * d * 2
    pairs = pairs_sparse(C, step.n_sel, P)
    flop = 14.0 * d * H_q * pairs
    n_sel_1m = step.n_sel
    step.free()
    hpool.free()

    # The same steps with the gradient pages in pinned host memory too: each head's backward
    # accumulates into device slots that the side stream adds to the host pages.
    log("[bench] host1m: refilling with gradient pages in host memory")
    hpool = pkv.Pool(wl.n_pages, P, H_kv, d, grads=True, host_tier=True, host_grads=True)
    for p0 in range(0, n_prior, 512):
        n = min(512, n_prior - p0)
        k, v = synth.kv_tokens(wl, p0, n)
        hpool.append(hbt, p0 * P, t16(k), t16(v))
    step = HostTierStep(hpool, hbt, n_prior, C, H_q, wl.top_k, wl.n_local, dev)
    ms_host_grads = timed(True)
    ms_host_grads_ahead = timed(True, lookahead=True)
    hpool.check()
    step.dev.check()
    step.free()
    # The earlier offload for comparison: one kernel adds the device slots into the host pages over
    # the host link (zero-copy loads and stores).
    step = HostTierStep(hpool, hbt, n_prior, C, H_q, wl.top_k, wl.n_local, dev, grad_offload="kernel")
    ms_host_grads_kernel = timed(True)
    hpool.check()
    step.dev.check()
    step.free()
    hpool.free()
    offload_bytes = (H_kv * n_sel_1m + H_kv * (C // P)) * 2 * P * d * 4  # fp32 dK+dV blocks
    log(f"[bench] host1m: {ms_host_grads:.3f} ms/step with gradient pages in host memory (staged), "
        f"{ms_host_grads_kernel:.3f} ms with the zero-copy offload kernel")
    log(f"[bench] host1m: {ms_host:.3f} ms/step with gathers ({ms_host_ahead:.3f} with lookahead), {ms_res:.3f} ms "
        f"resident, gathers alone {ms_gather:.3f} ms; host gradient pages with lookahead {ms_host_grads_ahead:.3f} ms")
    return {"workload": "host1m: 1M tokens, 8160 prior pages in pinned host memory, top-128 + 8 local per KV head, "
                        "per-head H2D gathers overlapped with the previous head's backward",
            "value": round(flop / (ms_host * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": round(ms_host, 4),
            "flop_per_step": flop, "ms_per_step_pages_resident": round(ms_res, 4),
            "overlap_overhead": round(ms_host / ms_res - 1.0, 4),
            "ms_per_step_lookahead": round(ms_host_ahead, 4),
            "overlap_overhead_lookahead": round(ms_host_ahead / ms_res - 1.0, 4),
            "h2d_bytes_per_step": h2d_bytes, "h2d_gather_ms": round(ms_gather, 4),
            "h2d_GBps": round(h2d_bytes / (ms_gather * 1e-3) / 1e9, 2),
            "h2d_pinned_memcpy_GBps": round(h2d_bytes / (ms_memcpy * 1e-3) / 1e9, 2),
            "ms_per_step_host_grads": round(ms_host_grads, 4),
            "host_grads_overhead": round(ms_host_grads / ms_host - 1.0, 4),
            "host_grads_overhead_vs_resident": round(ms_host_grads / ms_res - 1.0, 4),
            "ms_per_step_host_grads_lookahead": round(ms_host_grads_ahead, 4),
            "host_grads_overhead_lookahead": round(ms_host_grads_ahead / ms_host_ahead - 1.0, 4),
            "host_grads_overhead_lookahead_vs_resident": round(ms_host_grads_ahead / ms_res - 1.0, 4),
            "host_grads_offload": "device slots copied to pinned staging by the copy engines (one rectangular "
                                  "copy per head), added into the host pages by host threads",
            "ms_per_step_host_grads_zero_copy_kernel": round(ms_host_grads_kernel, 4),
            "host_grads_overhead_zero_copy_kernel": round(ms_host_grads_kernel / ms_host - 1.0, 4),
            "grad_offload_bytes_per_step": offload_bytes}


def bench_dense_host(args, pkv, synth, dev, t16):
    """Dense 1M-token steps over two layers whose KV and gradient pages live in pinned host memory:
    each step's forward+backward runs on one device pool while a copy engine loads the next layer's
    pages into the other and another writes the finished layer's gradient pages home."""
    import torch
    from paged_kv_cache_fwd_amd.host_tier import DenseLayerPrefetch

    wl = synth.WORKLOADS["host1m"]
    c = wl.chunks[0]
    C, P, H_q, H_kv, d = wl.chunk, wl.page, wl.h_q, wl.h_kv, wl.d
    n_prior, N = wl.n_prior(c), wl.n_pages
    log(f"[bench] dense1m-host: generating {N} pages (device-resident pool)")
    res = pkv.Pool(N, P, H_kv, d, grads=True)
    bt = torch.from_numpy(synth.page_permutation(wl)).to(dev)
    for p0 in range(0, N, 512):
        n = min(512, N - p0)
        k, v = synth.kv_tokens(wl, p0, n)
        res.append(bt, p0 * P, t16(k), t16(v))
    log("[bench] dense1m-host: two layers of KV + gradient pages in pinned host memory")
    hosts = [pkv.Pool(N, P, H_kv, d, grads=True, host_tier=True, host_grads=True) for _ in range(2)]
    for h in hosts:
        pkv.paged_kv_copy(res, h, pkv.PKV_COPY_KV)
    q, do = t16(synth.q_chunk(wl, c)), t16(synth.do_chunk(wl, c))
    o, dq = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((H_q, C), dtype=torch.float32, device=dev)
    ws_f = torch.empty(max(pkv.chunk_attn_fwd_ws_bytes(res, n_prior, -1, H_kv, C, H_q), 1), dtype=torch.uint8,
                       device=dev)
    ws_b = torch.empty(max(pkv.chunk_attn_bwd_ws_bytes(res, n_prior, -1, H_kv, C, H_q), 1), dtype=torch.uint8,
                       device=dev)
    n_steps = max(args.steps, 6)

    def timed(step):
        for i in range(2):
            step(i)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(n_steps):
            step(i)
            ev[i + 1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / n_steps * 1e3
        per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n_steps))
        return wall, per[len(per) // 2]

    def step_res(i):
        pkv.chunk_attn_fwd(res, bt, n_prior, q, wl.scale, o=o, lse=lse, ws=ws_f)
        pkv.chunk_attn_bwd(res, bt, n_prior, q, o, do, lse, wl.scale, dq=dq, ws=ws_b)

    log(f"[bench] dense1m-host: {n_steps} steps with all pages on the device")
    wall_res, med_res = timed(step_res)
    run = DenseLayerPrefetch(hosts, dev)

    def step_host(i):
        run.run(i % 2, (i + 1) % 2, bt, n_prior, q, do, wl.scale, o, lse, dq)

    log(f"[bench] dense1m-host: {n_steps} steps alternating two host-resident layers")
    wall_host, med_host = timed(step_host)
    # Each direction alone, for the link's rate.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    pkv.paged_kv_copy(hosts[0], run.dev[0], pkv.PKV_COPY_KV | pkv.PKV_COPY_GRAD)
    torch.cuda.synchronize()
    ms_h2d = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    pkv.paged_kv_copy(run.dev[0], hosts[0], pkv.PKV_COPY_GRAD)
    torch.cuda.synchronize()
    ms_d2h = (time.perf_counter() - t0) * 1e3
    for h in hosts:
        h.check()
    run.free()
    for h in hosts:
        h.free()
    res.free()
    kv_b, gr_b = N * H_kv * 2 * P * d * 2, N * H_kv * 2 * P * d * 4
    flop = 14.0 * d * H_q * pairs_dense(C, wl.q0(c))
    log(f"[bench] dense1m-host: {med_host:.2f} ms/step (wall {wall_host:.2f}) vs {med_res:.2f} resident "
        f"(wall {wall_res:.2f}); H2D {ms_h2d:.1f} ms, D2H {ms_d2h:.1f} ms per layer alone")
    return {"workload": "dense1m-host: final 4096-token chunk over 8160 prior pages + own block, 28/4 heads, d=128, "
                        "dense; two layers whose KV and gradient pages live in pinned host memory, each step "
                        "overlapping the next layer's page load and the finished layer's gradient write-back",
            "value": round(flop / (med_host * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(med_host, 3), "ms_per_step_wall": round(wall_host, 3),
            "ms_per_step_resident": round(med_res, 3), "ms_per_step_resident_wall": round(wall_res, 3),
            "overhead": round(med_host / med_res - 1.0, 4), "overhead_wall": round(wall_host / wall_res - 1.0, 4),
            "flop_per_step": flop, "steps": n_steps,
            "h2d_bytes_per_step": kv_b + gr_b, "d2h_bytes_per_step": gr_b,
            "h2d_alone_ms": round(ms_h2d, 2), "h2d_GBps": round((kv_b + gr_b) / (ms_h2d * 1e-3) / 1e9, 2),
            "d2h_alone_ms": round(ms_d2h, 2), "d2h_GBps": round(gr_b / (ms_d2h * 1e-3) / 1e9, 2),
            "note": "ms_per_step is the median interval between steps on the compute stream; the wall figure "
                    "also counts draining the last write-back"}


def bench_recurrent(args, pkv, dev):
    """Chunk-recurrent training of one attention layer with Qwen2.5-7B attention shapes (d_model
    3584, 28/4 heads, d=128, 4096-token chunks), float32 projections, dense attention: step time,
    the library kernels' share, and peak torch memory beyond the inputs at two context lengths
    (it stays flat: only the paged cache, allocated by the library, grows with the context)."""
    import torch
    from paged_kv_cache_fwd_amd.recurrent import ChunkRecurrentAttention

    out = {}
    for n_chunks in (4, 8):
        C, dm = 4096, 3584
        layer = ChunkRecurrentAttention(dm, 28, 4, 128, 128, C, C * n_chunks, seed=0)
        g = torch.Generator().manual_seed(7)
        xs = [torch.randn(C, dm, generator=g).to(dev) for _ in range(n_chunks)]
        rs = [torch.randn(C, dm, generator=g).to(dev) / 64.0 for _ in range(n_chunks)]

        def loss_fn(y, i):
            return (y * rs[i]).sum()

        layer.train_step(xs, loss_fn)  # warm-up
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        pkv.timing_enable(True)
        t0 = time.perf_counter()
        layer.train_step(xs, loss_fn)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3
        pkv.timing_enable(False)
        kt = pkv.timing_collect()
        # Beyond the inputs (and the returned dx, one input-sized tensor per chunk).
        peak = torch.cuda.max_memory_allocated() - base - n_chunks * C * dm * 4
        lib_ms = sum(v[1] for v in kt.values())
        pool_bytes = layer.n_pages * 4 * 2 * 128 * 128 * (2 + 4)
        ctx = C * n_chunks
        log(f"[bench] recurrent {ctx // 1024}K: {ms:.1f} ms/step, library kernels {lib_ms:.1f} ms, "
            f"peak torch memory beyond inputs and dx {peak / 2**20:.0f} MiB, pool {pool_bytes / 2**20:.0f} MiB")
        out[f"{ctx // 1024}k"] = {"ms_per_step": round(ms, 2), "tokens_per_s": round(ctx / (ms * 1e-3), 1),
                                  "library_kernel_ms": round(lib_ms, 2),
                                  "peak_torch_bytes_beyond_inputs_and_dx": int(peak), "pool_bytes": pool_bytes}
        layer.free()
        del xs, rs, layer
        torch.cuda.empty_cache()
    out["note"] = ("one attention layer (Qwen2.5-7B shapes), forward over 4096-token chunks then reverse "
                   "backward with recomputation; float32 projections via torch, attention in the library")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-tokens", type=int, default=1024, help="chunk tokens in the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-topk", action="store_true")
    ap.add_argument("--no-host1m", action="store_true", help="skip the 1M-token host-tier workload")
    ap.add_argument("--no-recurrent", action="store_true", help="skip the chunk-recurrent layer driver")
    ap.add_argument("--no-densehost", action="store_true",
                    help="skip the dense 1M-token workload over host-resident layers")
    ap.add_argument("--only", choices=("topk", "qpage", "host1m", "densehost"),
                    help="time only this workload (for per-workload profiles; prints no headline value)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="first run one plain streaming kernel (torch.neg on fp32) over this many MiB, as the "
                         "known-size reference for byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_fwd_amd as pkv
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    pkv.load()
    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib << 18
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] calibration kernel: reads {n * 4} B, writes {n * 4} B")
        del src, dst

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.only == "host1m":
        print(json.dumps(bench_host1m(args, pkv, synth, dev, t16)), flush=True)
        return
    if args.only == "densehost":
        print(json.dumps(bench_dense_host(args, pkv, synth, dev, t16)), flush=True)
        return
    wl = synth.WORKLOADS["dense256k"]
    wlk = synth.WORKLOADS["topk256k"]
    c = wl.chunks[0]
    C, P, H_q, H_kv, d = wl.chunk, wl.page, wl.h_q, wl.h_kv, wl.d
    q0, n_prior, n_pages = wl.q0(c), wl.n_prior(c), wl.n_pages

    log(f"[bench] generating {n_pages} pages of K/V ({wl.note})")
    t0 = time.time()
    k_np, v_np = synth.kv_tokens(wl, 0, n_pages)
    q_np, do_np = synth.q_chunk(wl, c), synth.do_chunk(wl, c)
    bt_np = synth.page_permutation(wl)
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s; appending prior pages")
    pool = pkv.Pool(n_pages, P, H_kv, d, grads=True)
    bt = torch.from_numpy(bt_np).to(dev)
    # One append over all prior pages: the bulk datapoint of the append, representative and
    # gradient-zeroing kernels (268 MB of keys in one launch, not launch-latency-sized pieces).
    per = n_prior
    kv_pieces = [(p0, t16(k_np[p0 * P:(p0 + min(per, n_prior - p0)) * P]),
                  t16(v_np[p0 * P:(p0 + min(per, n_prior - p0)) * P])) for p0 in range(0, n_prior, per)]
    # The pool is filled twice with the same pages: the first pass is the first touch of freshly
    # allocated memory (page-table walks), the second is timed.
    for p0, kp, vp in kv_pieces:
        pool.append(bt, p0 * P, kp, vp)
    torch.cuda.synchronize()
    pkv.timing_enable(True)
    for p0, kp, vp in kv_pieces:
        pool.append(bt, p0 * P, kp, vp)
    torch.cuda.synchronize()
    pkv.timing_enable(False)
    kt_fill = pkv.timing_collect()
    del kv_pieces
    # Bulk append of the prior pages in one call: K/V read and written, new gradient pages
    # zeroed, and one representative per (page, head) from the page's keys.
    pg = n_prior * H_kv * P * d
    fill = {"pages": n_prior, "calls": kt_fill.get("k_append", (0, 0))[0]}
    for kname, nbytes in (("k_append", pg * 2 * 2 * 2), ("k_page_reps", pg * 2 + n_prior * H_kv * d * 4),
                          ("k_zero_grad", pg * 2 * 4)):
        if kname in kt_fill:
            ms = kt_fill[kname][1]
            fill[kname] = {"ms": round(ms, 4), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                           "pct_hbm_peak": round(100.0 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)}
    log(f"[bench] pool fill: {fill}")
    k_own, v_own = t16(k_np[q0:q0 + C]), t16(v_np[q0:q0 + C])
    q, do = t16(q_np), t16(do_np)
    o = torch.empty_like(q)
    dq = torch.empty_like(q)
    lse = torch.empty((H_q, C), dtype=torch.float32, device=dev)
    top_k, n_local = wlk.top_k, wlk.n_local
    n_sel = min(top_k, n_prior - n_local) + n_local
    sel = torch.empty((H_kv, n_sel), dtype=torch.int32, device=dev)
    sel_l = torch.empty((H_kv, LOCAL_WINDOW), dtype=torch.int32, device=dev)
    n_qp = C // P
    sel_q = torch.empty((H_kv, n_qp, n_sel), dtype=torch.int32, device=dev)
    shapes = ((-1, 1), (n_sel, 1), (LOCAL_WINDOW, 1), (n_sel, n_qp))
    ws_f = torch.empty(max(max(pkv.chunk_attn_fwd_ws_bytes(pool, n_prior, ns, H_kv, C, H_q, nl)
                               for ns, nl in shapes), 1), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(max(pkv.chunk_attn_bwd_ws_bytes(pool, n_prior, ns, H_kv, C, H_q, nl)
                               for ns, nl in shapes), 1), dtype=torch.uint8, device=dev)
    ws_t = torch.empty(max(pkv.load().page_topk_ws_bytes(pool.handle, n_prior, C, H_q, n_qp), 1),
                       dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step_dense():
        pool.append(bt, q0, k_own, v_own)
        pkv.chunk_attn_fwd(pool, bt, n_prior, q, wl.scale, o=o, lse=lse, ws=ws_f)
        pkv.chunk_attn_bwd(pool, bt, n_prior, q, o, do, lse, wl.scale, dq=dq, ws=ws_b)

    def step_local():
        pool.append(bt, q0, k_own, v_own)
        s = pkv.page_topk_select(pool, bt, n_prior, q, 0, LOCAL_WINDOW, sel=sel_l, ws=ws_t)
        pkv.chunk_attn_fwd(pool, bt, n_prior, q, wl.scale, sel=s, o=o, lse=lse, ws=ws_f)
        pkv.chunk_attn_bwd(pool, bt, n_prior, q, o, do, lse, wl.scale, sel=s, dq=dq, ws=ws_b)

    def step_topk():
        pool.append(bt, q0, k_own, v_own)
        s = pkv.page_topk_select(pool, bt, n_prior, q, top_k, n_local, sel=sel, ws=ws_t)
        pkv.chunk_attn_fwd(pool, bt, n_prior, q, wl.scale, sel=s, o=o, lse=lse, ws=ws_f)
        pkv.chunk_attn_bwd(pool, bt, n_prior, q, o, do, lse, wl.scale, sel=s, dq=dq, ws=ws_b)

    def step_qpage():
        pool.append(bt, q0, k_own, v_own)
        s = pkv.page_topk_select(pool, bt, n_prior, q, top_k, n_local, sel=sel_q, ws=ws_t, per_query_page=True)
        pkv.chunk_attn_fwd(pool, bt, n_prior, q, wl.scale, sel=s, o=o, lse=lse, ws=ws_f)
        pkv.chunk_attn_bwd(pool, bt, n_prior, q, o, do, lse, wl.scale, sel=s, dq=dq, ws=ws_b)

    stats = {}

    def run(step, name):
        log(f"[bench] {name}: {args.warmup} warmup steps")
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        pool.zero_grad()
        torch.cuda.synchronize()
        pkv.timing_enable(True)
        log(f"[bench] {name}: {args.steps} timed steps")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        for k in range(args.steps):
            step()
            ev[k + 1].record()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        pkv.timing_enable(False)
        kt = pkv.timing_collect()
        pool.check()
        per = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps))
        stats[name] = {"median_ms": round(per[len(per) // 2], 4), "min_ms": round(per[0], 4)}
        return dt / args.steps * 1e3, kt

    def graph_ms(step):
        """The step recorded once into a HIP graph (torch.cuda.CUDAGraph) and replayed back to back:
        per-step time without host launch cost or gaps between the step's kernels."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step()
        for _ in range(args.warmup):
            gr.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        pool.check()
        del gr
        return round(e0.elapsed_time(e1) / args.steps, 4)

    def select_b2b(n=50, copy_gbps=None):
        """page_topk_select alone, n calls back to back: steady-state per-call time and GB/s."""
        for _ in range(3):
            pkv.page_topk_select(pool, bt, n_prior, q, top_k, n_local, sel=sel, ws=ws_t)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            pkv.page_topk_select(pool, bt, n_prior, q, top_k, n_local, sel=sel, ws=ws_t)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        b = C * H_q * d * 2 + (n_prior - n_local) * H_kv * d * 4
        return {"ms_per_call": round(ms, 4), "GBps": round(b / (ms * 1e-3) / 1e9, 1), "bytes": b,
                "pct_hbm_peak": round(100.0 * b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                "pct_streaming_copy": None if copy_gbps is None else round(100.0 * b / (ms * 1e-3) / 1e9 / copy_gbps, 2)}

    pd = pairs_dense(C, q0)
    flop_dense = 14.0 * d * H_q * pd
    if args.only == "topk":
        ps = pairs_sparse(C, n_sel, P)
        ms_topk, kt_topk = run(step_topk, "topk256k")
        print(json.dumps({"workload": "topk256k", "ms_per_step": round(ms_topk, 4),
                          "TFLOP/s": round(14.0 * d * H_q * ps / (ms_topk * 1e-3) / 1e12, 2),
                          "per_kernel_ms": {k: round(v[1] / v[0], 4) for k, v in kt_topk.items()},
                          "select_back_to_back": select_b2b()}), flush=True)
        pool.free()
        return
    if args.only == "qpage":
        ps = pairs_sparse(C, n_sel, P)
        ms_qp, kt_qp = run(step_qpage, "qpage256k")
        print(json.dumps({"workload": "qpage256k", "ms_per_step": round(ms_qp, 4),
                          "TFLOP/s": round(14.0 * d * H_q * ps / (ms_qp * 1e-3) / 1e12, 2),
                          "per_kernel_ms": {k: round(v[1] / v[0], 4) for k, v in kt_qp.items()}}), flush=True)
        pool.free()
        return
    ms_dense, kt_dense = run(step_dense, "dense256k")
    tflops_dense = flop_dense / (ms_dense * 1e-3) / 1e12
    mfma_peak = mfma_loop_peak(pkv, dev)
    log(f"[bench] sustained MFMA loop: {mfma_peak:.1f} TFLOP/s")
    atomic = atomic_probe_rates(pkv, dev, wl)
    log(f"[bench] fp32 atomic adds: {atomic}")
    # Streaming-copy reference (1 GiB read + 1 GiB written) and cold-cache step times: a 1 GiB write
    # before each step evicts the L2 caches and the 256 MB Infinity Cache; events bracket the step only.
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    flush2 = torch.empty_like(flush)
    for _ in range(2):
        flush2.copy_(flush)
    ec0, ec1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ec0.record()
    for _ in range(5):
        flush2.copy_(flush)
    ec1.record()
    torch.cuda.synchronize()
    copy_gbps = 2.0 * (1 << 30) / (ec0.elapsed_time(ec1) / 5 * 1e-3) / 1e9
    del flush2

    def cold(step, n):
        times = []
        for i in range(n):
            flush.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        return {"median_ms": round(times[len(times) // 2], 4), "min_ms": round(times[0], 4), "steps": n}

    cold_dense = cold(step_dense, 5)
    log(f"[bench] streaming copy {copy_gbps:.0f} GB/s; dense256k cold cache {cold_dense}")
    log(f"[bench] dense256k: {ms_dense:.3f} ms/step, {tflops_dense:.1f} TFLOP/s")
    for kname, (n, ms) in sorted(kt_dense.items(), key=lambda x: -x[1][1]):
        log(f"[bench]   {kname:18s} launches {n:4d}  avg {ms / n:.3f} ms")

    # Roofline of the dominant kernel: its own algorithmic MFMA work per launch / its average duration.
    kernel_flop = {"k_attn_fwd": 4.0 * d * H_q * pd, "k_attn_fwd64": 4.0 * d * H_q * pd,
                   "k_bwd_dq": 6.0 * d * H_q * pd, "k_bwd_dq64": 6.0 * d * H_q * pd, "k_bwd_dkdv": 8.0 * d * H_q * pd}
    dom = max(kt_dense.items(), key=lambda x: x[1][1])[0]
    n_l, tot_ms = kt_dense[dom]
    avg_ms = tot_ms / n_l
    def split_ms(kt):
        fwd = sum(v[1] / v[0] for k, v in kt.items() if k in ("k_attn_fwd", "k_attn_fwd64", "k_fwd_combine"))
        bwd = sum(v[1] / v[0] for k, v in kt.items() if k.startswith("k_bwd"))
        return round(fwd, 4), round(bwd, 4)

    fwd_ms, bwd_ms = split_ms(kt_dense)
    if dom in kernel_flop:
        ach = kernel_flop[dom] / (avg_ms * 1e-3) / 1e12
        tb = traffic_bytes(dom)
        credited = {"k_attn_fwd": "4*d (S, PV)", "k_attn_fwd64": "4*d (S, PV)",
                    "k_bwd_dq": "6*d (S and dP recomputed, dQ)", "k_bwd_dq64": "6*d (S and dP recomputed, dQ)",
                    "k_bwd_dkdv": "8*d (S and dP recomputed, dV, dK)"}[dom]
        bwd_flop = 10.0 * d * H_q * pd
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": None if tb is None else int(tb[0] + tb[1]),
                    "traffic_fetch_write": None if tb is None else [int(tb[0]), int(tb[1])],
                    "avg_launch_ms": round(avg_ms, 4),
                    "credited_flop_per_pair": credited,
                    "note": "achieved credits the dominant kernel with the MFMA work it executes per (row, key) "
                            "pair; the two-pass backward executes 14*d per pair against the method's 10*d, so the "
                            "step executes 18*d per pair and the headline value credits only the method's 14*d",
                    "measured_mfma_loop_TFLOPs": round(mfma_peak, 1),
                    "frac_of_measured_mfma_loop": round(ach / mfma_peak, 4),
                    "method_backward_frac_of_peak": round(bwd_flop / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "method_step_frac_of_peak": round(tflops_dense / PEAK_BF16_TFLOPS, 4),
                    "executed_over_method_flop": round(18.0 / 14.0, 4),
                    "structural_ceiling_frac_of_peak": round(mfma_peak / PEAK_BF16_TFLOPS * 14.0 / 18.0, 4),
                    "per_kernel_ms": {k: round(v[1] / v[0], 4) for k, v in kt_dense.items()}}
    else:
        roofline = {"bound": "hbm", "kernel": dom, "achieved": None, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": None, "traffic": None, "avg_launch_ms": round(avg_ms, 4)}

    topk = None
    if not args.no_topk:
        ps = pairs_sparse(C, n_sel, P)
        flop_topk = 14.0 * d * H_q * ps
        ms_topk, kt_topk = run(step_topk, "topk256k")
        log(f"[bench] topk256k: {ms_topk:.3f} ms/step, {flop_topk / (ms_topk * 1e-3) / 1e12:.1f} TFLOP/s")
        for kname, (n, ms) in sorted(kt_topk.items(), key=lambda x: -x[1][1]):
            log(f"[bench]   {kname:18s} launches {n:4d}  avg {ms / n:.3f} ms")
        sel_ms = sum(v[1] / v[0] for k, v in kt_topk.items() if k in ("k_qsum_part", "k_hsum", "k_scores", "k_topk"))
        sel_bytes = C * H_q * d * 2 + (n_prior - n_local) * H_kv * d * 4  # Q chunk + candidate reps
        topk = {"workload": "topk256k: top-64 + 4 local pages of 2016 by mean-key score, + own block",
                "value": round(flop_topk / (ms_topk * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                "ms_per_step": round(ms_topk, 4), "flop_per_step": flop_topk,
                "step_speedup_vs_dense": round(ms_dense / ms_topk, 2),
                "select_ms": round(sel_ms, 4),
                "select_GBps": round(sel_bytes / (sel_ms * 1e-3) / 1e9, 1) if sel_ms > 0 else None,
                "select_back_to_back": select_b2b(copy_gbps=copy_gbps),
                "cold_cache": cold(step_topk, 10),
                "fwd_ms": split_ms(kt_topk)[0], "bwd_ms": split_ms(kt_topk)[1],
                "step_stats": stats.get("topk256k"),
                "per_kernel_ms": {k: round(v[1] / v[0], 4) for k, v in kt_topk.items()}}

    qpage = None
    if not args.no_topk:
        # Same pair count as the shared-list step: every query page attends to n_sel prior pages.
        ms_qp, kt_qp = run(step_qpage, "qpage256k")
        log(f"[bench] qpage256k: {ms_qp:.3f} ms/step, {flop_topk / (ms_qp * 1e-3) / 1e12:.1f} TFLOP/s")
        for kname, (n, ms) in sorted(kt_qp.items(), key=lambda x: -x[1][1]):
            log(f"[bench]   {kname:18s} launches {n:4d}  avg {ms / n:.3f} ms")
        qpage = {"workload": f"qpage256k: top-64 + 4 local pages of 2016 chosen per query page ({n_qp} query "
                             "pages x 4 KV heads), + own block",
                 "value": round(flop_topk / (ms_qp * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                 "ms_per_step": round(ms_qp, 4), "flop_per_step": flop_topk,
                 "vs_shared_list_step": round(ms_qp / ms_topk, 3),
                 "select_ms": round(sum(v[1] / v[0] for k, v in kt_qp.items()
                                        if k in ("k_qsum_part", "k_hsum", "k_scores", "k_topk")), 4),
                 "fwd_ms": split_ms(kt_qp)[0], "bwd_ms": split_ms(kt_qp)[1],
                 "step_stats": stats.get("qpage256k"),
                 "per_kernel_ms": {k: round(v[1] / v[0], 4) for k, v in kt_qp.items()}}

    local = None
    if not args.no_topk:
        ms_local, kt_local = run(step_local, "local256k")
        flop_local = 14.0 * d * H_q * pairs_sparse(C, LOCAL_WINDOW, P)
        log(f"[bench] local256k: {ms_local:.3f} ms/step, {flop_local / (ms_local * 1e-3) / 1e12:.1f} TFLOP/s")
        local = {"workload": f"local256k: window of the {LOCAL_WINDOW} most recent prior page(s) "
                             f"({LOCAL_WINDOW * P} tokens) + causal own block, selected with top_k = 0",
                 "value": round(flop_local / (ms_local * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                 "ms_per_step": round(ms_local, 4), "flop_per_step": flop_local,
                 "fwd_ms": split_ms(kt_local)[0], "bwd_ms": split_ms(kt_local)[1],
                 "mixed_pair_ms": round(ms_local + topk["ms_per_step"], 4),
                 "mixed_pair_note": "one local layer + one top-K layer (alternating policies), per pair",
                 "step_stats": stats.get("local256k")}

    host1m = None if args.no_host1m else bench_host1m(args, pkv, synth, dev, t16)
    dense_host = None if args.no_densehost else bench_dense_host(args, pkv, synth, dev, t16)
    recurrent = None if args.no_recurrent else bench_recurrent(args, pkv, dev)

    # Graph-replayed steps last: recording creates HIP streams, and with a handful of hardware
    # queues per process a stream created here could share a queue with the copy streams of the
    # host-tier measurements above and serialise them.
    if topk is not None:
        topk["graph_ms_per_step"] = graph_ms(step_topk)
    if local is not None:
        local["graph_ms_per_step"] = graph_ms(step_local)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle sample ({args.cpu_tokens} tokens)")
        cpu = cpu_baseline(wl, k_np, v_np, q_np, do_np, c, args.cpu_tokens)
        log(f"[bench] CPU oracle: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")
    pool.free()

    out = {
        "metric": METRIC, "value": round(tflops_dense, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_dense, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "dense256k: final 4096-token chunk at position 258048 over 2016 prior 128-token pages "
                               "+ causal own block, 28/4 heads, d=128, K = N(0,1) + per-page N(0,0.5) offset",
                   "context": wl.context, "chunk": C, "page": P, "h_q": H_q, "h_kv": H_kv, "head_dim": d,
                   "flop_per_step": flop_dense, "pct_bf16_peak": round(100.0 * tflops_dense / PEAK_BF16_TFLOPS, 2),
                   "pct_measured_mfma_loop": round(100.0 * tflops_dense / mfma_peak, 2),
                   "step": "append own block + forward + backward (dK/dV accumulated into gradient pages)"},
        "roofline": roofline,
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms, "step_stats": stats.get("dense256k"),
        "cpu_baseline": cpu,
        "cold_cache": {"dense256k": cold_dense,
                       "note": "a 1 GiB write before each step evicts the L2 caches and the 256 MB Infinity Cache; "
                               "HIP events bracket the step only; the headline value is the warm back-to-back rate"},
        "streaming_copy_GBps": round(copy_gbps, 1),
        "fp32_atomic_adds": atomic,
        "pool_fill": fill,
        "topk256k": topk,
        "qpage256k": qpage,
        "local256k": local,
        "host1m": host1m,
        "dense1m_host": dense_host,
        "recurrent_layer": recurrent,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
