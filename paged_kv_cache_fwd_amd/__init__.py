"""Python binding of libpkv (paged chunk attention for MI355X): argument marshalling only.

Every computation runs in the HIP kernels behind the C ABI declared in include/pkv.h. PyTorch is
used for device memory and the current stream. The binding raises if the compiled library is
missing; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import warnings
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_OK, PKV_E_INVALID, PKV_E_UNSUPPORTED, PKV_E_NOMEM, PKV_E_RANGE, PKV_E_HIP, PKV_E_STATE, PKV_E_DEVICE = \
    0, -1, -2, -3, -4, -5, -6, -7
PKV_GRADS, PKV_HOST_TIER, PKV_HOST_GRADS = 1, 2, 4
PKV_COPY_KV, PKV_COPY_GRAD = 1, 2
PKV_K, PKV_V, PKV_DK, PKV_DV, PKV_REP = 0, 1, 2, 3, 4

EXPORTED = (
    "pkv_version", "pkv_last_error", "paged_kv_alloc", "paged_kv_free", "paged_kv_info", "paged_kv_data",
    "paged_kv_append", "paged_kv_zero_grad", "paged_kv_export", "paged_kv_check", "page_topk_ws_bytes",
    "page_topk_select", "chunk_attn_fwd_ws_bytes", "chunk_attn_fwd", "chunk_attn_bwd_ws_bytes",
    "chunk_attn_bwd", "paged_kv_gather", "paged_kv_grad_offload", "paged_kv_copy", "pkv_mfma_probe",
    "pkv_timing_enable", "pkv_timing_collect",
    "pkv_timing_get", "paged_kv_page_alloc", "paged_kv_page_release", "paged_kv_pages_available",
    "page_topk_select_noalloc", "pkv_atomic_probe", "paged_kv_grad_staging_bytes", "paged_kv_grad_stage",
    "paged_kv_grad_accumulate",
)


class PkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pkv error {code}: {msg}")
        self.code = code


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_U = ctypes.c_uint32
_S = ctypes.c_size_t
_F = ctypes.c_float


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the compiled library (once). Raises if it was not built. PKV_LIBRARY in the environment
    names another build of the same library to use instead of the in-tree one."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("PKV_LIBRARY") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m paged_kv_cache_fwd_amd.build` "
                           "or __graft_entry__.build(); there is no fallback implementation")
    lib = ctypes.CDLL(p)
    sig = {
        "pkv_version": (_I, []),
        "pkv_last_error": (ctypes.c_char_p, []),
        "paged_kv_alloc": (_I, [ctypes.POINTER(_P), _I, _I, _I, _I, _U]),
        "paged_kv_free": (_I, [_P]),
        "paged_kv_info": (_I, [_P, ctypes.POINTER(_I), ctypes.POINTER(_I), ctypes.POINTER(_I), ctypes.POINTER(_I),
                               ctypes.POINTER(_U)]),
        "paged_kv_data": (_P, [_P, _I]),
        "paged_kv_append": (_I, [_P, _P, _I, _I, _I, _P, _P, _P]),
        "paged_kv_zero_grad": (_I, [_P, _P, _I, _P]),
        "paged_kv_export": (_I, [_P, _I, _P, _I, _I, _I, _P, _P]),
        "paged_kv_check": (_I, [_P]),
        "page_topk_ws_bytes": (_S, [_P, _I, _I, _I, _I]),
        "page_topk_select": (_I, [_P, _P, _I, _I, _P, _I, _I, _I, _I, _I, _P, ctypes.POINTER(_I), _P, _S, _P]),
        "chunk_attn_fwd_ws_bytes": (_S, [_P, _I, _I, _I, _I, _I, _I]),
        "chunk_attn_fwd": (_I, [_P, _P, _I, _I, _P, _I, _I, _I, _I, _P, _I, _I, _F, _P, _P, _P, _S, _P]),
        "chunk_attn_bwd_ws_bytes": (_S, [_P, _I, _I, _I, _I, _I, _I]),
        "chunk_attn_bwd": (_I, [_P, _P, _I, _P, _P, _I, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _I, _I, _F, _P, _P, _S,
                                _P]),
        "paged_kv_gather": (_I, [_P, _P, _P, _I, _P, _I, _I, _P, _P, _I, _I, _P]),
        "paged_kv_grad_offload": (_I, [_P, _P, _I, _P, _P, _I, _P, _I, _I, _I, _P]),
        "paged_kv_copy": (_I, [_P, _P, _U, _I, _I, _P]),
        "pkv_mfma_probe": (_I, [_I, _I, _P, ctypes.POINTER(ctypes.c_double), _P]),
        "pkv_timing_enable": (_I, [ctypes.c_int]),
        "pkv_timing_collect": (ctypes.c_int, []),
        "pkv_timing_get": (_I, [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_I),
                                ctypes.POINTER(ctypes.c_double)]),
        "paged_kv_page_alloc": (_I, [_P, _I, ctypes.POINTER(_I)]),
        "paged_kv_page_release": (_I, [_P, _I, ctypes.POINTER(_I)]),
        "paged_kv_pages_available": (_I, [_P]),
        "page_topk_select_noalloc": (_I, [_P, _P, _I, _I, _P, _I, _I, _I, _I, _I, _P, ctypes.POINTER(_I), _P]),
        "pkv_atomic_probe": (_I, [_I, _I, _I, _P, ctypes.POINTER(ctypes.c_double), _P]),
        "paged_kv_grad_staging_bytes": (_S, [_P, _I]),
        "paged_kv_grad_stage": (_I, [_P, _I, _I, _I, _P, _P, _S, _P]),
        "paged_kv_grad_accumulate": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(rc: int):
    if rc != PKV_OK:
        raise PkvError(rc, load().pkv_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _sel_ptr(sel: Optional[torch.Tensor], other: torch.Tensor):
    """Selection pointer: NULL means dense, so an empty selection (no prior page) passes another
    valid device pointer instead; with n_sel = 0 it is never read."""
    if sel is None:
        return None
    return ctypes.c_void_p(sel.data_ptr() if sel.numel() > 0 else other.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, dtype, name: str, shape=None):
    """The library sees only pointers, so every tensor is checked here: dtype, device, layout and,
    where the call fixes it, the exact shape (a wrong shape would make a kernel read past it)."""
    if not t.is_cuda or not t.is_contiguous() or t.dtype != dtype:
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor, got {t.dtype} on {t.device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need_q(pool: "Pool", q: torch.Tensor):
    """q is [C][H_q][d] bf16 with d the pool's head dimension; returns (C, H_q)."""
    _need(q, torch.bfloat16, "q")
    if q.dim() != 3 or q.shape[2] != pool.d:
        raise ValueError(f"q must be [C][H_q][{pool.d}], got {tuple(q.shape)}")
    return q.shape[0], q.shape[1]


class Pool:
    """A paged KV pool (pages of K|V in bf16, optional fp32 gradient pages, fp32 page reps)."""

    def __init__(self, n_pages: int, page_size: int, n_kv_heads: int, head_dim: int, grads: bool = True,
                 host_tier: bool = False, host_grads: bool = False):
        lib = load()
        h = ctypes.c_void_p()
        flags = (PKV_GRADS if grads else 0) | (PKV_HOST_TIER if host_tier else 0) | (PKV_HOST_GRADS if host_grads else 0)
        _check(lib.paged_kv_alloc(ctypes.byref(h), n_pages, page_size, n_kv_heads, head_dim, flags))
        self.handle = h
        self.n_pages, self.page, self.h_kv, self.d = n_pages, page_size, n_kv_heads, head_dim
        self.grads, self.host_tier, self.host_grads = grads, host_tier, host_grads

    def free(self):
        if self.handle:
            _check(load().paged_kv_free(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    def append(self, bt: torch.Tensor, pos0: int, k: torch.Tensor, v: torch.Tensor, stream=None):
        _need(bt, torch.int32, "bt")
        n = k.shape[0] if k.dim() == 3 else -1
        _need(k, torch.bfloat16, "k", (n, self.h_kv, self.d))
        _need(v, torch.bfloat16, "v", (n, self.h_kv, self.d))
        _check(load().paged_kv_append(self.handle, _ptr(bt), bt.numel(), pos0, n, _ptr(k), _ptr(v), _stream(stream)))

    def zero_grad(self, bt: Optional[torch.Tensor] = None, n_pages: int = 0, stream=None):
        _check(load().paged_kv_zero_grad(self.handle, _ptr(bt), n_pages, _stream(stream)))

    def export(self, what: int, bt: torch.Tensor, first_page: int, n_pages: int, stream=None) -> torch.Tensor:
        _need(bt, torch.int32, "bt")
        if what in (PKV_K, PKV_V):
            out = torch.empty((n_pages * self.page, self.h_kv, self.d), dtype=torch.bfloat16, device=bt.device)
        elif what in (PKV_DK, PKV_DV):
            out = torch.empty((n_pages * self.page, self.h_kv, self.d), dtype=torch.float32, device=bt.device)
        else:
            out = torch.empty((n_pages, self.h_kv, self.d), dtype=torch.float32, device=bt.device)
        _check(load().paged_kv_export(self.handle, what, _ptr(bt), bt.numel(), first_page, n_pages, _ptr(out),
                                      _stream(stream)))
        return out

    def check(self):
        _check(load().paged_kv_check(self.handle))

    def alloc_pages(self, n: int) -> list:
        """Take n physical pages from the pool's free list (raises PkvError PKV_E_NOMEM, taking none,
        when fewer are free); returns their ids for the caller's block table."""
        buf = (_I * max(n, 1))()
        _check(load().paged_kv_page_alloc(self.handle, n, buf))
        return [int(buf[i]) for i in range(n)]

    def release_pages(self, pages) -> None:
        """Return pages to the free list (all or none: an id outside the pool, not allocated, or
        repeated raises PKV_E_INVALID)."""
        pages = [int(p) for p in pages]
        buf = (_I * max(len(pages), 1))(*pages)
        _check(load().paged_kv_page_release(self.handle, len(pages), buf))

    def pages_available(self) -> int:
        n = load().paged_kv_pages_available(self.handle)
        if n < 0:
            _check(n)
        return n


class WorkspaceAllocationWarning(UserWarning):
    """A hot-path call had to allocate its own device workspace (the caller passed none, or one too
    small): pass ws= (sized by the *_ws_bytes queries) to keep the step free of allocations."""


_warned_ws = set()


def _ws(nbytes: int, device, ws: Optional[torch.Tensor], call: str) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    if call not in _warned_ws:  # once per entry point
        _warned_ws.add(call)
        warnings.warn(f"{call}: no workspace of {nbytes} bytes was passed, so one is allocated on every such call; "
                      "pass ws= to avoid allocating on the hot path", WorkspaceAllocationWarning, stacklevel=3)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def page_topk_select(pool: Pool, bt: torch.Tensor, n_prior: int, q: torch.Tensor, top_k: int, n_local: int,
                     sel: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None,
                     per_query_page: bool = False):
    """Returns sel [H_kv][n_sel] int32 (logical page ids, ascending per head), or with
    per_query_page one list per query page: [H_kv][C / page][n_sel]. A given sel buffer must be
    contiguous and large enough; the result is a view of its first elements."""
    lib = load()
    _need(bt, torch.int32, "bt")
    C, H_q = _need_q(pool, q)
    n_cand = max(n_prior - n_local, 0)
    n_sel = min(top_k, n_cand) + (n_prior - n_cand)
    n_lists = C // pool.page if per_query_page else 1
    shape = (pool.h_kv, n_lists, n_sel) if per_query_page else (pool.h_kv, n_sel)
    need = pool.h_kv * n_lists * n_sel
    if sel is None:
        sel = torch.empty(shape, dtype=torch.int32, device=q.device)
    _need(sel, torch.int32, "sel")
    if sel.numel() < need:
        raise ValueError(f"sel holds {sel.numel()} entries, {need} needed")
    nb = lib.page_topk_ws_bytes(pool.handle, n_prior, C, H_q, n_lists)
    ws = _ws(nb, q.device, ws, "page_topk_select")
    out_n = _I(0)
    _check(lib.page_topk_select(pool.handle, _ptr(bt), bt.numel(), n_prior, _ptr(q), C, H_q, top_k, n_local,
                                n_lists, _ptr(sel), ctypes.byref(out_n), _ptr(ws), nb, _stream(stream)))
    assert out_n.value == n_sel
    return sel if tuple(sel.shape) == shape else sel.view(-1)[:need].view(shape)


def page_topk_ws_bytes(pool: Pool, n_prior: int, C: int, H_q: int, n_lists: int = 1) -> int:
    return load().page_topk_ws_bytes(pool.handle, n_prior, C, H_q, n_lists)


def page_topk_select_noalloc(pool: Pool, bt: torch.Tensor, n_prior: int, q: torch.Tensor, top_k: int, n_local: int,
                             sel: torch.Tensor, stream=None, per_query_page: bool = False) -> torch.Tensor:
    """page_topk_select with the library's static scratch instead of a workspace, for callers that
    cannot allocate: nothing is allocated here either, so the output buffer sel is required
    ([H_kv][n_sel] int32, or [H_kv][C / page][n_sel] with per_query_page)."""
    _need(bt, torch.int32, "bt")
    C, H_q = _need_q(pool, q)
    n_cand = max(n_prior - n_local, 0)
    n_sel = min(top_k, n_cand) + (n_prior - n_cand)
    n_lists = C // pool.page if per_query_page else 1
    shape = (pool.h_kv, n_lists, n_sel) if per_query_page else (pool.h_kv, n_sel)
    _need(sel, torch.int32, "sel", shape)
    out_n = _I(0)
    _check(load().page_topk_select_noalloc(pool.handle, _ptr(bt), bt.numel(), n_prior, _ptr(q), C, H_q, top_k, n_local,
                                           n_lists, _ptr(sel), ctypes.byref(out_n), _stream(stream)))
    return sel


def chunk_attn_fwd_ws_bytes(pool: Pool, n_prior: int, n_sel: int, n_kvh: int, C: int, H_q: int,
                            n_lists: int = 1) -> int:
    return load().chunk_attn_fwd_ws_bytes(pool.handle, n_prior, n_sel, n_lists, n_kvh, C, H_q)


def chunk_attn_bwd_ws_bytes(pool: Pool, n_prior: int, n_sel: int, n_kvh: int, C: int, H_q: int,
                            n_lists: int = 1) -> int:
    return load().chunk_attn_bwd_ws_bytes(pool.handle, n_prior, n_sel, n_lists, n_kvh, C, H_q)


def _sel_shape(sel: Optional[torch.Tensor], pool: Pool):
    """(n_sel, n_lists) of a selection: None -> dense; [H_kv][n_sel]; [H_kv][C/page][n_sel]. The
    kernels index it by absolute KV head, so it holds a row per KV head of the pool."""
    if sel is None:
        return -1, 1
    _need(sel, torch.int32, "sel")
    if sel.dim() not in (2, 3) or sel.shape[0] != pool.h_kv:
        raise ValueError(f"sel must be [{pool.h_kv}][n_sel] or [{pool.h_kv}][C/page][n_sel], "
                         f"got shape {tuple(sel.shape)}")
    return (sel.shape[1], 1) if sel.dim() == 2 else (sel.shape[2], sel.shape[1])


def chunk_attn_fwd(pool: Pool, bt: torch.Tensor, n_prior: int, q: torch.Tensor, scale: float,
                   sel: Optional[torch.Tensor] = None, kvh0: int = 0, n_kvh: Optional[int] = None,
                   o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None, stream=None):
    """Forward of one chunk; returns (o [C][H_q][d] bf16, lse [H_q][C] fp32). sel: None (dense),
    [H_kv][n_sel] (one list per KV head) or [H_kv][C/page][n_sel] (one list per query page)."""
    lib = load()
    _need(bt, torch.int32, "bt")
    C, H_q = _need_q(pool, q)
    n_kvh = pool.h_kv - kvh0 if n_kvh is None else n_kvh
    n_sel, n_lists = _sel_shape(sel, pool)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H_q, C), dtype=torch.float32, device=q.device)
    _need(o, torch.bfloat16, "o", q.shape)
    _need(lse, torch.float32, "lse", (H_q, C))
    nb = lib.chunk_attn_fwd_ws_bytes(pool.handle, n_prior, n_sel, n_lists, n_kvh, C, H_q)
    ws = _ws(nb, q.device, ws, "chunk_attn_fwd")
    _check(lib.chunk_attn_fwd(pool.handle, _ptr(bt), bt.numel(), n_prior, _sel_ptr(sel, bt), max(n_sel, 0), n_lists,
                              kvh0, n_kvh,
                              _ptr(q), C, H_q, float(scale), _ptr(o), _ptr(lse), _ptr(ws), nb, _stream(stream)))
    return o, lse


def chunk_attn_bwd(pool: Pool, bt: torch.Tensor, n_prior: int, q: torch.Tensor, o: torch.Tensor,
                   dout: torch.Tensor, lse: torch.Tensor, scale: float, sel: Optional[torch.Tensor] = None,
                   kvh0: int = 0, n_kvh: Optional[int] = None, gpool: Optional[Pool] = None,
                   gbt: Optional[torch.Tensor] = None, dq: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None, stream=None):
    """Backward of one chunk; returns dq. dK/dV are added into the gradient pages of gpool."""
    lib = load()
    _need(bt, torch.int32, "bt")
    C, H_q = _need_q(pool, q)
    for t, nm in ((o, "o"), (dout, "dout")):
        _need(t, torch.bfloat16, nm, q.shape)
    _need(lse, torch.float32, "lse", (H_q, C))
    n_kvh = pool.h_kv - kvh0 if n_kvh is None else n_kvh
    n_sel, n_lists = _sel_shape(sel, pool)
    gpool = pool if gpool is None else gpool
    gbt = bt if gbt is None else gbt
    _need(gbt, torch.int32, "gbt")
    if dq is None:
        dq = torch.empty_like(q)
    _need(dq, torch.bfloat16, "dq", q.shape)
    nb = lib.chunk_attn_bwd_ws_bytes(pool.handle, n_prior, n_sel, n_lists, n_kvh, C, H_q)
    ws = _ws(nb, q.device, ws, "chunk_attn_bwd")
    _check(lib.chunk_attn_bwd(pool.handle, _ptr(bt), bt.numel(), gpool.handle, _ptr(gbt), gbt.numel(), n_prior,
                              _sel_ptr(sel, bt), max(n_sel, 0), n_lists, kvh0, n_kvh, _ptr(q), _ptr(o), _ptr(dout), _ptr(lse), C,
                              H_q, float(scale), _ptr(dq), _ptr(ws), nb, _stream(stream)))
    return dq


def paged_kv_gather(host: Pool, dev: Pool, host_bt: torch.Tensor, sel_row: torch.Tensor, kvh: int,
                    dst_pages: torch.Tensor, dev_bt_out: Optional[torch.Tensor] = None, n_workgroups: int = 0,
                    stream=None):
    """Copy the (page, kvh) blocks of the logical pages sel_row from a host-tier pool into the device
    pool pages dst_pages (both int32 device vectors of equal length); optionally record
    dev_bt_out[sel_row[i]] = dst_pages[i]. n_workgroups: CUs the copy holds (0: 8, the host link's
    rate; 2 for a copy that runs beside attention kernels)."""
    _need(host_bt, torch.int32, "host_bt")
    _need(sel_row, torch.int32, "sel_row")
    _need(dst_pages, torch.int32, "dst_pages", sel_row.shape)
    if dev_bt_out is not None:
        _need(dev_bt_out, torch.int32, "dev_bt_out")
    _check(load().paged_kv_gather(host.handle, dev.handle, _ptr(host_bt), host_bt.numel(), _ptr(sel_row),
                                  sel_row.numel(), kvh, _ptr(dst_pages), _ptr(dev_bt_out),
                                  0 if dev_bt_out is None else dev_bt_out.numel(), n_workgroups, _stream(stream)))


def paged_kv_grad_offload(host: Pool, host_bt: torch.Tensor, dev: Pool, dev_bt: torch.Tensor, lps: torch.Tensor,
                          kvh0: int = 0, n_kvh: Optional[int] = None, stream=None):
    """host grad[host_bt[lp]][g] += dev grad[dev_bt[lp]][g] and the device block is cleared, for the
    logical pages lps (int32, distinct) and KV heads [kvh0, kvh0 + n_kvh)."""
    _need(host_bt, torch.int32, "host_bt")
    _need(dev_bt, torch.int32, "dev_bt")
    _need(lps, torch.int32, "lps")
    n_kvh = host.h_kv - kvh0 if n_kvh is None else n_kvh
    _check(load().paged_kv_grad_offload(host.handle, _ptr(host_bt), host_bt.numel(), dev.handle, _ptr(dev_bt),
                                        dev_bt.numel(), _ptr(lps), lps.numel(), kvh0, n_kvh, _stream(stream)))


def grad_staging_bytes(pool: Pool, n: int) -> int:
    return load().paged_kv_grad_staging_bytes(pool.handle, n)


def paged_kv_grad_stage(dev: Pool, dev_page0: int, n: int, kvh: int, lps: torch.Tensor, staging: torch.Tensor,
                        stream=None):
    """Copy head kvh's gradient blocks of device pages [dev_page0, dev_page0 + n) and the logical ids
    lps (int32, device) into pinned host staging (uint8, pinned), then clear those device blocks."""
    _need(lps, torch.int32, "lps")
    if lps.numel() < n:
        raise ValueError(f"lps holds {lps.numel()} ids, {n} needed")
    if staging.is_cuda or not staging.is_pinned() or not staging.is_contiguous():
        raise ValueError("staging must be a contiguous pinned host tensor")
    _check(load().paged_kv_grad_stage(dev.handle, dev_page0, n, kvh, _ptr(lps), _ptr(staging),
                                      staging.numel() * staging.element_size(), _stream(stream)))


def paged_kv_grad_accumulate(host: Pool, host_bt_host: torch.Tensor, n: int, kvh: int, staging: torch.Tensor,
                             stream=None):
    """Enqueue the host-side add of n staged blocks into the host pool's gradient pages, head kvh.
    host_bt_host (int32, host) and staging must stay alive until the stream has passed this call."""
    if host_bt_host.is_cuda or host_bt_host.dtype != torch.int32 or not host_bt_host.is_contiguous():
        raise ValueError("host_bt_host must be a contiguous int32 host tensor")
    if staging.is_cuda or not staging.is_pinned():
        raise ValueError("staging must be a pinned host tensor")
    _check(load().paged_kv_grad_accumulate(host.handle, _ptr(host_bt_host), host_bt_host.numel(), n, kvh,
                                           _ptr(staging), _stream(stream)))


def paged_kv_copy(src: Pool, dst: Pool, what: int, first_page: int = 0, n_pages: Optional[int] = None, stream=None):
    """Copy physical pages [first_page, first_page + n_pages) of src into the same pages of dst:
    KV pages with PKV_COPY_KV, gradient pages with PKV_COPY_GRAD (host or device pools alike)."""
    n_pages = min(src.n_pages, dst.n_pages) - first_page if n_pages is None else n_pages
    _check(load().paged_kv_copy(src.handle, dst.handle, what, first_page, n_pages, _stream(stream)))


def mfma_probe(n_workgroups: int, iters: int, out: torch.Tensor, stream=None) -> float:
    """Enqueue the sustained-MFMA diagnostic; returns its FLOP count (the caller times it)."""
    _need(out, torch.float32, "out", (n_workgroups * 512,))
    flop = ctypes.c_double(0.0)
    _check(load().pkv_mfma_probe(n_workgroups, iters, _ptr(out), ctypes.byref(flop), _stream(stream)))
    return flop.value


def atomic_probe(n_workgroups: int, n_regions: int, region_elems: int, buf: torch.Tensor, stream=None) -> float:
    """Enqueue the fp32 atomic-add diagnostic on buf ([n_regions * region_elems] float32); returns the
    bytes it adds (the caller times it)."""
    _need(buf, torch.float32, "buf", (n_regions * region_elems,))
    nbytes = ctypes.c_double(0.0)
    _check(load().pkv_atomic_probe(n_workgroups, n_regions, region_elems, _ptr(buf), ctypes.byref(nbytes),
                                   _stream(stream)))
    return nbytes.value


def timing_enable(on: bool = True):
    """Start (clearing earlier records) or stop per-kernel HIP-event timing inside the library."""
    _check(load().pkv_timing_enable(1 if on else 0))


def timing_collect() -> dict:
    """Wait for the recorded launches; return {kernel name: (launches, total ms)}."""
    lib = load()
    n = lib.pkv_timing_collect()
    if n < 0:
        _check(n)
    out = {}
    for i in range(n):
        name = ctypes.c_char_p()
        cnt = _I(0)
        ms = ctypes.c_double(0.0)
        _check(lib.pkv_timing_get(i, ctypes.byref(name), ctypes.byref(cnt), ctypes.byref(ms)))
        out[name.value.decode()] = (cnt.value, ms.value)
    return out
