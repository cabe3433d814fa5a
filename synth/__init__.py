"""Seeded synthetic inputs for paged chunk attention.

This module only draws random numbers and stores them as bf16 bit patterns. It holds none of the
attention, selection or paging arithmetic: both the HIP path and the CPU oracle receive exactly
the bytes produced here.

Workload shapes follow the synthetic recipe for OOMB-style training described in the web summaries
of "Out of the Memory Barrier: A Highly Memory Efficient Training System for LLMs with
Million-Token Contexts" (gist.science pt/es/it, section 2 "Methodology" and section 4 / 3
"Results": Qwen2.5-7B, 256K and 1M contexts). The pages print no data, so every tensor is drawn
from the distributions stated in the workload descriptions below.

Streams: each tensor piece comes from ``numpy.random.default_rng(SeedSequence([seed, tensor_id,
index]))`` so that any page or chunk can be regenerated on its own (tensor ids: Q=0, K=1, V=2,
dO=3, page offset=4, permutation=5).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

T_Q, T_K, T_V, T_DO, T_OFF, T_PERM = 0, 1, 2, 3, 4, 5


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even. Inputs are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = bits + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_widen(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, tensor_id: int, index: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tensor_id), int(index)]))


@dataclass(frozen=True)
class Workload:
    """Shape and data recipe of one synthetic paged-attention workload."""
    name: str
    h_q: int
    h_kv: int
    d: int
    page: int            # tokens per page
    context: int         # total tokens including the last chunk
    chunk: int           # tokens per query chunk
    chunks: tuple        # chunk indices processed (forward + backward)
    offset_std: float = 0.0   # std of the per-(page, kv head) key offset vector
    top_k: Optional[int] = None
    n_local: int = 0
    host_tier: bool = False
    seed: int = 0
    note: str = ""

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def n_pages(self) -> int:
        return self.context // self.page

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def q0(self, c: int) -> int:
        return c * self.chunk

    def n_prior(self, c: int) -> int:
        return self.q0(c) // self.page

    def with_seed(self, seed: int) -> "Workload":
        return replace(self, seed=seed)


WORKLOADS = {
    # 4 query heads / 1 KV head, d=64, 2048 tokens as 4 chunks of 512, page 64, dense.
    "tiny": Workload("tiny", 4, 1, 64, 64, 2048, 512, (0, 1, 2, 3),
                     note="4/1 heads, d=64, 2048 tokens as 4x512, page 64, dense"),
    # Qwen2.5-7B attention shape, 32K context as 8 chunks of 4096, page 128, dense.
    "qwen32k": Workload("qwen32k", 28, 4, 128, 128, 32768, 4096, tuple(range(8)),
                        note="28/4 heads, d=128, 32K as 8x4096, page 128, dense"),
    # Last 4096-token chunk at position 258048 (2016 prior pages), keys carry a per-page offset.
    "dense256k": Workload("dense256k", 28, 4, 128, 128, 262144, 4096, (63,), offset_std=0.5,
                          note="28/4 heads, d=128, final 4096-token chunk over 2016 prior pages + own block"),
    # Same data, top-64 pages by mean-key score plus the 4 most recent prior pages.
    "topk256k": Workload("topk256k", 28, 4, 128, 128, 262144, 4096, (63,), offset_std=0.5,
                         top_k=64, n_local=4,
                         note="as dense256k, top-64 + 4 local prior pages + own block"),
    # 1M tokens, prior pages in pinned host memory, top-128 + 8 local.
    "host1m": Workload("host1m", 28, 4, 128, 128, 1048576, 4096, (255,), offset_std=0.5,
                       top_k=128, n_local=8, host_tier=True,
                       note="28/4 heads, d=128, 8192 pages (8160 prior in pinned host memory), top-128 + 8 local"),
}


def k_page(wl: Workload, p: int) -> np.ndarray:
    """Keys of logical page p as bf16 bits, shape [page][h_kv][d].

    Values: N(0,1) float32, plus (if offset_std > 0) one N(0, offset_std^2) vector per (page, kv
    head) added to every token of the page, then a single bf16 rounding.
    """
    x = _rng(wl.seed, T_K, p).standard_normal((wl.page, wl.h_kv, wl.d), dtype=np.float32)
    if wl.offset_std > 0.0:
        off = _rng(wl.seed, T_OFF, p).standard_normal((wl.h_kv, wl.d), dtype=np.float32)
        x = x + np.float32(wl.offset_std) * off[None, :, :]
    return bf16_round(x)


def v_page(wl: Workload, p: int) -> np.ndarray:
    """Values of logical page p as bf16 bits, shape [page][h_kv][d], N(0,1)."""
    x = _rng(wl.seed, T_V, p).standard_normal((wl.page, wl.h_kv, wl.d), dtype=np.float32)
    return bf16_round(x)


def q_chunk(wl: Workload, c: int) -> np.ndarray:
    """Queries of chunk c as bf16 bits, shape [chunk][h_q][d], N(0,1)."""
    x = _rng(wl.seed, T_Q, c).standard_normal((wl.chunk, wl.h_q, wl.d), dtype=np.float32)
    return bf16_round(x)


def do_chunk(wl: Workload, c: int) -> np.ndarray:
    """Output gradient of chunk c as bf16 bits, shape [chunk][h_q][d], N(0,1)."""
    x = _rng(wl.seed, T_DO, c).standard_normal((wl.chunk, wl.h_q, wl.d), dtype=np.float32)
    return bf16_round(x)


def kv_tokens(wl: Workload, first_page: int, n_pages: int):
    """Keys and values for logical pages [first_page, first_page + n_pages) as contiguous
    [n_pages * page][h_kv][d] bf16 bit arrays."""
    ks = [k_page(wl, p) for p in range(first_page, first_page + n_pages)]
    vs = [v_page(wl, p) for p in range(first_page, first_page + n_pages)]
    shape = (n_pages * wl.page, wl.h_kv, wl.d)
    return np.concatenate(ks).reshape(shape), np.concatenate(vs).reshape(shape)


def page_permutation(wl: Workload, n_physical: Optional[int] = None) -> np.ndarray:
    """Block table: logical page -> physical page, a seeded random permutation (int32)."""
    n = wl.n_pages if n_physical is None else n_physical
    perm = _rng(wl.seed, T_PERM, 0).permutation(n).astype(np.int32)
    return perm[: wl.n_pages].copy()
