"""CPU oracle for chunk attention over a paged KV cache -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark may import or run
anything in this package. The product path (the HIP library and its Python binding) never calls
it and fails loudly when its compiled library is missing.

What it computes follows the web summaries of "Out of the Memory Barrier: A Highly Memory
Efficient Training System for LLMs with Million-Token Contexts" (gist.science, three language
editions: pt, es, it). Citations below name the edition and its section, e.g. "pt 2.A" is the
Portuguese edition, section 2 (Methodology), part A.

* ``attention``: forward and analytic backward of one query chunk against all earlier keys plus
  its own causal block (pt 2.A chunk-recurrent training; pt 2.B paged KV cache with gradients
  accumulated in place; es 2.B; it 2.A-2.B), optionally restricted to selected key pages
  (pt 2.C, es 2.B, it 2.D).
* ``selection``: page representatives (mean key per page), the query-chunk summary, dot-product
  page scores and the top-K page choice, in one fixed float32 operation order (es 2.B "Page-level
  sparse attention": a mean representative vector per key page, most relevant pages for the
  current queries).

Everything is plain NumPy. Nothing here is shared with, or imported from, the HIP path.
"""
from .attention import (
    widen_bf16,
    visible_keys,
    group_forward,
    group_backward,
    chunk_forward,
    chunk_backward,
    key_gradients,
)
from .selection import (
    page_key_sums,
    page_reps,
    query_sum,
    page_scores,
    select_pages,
    n_selected,
    topk_pages,
    topk_pages_per_query_page,
)

__all__ = [
    "widen_bf16", "visible_keys", "group_forward", "group_backward", "chunk_forward", "chunk_backward", "key_gradients",
    "page_key_sums", "page_reps", "query_sum", "page_scores", "select_pages", "n_selected", "topk_pages",
]
