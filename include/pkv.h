/*
 * pkv -- chunk attention over a paged KV cache, forward and backward, for AMD MI355X (gfx950).
 *
 * C ABI. Every pointer argument named *_dev is a device pointer (or a device-mapped pinned host
 * pointer where stated); every other pointer is host memory. Sizes are element counts unless the
 * name ends in _bytes. No call allocates memory except paged_kv_alloc. Compute calls enqueue work
 * on the caller's HIP stream (passed as void*; NULL is the default stream) and return without
 * synchronising; device faults surface at the caller's next synchronisation.
 *
 * Citations name the web summaries of "Out of the Memory Barrier: A Highly Memory Efficient
 * Training System for LLMs with Million-Token Contexts" (gist.science, editions pt / es / it)
 * and a section on them.
 *
 * Conventions shared by all calls:
 *  - bf16 values travel as uint16_t bit patterns.
 *  - A pool stores, per physical page p and KV head g, one contiguous block
 *      kv[p][g][0][t][d] = key, kv[p][g][1][t][d] = value   (bf16, t < page_size, d < head_dim)
 *    and, if created with PKV_GRADS, a gradient block of the same shape in fp32
 *      grad[p][g][0][t][d] = dK, grad[p][g][1][t][d] = dV,
 *    plus one fp32 representative key (mean key) per page and head, rep[p][g][d].
 *  - A block table bt_dev (int32, device) maps logical page i (token positions
 *    [i*page_size, (i+1)*page_size)) to a physical page bt_dev[i]. It is owned by the caller and
 *    may be any permutation. n_bt is its length.
 *  - Queries and query gradients of one chunk are [C][H_q][head_dim] bf16, row-major. Query head
 *    h reads KV head h / G with G = H_q / H_kv. The chunk starts at token q0 = n_prior*page_size.
 *  - lse is [H_q][C] fp32 natural-log log-sum-exp of the scaled scores.
 *  - Validation happens before anything is enqueued; a call that fails enqueues nothing.
 *    Block-table and selection entries live on the device and are checked there: an entry out of
 *    range is skipped (treated as an empty page) and recorded in the pool's error word, read by
 *    paged_kv_check.
 *  - Errors: the return value is a status code below; pkv_last_error() gives a message
 *    (thread-local, valid until the next call on the same thread).
 *  - HIP graphs: paged_kv_zero_grad, paged_kv_append, page_topk_select and chunk_attn_fwd / _bwd
 *    may be recorded into a HIP graph by stream capture (tested: a whole step, replayed) when the
 *    caller passes every workspace (ws_dev with enough ws_bytes) and the timing hooks are off:
 *    they then enqueue kernels only (memory is cleared by fill kernels, never by memset nodes),
 *    allocate nothing and never synchronise. paged_kv_alloc, paged_kv_free and paged_kv_check
 *    synchronise the device and must stay outside a capture.
 *  - Streams: overlap between calls on different streams (host-tier gathers, gradient offload,
 *    page copies beside attention) needs those streams on different hardware queues. HIP spreads
 *    a process's streams over a small number of hardware queues, so keep the number of live
 *    streams within it, or copies may run serialised behind the kernels of another stream.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK 0
#define PKV_E_INVALID (-1)     /* null pointer, bad shape, C % page_size != 0, H_q % H_kv != 0 */
#define PKV_E_UNSUPPORTED (-2) /* head_dim not in {64,128} or page_size not in {64,128} */
#define PKV_E_NOMEM (-3)       /* allocation failed or workspace too small */
#define PKV_E_RANGE (-4)       /* token positions or pages beyond the pool or block table */
#define PKV_E_HIP (-5)         /* a HIP runtime call failed; see pkv_last_error */
#define PKV_E_STATE (-6)       /* operation not valid for this pool (e.g. attention on a host-tier pool) */
#define PKV_E_DEVICE (-7)      /* paged_kv_check: a kernel met an out-of-range table entry */

#define PKV_GRADS 1u      /* allocate fp32 gradient pages (zero-initialised) on the device */
#define PKV_HOST_TIER 2u  /* keep the bf16 KV pages in pinned, device-mapped host memory */
#define PKV_HOST_GRADS 4u /* with PKV_GRADS: keep the fp32 gradient pages in pinned host memory */

/* paged_kv_copy selectors (bit mask) */
#define PKV_COPY_KV 1u   /* the bf16 KV pages */
#define PKV_COPY_GRAD 2u /* the fp32 gradient pages */

/* paged_kv_export / paged_kv_import selectors */
#define PKV_K 0
#define PKV_V 1
#define PKV_DK 2
#define PKV_DV 3
#define PKV_REP 4

typedef struct pkv_pool pkv_pool;

/* Library version (major*10000 + minor*100 + patch). */
int pkv_version(void);

/* Message for the last failed call on this thread ("" if none). Never NULL. */
const char* pkv_last_error(void);

/*
 * Create a pool of n_pages physical pages on the current HIP device.
 * Paged KV cache with gradients kept in pages too: pt 2.B, es 2.B ("paged memory manager"), it 2.B.
 * flags: PKV_GRADS adds fp32 gradient pages (zeroed); PKV_HOST_TIER places the KV pages in pinned
 * host memory that kernels read over the host link (pt 2.D, es 2.B "asynchronous CPU offloading",
 * it 2.C); gradients and representatives of such a pool stay on the device unless PKV_HOST_GRADS
 * (with PKV_GRADS) places the gradient pages in pinned, device-mapped host memory too (pt 2.D: the
 * gradients of the KV cache move to CPU memory as well). Backward passes never accumulate into
 * host gradient pages directly: they accumulate into a device pool's pages, which
 * paged_kv_grad_offload then adds to the host pages.
 * The pool owns all its memory; paged_kv_free releases it.
 */
int paged_kv_alloc(pkv_pool** out, int32_t n_pages, int32_t page_size, int32_t n_kv_heads,
                   int32_t head_dim, uint32_t flags);

/*
 * Gradient offload for a host tier (pt 2.D / es 2.B "asynchronous CPU offloading": the KV cache
 * and its gradients move between GPU and CPU memory on dedicated streams). For each of the n
 * logical pages lp = lp_dev[i] and KV heads g in [kvh0, kvh0 + n_kvh):
 *   host grad[host_bt[lp]][g] += dev grad[dev_bt[lp]][g]   (dK and dV blocks, fp32)
 *   dev grad[dev_bt[lp]][g] = 0                           (the device page is ready for reuse)
 * host must have PKV_GRADS | PKV_HOST_GRADS, dev PKV_GRADS without PKV_HOST_GRADS. The host pages are
 * read and written over the host link by the kernel; lp_dev lists distinct pages. Calls that
 * touch the same host page must not overlap (order them on one stream). Out-of-range table
 * entries are skipped and recorded (paged_kv_check on either pool).
 */
int paged_kv_grad_offload(pkv_pool* host, const int32_t* host_bt_dev, int32_t n_host_bt, pkv_pool* dev,
                          const int32_t* dev_bt_dev, int32_t n_dev_bt, const int32_t* lp_dev, int32_t n,
                          int32_t kvh0, int32_t n_kvh, void* stream);

/*
 * Gradient offload for a host tier through the copy engines, in two stream-ordered steps (pt 2.D /
 * es 2.B "asynchronous CPU offloading": the gradients of the KV cache move to CPU memory on
 * dedicated streams; it 2.C). Unlike paged_kv_grad_offload no kernel touches host memory: the host
 * pages receive the sums from host threads.
 *
 * paged_kv_grad_stage: for i < n, copies head kvh's gradient block (dK then dV, 2 * page_size *
 * head_dim floats) of device page dev_page0 + i into staging block i with one rectangular
 * device-to-host copy (a copy engine, no compute units), copies the n logical page ids lp_dev[0..n)
 * beside them, and then clears those device blocks with a fill kernel (ready for the next
 * backward). staging_host: pinned host memory of at least paged_kv_grad_staging_bytes(dev, n)
 * bytes, laid out as n int32 page ids (padded to 256 bytes) followed by the n blocks. dev: a pool
 * with device gradient pages; [dev_page0, dev_page0 + n) inside it.
 *
 * paged_kv_grad_accumulate: enqueues on stream a host function that, once the work before it on
 * the stream is done, adds staged block i into host grad[host_bt_host[lp[i]]][kvh] of host (a pool
 * with PKV_HOST_GRADS), lp being the ids staged beside the blocks. host_bt_host is a host copy of
 * the host pool's block table (n_host_bt entries); it and the staging must stay valid until the
 * function has run. The adds run on the library's host threads (PKV_HOST_THREADS in the
 * environment, default 8, sets their number). A staged id outside [0, n_host_bt) or a table entry
 * outside the pool is skipped and reported by paged_kv_check(host). Each host pool keeps 1024 job
 * slots, so enqueueing allocates nothing: a call made while 1024 earlier calls on the pool are still
 * pending waits on the host for the oldest to run, and fails with PKV_E_STATE after 60 s. The host
 * function makes this call unfit for HIP graph capture.
 *
 * Ordering is the caller's: stage after the backward that wrote the blocks, accumulate after the
 * stage (same stream, or an event), reuse a staging buffer only after its accumulation has run,
 * and let calls that add into the same host pages run one after another (the library runs one
 * accumulation at a time). Apart from that back-pressure nothing here waits on the host. Errors:
 * PKV_E_INVALID (NULL pointers, ranges, kvh), PKV_E_STATE (pool kinds, pending slots), PKV_E_NOMEM
 * (staging too small), PKV_E_HIP (a copy, kernel or host function could not be enqueued).
 */
size_t paged_kv_grad_staging_bytes(const pkv_pool* pool, int32_t n);
int paged_kv_grad_stage(pkv_pool* dev, int32_t dev_page0, int32_t n, int32_t kvh, const int32_t* lp_dev,
                        void* staging_host, size_t staging_bytes, void* stream);
int paged_kv_grad_accumulate(pkv_pool* host, const int32_t* host_bt_host, int32_t n_host_bt, int32_t n, int32_t kvh,
                             const void* staging_host, void* stream);

/*
 * Bulk page copy between two pools of the same page size, heads and dim, for dense attention over a
 * host tier (pt 2.D: with dense or local attention the next block is fetched while the current one
 * is computed; es 2.B: transfers overlap the next layer's compute). Copies physical pages
 * [first_page, first_page + n_pages) of src into the same physical pages of dst: the KV pages if
 * what has PKV_COPY_KV, the gradient pages if it has PKV_COPY_GRAD (both pools need gradient pages
 * then). Physical page numbers are kept, so one block table serves both pools. Either pool may live
 * in host or device memory; each range is one contiguous hipMemcpyAsync on stream, which the
 * runtime serves with its copy engines (no compute units). Nothing synchronises; src and dst must
 * be different pools, and the caller orders the copy against kernels that touch either range.
 * n_pages = 0 is a no-op. Errors: PKV_E_INVALID (NULL pool, same pool, shape mismatch, range
 * outside either pool, unknown bits), PKV_E_STATE (PKV_COPY_GRAD on a pool without gradients),
 * PKV_E_HIP (the copy could not be enqueued).
 */
int paged_kv_copy(const pkv_pool* src, pkv_pool* dst, uint32_t what, int32_t first_page, int32_t n_pages,
                  void* stream);

/* Release a pool and all its memory (the paged memory manager owns its pages: pt 2.B, it 2.B).
 * Synchronises the device first, so no enqueued kernel still reads the pages. NULL is a no-op
 * returning PKV_OK. */
int paged_kv_free(pkv_pool* pool);

/*
 * Page allocation from the pool's free list (pt 2.B, it 2.B: the paged memory manager hands out
 * fixed-size pages, so appending never reallocates or copies, and released pages are reused with no
 * fragmentation). A new pool has every physical page free; they are handed out from page 0 up, and
 * afterwards the most recently released page first. paged_kv_page_alloc takes n pages and writes
 * their physical ids to pages_host (host memory, n entries), which the caller places in its block
 * table; with fewer than n pages free it fails with PKV_E_NOMEM and takes none.
 * paged_kv_page_release returns n pages; an id outside the pool, a page that is not allocated or an
 * id listed twice fails the call with PKV_E_INVALID and releases none. paged_kv_pages_available
 * returns the number of free pages (a negative status for a NULL pool). These calls only keep host
 * bookkeeping: nothing is enqueued or synchronised, so the caller orders the reuse of a released
 * page after the kernels that still read or write it. The three calls are thread-safe per pool.
 * Block tables need not come from the allocator: kernels accept any table whose entries lie in
 * the pool.
 */
int paged_kv_page_alloc(pkv_pool* pool, int32_t n, int32_t* pages_host);
int paged_kv_page_release(pkv_pool* pool, int32_t n, const int32_t* pages_host);
int32_t paged_kv_pages_available(const pkv_pool* pool);

/* Shape of a pool (any output pointer may be NULL). */
int paged_kv_info(const pkv_pool* pool, int32_t* n_pages, int32_t* page_size, int32_t* n_kv_heads,
                  int32_t* head_dim, uint32_t* flags);

/*
 * Device address of a pool array: what = PKV_K/PKV_V give the bf16 KV base (both return the same
 * base, the [K|V] index is part of the layout above), PKV_DK/PKV_DV the fp32 gradient base,
 * PKV_REP the fp32 representative base. For PKV_HOST_TIER pools the KV base is the device-mapped
 * pointer of the pinned host array. Returns NULL on error.
 */
void* paged_kv_data(const pkv_pool* pool, int32_t what);

/*
 * Append n_tokens tokens at positions [pos0, pos0 + n_tokens) without moving any existing page
 * (pt 2.B: no reallocation or copy on append). k_dev, v_dev: [n_tokens][H_kv][head_dim] bf16.
 * For every page whose first token is written by this call, its gradient block is zeroed
 * (PKV_GRADS pools). For every page whose last token is written by this call, its representative
 * key is computed as the float32 sequential sum over the page's tokens times 1/page_size
 * (es 2.B: a mean representative vector per key page).
 */
int paged_kv_append(pkv_pool* pool, const int32_t* bt_dev, int32_t n_bt, int32_t pos0, int32_t n_tokens,
                    const uint16_t* k_dev, const uint16_t* v_dev, void* stream);

/* Zero the gradient blocks of logical pages [0, n_pages) through bt_dev, or of the whole pool when
 * bt_dev is NULL: the gradient pages accumulate in place across backward calls (pt 2.B, it 2.B), so
 * a new accumulation starts from cleared pages. Uses a fill kernel (no memset node), so it may be
 * captured in a graph. Errors: PKV_E_STATE (no gradient pages), PKV_E_INVALID (n_pages < 0). */
int paged_kv_zero_grad(pkv_pool* pool, const int32_t* bt_dev, int32_t n_pages, void* stream);

/*
 * Copy logical pages [first_page, first_page + n_pages) of one array into dst_dev in logical
 * order: PKV_K/PKV_V -> [n_pages*page_size][H_kv][head_dim] bf16; PKV_DK/PKV_DV -> same shape fp32;
 * PKV_REP -> [n_pages][H_kv][head_dim] fp32. For tests and checkpoint-style read-back.
 */
int paged_kv_export(const pkv_pool* pool, int32_t what, const int32_t* bt_dev, int32_t n_bt,
                    int32_t first_page, int32_t n_pages, void* dst_dev, void* stream);

/* Synchronise the device, return PKV_E_DEVICE if a kernel recorded an out-of-range table entry
 * since the last check (and clear the record), else PKV_OK. */
int paged_kv_check(pkv_pool* pool);

/*
 * Page-level top-K selection for one query chunk (pt 2.C, es 2.B "page-level sparse attention",
 * it 2.D). For each KV head g:
 *   qsum_g = float32 sum of the chunk's queries over tokens and the group's G heads, in the
 *            order: 64-token blocks summed sequentially, blocks summed sequentially, heads summed
 *            sequentially;
 *   score(p) = sequential float32 dot(qsum_g, rep[bt[p]][g]) with no fused multiply-add, for
 *            candidate logical pages p in [0, n_cand), n_cand = max(n_prior - n_local, 0);
 *   the min(top_k, n_cand) best candidates by (score descending, page id ascending; NaN lowest),
 *   sorted ascending, followed by the n_local most recent prior pages [n_cand, n_prior).
 * n_lists = 1 gives one selection per KV head for the whole chunk. n_lists = C / page_size gives
 * one per (KV head, query page) (pt 2.C: the most relevant key pages for each page of queries):
 * the chunk's tokens [i*page_size, (i+1)*page_size) form query page i, whose summary qsum_{g,i}
 * follows the order above over its own tokens only, and which ranks the candidates on its own.
 * Output sel_dev: [H_kv][n_lists][n_sel] int32 logical page ids, n_sel = min(top_k, n_cand) +
 * (n_prior - n_cand), also stored to *n_sel_out (host; known without synchronising).
 * q_dev: [C][H_q][head_dim] bf16, 16-byte aligned, C % 64 == 0. ws_dev: at least
 * page_topk_ws_bytes(...) bytes (same n_lists).
 * Errors: PKV_E_INVALID (shapes, n_lists other than 1 or C / page_size), PKV_E_UNSUPPORTED
 * (H_q / H_kv > 128), PKV_E_RANGE (n_prior > n_bt), PKV_E_NOMEM (workspace too small); nothing
 * is enqueued on error.
 */
size_t page_topk_ws_bytes(const pkv_pool* pool, int32_t n_prior, int32_t C, int32_t H_q, int32_t n_lists);
int page_topk_select(const pkv_pool* pool, const int32_t* bt_dev, int32_t n_bt, int32_t n_prior,
                     const uint16_t* q_dev, int32_t C, int32_t H_q, int32_t top_k, int32_t n_local,
                     int32_t n_lists, int32_t* sel_dev, int32_t* n_sel_out, void* ws_dev, size_t ws_bytes,
                     void* stream);

/*
 * page_topk_select for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same selection, the same arguments
 * except that there is no workspace argument, and bitwise the same output. Its scratch is a static
 * 16 MiB array compiled into the library, one copy per GPU, held until the process ends; the call
 * itself allocates nothing. A call whose page_topk_ws_bytes(...) exceeds 16 MiB (2^24 bytes) fails
 * with PKV_E_NOMEM and enqueues nothing. Every call on one GPU uses that GPU's single scratch array,
 * so calls that may overlap on one GPU (on different streams, or from several host threads) race
 * and must be ordered by the caller; calls on one stream are ordered by the stream. Other errors
 * are those of page_topk_select, plus PKV_E_HIP if the scratch's device address cannot be looked up
 * (done once per GPU, on the first call there).
 */
int page_topk_select_noalloc(const pkv_pool* pool, const int32_t* bt_dev, int32_t n_bt, int32_t n_prior,
                             const uint16_t* q_dev, int32_t C, int32_t H_q, int32_t top_k, int32_t n_local,
                             int32_t n_lists, int32_t* sel_dev, int32_t* n_sel_out, void* stream);

/*
 * Forward attention of one query chunk over the paged cache (pt 2.A, 2.B; es 2.B custom kernels).
 * Query head h (KV head g = h / G) at chunk row t (position q0 + t) attends to
 *   dense (sel_dev == NULL): every key at position <= q0 + t, i.e. logical pages [0, n_prior)
 *                            plus the chunk's own block;
 *   sparse: the pages sel_dev[(g*n_lists + l)*n_sel + i], i < n_sel (ascending logical ids <
 *           n_prior), plus the own block, causally, where l = 0 when n_lists == 1 and l = t /
 *           page_size (the row's query page, pt 2.C) when n_lists == C / page_size. A selection
 *           of no page (n_sel == 0: the own block only) still passes a non-NULL sel_dev, which
 *           is then not read. Dense calls take n_lists = 1.
 * with softmax(scale * q.k), scale > 0 and finite. The own block (logical pages [n_prior, n_prior + C/page_size)) must
 * already be appended. Only KV heads [kvh0, kvh0 + n_kvh) and their query heads are computed.
 * Outputs: o_dev [C][H_q][head_dim] bf16 and lse_dev [H_q][C] fp32 for those heads.
 * ws_dev: at least chunk_attn_fwd_ws_bytes(...) bytes of device scratch (may be NULL if 0). The
 * *_ws_bytes queries take n_sel < 0 for dense calls, and the call's n_lists.
 * Errors: PKV_E_INVALID (shapes, alignment, n_sel or n_lists out of range, scale not a positive
 * finite number), PKV_E_RANGE (block table too short), PKV_E_STATE (host-tier pool), PKV_E_NOMEM
 * (workspace too small).
 */
size_t chunk_attn_fwd_ws_bytes(const pkv_pool* pool, int32_t n_prior, int32_t n_sel, int32_t n_lists,
                               int32_t n_kvh, int32_t C, int32_t H_q);
int chunk_attn_fwd(const pkv_pool* pool, const int32_t* bt_dev, int32_t n_bt, int32_t n_prior,
                   const int32_t* sel_dev, int32_t n_sel, int32_t n_lists, int32_t kvh0, int32_t n_kvh,
                   const uint16_t* q_dev, int32_t C, int32_t H_q, float scale,
                   uint16_t* o_dev, float* lse_dev, void* ws_dev, size_t ws_bytes, void* stream);

/*
 * Backward attention of one query chunk (pt 2.A recomputation; pt 2.B, it 2.B in-place gradient
 * accumulation into gradient pages). Probabilities are recomputed from q, the pages and lse.
 * dq_dev [C][H_q][head_dim] bf16 is written. dK and dV of every attended key are ADDED (fp32) into
 * the gradient pages of gpool through gbt_dev (gpool may equal pool and gbt_dev may equal bt_dev;
 * gpool must have PKV_GRADS). sel_dev/n_sel/n_lists must equal the forward's. o_dev, dout_dev:
 * [C][H_q][head_dim] bf16; lse_dev as written by chunk_attn_fwd.
 * Calls that add into the same gradient pages commute (fp32 atomic adds).
 */
size_t chunk_attn_bwd_ws_bytes(const pkv_pool* pool, int32_t n_prior, int32_t n_sel, int32_t n_lists,
                               int32_t n_kvh, int32_t C, int32_t H_q);
int chunk_attn_bwd(const pkv_pool* pool, const int32_t* bt_dev, int32_t n_bt,
                   pkv_pool* gpool, const int32_t* gbt_dev, int32_t n_gbt, int32_t n_prior,
                   const int32_t* sel_dev, int32_t n_sel, int32_t n_lists, int32_t kvh0, int32_t n_kvh,
                   const uint16_t* q_dev, const uint16_t* o_dev, const uint16_t* dout_dev,
                   const float* lse_dev, int32_t C, int32_t H_q, float scale, uint16_t* dq_dev,
                   void* ws_dev, size_t ws_bytes, void* stream);

/*
 * Host-tier gather (pt 2.D, es 2.B, it 2.C: KV moves between host and GPU memory on dedicated
 * streams from pinned memory). For KV head kvh and i < n_sel, copies the (page, kvh) block of
 * logical page sel_dev[i] (host pool, physical page host_bt_dev[sel_dev[i]]) into the same head's
 * block of device pool page dst_pages_dev[i], and, when dev_bt_out_dev is not NULL, records the
 * mapping dev_bt_out_dev[sel_dev[i]] = dst_pages_dev[i] (a block table for the device pool; its
 * other entries are left as they are; entries >= n_dev_bt are skipped and flagged). Indices stay on
 * the device; nothing synchronises; order it against the compute stream with events.
 * host must be a PKV_HOST_TIER pool and dev a device pool of the same page size, heads and dim.
 * n_workgroups (0..64; 0 picks 8) sets how many workgroups copy, each keeping one CU to itself while
 * the copy runs (it reserves LDS that an attention workgroup would need there). Each moves about
 * 11 GB/s over the host link and 8 reach the link's own limit (about 55 GB/s measured on MI355X); a
 * gather that runs beside attention kernels slows them less on 2, one that they wait for is done
 * soonest on 8.
 * Other values fail with PKV_E_INVALID.
 */
int paged_kv_gather(const pkv_pool* host, pkv_pool* dev, const int32_t* host_bt_dev, int32_t n_host_bt,
                    const int32_t* sel_dev, int32_t n_sel, int32_t kvh, const int32_t* dst_pages_dev,
                    int32_t* dev_bt_out_dev, int32_t n_dev_bt, int32_t n_workgroups, void* stream);

/*
 * Diagnostic: the sustained bf16 MFMA rate of this GPU, the practical ceiling of the attention
 * kernels (its clock under MFMA load is below the one the datasheet peak assumes). Enqueues
 * n_workgroups workgroups of 512 threads (two waves per SIMD), each wave running iters steps of
 * four independent v_mfma_f32_32x32x16_bf16 on register operands filled with pseudo-random bf16
 * bits; no memory is touched in the loop. out_dev (float, n_workgroups * 512 entries, device)
 * receives one sum per thread so the work is not optimised away; its values carry no meaning.
 * *flop (host, may be NULL) receives the FLOP count of the launch; the caller times it.
 * Errors: PKV_E_INVALID for non-positive sizes or a NULL out_dev.
 */
int pkv_mfma_probe(int32_t n_workgroups, int32_t iters, float* out_dev, double* flop, void* stream);

/*
 * Diagnostic: the device's fp32 atomic-add rate in the pattern of a gradient flush into pages
 * (pt 2.B, it 2.B: key/value gradients are added in place with atomic adds). Enqueues n_workgroups
 * workgroups of 256 threads; workgroup w adds 1.0 to each of the region_elems floats of region
 * w % n_regions of buf_dev (n_regions * region_elems floats, device), consecutive threads on
 * consecutive floats. With n_regions == n_workgroups every float gets one add; with fewer regions,
 * n_workgroups / n_regions workgroups add into the same floats concurrently. After the launch each
 * float of region r has grown by the number of workgroups w < n_workgroups with w % n_regions == r.
 * *bytes (host, may be NULL) receives the bytes added (n_workgroups * region_elems * 4); the caller
 * times the launch. Errors: PKV_E_INVALID for non-positive sizes, n_regions > n_workgroups, a
 * buffer over 2^31 floats or a NULL buf_dev.
 */
int pkv_atomic_probe(int32_t n_workgroups, int32_t n_regions, int32_t region_elems, float* buf_dev, double* bytes,
                     void* stream);

/*
 * Per-kernel timing (tracing aid, off by default). While enabled, every kernel launch of the
 * library is bracketed by two HIP events recorded on the launch's own stream.
 * pkv_timing_enable(1) clears earlier records and starts recording; pkv_timing_enable(0) stops.
 * pkv_timing_collect() waits for the recorded events and aggregates them per kernel name; it
 * returns the number of names (or a negative status). pkv_timing_get(i, ...) returns name i,
 * its launch count and the summed duration in milliseconds. Records are process-wide and not
 * thread-safe against concurrent launches from several host threads.
 */
int pkv_timing_enable(int on);
int pkv_timing_collect(void);
int pkv_timing_get(int i, const char** name, int32_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
