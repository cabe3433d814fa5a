// Paged KV pool kernels: append (scatter through the block table), representative keys, gradient
// zeroing, logical-order export and the host-tier gather.
//
// Paged KV cache and gradient pages: "Out of the Memory Barrier" summaries, pt 2.B / es 2.B / it 2.B
// (pages are never moved when tokens are appended). Mean representative key per page: es 2.B.
// Host tier gathered over the host link from pinned memory: pt 2.D / es 2.B / it 2.C.
#include "pkv_device.h"

#pragma clang fp contract(off)

namespace pkv {

// One thread per 16-byte chunk (8 bf16) of K or V; idx is the chunk index.
__device__ __forceinline__ void append_chunk(uint16_t* __restrict__ kv, int32_t n_pool, int32_t P, int32_t H,
                                             int32_t D, const int32_t* __restrict__ bt, int32_t n_bt, int32_t pos0,
                                             int32_t n, const uint16_t* __restrict__ k,
                                             const uint16_t* __restrict__ v, int32_t* err, int64_t idx) {
  const int64_t per = (int64_t)n * H * (D / 8);
  if (idx >= 2 * per) return;
  const int which = idx >= per;
  const int64_t c = which ? idx - per : idx;
  const int32_t dc = (int32_t)(c % (D / 8));
  const int64_t tg = c / (D / 8);
  const int32_t g = (int32_t)(tg % H);
  const int32_t t = (int32_t)(tg / H);
  const int32_t pos = pos0 + t;
  const int32_t phys = phys_page(bt, n_bt, n_pool, pos / P, err);
  if (phys < 0) return;
  const uint16_t* src = (which ? v : k) + (tg * D + dc * 8);
  uint16_t* dst = kv + ((((int64_t)phys * H + g) * 2 + which) * P + (pos % P)) * D + dc * 8;
  *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
}

__global__ __launch_bounds__(256) void k_append(uint16_t* __restrict__ kv, int32_t n_pool, int32_t P, int32_t H,
                                                int32_t D, const int32_t* __restrict__ bt, int32_t n_bt,
                                                int32_t pos0, int32_t n, const uint16_t* __restrict__ k,
                                                const uint16_t* __restrict__ v, int32_t* err) {
  append_chunk(kv, n_pool, P, H, D, bt, n_bt, pos0, n, k, v, err, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// Representative key of each page completed by an append: float32 sequential sum over the page's
// tokens in token order starting from +0.0, times 1/P (exact: P is a power of two).
// One wave per (logical page, KV head) block, four blocks per workgroup (blk = 4 * wg + wave).
// Lane l owns key columns 2l and 2l+1: it loads its 4-byte column pair from every token row (a
// wave's load covers one whole 256-byte row), all P loads issued before the first add, then runs
// the two columns' sums side by side. No LDS and no barrier. Rows come from the pool, or, when
// ksrc is given, rows at positions >= pos0 come from the appended keys ksrc ([n][H][D], first row
// at pos0) instead, so the sums need nothing written by the same launch.
template <int P>
__device__ __forceinline__ void page_rep_block(const uint16_t* __restrict__ kv, float* __restrict__ rep,
                                               int32_t n_pool, int32_t H, int32_t D,
                                               const int32_t* __restrict__ bt, int32_t n_bt, int32_t lp0,
                                               int32_t n_lp, int32_t* err, const uint16_t* __restrict__ ksrc,
                                               int32_t pos0, int64_t blk, int32_t lane) {
  if (blk >= (int64_t)n_lp * H || 2 * lane >= D) return;
  const int32_t g = (int32_t)(blk % H);
  const int32_t lp = lp0 + (int32_t)(blk / H);
  const int32_t phys = phys_page(bt, n_bt, n_pool, lp, err);
  if (phys < 0) return;
  const uint32_t* kp = reinterpret_cast<const uint32_t*>(kv + (((int64_t)phys * H + g) * 2) * P * D) + lane;
  const int32_t row = D / 2;  // 4-byte words per token row
  uint32_t x[P];
  if (ksrc == nullptr) {
#pragma unroll
    for (int32_t t = 0; t < P; ++t) x[t] = kp[t * row];
  } else {
    // Row t of the page sits at position lp * P + t; rows from pos0 on are the appended keys.
    const int32_t t_src = pos0 - lp * P;  // first row taken from ksrc (may be <= 0)
    const uint32_t* ks = reinterpret_cast<const uint32_t*>(ksrc) + (int64_t)g * row + lane;
#pragma unroll
    for (int32_t t = 0; t < P; ++t) x[t] = t >= t_src ? ks[(int64_t)(t - t_src) * H * row] : kp[t * row];
  }
  float a0 = 0.0f, a1 = 0.0f;  // columns 2*lane (low half-word) and 2*lane + 1 (high half-word)
#pragma unroll
  for (int32_t t = 0; t < P; ++t) {
    a0 = __fadd_rn(a0, __uint_as_float(x[t] << 16));
    a1 = __fadd_rn(a1, __uint_as_float(x[t] & 0xFFFF0000u));
  }
  float* r = rep + ((int64_t)phys * H + g) * D + 2 * lane;
  r[0] = __fmul_rn(a0, 1.0f / (float)P);
  r[1] = __fmul_rn(a1, 1.0f / (float)P);
}

template <int P>
__global__ __launch_bounds__(256) void k_page_reps(const uint16_t* __restrict__ kv, float* __restrict__ rep,
                                                   int32_t n_pool, int32_t H, int32_t D,
                                                   const int32_t* __restrict__ bt, int32_t n_bt, int32_t lp0,
                                                   int32_t n_lp, int32_t* err) {
  page_rep_block<P>(kv, rep, n_pool, H, D, bt, n_bt, lp0, n_lp, err, nullptr, 0,
                    (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6), threadIdx.x & 63);
}

constexpr int kZeroPerThread = 8;
// Piece `piece` (8 x 256 16-byte chunks) of the gradient block of logical page lp.
__device__ __forceinline__ void zero_grad_piece(float* __restrict__ grad, int32_t n_pool, int32_t P, int32_t H,
                                                int32_t D, const int32_t* __restrict__ bt, int32_t n_bt,
                                                int32_t lp, int32_t piece, int32_t* err) {
  const int64_t per_page = (int64_t)H * 2 * P * D / 4;  // 16-byte chunks per page
  const int64_t i0 = (int64_t)piece * kZeroPerThread * 256 + threadIdx.x;
  const int32_t phys = bt ? phys_page(bt, n_bt, n_pool, lp, err) : lp;
  if (phys < 0 || phys >= n_pool) return;
  f32x4* base = reinterpret_cast<f32x4*>(grad) + (int64_t)phys * per_page;
#pragma unroll
  for (int u = 0; u < kZeroPerThread; ++u) {
    const int64_t i = i0 + (int64_t)u * 256;
    if (i < per_page) base[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
}

// Zero the gradient blocks of logical pages [lp0, lp0 + n_lp) (bt == NULL: physical = logical).
// Grid (x: 32 KiB pieces of a page, y: pages, striding when there are more than gridDim.y): one
// table lookup per workgroup, 8 16-byte stores per thread.
__global__ __launch_bounds__(256) void k_zero_grad(float* __restrict__ grad, int32_t n_pool, int32_t P, int32_t H,
                                                   int32_t D, const int32_t* __restrict__ bt, int32_t n_bt,
                                                   int32_t lp0, int32_t n_lp, int32_t* err) {
  for (int32_t r = blockIdx.y; r < n_lp; r += gridDim.y)
    zero_grad_piece(grad, n_pool, P, H, D, bt, n_bt, lp0 + r, blockIdx.x, err);
}

// A chunk-sized append in one launch: workgroups [0, nr) build the representatives of the pages
// it completes, reading the appended rows from k itself (dispatched first: each is a chain of
// dependent row loads), [nr, nr + nz) zero the gradient blocks of the pages the append starts
// (zp pieces per page), the rest copy K and V into the pages. None of the three reads what
// another writes.
template <int P>
__global__ __launch_bounds__(256) void k_append_fused(uint16_t* __restrict__ kv, float* __restrict__ grad,
                                                      float* __restrict__ rep, int32_t n_pool, int32_t H, int32_t D,
                                                      const int32_t* __restrict__ bt, int32_t n_bt, int32_t pos0,
                                                      int32_t n, const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v, int32_t first_new, int32_t zp,
                                                      int32_t nz, int32_t nr, int32_t lp_a, int32_t n_lp,
                                                      int32_t* err) {
  const int32_t b = blockIdx.x;
  if (b < nr) {
    page_rep_block<P>(kv, rep, n_pool, H, D, bt, n_bt, lp_a, n_lp, err, k, pos0,
                      (int64_t)b * 4 + (threadIdx.x >> 6), threadIdx.x & 63);
  } else if (b < nr + nz) {
    zero_grad_piece(grad, n_pool, P, H, D, bt, n_bt, first_new + (b - nr) / zp, (b - nr) % zp, err);
  } else {
    append_chunk(kv, n_pool, P, H, D, bt, n_bt, pos0, n, k, v, err, (int64_t)(b - nr - nz) * 256 + threadIdx.x);
  }
}

static dim3 zero_grid(const pkv_pool& pool, int32_t n_pages) {
  const int64_t per_page = (int64_t)pool.h_kv * 2 * pool.page * pool.d / 4;
  return dim3((unsigned)((per_page + kZeroPerThread * 256 - 1) / (kZeroPerThread * 256)),
              (unsigned)(n_pages < 65535 ? n_pages : 65535));
}

// Export K/V (bf16) in logical order: dst[(lp*P + t)*H + g][d].
__global__ __launch_bounds__(256) void k_export_kv(const uint16_t* __restrict__ kv, int32_t n_pool, int32_t P,
                                                   int32_t H, int32_t D, int32_t which,
                                                   const int32_t* __restrict__ bt, int32_t n_bt, int32_t lp0,
                                                   int32_t n_lp, uint16_t* __restrict__ dst, int32_t* err) {
  const int64_t total = (int64_t)n_lp * P * H * (D / 8);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int32_t dc = (int32_t)(idx % (D / 8));
  const int64_t row = idx / (D / 8);  // (lp_rel*P + t)*H + g
  const int32_t g = (int32_t)(row % H);
  const int32_t t = (int32_t)((row / H) % P);
  const int32_t lr = (int32_t)(row / ((int64_t)H * P));
  const int32_t phys = phys_page(bt, n_bt, n_pool, lp0 + lr, err);
  u32x4 val = (u32x4){0u, 0u, 0u, 0u};
  if (phys >= 0)
    val = *reinterpret_cast<const u32x4*>(kv + ((((int64_t)phys * H + g) * 2 + which) * P + t) * D + dc * 8);
  *reinterpret_cast<u32x4*>(dst + row * D + dc * 8) = val;
}

// Export dK/dV (fp32) in logical order.
__global__ __launch_bounds__(256) void k_export_grad(const float* __restrict__ grad, int32_t n_pool, int32_t P,
                                                     int32_t H, int32_t D, int32_t which,
                                                     const int32_t* __restrict__ bt, int32_t n_bt, int32_t lp0,
                                                     int32_t n_lp, float* __restrict__ dst, int32_t* err) {
  const int64_t total = (int64_t)n_lp * P * H * (D / 4);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int32_t dc = (int32_t)(idx % (D / 4));
  const int64_t row = idx / (D / 4);
  const int32_t g = (int32_t)(row % H);
  const int32_t t = (int32_t)((row / H) % P);
  const int32_t lr = (int32_t)(row / ((int64_t)H * P));
  const int32_t phys = phys_page(bt, n_bt, n_pool, lp0 + lr, err);
  f32x4 val = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (phys >= 0)
    val = *reinterpret_cast<const f32x4*>(grad + ((((int64_t)phys * H + g) * 2 + which) * P + t) * D + dc * 4);
  *reinterpret_cast<f32x4*>(dst + row * D + dc * 4) = val;
}

// Export representatives [lp][g][d].
__global__ __launch_bounds__(256) void k_export_rep(const float* __restrict__ rep, int32_t n_pool, int32_t H, int32_t D,
                                                    const int32_t* __restrict__ bt, int32_t n_bt, int32_t lp0,
                                                    int32_t n_lp, float* __restrict__ dst, int32_t* err) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n_lp * H * D) return;
  const int32_t lr = (int32_t)(idx / ((int64_t)H * D));
  const int32_t phys = phys_page(bt, n_bt, n_pool, lp0 + lr, err);
  dst[idx] = phys >= 0 ? rep[(int64_t)phys * H * D + idx % ((int64_t)H * D)] : 0.0f;
}

// Host tier -> device: a few workgroups stride over the selected pages, each copying a page's
// (page, kvh) K|V block with 16-byte loads of the device-mapped pinned host memory. The caller picks
// the workgroup count: one workgroup of 256 threads, 8 loads of 16 bytes in flight per thread, moves
// about 11 GB/s over the host link (a CU's outstanding misses, not its threads, set the rate), 4 move
// 44 GB/s and 8 move 54, as fast as 16: the link's own limit.
// Each workgroup also reserves kGatherLds bytes of LDS that it never touches, so that no attention
// workgroup (113 to 132 KB of LDS each) shares its CU. One that did ran its one wave per SIMD beside
// the copy's waves, which hold the CU's memory pipeline, and its whole grid waited for it: a forward
// or dQ pass beside a copy took up to 30% longer. With the reservation the copy takes an idle CU (the
// forward and dQ grids of a one-head call leave some) or waits for one.
constexpr size_t kGatherLds = 64 * 1024;
constexpr int kGatherBlocks = 8;
constexpr int kGatherThreads = 256;
__global__ __launch_bounds__(kGatherThreads) void k_gather(const uint16_t* __restrict__ host_kv, int32_t n_host_pool,
                                                uint16_t* __restrict__ dev_kv, int32_t n_dev_pool, int32_t P,
                                                int32_t H, int32_t D, const int32_t* __restrict__ host_bt,
                                                int32_t n_host_bt, const int32_t* __restrict__ sel, int32_t n_sel,
                                                const int32_t* __restrict__ dst_pages, int32_t kvh,
                                                int32_t* __restrict__ dev_bt_out, int32_t n_dev_bt, int32_t* err) {
  for (int32_t i = blockIdx.x; i < n_sel; i += gridDim.x) {
    const int32_t lp = sel[i];
    const int32_t hp = phys_page(host_bt, n_host_bt, n_host_pool, lp, err);
    const int32_t dp = dst_pages[i];
    if (hp < 0) continue;
    if (dp < 0 || dp >= n_dev_pool) {
      flag_error(err, 4);
      continue;
    }
    if (dev_bt_out != nullptr && threadIdx.x == 0) {
      if (lp < n_dev_bt)
        dev_bt_out[lp] = dp;
      else
        flag_error(err, 3);
    }
    const int64_t n16 = (int64_t)2 * P * D / 8;  // 16-byte chunks in one (page, head) block
    const u32x4* src = reinterpret_cast<const u32x4*>(host_kv + ((int64_t)hp * H + kvh) * 2 * P * D);
    u32x4* dst = reinterpret_cast<u32x4*>(dev_kv + ((int64_t)dp * H + kvh) * 2 * P * D);
    constexpr int kUnroll = 8;
    for (int64_t c0 = threadIdx.x; c0 < n16; c0 += kGatherThreads * kUnroll) {
      u32x4 buf[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = c0 + (int64_t)u * kGatherThreads;
        if (c < n16) buf[u] = __builtin_nontemporal_load(src + c);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = c0 + (int64_t)u * kGatherThreads;
        if (c < n16) dst[c] = buf[u];
      }
    }
  }
}

// Gradient offload: host[host_bt[lp]][g] += dev[dev_bt[lp]][g], then the device block is cleared.
// Workgroups stride over the (page, head) blocks; each fp32 block is 2*P*D floats. The host block
// is read and written over the host link (device-mapped pinned memory), 8 x 16 bytes in flight
// per thread.
constexpr int kOffloadBlocks = 32;
__global__ __launch_bounds__(256) void k_grad_offload(float* __restrict__ host_grad, int32_t n_host_pool,
                                                      float* __restrict__ dev_grad, int32_t n_dev_pool, int32_t P,
                                                      int32_t H, int32_t D, const int32_t* __restrict__ host_bt,
                                                      int32_t n_host_bt, const int32_t* __restrict__ dev_bt,
                                                      int32_t n_dev_bt, const int32_t* __restrict__ lps, int32_t n,
                                                      int32_t kvh0, int32_t n_kvh, int32_t* host_err,
                                                      int32_t* dev_err) {
  const int64_t n_blocks = (int64_t)n * n_kvh;
  const int64_t n16 = (int64_t)2 * P * D / 4;  // 16-byte chunks per (page, head) block
  for (int64_t bi = blockIdx.x; bi < n_blocks; bi += gridDim.x) {
    const int32_t lp = lps[bi / n_kvh];
    const int32_t g = kvh0 + (int32_t)(bi % n_kvh);
    const int32_t hp = phys_page(host_bt, n_host_bt, n_host_pool, lp, host_err);
    const int32_t dp = phys_page(dev_bt, n_dev_bt, n_dev_pool, lp, dev_err);
    if (hp < 0 || dp < 0) continue;
    f32x4* hb = reinterpret_cast<f32x4*>(host_grad + ((int64_t)hp * H + g) * 2 * P * D);
    f32x4* db = reinterpret_cast<f32x4*>(dev_grad + ((int64_t)dp * H + g) * 2 * P * D);
    constexpr int kUnroll = 8;
    for (int64_t c0 = threadIdx.x; c0 < n16; c0 += 256 * kUnroll) {
      f32x4 hv[kUnroll], dv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = c0 + (int64_t)u * 256;
        if (c < n16) {
          hv[u] = __builtin_nontemporal_load(hb + c);
          dv[u] = db[c];
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = c0 + (int64_t)u * 256;
        if (c < n16) {
          hb[c] = hv[u] + dv[u];
          db[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
}

static inline unsigned grid_for(int64_t n) { return (unsigned)((n + 255) / 256); }

// Appends of at most this many tokens (a chunk's own block) run as one fused launch; larger ones
// (pool fills) as three kernels, each with the whole grid to itself.
constexpr int32_t kFusedAppendMaxTokens = 16384;

hipError_t launch_append(const pkv_pool& pool, const int32_t* bt, int32_t n_bt, int32_t pos0, int32_t n,
                         const uint16_t* k, const uint16_t* v, hipStream_t s) {
  const int32_t P = pool.page, H = pool.h_kv, D = pool.d;
  // Pages whose first token is written here get zeroed gradients.
  const int32_t first_new = (pos0 + P - 1) / P;           // first page starting at or after pos0
  const int32_t end_new = (pos0 + n + P - 1) / P;         // pages starting before pos0 + n
  const int32_t n_new = (pool.grad && end_new > first_new) ? end_new - first_new : 0;
  const int64_t chunks = (int64_t)2 * n * H * (D / 8);
  // Pages whose last token is written here get their representative key.
  const int32_t first_full = pos0 / P;                    // candidate: page containing pos0
  const int32_t lp_a = ((first_full + 1) * P - 1 >= pos0) ? first_full : first_full + 1;
  const int32_t lp_b = (pos0 + n) / P;                    // pages fully ending before pos0 + n
  const int32_t n_lp = lp_b > lp_a ? lp_b - lp_a : 0;
  if (n <= kFusedAppendMaxTokens) {
    const int32_t zp = (int32_t)zero_grid(pool, 1).x;     // pieces per page
    const int32_t nz = n_new * zp;
    const int32_t na = (int32_t)grid_for(chunks);
    const int32_t nr = (int32_t)(((int64_t)n_lp * H + 3) / 4);
    TimerScope ts_("k_append_fused", s);
    if (P == 128)
      hipLaunchKernelGGL(k_append_fused<128>, dim3((unsigned)(nz + na + nr)), dim3(256), 0, s, pool.kv, pool.grad,
                         pool.rep, pool.n_pages, H, D, bt, n_bt, pos0, n, k, v, first_new, zp, nz, nr, lp_a, n_lp,
                         pool.err);
    else
      hipLaunchKernelGGL(k_append_fused<64>, dim3((unsigned)(nz + na + nr)), dim3(256), 0, s, pool.kv, pool.grad,
                         pool.rep, pool.n_pages, H, D, bt, n_bt, pos0, n, k, v, first_new, zp, nz, nr, lp_a, n_lp,
                         pool.err);
    return hipGetLastError();
  }
  if (n_new > 0) {
    TimerScope ts_("k_zero_grad", s);
    hipLaunchKernelGGL(k_zero_grad, zero_grid(pool, n_new), dim3(256), 0, s, pool.grad, pool.n_pages, P, H, D, bt,
                       n_bt, first_new, n_new, pool.err);
  }
  {
    TimerScope ts_("k_append", s);
    hipLaunchKernelGGL(k_append, dim3(grid_for(chunks)), dim3(256), 0, s, pool.kv, pool.n_pages, P, H, D, bt, n_bt,
                       pos0, n, k, v, pool.err);
  }
  if (n_lp > 0) {
    TimerScope ts_("k_page_reps", s);
    const dim3 grid((unsigned)(((int64_t)n_lp * H + 3) / 4));
    if (P == 128)
      hipLaunchKernelGGL(k_page_reps<128>, grid, dim3(256), 0, s, pool.kv, pool.rep, pool.n_pages, H, D, bt, n_bt,
                         lp_a, n_lp, pool.err);
    else
      hipLaunchKernelGGL(k_page_reps<64>, grid, dim3(256), 0, s, pool.kv, pool.rep, pool.n_pages, H, D, bt, n_bt,
                         lp_a, n_lp, pool.err);
  }
  return hipGetLastError();
}

hipError_t launch_zero_grad(const pkv_pool& pool, const int32_t* bt, int32_t first_page, int32_t n_pages,
                            hipStream_t s) {
  if (n_pages <= 0) return hipSuccess;
  {
    TimerScope ts_("k_zero_grad", s);
    hipLaunchKernelGGL(k_zero_grad, zero_grid(pool, n_pages), dim3(256), 0, s, pool.grad, pool.n_pages, pool.page,
                       pool.h_kv, pool.d, bt, first_page + n_pages, first_page, n_pages, pool.err);
  }
  return hipGetLastError();
}

hipError_t launch_export(const pkv_pool& pool, int32_t what, const int32_t* bt, int32_t first_page,
                         int32_t n_pages, void* dst, hipStream_t s) {
  const int32_t P = pool.page, H = pool.h_kv, D = pool.d;
  const int32_t n_bt = first_page + n_pages;
  if (what == 0 || what == 1) {
    const int64_t work = (int64_t)n_pages * P * H * (D / 8);
    {
      TimerScope ts_("k_export_kv", s);
      hipLaunchKernelGGL(k_export_kv, dim3(grid_for(work)), dim3(256), 0, s, pool.kv, pool.n_pages, P, H, D, what, bt,
                         n_bt, first_page, n_pages, (uint16_t*)dst, pool.err);
    }
  } else if (what == 2 || what == 3) {
    const int64_t work = (int64_t)n_pages * P * H * (D / 4);
    {
      TimerScope ts_("k_export_grad", s);
      hipLaunchKernelGGL(k_export_grad, dim3(grid_for(work)), dim3(256), 0, s, pool.grad, pool.n_pages, P, H, D,
                         what - 2, bt, n_bt, first_page, n_pages, (float*)dst, pool.err);
    }
  } else {
    const int64_t work = (int64_t)n_pages * H * D;
    {
      TimerScope ts_("k_export_rep", s);
      hipLaunchKernelGGL(k_export_rep, dim3(grid_for(work)), dim3(256), 0, s, pool.rep, pool.n_pages, H, D, bt, n_bt,
                         first_page, n_pages, (float*)dst, pool.err);
    }
  }
  return hipGetLastError();
}

hipError_t launch_gather(const pkv_pool& host, const pkv_pool& dev, const int32_t* host_bt, int32_t n_host_bt,
                         const int32_t* sel, int32_t n_sel, int32_t kvh, const int32_t* dst_pages,
                         int32_t* dev_bt_out, int32_t n_dev_bt, int32_t n_workgroups, hipStream_t s) {
  if (n_sel == 0) return hipSuccess;
  const int32_t n_wg = n_workgroups > 0 ? n_workgroups : kGatherBlocks;
  {
    TimerScope ts_("k_gather", s);
    hipLaunchKernelGGL(k_gather, dim3(n_sel < n_wg ? n_sel : n_wg), dim3(kGatherThreads), kGatherLds, s, host.kv,
                       host.n_pages, dev.kv, dev.n_pages, host.page, host.h_kv, host.d, host_bt, n_host_bt, sel, n_sel,
                       dst_pages, kvh, dev_bt_out, n_dev_bt, dev.err);
  }
  return hipGetLastError();
}

// Clear head g's gradient block (dK and dV, 2*P*D floats) of physical pages [page0, page0 + n):
// grid.y walks the pages, grid.x the block's 16-byte chunks.
__global__ __launch_bounds__(256) void k_zero_head_blocks(float* __restrict__ grad, int32_t P, int32_t H, int32_t D,
                                                          int32_t page0, int32_t n, int32_t g) {
  const int64_t n16 = (int64_t)2 * P * D / 4;
  for (int32_t r = blockIdx.y; r < n; r += gridDim.y) {
    f32x4* b = reinterpret_cast<f32x4*>(grad + (((int64_t)(page0 + r) * H + g) * 2) * P * D);
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n16; c += (int64_t)gridDim.x * 256)
      b[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
}

hipError_t launch_zero_head_blocks(const pkv_pool& pool, int32_t page0, int32_t n, int32_t g, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t n16 = (int64_t)2 * pool.page * pool.d / 4;
  {
    TimerScope ts_("k_zero_head_blocks", s);
    hipLaunchKernelGGL(k_zero_head_blocks, dim3((unsigned)((n16 + 255) / 256), (unsigned)(n < 65535 ? n : 65535)),
                       dim3(256), 0, s, pool.grad, pool.page, pool.h_kv, pool.d, page0, n, g);
  }
  return hipGetLastError();
}

hipError_t launch_grad_offload(const pkv_pool& host, const int32_t* host_bt, int32_t n_host_bt, const pkv_pool& dev,
                               const int32_t* dev_bt, int32_t n_dev_bt, const int32_t* lp, int32_t n, int32_t kvh0,
                               int32_t n_kvh, hipStream_t s) {
  const int64_t n_blocks = (int64_t)n * n_kvh;
  if (n_blocks == 0) return hipSuccess;
  {
    TimerScope ts_("k_grad_offload", s);
    hipLaunchKernelGGL(k_grad_offload, dim3((unsigned)(n_blocks < kOffloadBlocks ? n_blocks : kOffloadBlocks)),
                       dim3(256), 0, s, host.grad, host.n_pages, dev.grad, dev.n_pages, host.page, host.h_kv, host.d,
                       host_bt, n_host_bt, dev_bt, n_dev_bt, lp, n, kvh0, n_kvh, host.err, dev.err);
  }
  return hipGetLastError();
}

}  // namespace pkv
