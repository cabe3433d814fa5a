// Page-level top-K selection: query-chunk summary, dot-product page scores against the mean-key
// representatives, and an exact top-K by (score descending, logical page id ascending).
//
// "Out of the Memory Barrier" summaries: es 2.B (a mean representative vector per key page, the
// most relevant pages for the current queries), pt 2.C (top-K page retrieval approximating dense
// attention), it 2.D (recent pages kept for natively sparse models).
//
// Every float operation here is a single IEEE-rounded add or multiply in a fixed order (this file
// is compiled with contraction off as well), so the selected ids are reproducible bit for bit:
//   part[h][b][j] = sum_{t<64} Q[64b+t][h][j];  hsum[h][j] = sum_b part[h][b][j];
//   qsum[g][j] = sum_{hh<G} hsum[gG+hh][j];      score[g][p] = sum_j qsum[g][j] * rep[p][g][j].
// With one selection per query page (pt 2.C: the most relevant key pages for each page of
// queries) the chunk's 64-token blocks are cut into n_lists groups of consecutive blocks; group i
// is summarised, scored and selected on its own exactly as above (b running over its blocks).
#include <mutex>

#include "pkv_device.h"

#pragma clang fp contract(off)

namespace pkv {

// part[h][b][j]: one thread per (h, b, j), 64 sequential adds; lanes run along j (coalesced).
__global__ __launch_bounds__(256) void k_qsum_part(const uint16_t* __restrict__ q, int32_t H_q, int32_t D,
                                                   int32_t nb, float* __restrict__ part) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)H_q * nb * D) return;
  const int32_t j = (int32_t)(idx % D);
  const int32_t b = (int32_t)((idx / D) % nb);
  const int32_t h = (int32_t)(idx / ((int64_t)D * nb));
  const uint16_t* src = q + ((int64_t)(64 * b) * H_q + h) * D + j;
  // All 64 loads are issued before the first add, so each thread waits on memory once (the kernel
  // is latency-bound at this size).
  uint16_t x[64];
#pragma unroll
  for (int32_t t = 0; t < 64; ++t) x[t] = src[(int64_t)t * H_q * D];
  float acc = 0.0f;
#pragma unroll
  for (int32_t t = 0; t < 64; ++t) acc = __fadd_rn(acc, bf16_to_f32(x[t]));
  part[idx] = acc;
}

// hsum[h][i][j] = sum over the blocks b of list i, in order, of part[h][b][j]: one workgroup per
// (query head h, list i), one thread per column, with every part value of a group of 64 blocks
// fetched before its in-order adds. (The sum over the group's heads is formed by the scoring
// kernel.)
__global__ __launch_bounds__(256) void k_hsum(const float* __restrict__ part, int32_t D, int32_t nb,
                                              int32_t n_lists, float* __restrict__ hsum) {
  const int32_t h = blockIdx.x / n_lists, li = blockIdx.x % n_lists;
  const int32_t nbl = nb / n_lists;
  for (int32_t j = threadIdx.x; j < D; j += 256) {
    const float* ph = part + ((int64_t)h * nb + (int64_t)li * nbl) * D + j;
    float hs = 0.0f;
    int32_t b = 0;
    for (; b + 64 <= nbl; b += 64) {
      float v[64];
#pragma unroll
      for (int u = 0; u < 64; ++u) v[u] = ph[(int64_t)(b + u) * D];
#pragma unroll
      for (int u = 0; u < 64; ++u) hs = __fadd_rn(hs, v[u]);
    }
    for (; b < nbl; ++b) hs = __fadd_rn(hs, ph[(int64_t)b * D]);
    hsum[(int64_t)blockIdx.x * D + j] = hs;
  }
}

// score[g][i][p] for candidate logical pages p < n_cand (blockIdx.y = g * n_lists + i), one page
// per thread: the block-table read, then the page's representative row with every load in flight,
// while the workgroup forms qsum[g][i][j] = sum_{hh<G} hsum[gG+hh][i][j] in order into LDS; then
// the in-order dot product. An unreadable page scores NaN (ranks last). One list per KV head
// scores with one-wave workgroups (its few thousand pages spread over as many CUs as possible);
// one list per query page with four-wave ones (four times fewer qsum formations).
template <int D, int NT>
__global__ __launch_bounds__(NT) void k_scores(const float* __restrict__ hsum, const float* __restrict__ rep,
                                               int32_t n_pool, int32_t H_kv, int32_t G, int32_t n_lists,
                                               const int32_t* __restrict__ bt, int32_t n_bt, int32_t n_cand,
                                               float* __restrict__ scores, int32_t* err) {
  __shared__ float qs[D];
  const int32_t gl = blockIdx.y, g = gl / n_lists, li = gl % n_lists;
  const int tid = threadIdx.x;
  const int32_t p = blockIdx.x * NT + tid;
  const int32_t phys = (p < n_cand) ? phys_page(bt, n_bt, n_pool, p, err) : -1;
  f32x4 rv[D / 4];
  if (phys >= 0) {
    const f32x4* r = reinterpret_cast<const f32x4*>(rep + ((int64_t)phys * H_kv + g) * D);
#pragma unroll
    for (int j4 = 0; j4 < D / 4; ++j4) rv[j4] = r[j4];
  }
  for (int32_t j = tid; j < D; j += NT) {
    const float* hp = hsum + ((int64_t)g * G * n_lists + li) * D + j;
    float qv = 0.0f;
    for (int32_t hh = 0; hh < G; hh += 16) {  // 16 heads' values fetched ahead of their adds
      float hv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) hv[u] = (hh + u < G) ? hp[(int64_t)(hh + u) * n_lists * D] : 0.0f;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (hh + u < G) qv = __fadd_rn(qv, hv[u]);
    }
    qs[j] = qv;
  }
  __syncthreads();
  if (p >= n_cand) return;
  float acc = __uint_as_float(0x7fc00000u);
  if (phys >= 0) {
    acc = 0.0f;
#pragma unroll
    for (int32_t j4 = 0; j4 < D / 4; ++j4) {
      acc = __fadd_rn(acc, __fmul_rn(qs[4 * j4 + 0], rv[j4][0]));
      acc = __fadd_rn(acc, __fmul_rn(qs[4 * j4 + 1], rv[j4][1]));
      acc = __fadd_rn(acc, __fmul_rn(qs[4 * j4 + 2], rv[j4][2]));
      acc = __fadd_rn(acc, __fmul_rn(qs[4 * j4 + 3], rv[j4][3]));
    }
  }
  scores[(int64_t)gl * n_cand + p] = acc;
}

// Order key: larger is better. High word: score mapped to an order-preserving unsigned integer
// (+0 and -0 equal, NaN below everything); low word: ~page id, so equal scores prefer lower ids.
__device__ __forceinline__ uint64_t order_key(float s, int32_t id) {
  uint32_t hi;
  if (s != s) {
    hi = 0u;
  } else {
    uint32_t u = (s == 0.0f) ? 0u : __float_as_uint(s);
    hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((uint64_t)hi << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

constexpr int kSelThreads = 1024;

// One workgroup per (KV head, list): radix select (8 passes of 8 bits, most significant first)
// finds the K-th largest order key exactly; the winners are then compacted in ascending id order
// with a block-wide ballot scan, and the local pages are appended.
__global__ __launch_bounds__(kSelThreads) void k_topk(const float* __restrict__ scores, int32_t n_cand,
                                                      int32_t K, int32_t n_prior, int32_t n_sel,
                                                      int32_t* __restrict__ sel) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t s_prefix, s_mask;
  __shared__ uint32_t s_remaining, s_done;
  __shared__ uint32_t wave_tot[kSelThreads / 64];
  const int32_t gl = blockIdx.x;  // g * n_lists + list
  const int32_t tid = threadIdx.x;
  const float* sc = scores + (int64_t)gl * n_cand;
  int32_t* out = sel + (int64_t)gl * n_sel;

  uint64_t threshold = 0;  // select keys >= threshold
  const bool take_all = (K >= n_cand);
  if (!take_all && K > 0) {
    if (tid == 0) {
      s_prefix = 0;
      s_mask = 0;
      s_remaining = (uint32_t)K;
      s_done = 0u;
    }
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0u;
      __syncthreads();
      const uint64_t prefix = s_prefix, mask = s_mask;
      for (int32_t i = tid; i < n_cand; i += kSelThreads) {
        const uint64_t key = order_key(sc[i], i);
        if ((key & mask) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // Wave 0 finds the digit where the running count from the top reaches `remaining`:
        // lane l owns digits 4l..4l+3; suffix sums over lanes, then a walk down the lane's own 4.
        const uint32_t rem = s_remaining;
        uint32_t c[4], own = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c[i] = hist[4 * tid + i];
          own += c[i];
        }
        uint32_t suf = own;  // sum over lanes >= tid
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t v = __shfl_down(suf, off, 64);
          if (tid + off < 64) suf += v;
        }
        uint32_t cum = suf - own;  // digits above this lane's
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          if (cum < rem && cum + c[i] >= rem) {
            s_prefix = prefix | ((uint64_t)(4 * tid + i) << shift);
            s_remaining = rem - cum;
            // Every key of this digit is taken: keys >= prefix (lower digits zero) are the set.
            if (cum + c[i] == rem) s_done = 1u;
          }
          cum += c[i];
        }
        if (tid == 0) s_mask = mask | ((uint64_t)255 << shift);
      }
      __syncthreads();
      if (s_done) break;
    }
    threshold = s_prefix;
  }
  const int32_t kk = take_all ? n_cand : K;
  // Compaction in id order.
  const int lane = tid & 63, wave = tid >> 6;
  int32_t base = 0;
  if (kk > 0) {
    for (int32_t c0 = 0; c0 < n_cand; c0 += kSelThreads) {
      const int32_t i = c0 + tid;
      const bool f = (i < n_cand) && (take_all || order_key(sc[i], i) >= threshold);
      const uint64_t ball = __ballot(f);
      const uint32_t before = __popcll(ball & ((1ull << lane) - 1ull));
      if (lane == 0) wave_tot[wave] = __popcll(ball);
      __syncthreads();
      uint32_t wbase = 0, total = 0;
      for (int w = 0; w < kSelThreads / 64; ++w) {
        const uint32_t t = wave_tot[w];
        wbase += (w < wave) ? t : 0u;
        total += t;
      }
      if (f) {
        const int32_t pos = base + (int32_t)(wbase + before);
        if (pos < kk) out[pos] = i;
      }
      base += (int32_t)total;
      __syncthreads();
    }
  }
  for (int32_t u = tid; u < n_prior - n_cand; u += kSelThreads) out[kk + u] = n_cand + u;
}

// Scratch of page_topk_select_noalloc, for callers that cannot allocate: it lives with the code
// object, so each GPU the library runs on holds its own copy until the process ends. Host code
// never passes the array's name to a kernel (on the host it is only a stand-in for the symbol):
// topk_scratch_ptr looks up the device address of the current GPU's copy once and keeps it.
static __device__ __align__(256) unsigned char scratch[kTopkScratchBytes];

constexpr int kMaxScratchDevices = 64;

hipError_t topk_scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* ptrs[kMaxScratchDevices] = {};
  std::lock_guard<std::mutex> lk(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

size_t topk_ws_bytes(int32_t n_cand, int32_t C, int32_t h_q, int32_t h_kv, int32_t d, int32_t n_lists) {
  const size_t nb = (size_t)C / 64, nl = (size_t)(n_lists > 0 ? n_lists : 1);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al((size_t)h_q * nb * d * 4) + al((size_t)h_q * nl * d * 4) +
         al((size_t)h_kv * nl * (size_t)(n_cand > 0 ? n_cand : 1) * 4);
}

hipError_t launch_topk(const pkv_pool& pool, const int32_t* bt, int32_t n_bt, int32_t n_prior, const uint16_t* q,
                       int32_t C, int32_t h_q, int32_t top_k, int32_t n_local, int32_t n_lists, int32_t* sel,
                       void* ws, hipStream_t s) {
  const int32_t H = pool.h_kv, D = pool.d, G = h_q / H, HL = H * n_lists;
  const int32_t nb = C / 64;
  const int32_t n_cand = n_prior > n_local ? n_prior - n_local : 0;
  const int32_t K = top_k < n_cand ? top_k : n_cand;
  const int32_t n_sel = K + (n_prior - n_cand);
  if (n_sel == 0) return hipSuccess;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* w = (char*)ws;
  float* part = (float*)w;
  float* hsum = (float*)(w + al((size_t)h_q * nb * D * 4));
  float* scores = (float*)(w + al((size_t)h_q * nb * D * 4) + al((size_t)h_q * n_lists * D * 4));
  if (n_cand > 0 && K > 0 && K < n_cand) {
    const int64_t n1 = (int64_t)h_q * nb * D;
    {
      TimerScope ts_("k_qsum_part", s);
      hipLaunchKernelGGL(k_qsum_part, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s, q, h_q, D, nb, part);
    }
    {
      TimerScope ts_("k_hsum", s);
      hipLaunchKernelGGL(k_hsum, dim3((unsigned)(h_q * n_lists)), dim3(256), 0, s, part, D, nb, n_lists, hsum);
    }
    {
      TimerScope ts_("k_scores", s);
      auto launch = [&](auto kern, int nt) {
        hipLaunchKernelGGL(kern, dim3((unsigned)((n_cand + nt - 1) / nt), (unsigned)HL), dim3(nt), 0, s, hsum,
                           pool.rep, pool.n_pages, H, G, n_lists, bt, n_bt, n_cand, scores, pool.err);
      };
      if (D == 128)
        n_lists == 1 ? launch(k_scores<128, 64>, 64) : launch(k_scores<128, 256>, 256);
      else
        n_lists == 1 ? launch(k_scores<64, 64>, 64) : launch(k_scores<64, 256>, 256);
    }
  }
  {
    TimerScope ts_("k_topk", s);
    hipLaunchKernelGGL(k_topk, dim3(HL), dim3(kSelThreads), 0, s, scores, n_cand, K, n_prior, n_sel, sel);
  }
  return hipGetLastError();
}

}  // namespace pkv
