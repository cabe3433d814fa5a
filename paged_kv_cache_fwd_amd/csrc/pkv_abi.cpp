// C ABI of the paged chunk-attention library: argument validation, pool management and launch
// planning. Every check happens before anything is enqueued; kernels live in the *.hip files.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <tuple>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_internal.h"

// Free list of a pool's physical pages. Pages are all the same size, so a page freed anywhere can
// serve any later request: the pool never fragments and nothing is ever moved.
struct pkv_page_alloc {
  std::mutex mu;
  std::vector<int32_t> free_pages;  // stack: the most recently released page is handed out first
  std::vector<uint8_t> is_free;     // per physical page
};

// One host-side accumulation: staged gradient blocks added into a host pool's gradient pages.
struct pkv_add_job {
  std::atomic<int32_t> busy{0};
  float* grad_host = nullptr;        // host pool's gradient pages (host address)
  int32_t n_pages = 0, h = 0, blk = 0, kvh = 0;  // blk: floats per (page, head) block
  const int32_t* host_bt = nullptr;  // caller's host copy of the host pool's block table
  int32_t n_host_bt = 0;
  const unsigned char* staging = nullptr;
  int32_t n = 0;
  std::atomic<int32_t>* err = nullptr;
};

// Fixed ring of job slots per PKV_HOST_GRADS pool: enqueueing an accumulation allocates nothing.
// Host code may run far ahead of the stream; when every slot is still pending, the enqueueing call
// waits for the oldest to run.
constexpr int kHostJobs = 1024;
constexpr double kHostJobWaitSeconds = 60.0;
struct pkv_host_jobs {
  pkv_add_job slot[kHostJobs];
  std::atomic<uint32_t> next{0};
  std::atomic<int32_t> err{0};  // 5: a staged page id outside the block table or the pool
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PKV_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

void ok() { g_err.clear(); }

bool supported(int32_t page, int32_t d) { return (page == 64 || page == 128) && (d == 64 || d == 128); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t kv_bytes(const pkv_pool& p) { return (size_t)p.n_pages * p.h_kv * 2 * p.page * p.d * sizeof(uint16_t); }
size_t grad_bytes(const pkv_pool& p) { return (size_t)p.n_pages * p.h_kv * 2 * p.page * p.d * sizeof(float); }
size_t rep_bytes(const pkv_pool& p) { return (size_t)p.n_pages * p.h_kv * p.d * sizeof(float); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Shared checks of chunk_attn_fwd / chunk_attn_bwd.
int check_attn(const pkv_pool* pool, const int32_t* bt, int32_t n_bt, int32_t n_prior, const int32_t* sel,
               int32_t n_sel, int32_t n_lists, int32_t kvh0, int32_t n_kvh, const uint16_t* q, int32_t C,
               int32_t H_q, float scale) {
  // A non-positive scale has no softmax reading (scale 0 turns the running maximum into inf * 0,
  // a negative one inverts it), so it is rejected before anything else.
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PKV_E_INVALID, "scale=%g must be a positive finite number", (double)scale);
  if (!pool) return fail(PKV_E_INVALID, "pool is NULL");
  if (pool->flags & PKV_HOST_TIER)
    return fail(PKV_E_STATE, "attention reads device pages; gather host-tier pages into a device pool first");
  if (!bt) return fail(PKV_E_INVALID, "block table is NULL");
  if (!q) return fail(PKV_E_INVALID, "q is NULL");
  if (!aligned16(q)) return fail(PKV_E_INVALID, "q must be 16-byte aligned");
  if (C <= 0 || C % pool->page != 0) return fail(PKV_E_INVALID, "C=%d must be a positive multiple of the page size %d", C, pool->page);
  if (H_q <= 0 || H_q % pool->h_kv != 0) return fail(PKV_E_INVALID, "H_q=%d must be a positive multiple of H_kv=%d", H_q, pool->h_kv);
  if ((int64_t)C * (H_q / pool->h_kv) >= (int64_t)1 << 24)
    return fail(PKV_E_INVALID, "C * H_q / H_kv = %lld rows per KV head must be below 2^24", (long long)C * (H_q / pool->h_kv));
  if (n_prior < 0) return fail(PKV_E_INVALID, "n_prior < 0");
  if (n_bt < 0 || (int64_t)n_prior + C / pool->page > n_bt)
    return fail(PKV_E_RANGE, "pages [0, %d) exceed the block table (%d entries)", n_prior + C / pool->page, n_bt);
  if ((int64_t)(n_prior + C / pool->page) * pool->page > (int64_t)1 << 30) return fail(PKV_E_RANGE, "context too long");
  if (kvh0 < 0 || n_kvh <= 0 || kvh0 + n_kvh > pool->h_kv)
    return fail(PKV_E_INVALID, "KV head range [%d, %d) outside [0, %d)", kvh0, kvh0 + n_kvh, pool->h_kv);
  if (sel) {
    if (n_sel < 0 || n_sel > n_prior) return fail(PKV_E_INVALID, "n_sel=%d must be in [0, n_prior=%d]", n_sel, n_prior);
    if (n_lists != 1 && n_lists != C / pool->page)
      return fail(PKV_E_INVALID, "n_lists=%d must be 1 or C / page_size = %d", n_lists, C / pool->page);
  } else if (n_lists != 1) {
    return fail(PKV_E_INVALID, "dense attention takes n_lists = 1 (got %d)", n_lists);
  }
  return PKV_OK;
}

pkv::AttnArgs make_args(const pkv_pool* pool, const int32_t* bt, int32_t n_bt, int32_t n_prior, const int32_t* sel,
                        int32_t n_sel, int32_t n_lists, int32_t kvh0, int32_t n_kvh, const uint16_t* q, int32_t C,
                        int32_t H_q, float scale) {
  pkv::AttnArgs a;
  a.kv = pool->kv;
  a.n_pool_pages = pool->n_pages;
  a.page = pool->page;
  a.h_kv = pool->h_kv;
  a.d = pool->d;
  a.bt = bt;
  a.n_bt = n_bt;
  a.n_prior = n_prior;
  a.sel = sel;
  a.n_sel = sel ? n_sel : 0;
  a.n_lists = sel ? n_lists : 1;
  a.kvh0 = kvh0;
  a.n_kvh = n_kvh;
  a.q = q;
  a.C = C;
  a.h_q = H_q;
  a.G = H_q / pool->h_kv;
  a.scale = scale;
  a.err = pool->err;
  return a;
}

}  // namespace

namespace pkv {

namespace {
struct TimingRec {
  const char* name;
  hipEvent_t a, b;
};
bool g_timing = false;
std::vector<TimingRec> g_recs;     // recorded launches (events reused across enable cycles)
size_t g_nrec = 0;
std::vector<std::pair<std::string, std::pair<int32_t, double>>> g_summary;
std::mutex g_tmu;
}  // namespace

TimerScope::TimerScope(const char* name, hipStream_t s) : slot_(-1), s_(s) {
  if (!g_timing) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  if (g_nrec == g_recs.size()) {
    TimingRec r{name, nullptr, nullptr};
    if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) return;
    g_recs.push_back(r);
  }
  g_recs[g_nrec].name = name;
  if (hipEventRecord(g_recs[g_nrec].a, s) != hipSuccess) return;
  slot_ = (int)g_nrec++;
}

TimerScope::~TimerScope() {
  if (slot_ < 0) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  (void)hipEventRecord(g_recs[slot_].b, s_);
}

int num_cus() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cached = n;
    else
      cached = 256;
  }
  return cached;
}

// Pick the key-range split count: a workgroup costs (its tiles + fixed overhead), and workgroups
// run one per CU in waves, so minimise waves * per-workgroup cost.
static int32_t best_split(int64_t base_units, double tiles, double overhead, int32_t max_split, int per_cu) {
  const int64_t slots = (int64_t)num_cus() * per_cu;
  int32_t best = 1;
  double best_cost = 1e300;
  for (int32_t s = 1; s <= max_split; ++s) {
    const double waves = std::ceil((double)(base_units * s) / (double)slots);
    const double cost = waves * (std::ceil(tiles / s) + overhead) + (s > 1 ? 1.0 : 0.0);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

// Waves per workgroup of the forward and dQ passes. Eight waves (256 rows) share each staged K/V
// tile between twice the rows of four (128 rows, two workgroups per CU), halving the tile traffic
// into LDS; four are kept when a selection list's rows would leave a 256-row block half empty.
static int32_t pick_nw(int64_t rows, int32_t n_lists) {
  return (n_lists == 1 || (rows / n_lists) % 256 == 0) ? 8 : 4;
}

// Row blocks of 32*nw rows, cut at selection-list boundaries (n_lists groups of C*G/n_lists rows).
static int32_t row_blocks(int64_t rows, int32_t n_lists, int32_t nw) {
  const int64_t per_list = rows / n_lists, rb = 32 * nw;
  return (int32_t)(n_lists * ((per_list + rb - 1) / rb));
}

// Key-range split count of the forward and dQ passes. Their row blocks see different numbers of
// key tiles (the chunk's own keys up to each block's last row), so the count comes from a model of
// the dispatch: units u = (row block, split, KV head) in the kernels' order, row blocks last to
// first, cut into eight contiguous XCD shares, each run in rounds of (CUs per XCD x workgroups
// per CU) whose length is that round's longest workgroup (its tiles + a fixed 3), plus the
// combine or reduce pass for more than one split (4 + 4.3 per split, in tile times). The model
// runs once per shape.
static int32_t key_splits(int32_t n_kvh, int32_t n_lists, int64_t rows, int32_t nw, int32_t G, int32_t prior_tiles,
                          int32_t max_split) {
  struct Key {
    int32_t n_kvh, n_lists, nw, G, prior_tiles, max_split;
    int64_t rows;
    bool operator<(const Key& o) const {
      return std::tie(n_kvh, n_lists, nw, G, prior_tiles, max_split, rows) <
             std::tie(o.n_kvh, o.n_lists, o.nw, o.G, o.prior_tiles, o.max_split, o.rows);
    }
  };
  static std::mutex mu;
  static std::map<Key, int32_t> cache;
  const Key key{n_kvh, n_lists, nw, G, prior_tiles, max_split, rows};
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  const int64_t RL = rows / n_lists, rbw = 32 * (int64_t)nw, bpl = (RL + rbw - 1) / rbw, n_rb = n_lists * bpl;
  const int64_t slots = std::max<int64_t>(1, (int64_t)num_cus() / 8 * (8 / nw));
  std::vector<int32_t> tiles((size_t)n_rb);
  for (int64_t rb = 0; rb < n_rb; ++rb) {
    const int64_t li = rb / bpl, r0 = li * RL + (rb - li * bpl) * rbw;
    const int64_t r_last = std::min(r0 + rbw, (li + 1) * RL) - 1;
    tiles[(size_t)rb] = prior_tiles + (int32_t)((r_last / G) / 64) + 1;
  }
  int32_t best = 1;
  double best_cost = 1e300;
  for (int32_t s = 1; s <= std::min(max_split, 16); ++s) {
    const int64_t n = (int64_t)n_kvh * s * n_rb, q = n / 8, r = n % 8;
    double worst = 0;
    for (int64_t x = 0; x < 8; ++x) {
      const int64_t a = x * q + std::min(x, r), b = a + q + (x < r ? 1 : 0);
      double cost = 0;
      for (int64_t k0 = a; k0 < b; k0 += slots) {
        int64_t m = 0;
        for (int64_t u = k0; u < std::min(b, k0 + slots); ++u) {
          const int64_t rb = n_rb - 1 - u % n_rb, sp = (u / n_rb) % s, nt = tiles[(size_t)rb];
          m = std::max(m, nt * (sp + 1) / s - nt * sp / s);
        }
        cost += (double)m + 3.0;
      }
      worst = std::max(worst, cost);
    }
    const double total = worst + (s > 1 ? 4.0 + 4.3 * s : 0.0);
    if (total < best_cost - 1e-9) {
      best_cost = total;
      best = s;
    }
  }
  std::lock_guard<std::mutex> lk(mu);
  if (cache.size() > 256) cache.clear();
  cache[key] = best;
  return best;
}

FwdPlan plan_fwd(int32_t n_list_pages, int32_t n_lists, int32_t page, int32_t n_kvh, int32_t C, int32_t G,
                 int32_t d) {
  FwdPlan p;
  const int64_t rows = (int64_t)C * G;
  p.nw = pick_nw(rows, n_lists);
  p.n_rb = row_blocks(rows, n_lists, p.nw);
  const double tiles = (double)n_list_pages * (page / 64) + (C / 64 + 1) / 2.0;
  const int32_t max_split = (int32_t)std::max(1.0, std::min(32.0, tiles));
  p.splits = key_splits(n_kvh, n_lists, rows, p.nw, G, n_list_pages * (page / 64), max_split);
  p.ws_bytes = p.splits > 1 ? align256((size_t)p.splits * n_kvh * rows * d * 4) + align256((size_t)p.splits * n_kvh * rows * 4) : 0;
  return p;
}

// Row splits of equal work rather than equal rows for the dK/dV pass. A key unit (256 keys) with a
// prior key streams every row block; a unit of the chunk's own keys only starts at its causal
// diagonal, so later blocks carry more units. work(b) counts the (unit, block) pairs of one KV
// head before block b (of the own-key units only when own_only), and split r starts at the first
// block where work reaches r/R of the total, so the splits partition [0, n_blk) exactly. Own unit
// j >= n_full starts at block G * (j * 8 - prior_tiles) (32 keys per tile, 8 tiles per unit, 32
// rows per block): an arithmetic progression, so the sum over units has a closed form.
static RowSplits equal_work_splits(int32_t n_list_pages, int32_t page, int32_t n_ku, int32_t G, int64_t n_blk,
                                   int32_t R, bool own_only) {
  RowSplits s{};
  R = std::max(1, std::min(R, MAX_ROW_SPLITS));
  const int64_t prior_tiles = (int64_t)n_list_pages * (page / 32), per_unit = NKT_TILES_PER_WG;
  const int64_t n_full = std::min<int64_t>(n_ku, (prior_tiles + per_unit - 1) / per_unit);
  const int64_t s0 = G * (n_full * per_unit - prior_tiles), dlt = G * per_unit;
  auto work = [&](int64_t b) {
    int64_t w = own_only ? 0 : n_full * b;
    if (b > s0) {
      const int64_t k = std::min<int64_t>(n_ku - n_full, (b - s0 + dlt - 1) / dlt);  // units begun before b
      w += k * (b - s0) - dlt * k * (k - 1) / 2;
    }
    return w;
  };
  const int64_t total = work(n_blk);
  for (int32_t r = 0; r <= R; ++r) {
    if (r == R) {
      s.b[r] = (int32_t)n_blk;
      break;
    }
    const int64_t target = total * r / R;
    int64_t lo = 0, hi = n_blk;  // first b with work(b) >= target
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (work(mid) >= target) hi = mid;
      else lo = mid + 1;
    }
    s.b[r] = (int32_t)lo;
  }
  return s;
}

BwdPlan plan_bwd(int32_t n_list_pages, int32_t n_lists, int32_t page, int32_t n_kvh, int32_t C, int32_t G,
                 int32_t d) {
  BwdPlan p;
  const int64_t rows = (int64_t)C * G;
  p.dq_nw = pick_nw(rows, n_lists);
  p.n_rb = row_blocks(rows, n_lists, p.dq_nw);
  const double tiles = (double)n_list_pages * (page / 64) + (C / 64 + 1) / 2.0;
  const int32_t max_split = (int32_t)std::max(1.0, std::min(32.0, tiles));
  p.splits = key_splits(n_kvh, n_lists, rows, p.dq_nw, G, n_list_pages * (page / 64), max_split);
  const int64_t n_kt = (int64_t)(n_list_pages + C / page) * (page / 32);
  p.n_ku = (int32_t)((n_kt + NKT_TILES_PER_WG - 1) / NKT_TILES_PER_WG);
  const int64_t n_blk = (rows + 31) / 32;
  const int32_t max_rs = (int32_t)std::min<int64_t>(MAX_ROW_SPLITS, n_blk);
  // One page list per query page: the dK/dV pass splits rows exactly at the lists (each query
  // page's rows see only its list's pages).
  p.row_splits = n_lists > 1 ? n_lists : best_split((int64_t)n_kvh * p.n_ku, (double)n_blk, 2.0, max_rs, 1);
  // The units of only the chunk's own keys are seen alike by every query page, so with one list
  // per query page they run once over all rows instead of once per list, in n_lists / 16 row
  // splits: each such workgroup streams about eight times the rows of a list's workgroup (an own
  // unit sees half the chunk's rows on average), and their flushes drop by that factor. Measured
  // on the 256K per-query-page step (32 lists): 2 splits 1.47-1.52 ms, 1 split 1.57-1.58, 4 splits
  // 1.52-1.55, 8 splits 1.54-1.63, against 1.74-1.79 ms once per list.
  p.own_splits = n_lists > 1 ? std::max(1, n_lists / 16) : 0;
  p.work_splits = equal_work_splits(n_list_pages, page, p.n_ku, G, n_blk, n_lists > 1 ? p.own_splits : p.row_splits,
                                    n_lists > 1);
  // [H_q][C] row dots (H_q = n_kvh*G is enough for the heads computed, but the buffer is indexed by
  // absolute head, so size it for every head the pool can address), then dQ partials.
  p.ws_bytes = 0;  // filled by the caller, which knows H_q
  return p;
}

// Host threads that add staged gradient blocks into host gradient pages. A job is split by blocks
// (one (page, head) block each) over the workers and the thread that runs it; the threads are made
// on first use and live until the process ends. Jobs run one at a time.
namespace {
class HostAdder {
 public:
  static HostAdder& get() {
    static HostAdder* inst = new HostAdder();  // never destroyed: callbacks may run during exit
    return *inst;
  }

  void run(const pkv_add_job& j) {
    std::lock_guard<std::mutex> serial(run_mu_);
    {
      std::lock_guard<std::mutex> lk(mu_);
      job_ = &j;
      next_.store(0);
      ++gen_;
    }
    cv_.notify_all();
    work(j);
    std::unique_lock<std::mutex> lk(mu_);
    job_ = nullptr;  // late wakers find no job
    done_cv_.wait(lk, [&] { return active_ == 0; });
  }

 private:
  HostAdder() {
    int n = 8;
    if (const char* e = getenv("PKV_HOST_THREADS")) n = atoi(e);
    const int hw = (int)std::thread::hardware_concurrency();
    if (hw > 0) n = std::min(n, hw);
    n = std::max(0, std::min(n, 64));
    for (int i = 0; i < n; ++i) std::thread([this] { loop(); }).detach();
  }

  void loop() {
    uint64_t seen = 0;
    for (;;) {
      const pkv_add_job* j;
      {
        std::unique_lock<std::mutex> lk(mu_);
        cv_.wait(lk, [&] { return gen_ != seen; });
        seen = gen_;
        j = job_;
        if (!j) continue;
        ++active_;
      }
      work(*j);
      {
        std::lock_guard<std::mutex> lk(mu_);
        --active_;
      }
      done_cv_.notify_all();
    }
  }

  void work(const pkv_add_job& j) {
    const size_t lp_bytes = align256((size_t)j.n * sizeof(int32_t));
    const int32_t* lp = reinterpret_cast<const int32_t*>(j.staging);
    const float* blocks = reinterpret_cast<const float*>(j.staging + lp_bytes);
    for (;;) {
      const int32_t i = next_.fetch_add(1);
      if (i >= j.n) return;
      const int32_t l = lp[i];
      const int32_t hp = (l >= 0 && l < j.n_host_bt) ? j.host_bt[l] : -1;
      if (hp < 0 || hp >= j.n_pages) {
        int32_t zero = 0;
        j.err->compare_exchange_strong(zero, 5);
        continue;
      }
      float* dst = j.grad_host + ((size_t)hp * j.h + j.kvh) * j.blk;
      const float* src = blocks + (size_t)i * j.blk;
      for (int32_t k = 0; k < j.blk; ++k) dst[k] += src[k];
    }
  }

  std::mutex run_mu_, mu_;
  std::condition_variable cv_, done_cv_;
  const pkv_add_job* job_ = nullptr;
  uint64_t gen_ = 0;
  int active_ = 0;
  std::atomic<int32_t> next_{0};
};

void host_add_callback(void* arg) {
  pkv_add_job* j = static_cast<pkv_add_job*>(arg);
  HostAdder::get().run(*j);
  j->busy.store(0);
}
}  // namespace

}  // namespace pkv

extern "C" {

size_t paged_kv_grad_staging_bytes(const pkv_pool* pool, int32_t n) {
  if (!pool || n < 0) return 0;
  return align256((size_t)n * sizeof(int32_t)) + (size_t)n * 2 * pool->page * pool->d * sizeof(float);
}

int paged_kv_grad_stage(pkv_pool* dev, int32_t dev_page0, int32_t n, int32_t kvh, const int32_t* lp_dev,
                        void* staging_host, size_t staging_bytes, void* stream) {
  if (!dev) return fail(PKV_E_INVALID, "pool is NULL");
  if (!dev->grad || (dev->flags & PKV_HOST_GRADS)) return fail(PKV_E_STATE, "the pool needs device gradient pages");
  if (n < 0 || dev_page0 < 0 || (int64_t)dev_page0 + n > dev->n_pages)
    return fail(PKV_E_INVALID, "pages [%d, %lld) outside the pool (%d pages)", dev_page0, (long long)dev_page0 + n,
                dev->n_pages);
  if (kvh < 0 || kvh >= dev->h_kv) return fail(PKV_E_INVALID, "kvh=%d outside [0, %d)", kvh, dev->h_kv);
  if (n == 0) {
    ok();
    return PKV_OK;
  }
  if (!lp_dev || !staging_host) return fail(PKV_E_INVALID, "NULL page ids or staging");
  const size_t need = paged_kv_grad_staging_bytes(dev, n);
  if (staging_bytes < need) return fail(PKV_E_NOMEM, "staging too small: %zu < %zu bytes", staging_bytes, need);
  const size_t blk_bytes = (size_t)2 * dev->page * dev->d * sizeof(float);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(staging_host, lp_dev, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (staged page ids)");
  const char* src = reinterpret_cast<const char*>(dev->grad) + ((size_t)dev_page0 * dev->h_kv + kvh) * blk_bytes;
  e = hipMemcpy2DAsync(static_cast<char*>(staging_host) + align256((size_t)n * sizeof(int32_t)), blk_bytes, src,
                       blk_bytes * dev->h_kv, blk_bytes, (size_t)n, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy2DAsync (staged gradient blocks)");
  e = pkv::launch_zero_head_blocks(*dev, dev_page0, n, kvh, s);
  if (e != hipSuccess) return hip_fail(e, "clearing the staged blocks");
  ok();
  return PKV_OK;
}

int paged_kv_grad_accumulate(pkv_pool* host, const int32_t* host_bt_host, int32_t n_host_bt, int32_t n, int32_t kvh,
                             const void* staging_host, void* stream) {
  if (!host) return fail(PKV_E_INVALID, "pool is NULL");
  if (!(host->flags & PKV_HOST_GRADS) || !host->jobs) return fail(PKV_E_STATE, "the pool has no host gradient pages");
  if (kvh < 0 || kvh >= host->h_kv) return fail(PKV_E_INVALID, "kvh=%d outside [0, %d)", kvh, host->h_kv);
  if (n < 0 || n_host_bt < 0) return fail(PKV_E_INVALID, "negative count");
  if (n == 0) {
    ok();
    return PKV_OK;
  }
  if (!host_bt_host || !staging_host) return fail(PKV_E_INVALID, "NULL block table or staging");
  pkv_host_jobs& J = *host->jobs;
  pkv_add_job& j = J.slot[J.next.fetch_add(1) % kHostJobs];
  const auto t0 = std::chrono::steady_clock::now();
  for (;;) {
    int32_t idle = 0;
    if (j.busy.compare_exchange_strong(idle, 1)) break;
    if (std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() > kHostJobWaitSeconds)
      return fail(PKV_E_STATE, "%d accumulations pending on this pool for %.0f s", kHostJobs, kHostJobWaitSeconds);
    std::this_thread::sleep_for(std::chrono::microseconds(50));
  }
  j.grad_host = static_cast<float*>(host->grad_host);
  j.n_pages = host->n_pages;
  j.h = host->h_kv;
  j.blk = 2 * host->page * host->d;
  j.kvh = kvh;
  j.host_bt = host_bt_host;
  j.n_host_bt = n_host_bt;
  j.staging = static_cast<const unsigned char*>(staging_host);
  j.n = n;
  j.err = &J.err;
  hipError_t e = hipLaunchHostFunc((hipStream_t)stream, pkv::host_add_callback, &j);
  if (e != hipSuccess) {
    j.busy.store(0);
    return hip_fail(e, "hipLaunchHostFunc (gradient accumulation)");
  }
  ok();
  return PKV_OK;
}

int pkv_version(void) { return 100; }

int pkv_mfma_probe(int32_t n_workgroups, int32_t iters, float* out_dev, double* flop, void* stream) {
  if (n_workgroups <= 0 || iters <= 0) return fail(PKV_E_INVALID, "n_workgroups and iters must be > 0");
  if (!out_dev) return fail(PKV_E_INVALID, "out_dev is NULL");
  if (flop) *flop = pkv::mfma_probe_flop(n_workgroups, iters);
  hipError_t e = pkv::launch_mfma_probe(n_workgroups, iters, out_dev, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mfma probe launch");
  ok();
  return PKV_OK;
}

int pkv_atomic_probe(int32_t n_workgroups, int32_t n_regions, int32_t region_elems, float* buf_dev, double* bytes,
                     void* stream) {
  if (n_workgroups <= 0 || n_regions <= 0 || region_elems <= 0)
    return fail(PKV_E_INVALID, "n_workgroups, n_regions and region_elems must be > 0");
  if (n_regions > n_workgroups) return fail(PKV_E_INVALID, "n_regions=%d exceeds n_workgroups=%d", n_regions, n_workgroups);
  if ((int64_t)n_regions * region_elems > ((int64_t)1 << 31))
    return fail(PKV_E_INVALID, "buffer of %lld floats too large", (long long)n_regions * region_elems);
  if (!buf_dev) return fail(PKV_E_INVALID, "buf_dev is NULL");
  if (bytes) *bytes = (double)n_workgroups * region_elems * sizeof(float);
  hipError_t e = pkv::launch_atomic_probe(n_workgroups, n_regions, region_elems, buf_dev, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "atomic probe launch");
  ok();
  return PKV_OK;
}

int pkv_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(pkv::g_tmu);
  pkv::g_timing = on != 0;
  if (on) {
    pkv::g_nrec = 0;
    pkv::g_summary.clear();
  }
  ok();
  return PKV_OK;
}

int pkv_timing_collect(void) {
  std::lock_guard<std::mutex> lk(pkv::g_tmu);
  std::map<std::string, std::pair<int32_t, double>> agg;
  for (size_t i = 0; i < pkv::g_nrec; ++i) {
    hipError_t e = hipEventSynchronize(pkv::g_recs[i].b);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize (timing)");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, pkv::g_recs[i].a, pkv::g_recs[i].b);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime (timing)");
    auto& slot = agg[pkv::g_recs[i].name];
    slot.first += 1;
    slot.second += ms;
  }
  pkv::g_summary.assign(agg.begin(), agg.end());
  ok();
  return (int)pkv::g_summary.size();
}

int pkv_timing_get(int i, const char** name, int32_t* launches, double* total_ms) {
  std::lock_guard<std::mutex> lk(pkv::g_tmu);
  if (i < 0 || (size_t)i >= pkv::g_summary.size()) return fail(PKV_E_INVALID, "timing index %d out of range", i);
  if (name) *name = pkv::g_summary[i].first.c_str();
  if (launches) *launches = pkv::g_summary[i].second.first;
  if (total_ms) *total_ms = pkv::g_summary[i].second.second;
  ok();
  return PKV_OK;
}

const char* pkv_last_error(void) { return g_err.c_str(); }

int paged_kv_alloc(pkv_pool** out, int32_t n_pages, int32_t page_size, int32_t n_kv_heads, int32_t head_dim,
                   uint32_t flags) {
  if (!out) return fail(PKV_E_INVALID, "out is NULL");
  *out = nullptr;
  if (n_pages <= 0 || n_kv_heads <= 0) return fail(PKV_E_INVALID, "n_pages and n_kv_heads must be positive");
  if (!supported(page_size, head_dim))
    return fail(PKV_E_UNSUPPORTED, "page_size %d / head_dim %d not supported (both must be 64 or 128)", page_size,
                head_dim);
  if (flags & ~(PKV_GRADS | PKV_HOST_TIER | PKV_HOST_GRADS)) return fail(PKV_E_INVALID, "unknown flags 0x%x", flags);
  if ((flags & PKV_HOST_GRADS) && !(flags & PKV_GRADS)) return fail(PKV_E_INVALID, "PKV_HOST_GRADS needs PKV_GRADS");
  pkv_pool* p = new (std::nothrow) pkv_pool();
  if (!p) return fail(PKV_E_NOMEM, "out of host memory");
  p->n_pages = n_pages;
  p->page = page_size;
  p->h_kv = n_kv_heads;
  p->d = head_dim;
  p->flags = flags;
  p->kv = nullptr;
  p->kv_host = nullptr;
  p->grad = nullptr;
  p->grad_host = nullptr;
  p->rep = nullptr;
  p->err = nullptr;
  p->alloc = new (std::nothrow) pkv_page_alloc();
  p->jobs = (flags & PKV_HOST_GRADS) ? new (std::nothrow) pkv_host_jobs() : nullptr;
  if (!p->alloc || ((flags & PKV_HOST_GRADS) && !p->jobs)) {
    delete p->alloc;
    delete p->jobs;
    delete p;
    return fail(PKV_E_NOMEM, "out of host memory");
  }
  try {
    p->alloc->free_pages.resize((size_t)n_pages);
    p->alloc->is_free.assign((size_t)n_pages, 1);
  } catch (const std::bad_alloc&) {
    delete p->alloc;
    delete p->jobs;
    delete p;
    return fail(PKV_E_NOMEM, "out of host memory for the page free list");
  }
  for (int32_t i = 0; i < n_pages; ++i) p->alloc->free_pages[(size_t)i] = n_pages - 1 - i;  // page 0 first
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) {
    delete p->alloc;
    delete p->jobs;
    delete p;
    return hip_fail(e, "hipGetDevice");
  }
  // Sizes are taken before anything can fail: cleanup() deletes p, and the error messages below
  // still report them.
  const size_t kvb = kv_bytes(*p), gb = grad_bytes(*p);
  auto cleanup = [&]() {
    if (p->kv_host) (void)hipHostFree(p->kv_host);
    else if (p->kv) (void)hipFree(p->kv);
    if (p->grad_host) (void)hipHostFree(p->grad_host);
    else if (p->grad) (void)hipFree(p->grad);
    if (p->rep) (void)hipFree(p->rep);
    if (p->err) (void)hipFree(p->err);
    delete p->alloc;
    delete p->jobs;
    delete p;
  };
  if (getenv("PKV_FAIL_HOST_ALLOC") && (flags & PKV_HOST_TIER)) {
    cleanup();
    return fail(PKV_E_NOMEM, "pinned host allocation failed (injected by PKV_FAIL_HOST_ALLOC)");
  }
  if (flags & PKV_HOST_TIER) {
    e = hipHostMalloc(&p->kv_host, kv_bytes(*p), hipHostMallocMapped | hipHostMallocPortable);
    if (e != hipSuccess) {
      p->kv_host = nullptr;
      (void)hipGetLastError();
      cleanup();
      return fail(PKV_E_NOMEM, "hipHostMalloc(%zu bytes): %s", kvb, hipGetErrorString(e));
    }
    void* dptr = nullptr;
    e = hipHostGetDevicePointer(&dptr, p->kv_host, 0);
    if (e != hipSuccess) {
      cleanup();
      return hip_fail(e, "hipHostGetDevicePointer");
    }
    p->kv = (uint16_t*)dptr;
    memset(p->kv_host, 0, kv_bytes(*p));
  } else {
    e = hipMalloc((void**)&p->kv, kv_bytes(*p));
    if (e != hipSuccess) {
      p->kv = nullptr;
      (void)hipGetLastError();
      cleanup();
      return fail(PKV_E_NOMEM, "hipMalloc(%zu bytes) for KV pages: %s", kvb, hipGetErrorString(e));
    }
    e = hipMemset(p->kv, 0, kv_bytes(*p));
    if (e != hipSuccess) {
      cleanup();
      return hip_fail(e, "hipMemset(kv)");
    }
  }
  if (flags & PKV_HOST_GRADS) {
    e = hipHostMalloc(&p->grad_host, grad_bytes(*p), hipHostMallocMapped | hipHostMallocPortable);
    if (e != hipSuccess) {
      p->grad_host = nullptr;
      (void)hipGetLastError();
      cleanup();
      return fail(PKV_E_NOMEM, "hipHostMalloc(%zu bytes) for gradient pages: %s", gb,
                  hipGetErrorString(e));
    }
    void* gptr = nullptr;
    e = hipHostGetDevicePointer(&gptr, p->grad_host, 0);
    if (e != hipSuccess) {
      cleanup();
      return hip_fail(e, "hipHostGetDevicePointer(grad)");
    }
    p->grad = (float*)gptr;
    memset(p->grad_host, 0, grad_bytes(*p));
  } else if (flags & PKV_GRADS) {
    e = hipMalloc((void**)&p->grad, grad_bytes(*p));
    if (e != hipSuccess) {
      p->grad = nullptr;
      (void)hipGetLastError();
      cleanup();
      return fail(PKV_E_NOMEM, "hipMalloc(%zu bytes) for gradient pages: %s", gb, hipGetErrorString(e));
    }
    e = hipMemset(p->grad, 0, grad_bytes(*p));
    if (e != hipSuccess) {
      cleanup();
      return hip_fail(e, "hipMemset(grad)");
    }
  }
  e = hipMalloc((void**)&p->rep, rep_bytes(*p));
  if (e == hipSuccess) e = hipMemset(p->rep, 0, rep_bytes(*p));
  if (e == hipSuccess) e = hipMalloc((void**)&p->err, 256);
  if (e == hipSuccess) e = hipMemset(p->err, 0, 256);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipGetLastError();
    cleanup();
    return fail(PKV_E_NOMEM, "device allocation failed: %s", hipGetErrorString(e));
  }
  *out = p;
  ok();
  return PKV_OK;
}

int paged_kv_free(pkv_pool* pool) {
  if (!pool) {
    ok();
    return PKV_OK;
  }
  hipError_t e = hipDeviceSynchronize();
  if (pool->kv_host) (void)hipHostFree(pool->kv_host);
  else if (pool->kv) (void)hipFree(pool->kv);
  if (pool->grad_host) (void)hipHostFree(pool->grad_host);
  else if (pool->grad) (void)hipFree(pool->grad);
  if (pool->rep) (void)hipFree(pool->rep);
  if (pool->err) (void)hipFree(pool->err);
  delete pool->alloc;
  delete pool->jobs;
  delete pool;
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize in paged_kv_free");
  ok();
  return PKV_OK;
}

int paged_kv_page_alloc(pkv_pool* pool, int32_t n, int32_t* pages_host) {
  if (!pool) return fail(PKV_E_INVALID, "pool is NULL");
  if (n < 0) return fail(PKV_E_INVALID, "n=%d < 0", n);
  if (n > 0 && !pages_host) return fail(PKV_E_INVALID, "pages_host is NULL");
  std::lock_guard<std::mutex> lk(pool->alloc->mu);
  auto& fl = pool->alloc->free_pages;
  if ((size_t)n > fl.size())
    return fail(PKV_E_NOMEM, "%d pages requested, %zu of %d free", n, fl.size(), pool->n_pages);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t pg = fl.back();
    fl.pop_back();
    pool->alloc->is_free[(size_t)pg] = 0;
    pages_host[i] = pg;
  }
  ok();
  return PKV_OK;
}

int paged_kv_page_release(pkv_pool* pool, int32_t n, const int32_t* pages_host) {
  if (!pool) return fail(PKV_E_INVALID, "pool is NULL");
  if (n < 0) return fail(PKV_E_INVALID, "n=%d < 0", n);
  if (n > 0 && !pages_host) return fail(PKV_E_INVALID, "pages_host is NULL");
  std::lock_guard<std::mutex> lk(pool->alloc->mu);
  auto& fr = pool->alloc->is_free;
  // Validate everything first (ids in range, allocated, no repeats), then release: a failed call
  // changes nothing.
  int32_t i = 0;
  for (; i < n; ++i) {
    const int32_t pg = pages_host[i];
    if (pg < 0 || pg >= pool->n_pages || fr[(size_t)pg] != 0) break;
    fr[(size_t)pg] = 2;  // marked for this call
  }
  if (i < n) {
    const int32_t bad = pages_host[i];
    for (int32_t j = 0; j < i; ++j) fr[(size_t)pages_host[j]] = 0;
    if (bad < 0 || bad >= pool->n_pages) return fail(PKV_E_INVALID, "page %d outside the pool (%d pages)", bad, pool->n_pages);
    return fail(PKV_E_INVALID, "page %d is not allocated (already free, or listed twice)", bad);
  }
  for (int32_t j = 0; j < n; ++j) {
    fr[(size_t)pages_host[j]] = 1;
    pool->alloc->free_pages.push_back(pages_host[j]);
  }
  ok();
  return PKV_OK;
}

int32_t paged_kv_pages_available(const pkv_pool* pool) {
  if (!pool) return fail(PKV_E_INVALID, "pool is NULL");
  std::lock_guard<std::mutex> lk(pool->alloc->mu);
  ok();
  return (int32_t)pool->alloc->free_pages.size();
}

int paged_kv_info(const pkv_pool* pool, int32_t* n_pages, int32_t* page_size, int32_t* n_kv_heads,
                  int32_t* head_dim, uint32_t* flags) {
  if (!pool) return fail(PKV_E_INVALID, "pool is NULL");
  if (n_pages) *n_pages = pool->n_pages;
  if (page_size) *page_size = pool->page;
  if (n_kv_heads) *n_kv_heads = pool->h_kv;
  if (head_dim) *head_dim = pool->d;
  if (flags) *flags = pool->flags;
  ok();
  return PKV_OK;
}

void* paged_kv_data(const pkv_pool* pool, int32_t what) {
  if (!pool) {
    fail(PKV_E_INVALID, "pool is NULL");
    return nullptr;
  }
  ok();
  switch (what) {
    case PKV_K:
    case PKV_V:
      return pool->kv;
    case PKV_DK:
    case PKV_DV:
      if (!pool->grad) fail(PKV_E_STATE, "pool has no gradient pages");
      return pool->grad;
    case PKV_REP:
      return pool->rep;
    default:
      fail(PKV_E_INVALID, "unknown array selector %d", what);
      return nullptr;
  }
}

int paged_kv_append(pkv_pool* pool, const int32_t* bt_dev, int32_t n_bt, int32_t pos0, int32_t n_tokens,
                    const uint16_t* k_dev, const uint16_t* v_dev, void* stream) {
  if (!pool) return fail(PKV_E_INVALID, "pool is NULL");
  if (!bt_dev || !k_dev || !v_dev) return fail(PKV_E_INVALID, "NULL block table, k or v");
  if (!aligned16(k_dev) || !aligned16(v_dev)) return fail(PKV_E_INVALID, "k and v must be 16-byte aligned");
  if (pos0 < 0 || n_tokens < 0) return fail(PKV_E_INVALID, "pos0 and n_tokens must be >= 0");
  if (n_bt < 0 || (int64_t)pos0 + n_tokens > (int64_t)n_bt * pool->page)
    return fail(PKV_E_RANGE, "positions [%d, %lld) exceed the block table (%d pages of %d)", pos0,
                (long long)pos0 + n_tokens, n_bt, pool->page);
  if (n_tokens == 0) {
    ok();
    return PKV_OK;
  }
  hipError_t e = pkv::launch_append(*pool, bt_dev, n_bt, pos0, n_tokens, k_dev, v_dev, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  ok();
  return PKV_OK;
}

int paged_kv_zero_grad(pkv_pool* pool, const int32_t* bt_dev, int32_t n_pages, void* stream) {
  if (!pool) return fail(PKV_E_INVALID, "pool is NULL");
  if (!pool->grad) return fail(PKV_E_STATE, "pool has no gradient pages");
  int32_t n = n_pages;
  if (!bt_dev) n = pool->n_pages;
  if (n < 0) return fail(PKV_E_INVALID, "n_pages < 0");
  hipError_t e = pkv::launch_zero_grad(*pool, bt_dev, 0, n, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "zero_grad launch");
  ok();
  return PKV_OK;
}

int paged_kv_export(const pkv_pool* pool, int32_t what, const int32_t* bt_dev, int32_t n_bt, int32_t first_page,
                    int32_t n_pages, void* dst_dev, void* stream) {
  if (!pool) return fail(PKV_E_INVALID, "pool is NULL");
  if (!bt_dev || !dst_dev) return fail(PKV_E_INVALID, "NULL block table or destination");
  if (what < PKV_K || what > PKV_REP) return fail(PKV_E_INVALID, "unknown array selector %d", what);
  if ((what == PKV_DK || what == PKV_DV) && !pool->grad) return fail(PKV_E_STATE, "pool has no gradient pages");
  if (first_page < 0 || n_pages < 0 || (int64_t)first_page + n_pages > n_bt)
    return fail(PKV_E_RANGE, "pages [%d, %lld) exceed the block table (%d)", first_page,
                (long long)first_page + n_pages, n_bt);
  if (!aligned16(dst_dev)) return fail(PKV_E_INVALID, "destination must be 16-byte aligned");
  if (n_pages == 0) {
    ok();
    return PKV_OK;
  }
  hipError_t e = pkv::launch_export(*pool, what, bt_dev, first_page, n_pages, dst_dev, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "export launch");
  ok();
  return PKV_OK;
}

int paged_kv_check(pkv_pool* pool) {
  if (!pool) return fail(PKV_E_INVALID, "pool is NULL");
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  int32_t word = 0;
  e = hipMemcpy(&word, pool->err, sizeof(word), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading the error word");
  if (pool->jobs && word == 0) word = pool->jobs->err.exchange(0);
  if (word != 0) {
    const int32_t zero = 0;
    e = hipMemcpy(pool->err, &zero, sizeof(zero), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "clearing the error word");
    const char* what = word == 1   ? "block-table entry outside the pool"
                       : word == 2 ? "selected page outside [0, n_prior)"
                       : word == 3 ? "logical page beyond the block table"
                       : word == 5 ? "staged gradient page outside the host block table or pool"
                                   : "gather destination outside the device pool";
    return fail(PKV_E_DEVICE, "a kernel skipped a page: %s", what);
  }
  ok();
  return PKV_OK;
}

size_t page_topk_ws_bytes(const pkv_pool* pool, int32_t n_prior, int32_t C, int32_t H_q, int32_t n_lists) {
  if (!pool || C <= 0 || H_q <= 0 || n_prior < 0 || n_lists <= 0) return 0;
  return pkv::topk_ws_bytes(n_prior, C, H_q, pool->h_kv, pool->d, n_lists);
}

// Shared checks of page_topk_select and page_topk_select_noalloc; on success *ws_need is the
// scratch the call needs and *n_sel the selection length.
static int check_topk(const pkv_pool* pool, const int32_t* bt_dev, int32_t n_bt, int32_t n_prior, const uint16_t* q_dev,
                      int32_t C, int32_t H_q, int32_t top_k, int32_t n_local, int32_t n_lists, const int32_t* sel_dev,
                      const int32_t* n_sel_out, size_t* ws_need, int32_t* n_sel, bool* needs_ws) {
  if (!pool) return fail(PKV_E_INVALID, "pool is NULL");
  if (!bt_dev || !q_dev || !n_sel_out) return fail(PKV_E_INVALID, "NULL block table, q or n_sel_out");
  if (!aligned16(q_dev)) return fail(PKV_E_INVALID, "q must be 16-byte aligned");
  if (C <= 0 || C % 64 != 0) return fail(PKV_E_INVALID, "C=%d must be a positive multiple of 64", C);
  if (H_q <= 0 || H_q % pool->h_kv != 0) return fail(PKV_E_INVALID, "H_q=%d must be a multiple of H_kv=%d", H_q, pool->h_kv);
  if (top_k < 0 || n_local < 0 || n_prior < 0) return fail(PKV_E_INVALID, "top_k, n_local, n_prior must be >= 0");
  if (H_q / pool->h_kv > 128) return fail(PKV_E_UNSUPPORTED, "H_q/H_kv=%d exceeds 128", H_q / pool->h_kv);
  if (n_prior > n_bt) return fail(PKV_E_RANGE, "n_prior=%d exceeds the block table (%d)", n_prior, n_bt);
  if (n_lists != 1 && (C % pool->page != 0 || n_lists != C / pool->page))
    return fail(PKV_E_INVALID, "n_lists=%d must be 1 or C / page_size", n_lists);
  const int32_t n_cand = n_prior > n_local ? n_prior - n_local : 0;
  const int32_t kk = std::min(top_k, n_cand);
  *n_sel = kk + (n_prior - n_cand);
  if (*n_sel > 0 && !sel_dev) return fail(PKV_E_INVALID, "sel is NULL");
  *ws_need = pkv::topk_ws_bytes(n_prior, C, H_q, pool->h_kv, pool->d, n_lists);
  *needs_ws = kk > 0 && kk < n_cand;
  return PKV_OK;
}

int page_topk_select_noalloc(const pkv_pool* pool, const int32_t* bt_dev, int32_t n_bt, int32_t n_prior,
                             const uint16_t* q_dev, int32_t C, int32_t H_q, int32_t top_k, int32_t n_local,
                             int32_t n_lists, int32_t* sel_dev, int32_t* n_sel_out, void* stream) {
  size_t ws_need = 0;
  int32_t n_sel = 0;
  bool needs_ws = false;
  int rc = check_topk(pool, bt_dev, n_bt, n_prior, q_dev, C, H_q, top_k, n_local, n_lists, sel_dev, n_sel_out,
                      &ws_need, &n_sel, &needs_ws);
  if (rc != PKV_OK) return rc;
  if (ws_need > pkv::kTopkScratchBytes)
    return fail(PKV_E_NOMEM, "this selection needs %zu bytes of scratch; the static scratch holds %zu", ws_need,
                pkv::kTopkScratchBytes);
  void* scratch = nullptr;
  hipError_t e = pkv::topk_scratch_ptr(&scratch);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (selection scratch)");
  *n_sel_out = n_sel;
  e = pkv::launch_topk(*pool, bt_dev, n_bt, n_prior, q_dev, C, H_q, top_k, n_local, n_lists, sel_dev, scratch,
                       (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  ok();
  return PKV_OK;
}

int page_topk_select(const pkv_pool* pool, const int32_t* bt_dev, int32_t n_bt, int32_t n_prior,
                     const uint16_t* q_dev, int32_t C, int32_t H_q, int32_t top_k, int32_t n_local,
                     int32_t n_lists, int32_t* sel_dev, int32_t* n_sel_out, void* ws_dev, size_t ws_bytes,
                     void* stream) {
  size_t ws_need = 0;
  int32_t n_sel = 0;
  bool needs_ws = false;
  int rc = check_topk(pool, bt_dev, n_bt, n_prior, q_dev, C, H_q, top_k, n_local, n_lists, sel_dev, n_sel_out,
                      &ws_need, &n_sel, &needs_ws);
  if (rc != PKV_OK) return rc;
  if (ws_bytes < ws_need || (!ws_dev && needs_ws))
    return fail(PKV_E_NOMEM, "workspace too small: %zu < %zu bytes", ws_bytes, ws_need);
  *n_sel_out = n_sel;
  hipError_t e = pkv::launch_topk(*pool, bt_dev, n_bt, n_prior, q_dev, C, H_q, top_k, n_local, n_lists, sel_dev,
                                  ws_dev, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  ok();
  return PKV_OK;
}

// Selection lists per KV head as the plan sees them: 1 for dense calls and malformed counts (the
// entry points reject those before planning).
static int32_t plan_lists(int32_t n_sel, int32_t n_lists, int32_t C, int32_t page) {
  return (n_sel >= 0 && n_lists > 1 && C % page == 0 && n_lists == C / page) ? n_lists : 1;
}

size_t chunk_attn_fwd_ws_bytes(const pkv_pool* pool, int32_t n_prior, int32_t n_sel, int32_t n_lists, int32_t n_kvh,
                               int32_t C, int32_t H_q) {
  if (!pool || C <= 0 || H_q <= 0 || n_kvh <= 0 || H_q % pool->h_kv != 0) return 0;
  const int32_t n_list = n_sel >= 0 ? n_sel : n_prior;
  return pkv::plan_fwd(n_list, plan_lists(n_sel, n_lists, C, pool->page), pool->page, n_kvh, C, H_q / pool->h_kv,
                       pool->d).ws_bytes;
}

int chunk_attn_fwd(const pkv_pool* pool, const int32_t* bt_dev, int32_t n_bt, int32_t n_prior, const int32_t* sel_dev,
                   int32_t n_sel, int32_t n_lists, int32_t kvh0, int32_t n_kvh, const uint16_t* q_dev, int32_t C,
                   int32_t H_q, float scale, uint16_t* o_dev, float* lse_dev, void* ws_dev, size_t ws_bytes,
                   void* stream) {
  int rc = check_attn(pool, bt_dev, n_bt, n_prior, sel_dev, n_sel, n_lists, kvh0, n_kvh, q_dev, C, H_q, scale);
  if (rc != PKV_OK) return rc;
  if (!o_dev || !lse_dev) return fail(PKV_E_INVALID, "NULL o or lse");
  if (!aligned16(o_dev)) return fail(PKV_E_INVALID, "o must be 16-byte aligned");
  const int32_t n_list = sel_dev ? n_sel : n_prior;
  const pkv::FwdPlan plan = pkv::plan_fwd(n_list, sel_dev ? n_lists : 1, pool->page, n_kvh, C, H_q / pool->h_kv,
                                          pool->d);
  if (plan.ws_bytes > 0 && (!ws_dev || ws_bytes < plan.ws_bytes))
    return fail(PKV_E_NOMEM, "workspace too small: %zu < %zu bytes", ws_bytes, plan.ws_bytes);
  const pkv::AttnArgs a =
      make_args(pool, bt_dev, n_bt, n_prior, sel_dev, n_sel, n_lists, kvh0, n_kvh, q_dev, C, H_q, scale);
  hipError_t e = pkv::launch_fwd(a, plan, o_dev, lse_dev, ws_dev, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  ok();
  return PKV_OK;
}

static size_t bwd_ws(const pkv_pool* pool, const pkv::BwdPlan& plan, int32_t n_kvh, int32_t C, int32_t H_q) {
  // -D, lse * log2 e and -lse / scale, each with 64 padding entries
  const size_t dbytes = 3 * ((((size_t)H_q * C + 63) & ~(size_t)63) + 64) * 4;
  const size_t dq = plan.splits > 1 ? (size_t)plan.splits * n_kvh * C * (H_q / pool->h_kv) * pool->d * 4 : 0;
  return align256(dbytes + dq);
}

size_t chunk_attn_bwd_ws_bytes(const pkv_pool* pool, int32_t n_prior, int32_t n_sel, int32_t n_lists, int32_t n_kvh,
                               int32_t C, int32_t H_q) {
  if (!pool || C <= 0 || H_q <= 0 || n_kvh <= 0 || H_q % pool->h_kv != 0) return 0;
  const int32_t n_list = n_sel >= 0 ? n_sel : n_prior;
  const pkv::BwdPlan plan = pkv::plan_bwd(n_list, plan_lists(n_sel, n_lists, C, pool->page), pool->page, n_kvh, C,
                                          H_q / pool->h_kv, pool->d);
  return bwd_ws(pool, plan, n_kvh, C, H_q);
}

int chunk_attn_bwd(const pkv_pool* pool, const int32_t* bt_dev, int32_t n_bt, pkv_pool* gpool, const int32_t* gbt_dev,
                   int32_t n_gbt, int32_t n_prior, const int32_t* sel_dev, int32_t n_sel, int32_t n_lists, int32_t kvh0,
                   int32_t n_kvh, const uint16_t* q_dev, const uint16_t* o_dev, const uint16_t* dout_dev, const float* lse_dev,
                   int32_t C, int32_t H_q, float scale, uint16_t* dq_dev, void* ws_dev, size_t ws_bytes,
                   void* stream) {
  int rc = check_attn(pool, bt_dev, n_bt, n_prior, sel_dev, n_sel, n_lists, kvh0, n_kvh, q_dev, C, H_q, scale);
  if (rc != PKV_OK) return rc;
  if (!gpool) return fail(PKV_E_INVALID, "gradient pool is NULL");
  if (!gpool->grad) return fail(PKV_E_STATE, "gradient pool has no gradient pages");
  if (gpool->flags & PKV_HOST_GRADS)
    return fail(PKV_E_STATE, "gradient pages in host memory: accumulate into a device pool, then paged_kv_grad_offload");
  if (gpool->page != pool->page || gpool->h_kv != pool->h_kv || gpool->d != pool->d)
    return fail(PKV_E_INVALID, "gradient pool shape differs from the KV pool");
  if (!gbt_dev) return fail(PKV_E_INVALID, "gradient block table is NULL");
  if ((int64_t)n_prior + C / pool->page > n_gbt)
    return fail(PKV_E_RANGE, "pages [0, %d) exceed the gradient block table (%d)", n_prior + C / pool->page, n_gbt);
  if (!o_dev || !dout_dev || !lse_dev || !dq_dev) return fail(PKV_E_INVALID, "NULL o, dout, lse or dq");
  if (!aligned16(o_dev) || !aligned16(dout_dev) || !aligned16(dq_dev))
    return fail(PKV_E_INVALID, "o, dout and dq must be 16-byte aligned");
  const int32_t n_list = sel_dev ? n_sel : n_prior;
  const pkv::BwdPlan plan = pkv::plan_bwd(n_list, sel_dev ? n_lists : 1, pool->page, n_kvh, C, H_q / pool->h_kv,
                                          pool->d);
  const size_t need = bwd_ws(pool, plan, n_kvh, C, H_q);
  if (!ws_dev || ws_bytes < need) return fail(PKV_E_NOMEM, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  const pkv::AttnArgs a =
      make_args(pool, bt_dev, n_bt, n_prior, sel_dev, n_sel, n_lists, kvh0, n_kvh, q_dev, C, H_q, scale);
  pkv::BwdExtra x;
  x.o = o_dev;
  x.dout = dout_dev;
  x.lse = lse_dev;
  x.dq = dq_dev;
  x.grad = gpool->grad;
  x.gbt = gbt_dev;
  x.n_gbt = n_gbt;
  x.n_gpool_pages = gpool->n_pages;
  hipError_t e = pkv::launch_bwd(a, x, plan, ws_dev, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  ok();
  return PKV_OK;
}

int paged_kv_gather(const pkv_pool* host, pkv_pool* dev, const int32_t* host_bt_dev, int32_t n_host_bt,
                    const int32_t* sel_dev, int32_t n_sel, int32_t kvh, const int32_t* dst_pages_dev,
                    int32_t* dev_bt_out_dev, int32_t n_dev_bt, int32_t n_workgroups, void* stream) {
  if (!host || !dev) return fail(PKV_E_INVALID, "NULL pool");
  if (!(host->flags & PKV_HOST_TIER)) return fail(PKV_E_STATE, "source pool is not a host-tier pool");
  if (dev->flags & PKV_HOST_TIER) return fail(PKV_E_STATE, "destination pool must be a device pool");
  if (host->page != dev->page || host->h_kv != dev->h_kv || host->d != dev->d)
    return fail(PKV_E_INVALID, "pool shapes differ");
  if (kvh < 0 || kvh >= host->h_kv) return fail(PKV_E_INVALID, "kvh=%d outside [0, %d)", kvh, host->h_kv);
  if (n_sel < 0) return fail(PKV_E_INVALID, "n_sel < 0");
  if (n_sel > 0 && (!host_bt_dev || !sel_dev || !dst_pages_dev)) return fail(PKV_E_INVALID, "NULL table");
  if (dev_bt_out_dev && n_dev_bt < 0) return fail(PKV_E_INVALID, "n_dev_bt < 0");
  if (n_workgroups < 0 || n_workgroups > pkv::kGatherMaxWorkgroups)
    return fail(PKV_E_INVALID, "n_workgroups=%d outside [0, %d]", n_workgroups, pkv::kGatherMaxWorkgroups);
  hipError_t e = pkv::launch_gather(*host, *dev, host_bt_dev, n_host_bt, sel_dev, n_sel, kvh, dst_pages_dev,
                                    dev_bt_out_dev, n_dev_bt, n_workgroups, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  ok();
  return PKV_OK;
}

int paged_kv_grad_offload(pkv_pool* host, const int32_t* host_bt_dev, int32_t n_host_bt, pkv_pool* dev,
                          const int32_t* dev_bt_dev, int32_t n_dev_bt, const int32_t* lp_dev, int32_t n,
                          int32_t kvh0, int32_t n_kvh, void* stream) {
  if (!host || !dev) return fail(PKV_E_INVALID, "NULL pool");
  if (!(host->flags & PKV_HOST_GRADS)) return fail(PKV_E_STATE, "destination pool has no host gradient pages");
  if (!dev->grad || (dev->flags & PKV_HOST_GRADS)) return fail(PKV_E_STATE, "source pool needs device gradient pages");
  if (host->page != dev->page || host->h_kv != dev->h_kv || host->d != dev->d)
    return fail(PKV_E_INVALID, "pool shapes differ");
  if (kvh0 < 0 || n_kvh <= 0 || kvh0 + n_kvh > host->h_kv)
    return fail(PKV_E_INVALID, "KV head range [%d, %d) outside [0, %d)", kvh0, kvh0 + n_kvh, host->h_kv);
  if (n < 0 || n_host_bt < 0 || n_dev_bt < 0) return fail(PKV_E_INVALID, "negative count");
  if (n > 0 && (!host_bt_dev || !dev_bt_dev || !lp_dev)) return fail(PKV_E_INVALID, "NULL table");
  hipError_t e = pkv::launch_grad_offload(*host, host_bt_dev, n_host_bt, *dev, dev_bt_dev, n_dev_bt, lp_dev, n, kvh0,
                                          n_kvh, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "gradient offload launch");
  ok();
  return PKV_OK;
}

int paged_kv_copy(const pkv_pool* src, pkv_pool* dst, uint32_t what, int32_t first_page, int32_t n_pages,
                  void* stream) {
  if (!src || !dst) return fail(PKV_E_INVALID, "NULL pool");
  if (src == dst) return fail(PKV_E_INVALID, "source and destination are the same pool");
  if (what & ~(PKV_COPY_KV | PKV_COPY_GRAD)) return fail(PKV_E_INVALID, "unknown copy bits 0x%x", what);
  if (src->page != dst->page || src->h_kv != dst->h_kv || src->d != dst->d)
    return fail(PKV_E_INVALID, "pool shapes differ");
  if (first_page < 0 || n_pages < 0 || (int64_t)first_page + n_pages > src->n_pages ||
      (int64_t)first_page + n_pages > dst->n_pages)
    return fail(PKV_E_INVALID, "pages [%d, %d) outside a pool (%d and %d pages)", first_page,
                first_page + n_pages, src->n_pages, dst->n_pages);
  if ((what & PKV_COPY_GRAD) && (!src->grad || !dst->grad))
    return fail(PKV_E_STATE, "gradient copy needs gradient pages in both pools");
  if (n_pages == 0 || what == 0) {
    ok();
    return PKV_OK;
  }
  // Host allocations are addressed by their host pointers, so the runtime sees pinned host memory
  // and uses a copy engine.
  const size_t page_elems = (size_t)src->h_kv * 2 * src->page * src->d;
  if (what & PKV_COPY_KV) {
    const size_t bytes = page_elems * sizeof(uint16_t);
    const char* s = (const char*)(src->kv_host ? src->kv_host : (void*)src->kv) + bytes * first_page;
    char* d = (char*)(dst->kv_host ? dst->kv_host : (void*)dst->kv) + bytes * first_page;
    hipError_t e = hipMemcpyAsync(d, s, bytes * n_pages, hipMemcpyDefault, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (KV pages)");
  }
  if (what & PKV_COPY_GRAD) {
    const size_t bytes = page_elems * sizeof(float);
    const char* s = (const char*)(src->grad_host ? src->grad_host : (void*)src->grad) + bytes * first_page;
    char* d = (char*)(dst->grad_host ? dst->grad_host : (void*)dst->grad) + bytes * first_page;
    hipError_t e = hipMemcpyAsync(d, s, bytes * n_pages, hipMemcpyDefault, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (gradient pages)");
  }
  ok();
  return PKV_OK;
}

}  // extern "C"
