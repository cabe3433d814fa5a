// Internal declarations shared by the host ABI (pkv_abi.cpp) and the kernel files (*.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

struct pkv_page_alloc;  // host-side free list of physical pages (pkv_abi.cpp)
struct pkv_host_jobs;   // host-side gradient accumulation jobs of a PKV_HOST_GRADS pool (pkv_abi.cpp)

struct pkv_pool {
  int32_t n_pages;
  int32_t page;
  int32_t h_kv;
  int32_t d;
  uint32_t flags;
  int device;
  uint16_t* kv;       // device address of the bf16 KV pages (device-mapped pinned host for host tier)
  void* kv_host;      // host allocation of a host-tier pool (NULL otherwise)
  float* grad;        // fp32 gradient pages (NULL without PKV_GRADS; device-mapped host for PKV_HOST_GRADS)
  void* grad_host;    // host allocation of PKV_HOST_GRADS gradient pages (NULL otherwise)
  float* rep;         // fp32 representative key per (page, head)
  int32_t* err;       // device word: nonzero once a kernel met an out-of-range table entry
  pkv_page_alloc* alloc;  // free list of physical pages handed out by paged_kv_page_alloc
  pkv_host_jobs* jobs;    // host gradient accumulation (PKV_HOST_GRADS pools only, else NULL)
};

namespace pkv {

// Everything a chunk-attention kernel needs to walk one chunk's key list.
struct AttnArgs {
  const uint16_t* kv;
  int32_t n_pool_pages;
  int32_t page;
  int32_t h_kv;
  int32_t d;
  const int32_t* bt;
  int32_t n_bt;
  int32_t n_prior;
  const int32_t* sel;  // NULL = dense; else [h_kv][n_lists][n_sel] logical page ids
  int32_t n_sel;
  int32_t n_lists;     // selection lists per KV head: 1, or one per query page (C / page)
  int32_t kvh0;
  int32_t n_kvh;
  const uint16_t* q;
  int32_t C;
  int32_t h_q;
  int32_t G;
  float scale;
  int32_t* err;
};

struct BwdExtra {
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  float* grad;          // gradient pool base
  const int32_t* gbt;   // gradient block table
  int32_t n_gbt;
  int32_t n_gpool_pages;
};

// Brackets one kernel launch with HIP events on its stream while timing is enabled.
class TimerScope {
 public:
  TimerScope(const char* name, hipStream_t s);
  ~TimerScope();

 private:
  int slot_;
  hipStream_t s_;
};

// Launch-shape decisions, computed on the host from the shapes alone.
struct FwdPlan {
  int32_t nw;         // waves per workgroup: 8 (256-row blocks) or 4 (128-row blocks)
  int32_t n_rb;       // row blocks per KV head (n_lists x blocks per list)
  int32_t splits;     // key-range splits (>1 needs the combine kernel and workspace)
  size_t ws_bytes;
};
// First row block of each equal-work row split of the dK/dV pass, and n_blk after the last
// (passed by value as a kernel argument).
constexpr int MAX_ROW_SPLITS = 64;
struct RowSplits {
  int32_t b[MAX_ROW_SPLITS + 1];
};

struct BwdPlan {
  int32_t dq_nw;       // dQ pass: waves per workgroup, as the forward's nw
  int32_t n_rb;        // dQ pass: row blocks per KV head (n_lists x blocks per list)
  int32_t splits;      // dQ pass: key-range splits
  int32_t n_ku;        // dK/dV pass: key units of 256 keys per KV head
  int32_t row_splits;  // dK/dV pass: row-range splits (one per selection list when n_lists > 1)
  int32_t own_splits;  // dK/dV pass with n_lists > 1: row splits of the units of only the chunk's
                       // own keys, run once over all rows (0: they run per list like the others)
  RowSplits work_splits;  // boundaries of the equal-work splits: of all units with one list (when
                          // row_splits > 1), of the own-key units with one list per query page
  size_t ws_bytes;
};

int num_cus();
// 32-key tiles per workgroup of the key-major dK/dV pass (4 waves x 2 tiles).
constexpr int NKT_TILES_PER_WG = 8;
FwdPlan plan_fwd(int32_t n_list_pages, int32_t n_lists, int32_t page, int32_t n_kvh, int32_t C, int32_t G, int32_t d);
BwdPlan plan_bwd(int32_t n_list_pages, int32_t n_lists, int32_t page, int32_t n_kvh, int32_t C, int32_t G, int32_t d);

hipError_t launch_append(const pkv_pool& pool, const int32_t* bt, int32_t n_bt, int32_t pos0, int32_t n,
                         const uint16_t* k, const uint16_t* v, hipStream_t s);
hipError_t launch_zero_grad(const pkv_pool& pool, const int32_t* bt, int32_t first_page, int32_t n_pages,
                            hipStream_t s);
hipError_t launch_export(const pkv_pool& pool, int32_t what, const int32_t* bt, int32_t first_page,
                         int32_t n_pages, void* dst, hipStream_t s);
hipError_t launch_gather(const pkv_pool& host, const pkv_pool& dev, const int32_t* host_bt, int32_t n_host_bt,
                         const int32_t* sel, int32_t n_sel, int32_t kvh, const int32_t* dst_pages,
                         int32_t* dev_bt_out, int32_t n_dev_bt, int32_t n_workgroups, hipStream_t s);
constexpr int32_t kGatherMaxWorkgroups = 64;
hipError_t launch_grad_offload(const pkv_pool& host, const int32_t* host_bt, int32_t n_host_bt, const pkv_pool& dev,
                               const int32_t* dev_bt, int32_t n_dev_bt, const int32_t* lp, int32_t n, int32_t kvh0,
                               int32_t n_kvh, hipStream_t s);
hipError_t launch_zero_head_blocks(const pkv_pool& pool, int32_t page0, int32_t n, int32_t g, hipStream_t s);
size_t topk_ws_bytes(int32_t n_cand, int32_t C, int32_t h_q, int32_t h_kv, int32_t d, int32_t n_lists);
// Static scratch of page_topk_select_noalloc: a file-scope device array in k_select.hip, one copy per
// GPU. topk_scratch_ptr returns the current device's copy (looked up once per device).
constexpr size_t kTopkScratchBytes = (size_t)16 << 20;
hipError_t topk_scratch_ptr(void** out);
hipError_t launch_topk(const pkv_pool& pool, const int32_t* bt, int32_t n_bt, int32_t n_prior, const uint16_t* q,
                       int32_t C, int32_t h_q, int32_t top_k, int32_t n_local, int32_t n_lists, int32_t* sel,
                       void* ws, hipStream_t s);
hipError_t launch_fwd(const AttnArgs& a, const FwdPlan& plan, uint16_t* o, float* lse, void* ws, hipStream_t s);
// The forward of 256-row blocks with one wave per SIMD (64 rows per wave); the same work units,
// outputs and split partials as k_attn_fwd with 8 waves.
template <int D>
hipError_t launch_fwd64(const AttnArgs& a, int32_t n_rb, int32_t splits, uint16_t* o, float* lse, float* ws_o,
                        float* ws_lse, hipStream_t s);
// Which kernel runs 256-row forward blocks: true (default) for launch_fwd64, false for k_attn_fwd
// with 8 waves; PKV_FWD_KERNEL=w8 selects the latter (read once).
bool fwd_one_wave_per_simd();
// The dQ pass of 256-row blocks with one wave per SIMD (64 rows per wave); the same work units,
// outputs and split partials as k_bwd_dq with 8 waves.
template <int D>
hipError_t launch_dq64(const AttnArgs& a, const BwdExtra& e, int32_t n_rb, int32_t splits, const float* ndbuf,
                       const float* lse2buf, float* ws_dq, hipStream_t s);
// Which kernel runs 256-row dQ blocks: true (default) for launch_dq64, false for k_bwd_dq with 8
// waves; PKV_DQ_KERNEL=w8 selects the latter (read once).
bool dq_one_wave_per_simd();
hipError_t launch_mfma_probe(int32_t n_wg, int32_t iters, float* out, hipStream_t s);
double mfma_probe_flop(int32_t n_wg, int32_t iters);
hipError_t launch_atomic_probe(int32_t n_wg, int32_t n_regions, int32_t region_elems, float* buf, hipStream_t s);
hipError_t launch_bwd(const AttnArgs& a, const BwdExtra& e, const BwdPlan& plan, void* ws, hipStream_t s);
template <int D>
hipError_t launch_dkdv(const AttnArgs& a, const BwdExtra& e, const BwdPlan& plan, const float* ndbuf,
                       const float* nlsbuf, int32_t pad_row, hipStream_t s);

}  // namespace pkv
