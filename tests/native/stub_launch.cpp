// Stand-ins for the library's kernel launchers (the *.hip files), for checking the host ABI on a
// machine without a GPU: each records that something was enqueued instead of launching. The
// checks use the count to assert that a call which fails validation enqueues nothing.
// Test infrastructure only.
#include "../../paged_kv_cache_fwd_amd/csrc/pkv_internal.h"

long g_stub_launches = 0;

namespace pkv {

hipError_t launch_append(const pkv_pool&, const int32_t*, int32_t, int32_t, int32_t, const uint16_t*,
                         const uint16_t*, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
hipError_t launch_zero_grad(const pkv_pool&, const int32_t*, int32_t, int32_t, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
hipError_t launch_export(const pkv_pool&, int32_t, const int32_t*, int32_t, int32_t, void*, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
hipError_t launch_gather(const pkv_pool&, const pkv_pool&, const int32_t*, int32_t, const int32_t*, int32_t, int32_t,
                         const int32_t*, int32_t*, int32_t, int32_t, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
// Clears the blocks for real (the fake device memory is host memory), so the checks can follow
// the staged offload's data.
hipError_t launch_zero_head_blocks(const pkv_pool& pool, int32_t page0, int32_t n, int32_t g, hipStream_t) {
  ++g_stub_launches;
  const size_t blk = (size_t)2 * pool.page * pool.d;
  for (int32_t i = 0; i < n; ++i)
    for (size_t k = 0; k < blk; ++k) pool.grad[((size_t)(page0 + i) * pool.h_kv + g) * blk + k] = 0.f;
  return hipSuccess;
}
hipError_t launch_grad_offload(const pkv_pool&, const int32_t*, int32_t, const pkv_pool&, const int32_t*, int32_t,
                               const int32_t*, int32_t, int32_t, int32_t, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
// Any positive size: the checks only need "too small" to be detectable.
size_t topk_ws_bytes(int32_t n_cand, int32_t C, int32_t h_q, int32_t, int32_t d, int32_t n_lists) {
  return 256 + (size_t)n_lists * ((size_t)n_cand + (size_t)C / 64 * h_q) * d * 4;
}
// The static selection scratch: any host buffer stands in for it here.
hipError_t topk_scratch_ptr(void** out) {
  static unsigned char buf[256];
  *out = buf;
  return hipSuccess;
}
hipError_t launch_topk(const pkv_pool&, const int32_t*, int32_t, int32_t, const uint16_t*, int32_t, int32_t, int32_t,
                       int32_t, int32_t, int32_t*, void*, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
hipError_t launch_fwd(const AttnArgs&, const FwdPlan&, uint16_t*, float*, void*, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
hipError_t launch_mfma_probe(int32_t, int32_t, float*, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
double mfma_probe_flop(int32_t n_wg, int32_t iters) { return (double)n_wg * iters; }
hipError_t launch_atomic_probe(int32_t, int32_t, int32_t, float*, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
hipError_t launch_bwd(const AttnArgs&, const BwdExtra&, const BwdPlan&, void*, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}

}  // namespace pkv
