// Host-side checks of the library's C ABI (pkv_abi.cpp) against the fake HIP runtime and stub
// launchers, built with the address and undefined-behaviour sanitizers (tests/test_abi_sanitized.py).
// What is checked: every entry point's argument errors and status codes, that a call failing
// validation enqueues nothing, allocation failure at every allocation of paged_kv_alloc (including
// the injected pinned-host failure) returning PKV_E_NOMEM with nothing left allocated, and the
// page free list. Test infrastructure only.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "../../include/pkv.h"

extern long g_stub_launches;
extern "C" {
void fake_hip_set_limit(size_t dev_bytes, size_t host_bytes);
void fake_hip_fail_nth(long dev_nth, long host_nth);
long fake_hip_live_device(void);
long fake_hip_live_host(void);
}

static int g_failures = 0;
static int g_checks = 0;

#define CHECK(cond)                                                                  \
  do {                                                                               \
    ++g_checks;                                                                      \
    if (!(cond)) {                                                                   \
      ++g_failures;                                                                  \
      std::fprintf(stderr, "%s:%d: check failed: %s (last error: %s)\n", __FILE__, __LINE__, #cond, \
                   pkv_last_error());                                                \
    }                                                                                \
  } while (0)

// The call fails with `code`, sets a message and enqueues nothing.
#define FAILS(code, call)                          \
  do {                                             \
    const long before_ = g_stub_launches;          \
    const int rc_ = (call);                        \
    CHECK(rc_ == (code));                          \
    CHECK(pkv_last_error()[0] != '\0');            \
    CHECK(g_stub_launches == before_);             \
  } while (0)

// The call succeeds and enqueues exactly `n` launches.
#define ENQUEUES(n, call)                          \
  do {                                             \
    const long before_ = g_stub_launches;          \
    const int rc_ = (call);                        \
    CHECK(rc_ == PKV_OK);                          \
    CHECK(pkv_last_error()[0] == '\0');            \
    CHECK(g_stub_launches == before_ + (n));       \
  } while (0)

static void check_alloc_errors() {
  pkv_pool* p = nullptr;
  FAILS(PKV_E_INVALID, paged_kv_alloc(nullptr, 4, 64, 1, 64, 0));
  FAILS(PKV_E_INVALID, paged_kv_alloc(&p, 0, 64, 1, 64, 0));
  FAILS(PKV_E_INVALID, paged_kv_alloc(&p, 4, 64, 0, 64, 0));
  FAILS(PKV_E_UNSUPPORTED, paged_kv_alloc(&p, 4, 96, 1, 64, 0));
  FAILS(PKV_E_UNSUPPORTED, paged_kv_alloc(&p, 4, 64, 1, 32, 0));
  FAILS(PKV_E_INVALID, paged_kv_alloc(&p, 4, 64, 1, 64, 0x80));
  FAILS(PKV_E_INVALID, paged_kv_alloc(&p, 4, 64, 1, 64, PKV_HOST_GRADS));
  CHECK(p == nullptr);
  CHECK(paged_kv_free(nullptr) == PKV_OK);
}

// Allocation failure at each allocation of paged_kv_alloc: PKV_E_NOMEM, no pool, nothing leaked.
static void check_alloc_failures() {
  const uint32_t flag_sets[] = {0u, PKV_GRADS, PKV_HOST_TIER | PKV_GRADS, PKV_HOST_TIER | PKV_GRADS | PKV_HOST_GRADS};
  for (uint32_t flags : flag_sets) {
    for (long nth = 1; nth <= 4; ++nth) {
      for (int host = 0; host < 2; ++host) {
        fake_hip_fail_nth(host ? -1 : nth, host ? nth : -1);
        pkv_pool* p = nullptr;
        const int rc = paged_kv_alloc(&p, 8, 64, 2, 64, flags);
        if (rc == PKV_OK) {  // this allocation index did not exist for these flags
          CHECK(p != nullptr);
          CHECK(paged_kv_free(p) == PKV_OK);
        } else {
          CHECK(rc == PKV_E_NOMEM);
          CHECK(p == nullptr);
        }
        CHECK(fake_hip_live_device() == 0);
        CHECK(fake_hip_live_host() == 0);
      }
    }
  }
  fake_hip_fail_nth(-1, -1);
  // A pool larger than the device can hold.
  fake_hip_set_limit(1 << 20, (size_t)-1);
  pkv_pool* p = nullptr;
  FAILS(PKV_E_NOMEM, paged_kv_alloc(&p, 64, 128, 4, 128, PKV_GRADS));
  CHECK(p == nullptr && fake_hip_live_device() == 0);
  fake_hip_set_limit((size_t)-1, (size_t)-1);
  // The injected pinned-host failure of a host-tier pool.
  setenv("PKV_FAIL_HOST_ALLOC", "1", 1);
  FAILS(PKV_E_NOMEM, paged_kv_alloc(&p, 8, 64, 2, 64, PKV_HOST_TIER));
  CHECK(p == nullptr && fake_hip_live_device() == 0 && fake_hip_live_host() == 0);
  CHECK(std::strstr(pkv_last_error(), "PKV_FAIL_HOST_ALLOC") != nullptr);
  // It applies to host-tier pools only.
  CHECK(paged_kv_alloc(&p, 8, 64, 2, 64, PKV_GRADS) == PKV_OK);
  CHECK(paged_kv_free(p) == PKV_OK);
  unsetenv("PKV_FAIL_HOST_ALLOC");
  CHECK(fake_hip_live_device() == 0 && fake_hip_live_host() == 0);
}

static void check_page_allocator() {
  pkv_pool* p = nullptr;
  CHECK(paged_kv_alloc(&p, 6, 64, 1, 64, PKV_GRADS) == PKV_OK);
  CHECK(paged_kv_pages_available(p) == 6);
  CHECK(paged_kv_pages_available(nullptr) == PKV_E_INVALID);
  int32_t got[8] = {-1, -1, -1, -1, -1, -1, -1, -1};
  CHECK(paged_kv_page_alloc(p, 0, nullptr) == PKV_OK);
  CHECK(paged_kv_page_alloc(p, 4, got) == PKV_OK);
  CHECK(got[0] == 0 && got[1] == 1 && got[2] == 2 && got[3] == 3);
  CHECK(paged_kv_pages_available(p) == 2);
  int32_t more[3] = {-1, -1, -1};
  FAILS(PKV_E_NOMEM, paged_kv_page_alloc(p, 3, more));  // 3 > 2 free: takes none
  CHECK(more[0] == -1 && paged_kv_pages_available(p) == 2);
  FAILS(PKV_E_INVALID, paged_kv_page_alloc(p, -1, more));
  FAILS(PKV_E_INVALID, paged_kv_page_alloc(p, 1, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_page_alloc(nullptr, 1, more));
  // Release: all or nothing.
  const int32_t rel_bad_range[2] = {1, 6};
  FAILS(PKV_E_INVALID, paged_kv_page_release(p, 2, rel_bad_range));
  const int32_t rel_free[2] = {1, 4};  // page 4 was never handed out
  FAILS(PKV_E_INVALID, paged_kv_page_release(p, 2, rel_free));
  const int32_t rel_twice[2] = {2, 2};
  FAILS(PKV_E_INVALID, paged_kv_page_release(p, 2, rel_twice));
  CHECK(paged_kv_pages_available(p) == 2);
  const int32_t rel[2] = {1, 3};
  CHECK(paged_kv_page_release(p, 2, rel) == PKV_OK);
  CHECK(paged_kv_pages_available(p) == 4);
  FAILS(PKV_E_INVALID, paged_kv_page_release(p, 1, rel));  // already free
  // Most recently released first, so a freed hole is reused before untouched pages.
  int32_t again[4] = {-1, -1, -1, -1};
  CHECK(paged_kv_page_alloc(p, 4, again) == PKV_OK);
  CHECK(again[0] == 3 && again[1] == 1 && again[2] == 4 && again[3] == 5);
  CHECK(paged_kv_pages_available(p) == 0);
  // Churn: every page allocated and released many times, never more than the pool.
  std::vector<int32_t> all(6);
  const int32_t live[6] = {0, 2, 3, 1, 4, 5};
  CHECK(paged_kv_page_release(p, 6, live) == PKV_OK);
  for (int it = 0; it < 100; ++it) {
    const int32_t n = 1 + it % 6;
    CHECK(paged_kv_page_alloc(p, n, all.data()) == PKV_OK);
    std::vector<int> seen(6, 0);
    for (int32_t i = 0; i < n; ++i) CHECK(all[i] >= 0 && all[i] < 6 && seen[all[i]]++ == 0);
    CHECK(paged_kv_page_release(p, n, all.data()) == PKV_OK);
    CHECK(paged_kv_pages_available(p) == 6);
  }
  CHECK(paged_kv_free(p) == PKV_OK);
}

static void check_compute_validation() {
  // A 64-token page, 2 KV heads, d = 64 pool with gradients; 16 pages.
  pkv_pool* p = nullptr;
  CHECK(paged_kv_alloc(&p, 16, 64, 2, 64, PKV_GRADS) == PKV_OK);
  pkv_pool* nog = nullptr;
  CHECK(paged_kv_alloc(&nog, 16, 64, 2, 64, 0) == PKV_OK);
  pkv_pool* host = nullptr;
  CHECK(paged_kv_alloc(&host, 16, 64, 2, 64, PKV_HOST_TIER | PKV_GRADS) == PKV_OK);
  pkv_pool* hg = nullptr;
  CHECK(paged_kv_alloc(&hg, 16, 64, 2, 64, PKV_HOST_TIER | PKV_GRADS | PKV_HOST_GRADS) == PKV_OK);
  pkv_pool* other = nullptr;
  CHECK(paged_kv_alloc(&other, 16, 128, 2, 64, PKV_GRADS) == PKV_OK);

  // Device-side buffers are never dereferenced by the host ABI; any aligned host memory serves.
  alignas(256) static uint16_t q[256 * 8 * 64], o[256 * 8 * 64], dout[256 * 8 * 64], dq[256 * 8 * 64];
  alignas(256) static float lse[8 * 256];
  alignas(256) static int32_t bt[16], sel[2 * 4 * 8];
  alignas(256) static unsigned char ws[1 << 22];
  const int32_t C = 256, Hq = 8, n_prior = 8, n_bt = 12;
  const float sc = 0.125f;
  const float nan = std::numeric_limits<float>::quiet_NaN(), inf = std::numeric_limits<float>::infinity();

  // Forward.
  const size_t fws = chunk_attn_fwd_ws_bytes(p, n_prior, -1, 1, 2, C, Hq);
  ENQUEUES(1, chunk_attn_fwd(p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, C, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  for (float bad : {0.f, -0.125f, nan, inf, -0.f})
    FAILS(PKV_E_INVALID, chunk_attn_fwd(p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, C, Hq, bad, o, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_fwd(nullptr, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, C, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_fwd(p, nullptr, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, C, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_fwd(p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q + 1, C, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_fwd(p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, 100, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_fwd(p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, C, 7, sc, o, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_RANGE, chunk_attn_fwd(p, bt, 11, n_prior, nullptr, 0, 1, 0, 2, q, C, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_fwd(p, bt, n_bt, -1, nullptr, 0, 1, 0, 2, q, C, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_fwd(p, bt, n_bt, n_prior, nullptr, 0, 1, 1, 2, q, C, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_fwd(p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 0, q, C, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_fwd(p, bt, n_bt, n_prior, nullptr, 0, 2, 0, 2, q, C, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_fwd(p, bt, n_bt, n_prior, sel, 9, 1, 0, 2, q, C, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_fwd(p, bt, n_bt, n_prior, sel, 4, 3, 0, 2, q, C, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  ENQUEUES(1, chunk_attn_fwd(p, bt, n_bt, n_prior, sel, 4, 4, 0, 2, q, C, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_fwd(p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, C, Hq, sc, nullptr, lse, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_STATE, chunk_attn_fwd(host, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, C, Hq, sc, o, lse, ws, sizeof(ws), nullptr));
  if (fws > 0) {
    FAILS(PKV_E_NOMEM, chunk_attn_fwd(p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, C, Hq, sc, o, lse, ws, fws - 1, nullptr));
    FAILS(PKV_E_NOMEM, chunk_attn_fwd(p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, C, Hq, sc, o, lse, nullptr, 0, nullptr));
  }

  // Backward.
  const size_t bws = chunk_attn_bwd_ws_bytes(p, n_prior, -1, 1, 2, C, Hq);
  CHECK(bws > 0);
  ENQUEUES(1, chunk_attn_bwd(p, bt, n_bt, p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, o, dout, lse, C, Hq, sc, dq, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_bwd(p, bt, n_bt, p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, o, dout, lse, C, Hq, 0.f, dq, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_bwd(p, bt, n_bt, nullptr, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, o, dout, lse, C, Hq, sc, dq, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_STATE, chunk_attn_bwd(p, bt, n_bt, nog, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, o, dout, lse, C, Hq, sc, dq, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_STATE, chunk_attn_bwd(p, bt, n_bt, hg, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, o, dout, lse, C, Hq, sc, dq, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_bwd(p, bt, n_bt, other, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, o, dout, lse, C, Hq, sc, dq, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_RANGE, chunk_attn_bwd(p, bt, n_bt, p, bt, 11, n_prior, nullptr, 0, 1, 0, 2, q, o, dout, lse, C, Hq, sc, dq, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_bwd(p, bt, n_bt, p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, o, nullptr, lse, C, Hq, sc, dq, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, chunk_attn_bwd(p, bt, n_bt, p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, o, dout, lse, C, Hq, sc, dq + 1, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_NOMEM, chunk_attn_bwd(p, bt, n_bt, p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, o, dout, lse, C, Hq, sc, dq, ws, bws - 1, nullptr));
  FAILS(PKV_E_NOMEM, chunk_attn_bwd(p, bt, n_bt, p, bt, n_bt, n_prior, nullptr, 0, 1, 0, 2, q, o, dout, lse, C, Hq, sc, dq, nullptr, 0, nullptr));

  // Selection.
  int32_t n_sel = -1;
  const size_t tws = page_topk_ws_bytes(p, n_prior, C, Hq, 1);
  ENQUEUES(1, page_topk_select(p, bt, n_bt, n_prior, q, C, Hq, 3, 1, 1, sel, &n_sel, ws, sizeof(ws), nullptr));
  CHECK(n_sel == 4);
  ENQUEUES(1, page_topk_select(p, bt, n_bt, n_prior, q, C, Hq, 30, 1, 1, sel, &n_sel, ws, sizeof(ws), nullptr));
  CHECK(n_sel == 8);  // every candidate is taken
  FAILS(PKV_E_INVALID, page_topk_select(p, bt, n_bt, n_prior, q, 96, Hq, 3, 1, 1, sel, &n_sel, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, page_topk_select(p, bt, n_bt, n_prior, q, C, 7, 3, 1, 1, sel, &n_sel, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_UNSUPPORTED, page_topk_select(p, bt, n_bt, n_prior, q, C, 2 * 129, 3, 1, 1, sel, &n_sel, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_RANGE, page_topk_select(p, bt, 7, n_prior, q, C, Hq, 3, 1, 1, sel, &n_sel, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, page_topk_select(p, bt, n_bt, n_prior, q, C, Hq, -1, 1, 1, sel, &n_sel, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, page_topk_select(p, bt, n_bt, n_prior, q, C, Hq, 3, 1, 3, sel, &n_sel, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_INVALID, page_topk_select(p, bt, n_bt, n_prior, q, C, Hq, 3, 1, 1, nullptr, &n_sel, ws, sizeof(ws), nullptr));
  FAILS(PKV_E_NOMEM, page_topk_select(p, bt, n_bt, n_prior, q, C, Hq, 3, 1, 1, sel, &n_sel, ws, tws - 1, nullptr));
  // The static-scratch variant: the same checks, and requests beyond its 16 MiB refused up front.
  n_sel = -1;
  ENQUEUES(1, page_topk_select_noalloc(p, bt, n_bt, n_prior, q, C, Hq, 3, 1, 1, sel, &n_sel, nullptr));
  CHECK(n_sel == 4);
  FAILS(PKV_E_INVALID, page_topk_select_noalloc(p, bt, n_bt, n_prior, q, 96, Hq, 3, 1, 1, sel, &n_sel, nullptr));
  FAILS(PKV_E_RANGE, page_topk_select_noalloc(p, bt, 7, n_prior, q, C, Hq, 3, 1, 1, sel, &n_sel, nullptr));
  FAILS(PKV_E_INVALID, page_topk_select_noalloc(p, bt, n_bt, n_prior, q, C, Hq, 3, 1, 1, nullptr, &n_sel, nullptr));
  FAILS(PKV_E_INVALID, page_topk_select_noalloc(nullptr, bt, n_bt, n_prior, q, C, Hq, 3, 1, 1, sel, &n_sel, nullptr));
  {
    // 2^17 chunk tokens of 64 query heads: the query partial sums alone exceed the scratch.
    alignas(256) static int32_t big_bt[1 << 12];
    FAILS(PKV_E_NOMEM, page_topk_select_noalloc(p, big_bt, 1 << 12, 1 << 12, q, 1 << 17, 64, 3, 1, 1, sel, &n_sel, nullptr));
    CHECK(std::strstr(pkv_last_error(), "scratch") != nullptr);
  }

  // Append, zeroing, export, check.
  ENQUEUES(1, paged_kv_append(p, bt, n_bt, 0, 128, q, o, nullptr));
  ENQUEUES(0, paged_kv_append(p, bt, n_bt, 64, 0, q, o, nullptr));
  FAILS(PKV_E_RANGE, paged_kv_append(p, bt, 2, 64, 128, q, o, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_append(p, bt, n_bt, -1, 1, q, o, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_append(p, bt, n_bt, 0, 64, q + 1, o, nullptr));
  ENQUEUES(1, paged_kv_zero_grad(p, nullptr, 0, nullptr));
  ENQUEUES(1, paged_kv_zero_grad(p, bt, 4, nullptr));
  FAILS(PKV_E_STATE, paged_kv_zero_grad(nog, nullptr, 0, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_zero_grad(p, bt, -1, nullptr));
  ENQUEUES(1, paged_kv_export(p, PKV_REP, bt, n_bt, 0, 2, ws, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_export(p, 9, bt, n_bt, 0, 2, ws, nullptr));
  FAILS(PKV_E_STATE, paged_kv_export(nog, PKV_DK, bt, n_bt, 0, 2, ws, nullptr));
  FAILS(PKV_E_RANGE, paged_kv_export(p, PKV_K, bt, n_bt, 11, 2, ws, nullptr));
  CHECK(paged_kv_check(p) == PKV_OK);

  // Host tier: gather and gradient offload.
  ENQUEUES(1, paged_kv_gather(host, p, bt, n_bt, sel, 4, 1, bt, nullptr, 0, 0, nullptr));
  FAILS(PKV_E_STATE, paged_kv_gather(p, p, bt, n_bt, sel, 4, 1, bt, nullptr, 0, 0, nullptr));
  FAILS(PKV_E_STATE, paged_kv_gather(host, host, bt, n_bt, sel, 4, 1, bt, nullptr, 0, 0, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_gather(host, p, bt, n_bt, sel, 4, 2, bt, nullptr, 0, 0, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_gather(host, other, bt, n_bt, sel, 4, 0, bt, nullptr, 0, 0, nullptr));
  ENQUEUES(1, paged_kv_gather(host, p, bt, n_bt, sel, 4, 1, bt, nullptr, 0, 64, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_gather(host, p, bt, n_bt, sel, 4, 1, bt, nullptr, 0, -1, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_gather(host, p, bt, n_bt, sel, 4, 1, bt, nullptr, 0, 65, nullptr));
  ENQUEUES(1, paged_kv_grad_offload(hg, bt, n_bt, p, bt, n_bt, sel, 4, 0, 2, nullptr));
  FAILS(PKV_E_STATE, paged_kv_grad_offload(host, bt, n_bt, p, bt, n_bt, sel, 4, 0, 2, nullptr));
  FAILS(PKV_E_STATE, paged_kv_grad_offload(hg, bt, n_bt, nog, bt, n_bt, sel, 4, 0, 2, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_grad_offload(hg, bt, n_bt, p, bt, n_bt, sel, 4, 1, 2, nullptr));

  // Page copies go to the copy engine (hipMemcpyAsync), never to a kernel.
  ENQUEUES(0, paged_kv_copy(hg, p, PKV_COPY_KV | PKV_COPY_GRAD, 0, 16, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_copy(p, p, PKV_COPY_KV, 0, 1, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_copy(hg, p, PKV_COPY_KV, 10, 7, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_copy(hg, p, 4u, 0, 1, nullptr));
  FAILS(PKV_E_STATE, paged_kv_copy(hg, nog, PKV_COPY_GRAD, 0, 1, nullptr));

  FAILS(PKV_E_INVALID, pkv_mfma_probe(0, 1, lse, nullptr, nullptr));
  double nbytes = 0.0;
  ENQUEUES(1, pkv_atomic_probe(8, 2, 64, lse, &nbytes, nullptr));
  CHECK(nbytes == 8.0 * 64 * 4);
  FAILS(PKV_E_INVALID, pkv_atomic_probe(8, 9, 64, lse, nullptr, nullptr));
  FAILS(PKV_E_INVALID, pkv_atomic_probe(8, 2, 0, lse, nullptr, nullptr));
  FAILS(PKV_E_INVALID, pkv_atomic_probe(8, 2, 64, nullptr, nullptr, nullptr));

  for (pkv_pool* x : {p, nog, host, hg, other}) CHECK(paged_kv_free(x) == PKV_OK);
  CHECK(fake_hip_live_device() == 0 && fake_hip_live_host() == 0);
}

// The staged gradient offload: a rectangular copy of one head's device blocks to staging, the
// device blocks cleared, and the host threads' adds into the host pages the staged ids name.
static void check_staged_offload() {
  const int32_t NP = 16, P = 64, H = 2, D = 64, blk = 2 * P * D;
  pkv_pool* dev = nullptr;
  pkv_pool* hg = nullptr;
  pkv_pool* ho = nullptr;
  CHECK(paged_kv_alloc(&dev, NP, P, H, D, PKV_GRADS) == PKV_OK);
  CHECK(paged_kv_alloc(&hg, NP, P, H, D, PKV_HOST_TIER | PKV_GRADS | PKV_HOST_GRADS) == PKV_OK);
  CHECK(paged_kv_alloc(&ho, NP, P, H, D, PKV_HOST_TIER | PKV_GRADS) == PKV_OK);
  float* dg = static_cast<float*>(paged_kv_data(dev, PKV_DK));
  float* hgr = static_cast<float*>(paged_kv_data(hg, PKV_DK));  // the fake maps host memory 1:1
  for (int32_t pg = 0; pg < NP; ++pg)
    for (int32_t g = 0; g < H; ++g)
      for (int32_t k = 0; k < blk; ++k) dg[((size_t)pg * H + g) * blk + k] = 1000.f * pg + 100.f * g + (float)(k % 7);
  int32_t host_bt[NP];
  for (int32_t i = 0; i < NP; ++i) host_bt[i] = (i * 5 + 3) % NP;  // a permutation
  alignas(256) static int32_t lp[3] = {3, 7, 11};
  const size_t need = paged_kv_grad_staging_bytes(dev, 3);
  CHECK(need == 256 + 3 * (size_t)blk * 4);
  void* stg = nullptr;
  CHECK(hipHostMalloc(&stg, need, 0) == hipSuccess);
  for (int rep = 1; rep <= 2; ++rep) {
    if (rep == 2)  // refill the device blocks the first stage cleared
      for (int32_t i = 0; i < 3; ++i)
        for (int32_t k = 0; k < blk; ++k) dg[((size_t)(2 + i) * H + 1) * blk + k] = 1000.f * (2 + i) + 100.f + (float)(k % 7);
    ENQUEUES(1, paged_kv_grad_stage(dev, 2, 3, 1, lp, stg, need, nullptr));
    ENQUEUES(0, paged_kv_grad_accumulate(hg, host_bt, NP, 3, 1, stg, nullptr));
    bool ok_host = true, ok_dev = true, ok_rest = true;
    for (int32_t i = 0; i < 3; ++i)
      for (int32_t k = 0; k < blk; ++k) {
        const float want = rep * (1000.f * (2 + i) + 100.f + (float)(k % 7));
        ok_host &= hgr[((size_t)host_bt[lp[i]] * H + 1) * blk + k] == want;
        ok_dev &= dg[((size_t)(2 + i) * H + 1) * blk + k] == 0.f;
        ok_rest &= dg[((size_t)(2 + i) * H + 0) * blk + k] == 1000.f * (2 + i) + (float)(k % 7);
      }
    CHECK(ok_host);
    CHECK(ok_dev);
    CHECK(ok_rest);
  }
  double other = 0.0;  // host blocks nobody staged stay zero
  for (int32_t pg = 0; pg < NP; ++pg)
    for (int32_t g = 0; g < H; ++g) {
      const bool staged = g == 1 && (pg == host_bt[3] || pg == host_bt[7] || pg == host_bt[11]);
      if (!staged)
        for (int32_t k = 0; k < blk; ++k) other += std::fabs(hgr[((size_t)pg * H + g) * blk + k]);
    }
  CHECK(other == 0.0);
  CHECK(paged_kv_check(hg) == PKV_OK);
  // A staged id outside the host table is skipped and reported.
  alignas(256) static int32_t bad_lp[1] = {99};
  ENQUEUES(1, paged_kv_grad_stage(dev, 0, 1, 0, bad_lp, stg, need, nullptr));
  ENQUEUES(0, paged_kv_grad_accumulate(hg, host_bt, NP, 1, 0, stg, nullptr));
  CHECK(paged_kv_check(hg) == PKV_E_DEVICE);
  CHECK(paged_kv_check(hg) == PKV_OK);
  // Argument errors: nothing enqueued.
  FAILS(PKV_E_NOMEM, paged_kv_grad_stage(dev, 2, 3, 1, lp, stg, need - 1, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_grad_stage(dev, 14, 3, 1, lp, stg, need, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_grad_stage(dev, 2, 3, 2, lp, stg, need, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_grad_stage(dev, 2, 3, 1, nullptr, stg, need, nullptr));
  FAILS(PKV_E_STATE, paged_kv_grad_stage(hg, 2, 3, 1, lp, stg, need, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_grad_stage(nullptr, 2, 3, 1, lp, stg, need, nullptr));
  FAILS(PKV_E_STATE, paged_kv_grad_accumulate(ho, host_bt, NP, 3, 1, stg, nullptr));
  FAILS(PKV_E_STATE, paged_kv_grad_accumulate(dev, host_bt, NP, 3, 1, stg, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_grad_accumulate(hg, host_bt, NP, 3, 2, stg, nullptr));
  FAILS(PKV_E_INVALID, paged_kv_grad_accumulate(hg, nullptr, NP, 3, 1, stg, nullptr));
  CHECK(paged_kv_grad_staging_bytes(nullptr, 3) == 0);
  CHECK(hipHostFree(stg) == hipSuccess);
  for (pkv_pool* x : {dev, hg, ho}) CHECK(paged_kv_free(x) == PKV_OK);
  CHECK(fake_hip_live_device() == 0 && fake_hip_live_host() == 0);
}

int main() {
  CHECK(pkv_version() > 0);
  check_alloc_errors();
  check_alloc_failures();
  check_page_allocator();
  check_compute_validation();
  check_staged_offload();
  std::printf("%d checks, %d failed\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
