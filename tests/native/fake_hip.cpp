// A host-only stand-in for the HIP runtime calls the library's host ABI (pkv_abi.cpp) makes, so
// that pool management and argument validation can run on a machine without a GPU, under the
// address and undefined-behaviour sanitizers. Test infrastructure only.
//
// "Device" and pinned "host" allocations are plain host allocations. Every allocation is tracked,
// so the checks can assert that a failed call left nothing behind. Failures are injected by
// size (fake_hip_set_limit) or by count (fake_hip_fail_nth).
#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>

namespace {
std::mutex g_mu;
std::map<void*, size_t> g_dev, g_host;
size_t g_dev_limit = (size_t)-1, g_host_limit = (size_t)-1;
long g_fail_nth_dev = -1, g_fail_nth_host = -1;  // 1-based index of the next call to fail
long g_n_dev = 0, g_n_host = 0;
hipError_t g_last = hipSuccess;

bool fail_now(long& nth, long& count) {
  ++count;
  if (nth > 0 && count == nth) {
    nth = -1;
    return true;
  }
  return false;
}
}  // namespace

extern "C" {

// Controls and counters for the checks.
void fake_hip_set_limit(size_t dev_bytes, size_t host_bytes) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_dev_limit = dev_bytes;
  g_host_limit = host_bytes;
}
void fake_hip_fail_nth(long dev_nth, long host_nth) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_fail_nth_dev = dev_nth;
  g_fail_nth_host = host_nth;
  g_n_dev = 0;
  g_n_host = 0;
}
long fake_hip_live_device(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  return (long)g_dev.size();
}
long fake_hip_live_host(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  return (long)g_host.size();
}

hipError_t hipGetDevice(int* deviceId) {
  if (!deviceId) return hipErrorInvalidValue;
  *deviceId = 0;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* pi, hipDeviceAttribute_t attr, int deviceId) {
  (void)deviceId;
  if (!pi) return hipErrorInvalidValue;
  *pi = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return hipSuccess;
}

hipError_t hipMalloc(void** ptr, size_t size) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!ptr) return hipErrorInvalidValue;
  *ptr = nullptr;
  if (size > g_dev_limit || fail_now(g_fail_nth_dev, g_n_dev)) return g_last = hipErrorOutOfMemory;
  void* p = std::malloc(size ? size : 1);
  if (!p) return g_last = hipErrorOutOfMemory;
  g_dev[p] = size;
  *ptr = p;
  return hipSuccess;
}

hipError_t hipFree(void* ptr) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!ptr) return hipSuccess;
  auto it = g_dev.find(ptr);
  if (it == g_dev.end()) std::abort();  // freeing something that is not a device allocation
  g_dev.erase(it);
  std::free(ptr);
  return hipSuccess;
}

hipError_t hipHostMalloc(void** ptr, size_t size, unsigned int flags) {
  (void)flags;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!ptr) return hipErrorInvalidValue;
  *ptr = nullptr;
  if (size > g_host_limit || fail_now(g_fail_nth_host, g_n_host)) return g_last = hipErrorOutOfMemory;
  void* p = std::malloc(size ? size : 1);
  if (!p) return g_last = hipErrorOutOfMemory;
  g_host[p] = size;
  *ptr = p;
  return hipSuccess;
}

hipError_t hipHostFree(void* ptr) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!ptr) return hipSuccess;
  auto it = g_host.find(ptr);
  if (it == g_host.end()) std::abort();  // freeing something that is not a pinned host allocation
  g_host.erase(it);
  std::free(ptr);
  return hipSuccess;
}

hipError_t hipHostGetDevicePointer(void** devPtr, void* hstPtr, unsigned int flags) {
  (void)flags;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!devPtr || g_host.find(hstPtr) == g_host.end()) return hipErrorInvalidValue;
  *devPtr = hstPtr;
  return hipSuccess;
}

static bool in_block(const std::map<void*, size_t>& m, const void* p, size_t n) {
  auto it = m.upper_bound(const_cast<void*>(p));
  if (it == m.begin()) return false;
  --it;
  const char* b = (const char*)it->first;
  return (const char*)p >= b && (const char*)p + n <= b + it->second;
}

hipError_t hipMemset(void* dst, int value, size_t sizeBytes) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!in_block(g_dev, dst, sizeBytes)) std::abort();
  std::memset(dst, value, sizeBytes);
  return hipSuccess;
}

hipError_t hipMemcpy(void* dst, const void* src, size_t sizeBytes, hipMemcpyKind kind) {
  (void)kind;
  std::memcpy(dst, src, sizeBytes);
  return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t sizeBytes, hipMemcpyKind kind, hipStream_t stream) {
  (void)kind;
  (void)stream;
  std::memcpy(dst, src, sizeBytes);
  return hipSuccess;
}

hipError_t hipMemcpy2DAsync(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height,
                             hipMemcpyKind kind, hipStream_t stream) {
  (void)kind;
  (void)stream;
  if (width > dpitch || width > spitch) return hipErrorInvalidValue;
  for (size_t r = 0; r < height; ++r)
    std::memcpy((char*)dst + r * dpitch, (const char*)src + r * spitch, width);
  return hipSuccess;
}

// Host functions run at once: with no device work pending, stream order is call order.
hipError_t hipLaunchHostFunc(hipStream_t stream, hipHostFn_t fn, void* userData) {
  (void)stream;
  fn(userData);
  return hipSuccess;
}

hipError_t hipDeviceSynchronize(void) { return hipSuccess; }

hipError_t hipGetLastError(void) {
  const hipError_t e = g_last;
  g_last = hipSuccess;
  return e;
}

const char* hipGetErrorString(hipError_t hipError) {
  return hipError == hipSuccess ? "no error" : hipError == hipErrorOutOfMemory ? "out of memory" : "fake HIP error";
}

hipError_t hipEventCreate(hipEvent_t* event) {
  if (!event) return hipErrorInvalidValue;
  *event = (hipEvent_t)std::malloc(16);
  return hipSuccess;
}

hipError_t hipEventRecord(hipEvent_t event, hipStream_t stream) {
  (void)event;
  (void)stream;
  return hipSuccess;
}

hipError_t hipEventSynchronize(hipEvent_t event) {
  (void)event;
  return hipSuccess;
}

hipError_t hipEventElapsedTime(float* ms, hipEvent_t start, hipEvent_t stop) {
  (void)start;
  (void)stop;
  if (ms) *ms = 0.f;
  return hipSuccess;
}

}  // extern "C"
