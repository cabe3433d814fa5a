// Diagnostic: a sustained bf16 MFMA loop, the reference against which the attention kernels'
// matrix rates are read (the clock under sustained MFMA load sits well below the one the
// datasheet peak assumes). Each wave keeps four independent 32x32 accumulators busy with
// v_mfma_f32_32x32x16_bf16 on operands filled with pseudo-random bf16 bits: the chip's power
// limit, and so its clock, depends on the data the MFMAs see. No memory traffic in the loop.
#include "pkv_device.h"

namespace pkv {

constexpr int kProbeThreads = 512;  // 8 waves: two per SIMD, like the forward and dQ kernels
constexpr int kProbeChains = 4;

// Finite bf16 bit pattern from a 32-bit hash: sign and mantissa random, exponent in [2^-8, 2^7].
__device__ __forceinline__ uint32_t probe_bits(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  const uint32_t lo = (x & 0x807fu) | ((119u + ((x >> 8) & 15u)) << 7);
  const uint32_t hi = ((x >> 16) & 0x807fu) | ((119u + ((x >> 24) & 15u)) << 7);
  return lo | (hi << 16);
}

__global__ __launch_bounds__(kProbeThreads) void k_mfma_probe(int32_t iters, float* __restrict__ out) {
  const uint32_t t = blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = probe_bits(t * 8u + (uint32_t)i);
    b[i] = probe_bits(t * 8u + 4u + (uint32_t)i);
  }
  const bf16x8 av = as_bf16x8(a), bv = as_bf16x8(b);
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = (f32x16){};
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = mfma32(av, bv, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[t] = s;
}

hipError_t launch_mfma_probe(int32_t n_wg, int32_t iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma_probe, dim3((unsigned)n_wg), dim3(kProbeThreads), 0, s, iters, out);
  return hipGetLastError();
}

double mfma_probe_flop(int32_t n_wg, int32_t iters) {
  return (double)n_wg * (kProbeThreads / 64) * (double)iters * kProbeChains * (32.0 * 32.0 * 16.0 * 2.0);
}

// Diagnostic: the rate of fp32 atomic adds into global memory, in the pattern a gradient flush
// makes: workgroup w adds 1.0 to every element of region w % n_regions, 256 threads striding over
// it, so consecutive lanes hit consecutive addresses. With n_regions equal to the workgroup count
// every element receives one add (the key-major dK/dV pass's single flush per gradient element);
// with fewer regions n_workgroups / n_regions workgroups add into each element (a query-major
// backward's per-row-block partials of one key tile).
constexpr int kAtomicProbeThreads = 256;

__global__ __launch_bounds__(kAtomicProbeThreads) void k_atomic_probe(float* __restrict__ buf, int32_t n_regions,
                                                                    int32_t region_elems) {
  float* r = buf + (int64_t)(blockIdx.x % (uint32_t)n_regions) * region_elems;
  for (int32_t i = threadIdx.x; i < region_elems; i += kAtomicProbeThreads) unsafeAtomicAdd(r + i, 1.0f);
}

hipError_t launch_atomic_probe(int32_t n_wg, int32_t n_regions, int32_t region_elems, float* buf, hipStream_t s) {
  hipLaunchKernelGGL(k_atomic_probe, dim3((unsigned)n_wg), dim3(kAtomicProbeThreads), 0, s, buf, n_regions,
                     region_elems);
  return hipGetLastError();
}

}  // namespace pkv
