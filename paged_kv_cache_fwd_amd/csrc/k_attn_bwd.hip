// Chunk attention backward over the paged KV cache, bf16 MFMA (gfx950).
//
// "Out of the Memory Barrier" summaries: pt 2.A / es 2.A / it 2.A (what the forward dropped is
// recomputed in backward: here the probabilities, from the stored log-sum-exp), pt 2.B / es 2.B /
// it 2.B (custom kernels add the key/value gradients in place into gradient pages, outside
// autograd, with atomic adds).
//
// Kernels here:
//  k_bwd_rowdot  per (head, token): -D with D = rowsum(dO * O), lse * log2 e, -lse / scale.
//  k_bwd_dq      query-major, workgroups of 8 (or 4) waves like the forward: each wave keeps dQ^T
//                for 32 rows in registers while walking the key list (S^T = K Q^T, P^T = exp(S^T - LSE), dP^T = V dO^T, dS^T = P^T (dP^T - D),
//                dQ^T += K^T dS^T). Split over key ranges like the forward; partials (fp32) are
//                summed by k_bwd_dq_reduce.
// The key-major dK/dV pass (k_attn_dkdv.hip) keeps dK/dV of its keys on chip for all rows and
// adds them to the gradient pages with one fp32 atomic add per element.
// Splitting the backward this way recomputes S and dP once more than a fused kernel, but keeps
// every partial sum on chip: a fused query-major kernel would stream one fp32 dK/dV partial per
// 256 query rows through global atomics, about 120 GB at a 256K context.
#include <cstdlib>
#include <cstring>

#include "pkv_device.h"

namespace pkv {

// ---------------------------------------------------------------------------------------------
// Row values of the backward for the query heads of KV heads [kvh0, kvh0 + n_kvh): -D with
// D[h][t] = sum_d dO[t][h][d] * O[t][h][d], lse * log2 e (dQ pass) and -lse / scale (dK/dV pass,
// which accumulates S onto it). Entries [pad_row, pad_row + 64) of -D and -lse/scale hold 0 and
// -inf: rows past the end of the chunk read them.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_rowdot(AttnArgs a, const uint16_t* __restrict__ o,
                                                    const uint16_t* __restrict__ dout, const float* __restrict__ lse,
                                                    float* __restrict__ ndbuf, float* __restrict__ lse2buf,
                                                    float* __restrict__ nlsbuf, int32_t pad_row) {
  const int32_t nh = a.n_kvh * a.G;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < 64) {
    ndbuf[pad_row + idx] = 0.f;
    nlsbuf[pad_row + idx] = -INFINITY;
  }
  if (idx >= (int64_t)a.C * nh) return;
  const int32_t h = a.kvh0 * a.G + (int32_t)(idx % nh);
  const int32_t t = (int32_t)(idx / nh);
  const u32x4* op = reinterpret_cast<const u32x4*>(o + ((int64_t)t * a.h_q + h) * D);
  const u32x4* dp = reinterpret_cast<const u32x4*>(dout + ((int64_t)t * a.h_q + h) * D);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const u32x4 x = op[c], y = dp[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc += __uint_as_float(x[j] << 16) * __uint_as_float(y[j] << 16);
      acc += __uint_as_float(x[j] & 0xffff0000u) * __uint_as_float(y[j] & 0xffff0000u);
    }
  }
  ndbuf[(int64_t)h * a.C + t] = -acc;
  const float lv = lse[(int64_t)h * a.C + t];
  lse2buf[(int64_t)h * a.C + t] = lv * kLog2e;
  nlsbuf[(int64_t)h * a.C + t] = -lv / a.scale;
}

// ---------------------------------------------------------------------------------------------
template <int D, int NWAVES>
struct DqCfg {
  static constexpr int NW = NWAVES;                  // waves per workgroup (32 rows each)
  static constexpr int BK = 64;                      // keys per tile
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int CHR = D / 8;
  static constexpr int TILE = BK * D;                // elements of one K or V tile
  static constexpr int SEG_PER_WAVE = TILE * 2 / 1024 / NW;
  static constexpr int ROWS_PER_SEG = 1024 / (2 * D);
};

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_dq(
    AttnArgs a, BwdExtra e, int32_t n_rb, int32_t splits, const float* __restrict__ ndbuf,
    const float* __restrict__ lse2buf, float* __restrict__ ws_dq) {
  using T = DqCfg<D, NW>;
  constexpr int BK = T::BK;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * 2 * T::TILE];  // [stage][K|V]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lg = lane >> 5, l32 = lane & 31;
  const int32_t n_units = a.n_kvh * splits * n_rb;
  const int32_t u = xcd_remap(blockIdx.x, n_units);
  // Row blocks run last to first within each (split, KV head): later rows see more of the chunk's
  // own keys, so the longest workgroups are dispatched first and the short ones fill the tail.
  const int32_t rb = n_rb - 1 - u % n_rb;
  const int32_t sp = (u / n_rb) % splits;
  const int32_t gi = u / (n_rb * splits);
  const int32_t g = a.kvh0 + gi;
  const int32_t G = a.G, CG = a.C * G, P = a.page;
  // Row blocks never straddle two selection lists: list li owns rows [li*RL, (li+1)*RL).
  const int32_t RL = CG / a.n_lists;
  const int32_t bpl = (RL + 32 * T::NW - 1) / (32 * T::NW);
  const int32_t li = rb / bpl;
  const int32_t r0 = li * RL + (rb - li * bpl) * 32 * T::NW;
  const int32_t r_end = min(r0 + 32 * T::NW, (li + 1) * RL);
  const int32_t r_last = r_end - 1;
  const int32_t t_min = r0 / G, t_max = r_last / G;
  const int32_t q0 = a.n_prior * P;
  const int tsh = (P == 128) ? 1 : 0;  // log2(64-key tiles per page)
  const int32_t n_prior_tiles = list_prior(a) << tsh;
  const int32_t n_tiles = n_prior_tiles + t_max / BK + 1;
  const int32_t tb = (int32_t)((int64_t)n_tiles * sp / splits);
  const int32_t te = (int32_t)((int64_t)n_tiles * (sp + 1) / splits);

  const int32_t row = r0 + wave * 32 + l32;
  const bool rvalid = row < r_end;
  const int32_t rr = rvalid ? row : r_last;
  const int32_t tq = rr / G;
  const int32_t h = g * G + (rr - tq * G);
  bf16x8 qreg[T::KS], doreg[T::KS];
  {
    const int64_t off = ((int64_t)tq * a.h_q + h) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      u32x4 x = *reinterpret_cast<const u32x4*>(a.q + off + ks * 16);
      u32x4 y = *reinterpret_cast<const u32x4*>(e.dout + off + ks * 16);
      if (!rvalid) {
        x = (u32x4){0u, 0u, 0u, 0u};
        y = (u32x4){0u, 0u, 0u, 0u};
      }
      qreg[ks] = as_bf16x8(x);
      doreg[ks] = as_bf16x8(y);
    }
  }
  const int64_t si = (int64_t)h * a.C + tq;
  const float lse2 = rvalid ? lse2buf[si] : INFINITY;
  const float ndval = rvalid ? ndbuf[si] : 0.f;

  // Tiles of the key list in order, with their table reads issued a tile ahead.
  KeyWalk walk = walk_begin(a, g, li, tsh, tb, te);
  int32_t seg_off[T::SEG_PER_WAVE];
#pragma unroll
  for (int j = 0; j < T::SEG_PER_WAVE; ++j) {
    const int rl = (wave * T::SEG_PER_WAVE + j) * T::ROWS_PER_SEG + lane / T::CHR;
    seg_off[j] = rl * D + (((lane % T::CHR) ^ swz<D>(rl)) << 3);
  }
  // Stage the walk's next tile (kp: its first key position, -1 when unreadable).
  auto load_tile = [&](int stage, int32_t& kp) {
    const uint16_t* src = walk_take<D>(a, walk, kp);
    if (src == nullptr) src = a.kv;  // unreadable page: any in-bounds bytes, the tile is masked
    uint16_t* kt = lds + stage * 2 * T::TILE;
#pragma unroll
    for (int j = 0; j < T::SEG_PER_WAVE; ++j) {
      const int seg = wave * T::SEG_PER_WAVE + j;
      g2lds16(src + seg_off[j], kt + seg * 512);
      g2lds16(src + (int64_t)P * D + seg_off[j], kt + T::TILE + seg * 512);
    }
  };

  // Loop-invariant LDS byte offsets of this lane's MFMA operands within a stage. The swizzle of a
  // tile row depends only on the row's low four bits, which the 32-key half (k2) and the 16-key
  // step (hf) never change, so every operand address is one of these plus a constant.
  uint32_t koff[T::KS];     // K and V rows l32, columns 16 ks + 8 lg
  uint32_t toff_t[T::DT][2];  // K^T: rows 4 lg + rr (+8), columns 32 dt + 16 b4 + 4 (lane%4)
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) koff[ks] = 2u * (uint32_t)toff<D>(l32, ks * 16 + 8 * lg);
  {
    const int rr = (lane & 15) >> 2, cb = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) toff_t[dt][kh] = 2u * (uint32_t)toff<D>(4 * lg + rr + 8 * kh, dt * 32 + cb);
  }

  const float sl2 = a.scale * kLog2e;
  f32x16 dq[T::DT];
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) dq[dt] = (f32x16){};

  int32_t kpos_next = -1;
  if (tb < te) load_tile(0, kpos_next);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int32_t i = tb; i < te; ++i) {
    const int cur = (i - tb) & 1;
    const int32_t kpos_t = kpos_next;
    if (i + 1 < te) load_tile(cur ^ 1, kpos_next);
    const char* kt = reinterpret_cast<const char*>(lds + cur * 2 * T::TILE);
    const char* vt = kt + 2 * T::TILE;
    const bool bad = kpos_t < 0;
    const bool need_mask = bad || (kpos_t + BK - 1 > q0 + t_min);
    const int32_t lim = q0 + tq;

    // The two 32-key halves of the tile run one after the other to bound register use.
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      f32x16 sacc = (f32x16){}, pacc = (f32x16){};
      __builtin_amdgcn_s_setprio(1);
      // The K and V operands of k-step ks + 1 are read while the MFMAs of ks run.
      bf16x8 ka[2], va[2];
      ka[0] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + koff[0] + k2 * 32 * D * 2));
      va[0] = as_bf16x8(*reinterpret_cast<const u32x4*>(vt + koff[0] + k2 * 32 * D * 2));
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        if (ks + 1 < T::KS) {
          const uint32_t off = koff[ks + 1] + k2 * 32 * D * 2;
          ka[(ks + 1) & 1] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + off));
          va[(ks + 1) & 1] = as_bf16x8(*reinterpret_cast<const u32x4*>(vt + off));
        }
        sacc = mfma32(ka[ks & 1], qreg[ks], sacc);
        pacc = mfma32(va[ks & 1], doreg[ks], pacc);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        if (ks + 1 < T::KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      float p[16];
#pragma unroll
      for (int el = 0; el < 16; ++el) p[el] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[el], sl2, -lse2));
      if (need_mask) {
#pragma unroll
        for (int el = 0; el < 16; ++el) {
          const int32_t key = kpos_t + k2 * 32 + 8 * (el >> 2) + 4 * lg + (el & 3);
          if (bad || key > lim) p[el] = 0.f;
        }
      }
      bf16x8 dsb[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int el = hf * 8 + 2 * j;
          w[j] = cvt_pk_bf16(p[el] * (pacc[el] + ndval), p[el + 1] * (pacc[el + 1] + ndval));
        }
        dsb[hf] = as_bf16x8(w);
      }
      // dQ^T[dt] += K^T[dt rows][16 keys] dS^T[16 keys]
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int rowb = (k2 * 32 + hf * 16) * D * 2;  // bytes
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
          const u32x2 lo = lds_tr16(reinterpret_cast<const uint16_t*>(kt + toff_t[dt][0] + rowb));
          const u32x2 hi = lds_tr16(reinterpret_cast<const uint16_t*>(kt + toff_t[dt][1] + rowb));
          const bf16x8 kta = as_bf16x8((u32x4){lo[0], lo[1], hi[0], hi[1]});
          dq[dt] = mfma32(kta, dsb[hf], dq[dt]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (!rvalid) return;
  if (splits == 1) {
    uint16_t* dp = e.dq + ((int64_t)tq * a.h_q + h) * D;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        u32x2 w;
        w[0] = cvt_pk_bf16(dq[dt][grp * 4 + 0] * a.scale, dq[dt][grp * 4 + 1] * a.scale);
        w[1] = cvt_pk_bf16(dq[dt][grp * 4 + 2] * a.scale, dq[dt][grp * 4 + 3] * a.scale);
        *reinterpret_cast<u32x2*>(dp + dt * 32 + grp * 8 + 4 * lg) = w;
      }
  } else {
    const int64_t rows_total = (int64_t)a.n_kvh * CG;
    float* wp = ws_dq + ((int64_t)sp * rows_total + (int64_t)gi * CG + row) * D;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = dq[dt][grp * 4 + j];
        *reinterpret_cast<f32x4*>(wp + dt * 32 + grp * 8 + 4 * lg) = w;
      }
  }
}

// Sum the dQ partials of all splits, scale, round to bf16.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_dq_reduce(AttnArgs a, int32_t splits, const float* __restrict__ ws_dq,
                                                       uint16_t* __restrict__ dq) {
  const int32_t G = a.G, CG = a.C * G;
  const int64_t rows_total = (int64_t)a.n_kvh * CG;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows_total * (D / 8)) return;
  const int32_t dc = (int32_t)(idx % (D / 8));
  const int64_t R = idx / (D / 8);
  const int32_t gi = (int32_t)(R / CG), r = (int32_t)(R % CG);
  const int32_t t = r / G, h = (a.kvh0 + gi) * G + (r - (r / G) * G);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    const f32x4* src = reinterpret_cast<const f32x4*>(ws_dq + ((int64_t)s * rows_total + R) * D + dc * 8);
    const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] += x0[j];
      acc[4 + j] += x1[j];
    }
  }
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = cvt_pk_bf16(acc[2 * j] * a.scale, acc[2 * j + 1] * a.scale);
  *reinterpret_cast<u32x4*>(dq + ((int64_t)t * a.h_q + h) * D + dc * 8) = out;
}

template <int D>
static hipError_t launch_bwd_d(const AttnArgs& a, const BwdExtra& e, const BwdPlan& plan, void* ws, hipStream_t s) {
  const int64_t rows_total = (int64_t)a.n_kvh * a.C * a.G;
  const size_t nrow = ((size_t)a.h_q * a.C + 63) & ~(size_t)63;  // + 64 padding entries each
  float* ndbuf = (float*)ws;            // [H_q][C] -D
  float* lse2buf = ndbuf + nrow + 64;   // [H_q][C] lse * log2 e
  float* nlsbuf = lse2buf + nrow + 64;  // [H_q][C] -lse / scale
  float* ws_dq = nlsbuf + nrow + 64;
  {
    const int64_t work = (int64_t)a.C * a.n_kvh * a.G;
    TimerScope ts_("k_bwd_rowdot", s);
    hipLaunchKernelGGL(k_bwd_rowdot<D>, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, a, e.o, e.dout,
                       e.lse, ndbuf, lse2buf, nlsbuf, (int32_t)nrow);
  }
  {
    const int32_t n_units = a.n_kvh * plan.splits * plan.n_rb;
    if (plan.dq_nw == 8 && dq_one_wave_per_simd()) {
      TimerScope ts_("k_bwd_dq64", s);
      const hipError_t err = launch_dq64<D>(a, e, plan.n_rb, plan.splits, ndbuf, lse2buf, ws_dq, s);
      if (err != hipSuccess) return err;
    } else {
      TimerScope ts_("k_bwd_dq", s);
      if (plan.dq_nw == 8)
        hipLaunchKernelGGL((k_bwd_dq<D, 8>), dim3(n_units), dim3(64 * 8), 0, s, a, e, plan.n_rb, plan.splits, ndbuf,
                           lse2buf, ws_dq);
      else
        hipLaunchKernelGGL((k_bwd_dq<D, 4>), dim3(n_units), dim3(64 * 4), 0, s, a, e, plan.n_rb, plan.splits, ndbuf,
                           lse2buf, ws_dq);
    }
    if (plan.splits > 1) {
      const int64_t work = rows_total * (D / 8);
      TimerScope ts_("k_bwd_dq_reduce", s);
      hipLaunchKernelGGL(k_bwd_dq_reduce<D>, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, a, plan.splits,
                         ws_dq, e.dq);
    }
  }
  {
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return launch_dkdv<D>(a, e, plan, ndbuf, nlsbuf, (int32_t)nrow, s);
}

bool dq_one_wave_per_simd() {
  static const bool v = [] {
    const char* e = getenv("PKV_DQ_KERNEL");
    return !(e && strcmp(e, "w8") == 0);
  }();
  return v;
}

hipError_t launch_bwd(const AttnArgs& a, const BwdExtra& e, const BwdPlan& plan, void* ws, hipStream_t s) {
  if (a.d == 128) return launch_bwd_d<128>(a, e, plan, ws, s);
  return launch_bwd_d<64>(a, e, plan, ws, s);
}

}  // namespace pkv
