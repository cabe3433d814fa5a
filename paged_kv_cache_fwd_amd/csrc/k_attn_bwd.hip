// Chunk attention backward over the paged KV cache, bf16 MFMA (gfx950).
//
// "Out of the Memory Barrier" summaries: pt 2.A / es 2.A / it 2.A (what the forward dropped is
// recomputed in backward: here the probabilities, from the stored log-sum-exp), pt 2.B / es 2.B /
// it 2.B (custom kernels add the key/value gradients in place into gradient pages, outside
// autograd, with atomic adds).
//
// Three kernels:
//  k_bwd_rowdot  D = rowsum(dO * O) per (head, token), fp32.
//  k_bwd_dq      query-major: each wave keeps dQ^T for 64 rows in registers while walking the key
//                list (S^T = K Q^T, P^T = exp(S^T - LSE), dP^T = V dO^T, dS^T = P^T (dP^T - D),
//                dQ^T += K^T dS^T). Split over key ranges like the forward; partials (fp32) are
//                summed by k_bwd_dq_reduce.
//  k_bwd_dkdv    key-major: each wave owns 32 keys (K, V in registers, dK/dV accumulators in
//                registers) and walks all rows of the chunk's query heads in 64-row blocks staged
//                in LDS (Q, dO row-major and transposed). The finished dK/dV are added to the
//                gradient pages with fp32 atomic adds, once per key per workgroup.
// Splitting the backward this way recomputes S and dP once more than a fused kernel, but keeps
// every partial sum on chip: a fused query-major kernel would stream one fp32 dK/dV partial per
// 256 query rows through global atomics, about 120 GB at a 256K context.
#include "pkv_device.h"

namespace pkv {

// ---------------------------------------------------------------------------------------------
// D[h][t] = sum_d dO[t][h][d] * O[t][h][d] for the query heads of KV heads [kvh0, kvh0 + n_kvh),
// and the log-sum-exp in base 2 (lse * log2 e) that the backward passes exponentiate against.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_rowdot(AttnArgs a, const uint16_t* __restrict__ o,
                                                    const uint16_t* __restrict__ dout, const float* __restrict__ lse,
                                                    float* __restrict__ dbuf, float* __restrict__ lse2buf) {
  const int32_t nh = a.n_kvh * a.G;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
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
  dbuf[(int64_t)h * a.C + t] = acc;
  lse2buf[(int64_t)h * a.C + t] = lse[(int64_t)h * a.C + t] * kLog2e;
}

// ---------------------------------------------------------------------------------------------
template <int D>
struct DqCfg {
  static constexpr int NW = 4;                       // waves per workgroup (32 rows each)
  static constexpr int BK = 64;                      // keys per tile
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int CHR = D / 8;
  static constexpr int TILE = BK * D;                // elements of one K or V tile
  static constexpr int SEG_PER_WAVE = TILE * 2 / 1024 / NW;
  static constexpr int ROWS_PER_SEG = 1024 / (2 * D);
};

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_dq(AttnArgs a, BwdExtra e, int32_t n_rb, int32_t splits,
                                                   const float* __restrict__ dbuf, const float* __restrict__ lse2buf,
                                                   float* __restrict__ ws_dq) {
  using T = DqCfg<D>;
  constexpr int BK = T::BK;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * 2 * T::TILE];  // [stage][K|V]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lg = lane >> 5, l32 = lane & 31;
  const int32_t n_units = a.n_kvh * splits * n_rb;
  const int32_t u = xcd_remap(blockIdx.x, n_units);
  const int32_t rb = u % n_rb;
  const int32_t sp = (u / n_rb) % splits;
  const int32_t gi = u / (n_rb * splits);
  const int32_t g = a.kvh0 + gi;
  const int32_t G = a.G, CG = a.C * G, P = a.page, H = a.h_kv;
  const int32_t r0 = rb * 32 * T::NW;
  const int32_t r_last = min(r0 + 32 * T::NW - 1, CG - 1);
  const int32_t t_min = r0 / G, t_max = r_last / G;
  const int32_t q0 = a.n_prior * P;
  const int tsh = (P == 128) ? 1 : 0;  // log2(64-key tiles per page)
  const int32_t n_prior_tiles = list_prior(a) << tsh;
  const int32_t n_tiles = n_prior_tiles + t_max / BK + 1;
  const int32_t tb = (int32_t)((int64_t)n_tiles * sp / splits);
  const int32_t te = (int32_t)((int64_t)n_tiles * (sp + 1) / splits);

  const int32_t row = r0 + wave * 32 + l32;
  const bool rvalid = row < CG;
  const int32_t rr = rvalid ? row : CG - 1;
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
  const float dval = rvalid ? dbuf[si] : 0.f;

  auto tile_src = [&](int32_t i, int32_t& kpos0) -> const uint16_t* {
    const int32_t pi = i >> tsh, sub = i & ((1 << tsh) - 1);
    const int32_t lp = list_page(a, g, pi);
    const int32_t ph = phys_page(a.bt, a.n_bt, a.n_pool_pages, lp, a.err);
    if (ph < 0) {
      kpos0 = -1;
      return nullptr;
    }
    kpos0 = lp * P + sub * BK;
    return a.kv + (((int64_t)ph * H + g) * 2) * P * D + (int64_t)sub * BK * D;
  };
  int32_t seg_off[T::SEG_PER_WAVE];
#pragma unroll
  for (int j = 0; j < T::SEG_PER_WAVE; ++j) {
    const int rl = (wave * T::SEG_PER_WAVE + j) * T::ROWS_PER_SEG + lane / T::CHR;
    seg_off[j] = rl * D + (((lane % T::CHR) ^ swz<D>(rl)) << 3);
  }
  auto load_tile = [&](int32_t i, int stage, int32_t& kp) {
    const uint16_t* src = tile_src(i, kp);
    if (src == nullptr) src = a.kv;  // unreadable page: any in-bounds bytes, the tile is masked
    uint16_t* kt = lds + stage * 2 * T::TILE;
#pragma unroll
    for (int j = 0; j < T::SEG_PER_WAVE; ++j) {
      const int seg = wave * T::SEG_PER_WAVE + j;
      g2lds16(src + seg_off[j], kt + seg * 512);
      g2lds16(src + (int64_t)P * D + seg_off[j], kt + T::TILE + seg * 512);
    }
  };

  const float sl2 = a.scale * kLog2e;
  f32x16 dq[T::DT];
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) dq[dt] = (f32x16){};

  int32_t kpos_next = -1;
  if (tb < te) load_tile(tb, 0, kpos_next);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int32_t i = tb; i < te; ++i) {
    const int cur = (i - tb) & 1;
    const int32_t kpos_t = kpos_next;
    if (i + 1 < te) load_tile(i + 1, cur ^ 1, kpos_next);
    const uint16_t* kt = lds + cur * 2 * T::TILE;
    const uint16_t* vt = kt + T::TILE;
    const bool bad = kpos_t < 0;
    const bool need_mask = bad || (kpos_t + BK - 1 > q0 + t_min);
    const int32_t lim = q0 + tq;

    // The two 32-key halves of the tile run one after the other to bound register use.
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      f32x16 sacc = (f32x16){}, pacc = (f32x16){};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const int off = toff<D>(k2 * 32 + l32, ks * 16 + 8 * lg);
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + off));
        const bf16x8 va = as_bf16x8(*reinterpret_cast<const u32x4*>(vt + off));
        sacc = mfma32(ka, qreg[ks], sacc);
        pacc = mfma32(va, doreg[ks], pacc);
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
          w[j] = cvt_pk_bf16(p[el] * (pacc[el] - dval), p[el + 1] * (pacc[el + 1] - dval));
        }
        dsb[hf] = as_bf16x8(w);
      }
      // dQ^T[dt] += K^T[dt rows][16 keys] dS^T[16 keys]
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int k_lo = k2 * 32 + hf * 16 + 4 * lg;
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
          const bf16x8 kta = tr_operand<D>(kt, k_lo, k_lo + 8, dt * 32, lane);
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

// ---------------------------------------------------------------------------------------------
template <int D>
struct DkvCfg {
  static constexpr int NW = dkdv_waves(D);     // waves per workgroup, 32 keys each
  static constexpr int BQ = (D == 128) ? 32 : 64;  // rows per staged block
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int CHR = D / 8;            // 16-byte chunks per row
  static constexpr int TILE = BQ * D;          // elements of one staged Q or dO block
  static constexpr int SEGS = TILE * 2 / 1024; // 1 KiB segments per block (one wave-wide load each)
  static constexpr int SEG_PER_WAVE = SEGS / NW;
  static constexpr int ROWS_PER_SEG = 1024 / (2 * D);
  static constexpr int STAGE_BYTES = 2 * TILE * 2 + 2 * BQ * 4;
  static constexpr int VRES = 32 * D;           // resident V rows of one wave's keys (elements)
};

// x / G for 0 <= x < 2^24 from a float reciprocal, corrected to the exact quotient.
__device__ __forceinline__ int32_t div_small(int32_t x, int32_t G, float invG) {
  int32_t q = (int32_t)((float)x * invG);
  q -= (q * G > x) ? 1 : 0;
  q += ((q + 1) * G <= x) ? 1 : 0;
  return q;
}

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_dkdv(AttnArgs a, BwdExtra e, int32_t n_ku, int32_t row_splits,
                                                     const float* __restrict__ dbuf, const float* __restrict__ lse2buf) {
  using T = DkvCfg<D>;
  constexpr int BQ = T::BQ;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * T::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint16_t vres[T::NW * T::VRES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lg = lane >> 5, l32 = lane & 31;
  const int32_t n_units = a.n_kvh * n_ku * row_splits;
  const int32_t u = xcd_remap(blockIdx.x, n_units);
  const int32_t rs = u % row_splits;
  const int32_t ku = (u / row_splits) % n_ku;
  const int32_t gi = u / (row_splits * n_ku);
  const int32_t g = a.kvh0 + gi;
  const int32_t G = a.G, CG = a.C * G, P = a.page, H = a.h_kv;
  const float invG = 1.0f / (float)G;
  const int32_t q0 = a.n_prior * P;
  const int tsh = (P == 128) ? 2 : 1;  // log2(32-key tiles per page)
  const int32_t n_kt = (list_prior(a) + a.C / P) << tsh;

  // This wave's 32 keys.
  const int32_t kt_idx = ku * T::NW + wave;
  bool kvalid = kt_idx < n_kt;
  int32_t kpos0 = 0, gphys = -1, sub = 0;
  const uint16_t* kbase = nullptr;
  if (kvalid) {
    const int32_t pi = kt_idx >> tsh;
    sub = kt_idx & ((1 << tsh) - 1);
    const int32_t lp = list_page(a, g, pi);
    const int32_t ph = phys_page(a.bt, a.n_bt, a.n_pool_pages, lp, a.err);
    gphys = phys_page(e.gbt, e.n_gbt, e.n_gpool_pages, lp, a.err);
    kvalid = (ph >= 0) && (gphys >= 0);
    kpos0 = (lp < 0 ? 0 : lp) * P + sub * 32;
    if (kvalid) kbase = a.kv + (((int64_t)ph * H + g) * 2) * P * D + (int64_t)sub * 32 * D;
  }
  // First row any key of this workgroup can see (keys ascend along the list).
  int32_t wg_kpos_min;
  {
    const int32_t pi0 = (ku * T::NW) >> tsh;
    const int32_t lp0 = (pi0 < list_prior(a)) ? -1 : a.n_prior + (pi0 - list_prior(a));
    wg_kpos_min = (lp0 < 0) ? 0 : lp0 * P + (((ku * T::NW) - (pi0 << tsh)) * 32);
  }
  const int32_t n_blk = (CG + BQ - 1) / BQ;
  int32_t blk_b = (int32_t)((int64_t)n_blk * rs / row_splits);
  const int32_t blk_e = (int32_t)((int64_t)n_blk * (rs + 1) / row_splits);
  if (wg_kpos_min > q0) blk_b = max(blk_b, (G * (wg_kpos_min - q0)) / BQ);
  // Row r sees key k iff r >= G * (k - q0); rows r >= CG do not exist.
  const int32_t my_rmin = G * (kpos0 + l32 - q0);
  const int32_t wave_rmin = G * (kpos0 - q0);
  const int32_t wave_rmax = G * (kpos0 + 31 - q0);

  // K of this wave's keys stays in registers (B operand of S = Q K^T); V goes to LDS once (B
  // operand of dP = dO V^T, read back as rows).
  bf16x8 kreg[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    u32x4 x = (u32x4){0u, 0u, 0u, 0u};
    if (kvalid) x = *reinterpret_cast<const u32x4*>(kbase + (int64_t)l32 * D + ks * 16 + 8 * lg);
    kreg[ks] = as_bf16x8(x);
  }
  uint16_t* vmine = vres + wave * T::VRES;
  {
    const uint16_t* vsrc = kvalid ? kbase + (int64_t)P * D : a.kv;  // invalid tiles: any bytes
#pragma unroll
    for (int sg = 0; sg < T::VRES * 2 / 1024; ++sg) {
      const int rl = sg * T::ROWS_PER_SEG + lane / T::CHR;
      g2lds16(vsrc + rl * D + (((lane % T::CHR) ^ swz<D>(rl)) << 3), vmine + sg * 512);
    }
  }

  // Staging with direct global->LDS loads. Wave w fills 1 KiB segments w*SEG_PER_WAVE + j of the
  // Q and dO blocks; lane L lands at segment offset 16 L = (row L / CHR of the segment, physical
  // chunk L % CHR), so it fetches the logical chunk that the swizzle places there. Each lane
  // tracks (token, head) of its rows incrementally from block to block. Rows past the end of the
  // chunk re-read the last row and are masked out in the compute.
  const uint16_t* qg = a.q + (int64_t)g * G * D;
  const uint16_t* dg = e.dout + (int64_t)g * G * D;
  const int32_t step_q = BQ / G, step_r = BQ - (BQ / G) * G;  // BQ = step_q * G + step_r
  int32_t st_t[T::SEG_PER_WAVE], st_h[T::SEG_PER_WAVE], st_c[T::SEG_PER_WAVE];
#pragma unroll
  for (int j = 0; j < T::SEG_PER_WAVE; ++j) {
    const int seg = wave * T::SEG_PER_WAVE + j;
    const int rl = seg * T::ROWS_PER_SEG + lane / T::CHR;
    const int32_t r = blk_b * BQ + rl;
    st_t[j] = div_small(r, G, invG);
    st_h[j] = r - st_t[j] * G;
    st_c[j] = ((lane % T::CHR) ^ swz<D>(rl)) * 8;  // logical column of this lane's chunk
  }
  // LSE / D rows: element e = wave * 64 + lane < 2 * BQ of the block's [lse2 | D] array.
  constexpr int LW = (2 * BQ + 63) / 64;  // waves that fetch them
  const int e_ld = wave * 64 + lane;
  const bool is_lse = e_ld < BQ;
  int32_t sl_t = 0, sl_h = 0;
  {
    const int32_t r = blk_b * BQ + (is_lse ? e_ld : e_ld - BQ);
    sl_t = div_small(r, G, invG);
    sl_h = r - sl_t * G;
  }
  const int32_t last_t = (CG - 1) / G, last_h = (CG - 1) - ((CG - 1) / G) * G;
  auto advance = [&](int32_t& t, int32_t& hh) {
    hh += step_r;
    t += step_q;
    if (hh >= G) {
      hh -= G;
      t += 1;
    }
  };
  auto load_blk = [&](int stage) {
    unsigned char* bs = smem + stage * T::STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < T::SEG_PER_WAVE; ++j) {
      const int seg = wave * T::SEG_PER_WAVE + j;
      const bool past = st_t[j] > last_t || (st_t[j] == last_t && st_h[j] > last_h);
      const int32_t t = past ? last_t : st_t[j], hh = past ? last_h : st_h[j];
      const int32_t off = (t * a.h_q + hh) * D + st_c[j];
      g2lds16(qg + off, bs + seg * 1024);
      g2lds16(dg + off, bs + T::TILE * 2 + seg * 1024);
      advance(st_t[j], st_h[j]);
    }
    if (wave < LW) {
      const bool past = sl_t > last_t || (sl_t == last_t && sl_h > last_h);
      const int32_t t = past ? last_t : sl_t, hh = past ? last_h : sl_h;
      const int32_t si = (g * G + hh) * a.C + t;
      g2lds4(is_lse ? (const void*)(lse2buf + si) : (const void*)(dbuf + si), bs + 2 * T::TILE * 2 + wave * 256);
    }
    advance(sl_t, sl_h);
  };

  const float sl2 = a.scale * kLog2e;
  f32x16 dk[T::DT], dv[T::DT];
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) {
    dk[dt] = (f32x16){};
    dv[dt] = (f32x16){};
  }

  if (blk_b < blk_e) load_blk(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int32_t blk = blk_b; blk < blk_e; ++blk) {
    const int cur = (blk - blk_b) & 1;
    if (blk + 1 < blk_e) load_blk(cur ^ 1);
    const unsigned char* bs = smem + cur * T::STAGE_BYTES;
    const uint16_t* qs = reinterpret_cast<const uint16_t*>(bs);
    const uint16_t* ds_ = qs + T::TILE;
    const float* ls = reinterpret_cast<const float*>(bs + 2 * T::TILE * 2);
    const float* dd = ls + BQ;

    // Blocks no key of this wave can see, and invalid key tiles, are masked rather than skipped,
    // so the loop body has a single path (their contributions are never flushed or are zero).
    {
      const bool need_mask = (blk * BQ < wave_rmax) || (blk * BQ + BQ > CG);
      (void)wave_rmin;
      const int32_t rlim = CG - blk * BQ;  // rows at or past this index do not exist
#pragma unroll
      for (int rt = 0; rt < BQ / 32; ++rt) {
        f32x16 sacc = (f32x16){}, pacc = (f32x16){};
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
          const int off = toff<D>(rt * 32 + l32, ks * 16 + 8 * lg);
          const bf16x8 qa = as_bf16x8(*reinterpret_cast<const u32x4*>(qs + off));
          const bf16x8 da = as_bf16x8(*reinterpret_cast<const u32x4*>(ds_ + off));
          const bf16x8 vb = as_bf16x8(*reinterpret_cast<const u32x4*>(vmine + toff<D>(l32, ks * 16 + 8 * lg)));
          sacc = mfma32(qa, kreg[ks], sacc);
          pacc = mfma32(da, vb, pacc);
        }
        float pv[16], dsv[16];
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int rr = rt * 32 + 8 * grp + 4 * lg;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + rr);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int el = grp * 4 + j;
            pv[el] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[el], sl2, -l4[j]));
          }
        }
        if (need_mask) {
          // Keep rows lo <= row < hi of this block: lo from the lane's key, hi from the chunk end.
          const uint32_t lo = (uint32_t)(my_rmin - blk * BQ), span = (uint32_t)(rlim - (my_rmin - blk * BQ));
#pragma unroll
          for (int el = 0; el < 16; ++el) {
            const int rr = rt * 32 + 8 * (el >> 2) + 4 * lg + (el & 3);
            if ((uint32_t)rr - lo >= span) pv[el] = 0.f;
          }
        }
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int rr = rt * 32 + 8 * grp + 4 * lg;
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dd + rr);
#pragma unroll
          for (int j = 0; j < 4; ++j) dsv[grp * 4 + j] = pv[grp * 4 + j] * (pacc[grp * 4 + j] - d4[j]);
        }
        bf16x8 pb[2], dsb[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          u32x4 w, x;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            w[j] = cvt_pk_bf16(pv[hf * 8 + 2 * j], pv[hf * 8 + 2 * j + 1]);
            x[j] = cvt_pk_bf16(dsv[hf * 8 + 2 * j], dsv[hf * 8 + 2 * j + 1]);
          }
          pb[hf] = as_bf16x8(w);
          dsb[hf] = as_bf16x8(x);
        }
        // dV[keys][d] += P^T[keys][16 rows] dO[16 rows][d]; dK[keys][d] += dS^T Q likewise. The B
        // operands (rows along the contraction) come from transposed reads of the staged blocks,
        // in the row order of the accumulator layout.
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int k_lo = rt * 32 + hf * 16 + 4 * lg;
#pragma unroll
          for (int dt = 0; dt < T::DT; ++dt) {
            const bf16x8 dob_t = tr_operand<D>(ds_, k_lo, k_lo + 8, dt * 32, lane);
            const bf16x8 qb_t = tr_operand<D>(qs, k_lo, k_lo + 8, dt * 32, lane);
            dv[dt] = mfma32(pb[hf], dob_t, dv[dt]);
            dk[dt] = mfma32(dsb[hf], qb_t, dk[dt]);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Accumulate into the gradient pages: element (key, d) of dK/dV goes to
  // grad[gphys][g][0/1][sub*32 + key][d]. Lanes of one instruction cover 32 consecutive d.
  if (kvalid && blk_b < blk_e) {
    float* gk = e.grad + (((int64_t)gphys * H + g) * 2) * P * D + (int64_t)sub * 32 * D;
    float* gv = gk + (int64_t)P * D;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
      for (int el = 0; el < 16; ++el) {
        const int key = 8 * (el >> 2) + 4 * lg + (el & 3);
        const int64_t off = (int64_t)key * D + dt * 32 + l32;
        unsafeAtomicAdd(gk + off, dk[dt][el] * a.scale);
        unsafeAtomicAdd(gv + off, dv[dt][el]);
      }
  }
}

template <int D>
static hipError_t launch_bwd_d(const AttnArgs& a, const BwdExtra& e, const BwdPlan& plan, void* ws, hipStream_t s) {
  const int64_t rows_total = (int64_t)a.n_kvh * a.C * a.G;
  const size_t nrow = ((size_t)a.h_q * a.C + 63) & ~(size_t)63;
  float* dbuf = (float*)ws;        // [H_q][C] row dots
  float* lse2buf = dbuf + nrow;    // [H_q][C] lse * log2 e
  float* ws_dq = lse2buf + nrow;
  {
    const int64_t work = (int64_t)a.C * a.n_kvh * a.G;
    TimerScope ts_("k_bwd_rowdot", s);
    hipLaunchKernelGGL(k_bwd_rowdot<D>, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, a, e.o, e.dout,
                       e.lse, dbuf, lse2buf);
  }
  {
    const int32_t n_units = a.n_kvh * plan.splits * plan.n_rb;
    {
      TimerScope ts_("k_bwd_dq", s);
      hipLaunchKernelGGL(k_bwd_dq<D>, dim3(n_units), dim3(64 * DqCfg<D>::NW), 0, s, a, e, plan.n_rb, plan.splits,
                         dbuf, lse2buf, ws_dq);
    }
    if (plan.splits > 1) {
      const int64_t work = rows_total * (D / 8);
      TimerScope ts_("k_bwd_dq_reduce", s);
      hipLaunchKernelGGL(k_bwd_dq_reduce<D>, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, a, plan.splits,
                         ws_dq, e.dq);
    }
  }
  {
    const int32_t n_units = a.n_kvh * plan.n_ku * plan.row_splits;
    TimerScope ts_("k_bwd_dkdv", s);
    hipLaunchKernelGGL(k_bwd_dkdv<D>, dim3(n_units), dim3(64 * DkvCfg<D>::NW), 0, s, a, e, plan.n_ku,
                       plan.row_splits, dbuf, lse2buf);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const AttnArgs& a, const BwdExtra& e, const BwdPlan& plan, void* ws, hipStream_t s) {
  if (a.d == 128) return launch_bwd_d<128>(a, e, plan, ws, s);
  return launch_bwd_d<64>(a, e, plan, ws, s);
}

}  // namespace pkv
