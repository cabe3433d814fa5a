// Chunk attention forward over the paged KV cache, bf16 MFMA (gfx950), online softmax.
//
// "Out of the Memory Barrier" summaries: pt 2.A / es 2.A / it 2.A (one chunk attends to every
// earlier key and its own causal block), pt 2.B / es 2.B / it 2.B (keys and values read in place
// from non-contiguous pages through the block table), pt 2.C / es 2.B / it 2.D (sparse mode:
// only the selected pages plus the own block).
//
// Work decomposition. The G query heads sharing a KV head are packed into one row space:
// row r = t*G + hh (t = chunk token, hh = head within the group), so every K/V tile staged in LDS
// feeds 256 rows (4 waves x 64 rows). A workgroup = (KV head, key-range split, 256-row block);
// splits > 1 write normalised partial outputs plus their log-sum-exp, merged by k_fwd_combine.
//
// Per wave and 64-key tile: S^T (keys x queries) = K Q^T as 2x2 tiles of 32x32 (A = K rows from
// LDS, B = Q^T held in registers), so each lane owns one query column and the softmax statistics
// are per lane (plus one exchange with lane l^32). P^T is fed straight back as the B operand of
// O^T += V^T P^T, with V^T staged transposed in LDS. The key order inside each 16-key MFMA step
// follows the accumulator layout (4 keys from each half-wave, twice); V^T reads use that order.
#include "pkv_device.h"

namespace pkv {

template <int D>
struct FwdTile {
  static constexpr int BK = 64;             // keys per tile
  static constexpr int KSTR = D + 8;        // K row stride (bf16) in LDS
  static constexpr int VSTR = BK + 4;       // V^T row stride (bf16) in LDS
  static constexpr int K_EL = BK * KSTR;
  static constexpr int V_EL = D * VSTR;
  static constexpr int STAGE = K_EL + V_EL;
  static constexpr int KCH = BK * D / 8 / 256;  // 16-byte K chunks per thread
  static constexpr int VKB = D / 32;            // keys per thread in the V^T transpose
  static constexpr int KS = D / 16;             // contraction steps over d
  static constexpr int DT = D / 32;             // 32-row tiles of O^T
};

template <int D>
__global__ __launch_bounds__(256, 1) void k_attn_fwd(AttnArgs a, int32_t n_rb, int32_t splits,
                                                     uint16_t* __restrict__ o, float* __restrict__ lse,
                                                     float* __restrict__ ws_o, float* __restrict__ ws_lse) {
  using T = FwdTile<D>;
  constexpr int BK = T::BK;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lg = lane >> 5, l32 = lane & 31;
  const int32_t n_units = a.n_kvh * splits * n_rb;
  const int32_t u = xcd_remap(blockIdx.x, n_units);
  const int32_t rb = u % n_rb;
  const int32_t sp = (u / n_rb) % splits;
  const int32_t gi = u / (n_rb * splits);
  const int32_t g = a.kvh0 + gi;
  const int32_t G = a.G, CG = a.C * G, P = a.page, H = a.h_kv;
  const int32_t r0 = rb * 256;
  const int32_t r_last = min(r0 + 255, CG - 1);
  const int32_t t_min = r0 / G, t_max = r_last / G;
  const int32_t q0 = a.n_prior * P;
  const int32_t tpp = P / BK;
  const int32_t n_prior_tiles = list_prior(a) * tpp;
  const int32_t n_tiles = n_prior_tiles + t_max / BK + 1;
  const int32_t tb = (int32_t)((int64_t)n_tiles * sp / splits);
  const int32_t te = (int32_t)((int64_t)n_tiles * (sp + 1) / splits);

  // This lane's query rows (one per 32-column tile) and their positions.
  int32_t row[2], tpos[2];
  bool rvalid[2];
  bf16x8 qreg[2][T::KS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    row[qt] = r0 + wave * 64 + qt * 32 + l32;
    rvalid[qt] = row[qt] < CG;
    const int32_t rr = rvalid[qt] ? row[qt] : CG - 1;
    tpos[qt] = rr / G;
    const int32_t h = g * G + (rr - tpos[qt] * G);
    const uint16_t* qp = a.q + ((int64_t)tpos[qt] * a.h_q + h) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + ks * 16);
      if (!rvalid[qt]) v = (u32x4){0u, 0u, 0u, 0u};
      qreg[qt][ks] = as_bf16x8(v);
    }
  }

  // Tile loader: K chunks and V^T transpose blocks held in registers between load and store.
  u32x4 kbuf[T::KCH];
  u32x4 vbuf[T::VKB];
  const int vdc = tid % (D / 8), vkb = tid / (D / 8);  // V^T block: keys vkb*VKB.., dims vdc*8..

  auto tile_base = [&](int32_t i, int32_t& kpos0) -> const uint16_t* {
    const int32_t pi = i / tpp, sub = i - (i / tpp) * tpp;
    const int32_t lp = list_page(a, g, pi);
    kpos0 = (lp < 0 ? 0 : lp) * P + sub * BK;
    const int32_t ph = phys_page(a.bt, a.n_bt, a.n_pool_pages, lp, a.err);
    if (ph < 0) {
      kpos0 = -1;
      return nullptr;
    }
    return a.kv + (((int64_t)ph * H + g) * 2) * P * D + (int64_t)sub * BK * D;
  };
  auto load_tile = [&](int32_t i) {
    int32_t kp;
    const uint16_t* base = tile_base(i, kp);
    if (base == nullptr) {
#pragma unroll
      for (int c = 0; c < T::KCH; ++c) kbuf[c] = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
      for (int c = 0; c < T::VKB; ++c) vbuf[c] = (u32x4){0u, 0u, 0u, 0u};
      return;
    }
#pragma unroll
    for (int c = 0; c < T::KCH; ++c) kbuf[c] = reinterpret_cast<const u32x4*>(base)[tid + 256 * c];
    const uint16_t* vb = base + (int64_t)P * D;
#pragma unroll
    for (int c = 0; c < T::VKB; ++c)
      vbuf[c] = *reinterpret_cast<const u32x4*>(vb + (int64_t)(vkb * T::VKB + c) * D + vdc * 8);
  };
  auto store_tile = [&](int stage) {
    uint16_t* ks = lds + stage * T::STAGE;
    uint16_t* vt = ks + T::K_EL;
#pragma unroll
    for (int c = 0; c < T::KCH; ++c) {
      const int ch = tid + 256 * c;
      const int key = ch / (D / 8), dc = ch % (D / 8);
      *reinterpret_cast<u32x4*>(ks + key * T::KSTR + dc * 8) = kbuf[c];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = 16 * (e & 1);
      uint16_t* dst = vt + (vdc * 8 + e) * T::VSTR + vkb * T::VKB;
      if constexpr (T::VKB == 4) {
        u32x2 w;
        w[0] = ((vbuf[0][e >> 1] >> sh) & 0xffffu) | (((vbuf[1][e >> 1] >> sh) & 0xffffu) << 16);
        w[1] = ((vbuf[2][e >> 1] >> sh) & 0xffffu) | (((vbuf[3][e >> 1] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<u32x2*>(dst) = w;
      } else {
        *reinterpret_cast<uint32_t*>(dst) =
            ((vbuf[0][e >> 1] >> sh) & 0xffffu) | (((vbuf[1][e >> 1] >> sh) & 0xffffu) << 16);
      }
    }
  };

  const float sl2 = a.scale * kLog2e;
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x16 oacc[T::DT][2];
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) oacc[dt][qt] = (f32x16){};

  if (tb < te) {
    load_tile(tb);
    store_tile(0);
  }
  __syncthreads();

  for (int32_t i = tb; i < te; ++i) {
    const int cur = (i - tb) & 1;
    int32_t kpos0;
    (void)tile_base(i, kpos0);  // position of this tile's first key (-1: unreadable page)
    if (i + 1 < te) load_tile(i + 1);

    const uint16_t* ks_l = lds + cur * T::STAGE;
    const uint16_t* vt_l = ks_l + T::K_EL;

    // S^T tiles [kt][qt]
    f32x16 sacc[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) sacc[kt][qt] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 ka =
            as_bf16x8(*reinterpret_cast<const u32x4*>(ks_l + (kt * 32 + l32) * T::KSTR + ks * 16 + 8 * lg));
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) sacc[kt][qt] = mfma32(ka, qreg[qt][ks], sacc[kt][qt]);
      }
    }

    const bool bad = kpos0 < 0;
    const bool need_mask = bad || (kpos0 + BK - 1 > q0 + t_min);
    bf16x8 pb[2][2][2];  // [kt][qt][half]
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int32_t lim = q0 + tpos[qt];
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float s = sacc[kt][qt][e] * sl2;
          if (need_mask) {
            const int32_t key = kpos0 + kt * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
            if (bad || key > lim) s = -INFINITY;
          }
          sacc[kt][qt][e] = s;
          mx = fmaxf(mx, s);
        }
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m[qt], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m[qt] - m_use);
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(sacc[kt][qt][e] - m_use);
          sacc[kt][qt][e] = p;
          rs += p;
        }
      l[qt] = l[qt] * alpha + rs;
      m[qt] = m_new;
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) oacc[dt][qt] *= alpha;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          u32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(sacc[kt][qt][hf * 8 + 2 * j], sacc[kt][qt][hf * 8 + 2 * j + 1]);
          pb[kt][qt][hf] = as_bf16x8(w);
        }
    }

    // O^T[dt][qt] += V^T[dt rows][16 keys] * P^T[16 keys][qt]
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int key0 = kt * 32 + hf * 16 + 4 * lg;
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
          const uint16_t* vr = vt_l + (dt * 32 + l32) * T::VSTR + key0;
          u32x4 w;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
          w[0] = lo[0];
          w[1] = lo[1];
          w[2] = hi[0];
          w[3] = hi[1];
          const bf16x8 va = as_bf16x8(w);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) oacc[dt][qt] = mfma32(va, pb[kt][qt][hf], oacc[dt][qt]);
        }
      }

    if (i + 1 < te) store_tile(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float lt = l[qt] + wave_xor32(l[qt]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m[qt] + __log2f(lt)) * kLn2 : -INFINITY;
    if (!rvalid[qt]) continue;
    const int32_t t = tpos[qt];
    const int32_t h = g * G + (row[qt] - t * G);
    if (splits == 1) {
      uint16_t* op = o + ((int64_t)t * a.h_q + h) * D;
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          u32x2 w;
          w[0] = pack_bf16x2(oacc[dt][qt][grp * 4 + 0] * inv, oacc[dt][qt][grp * 4 + 1] * inv);
          w[1] = pack_bf16x2(oacc[dt][qt][grp * 4 + 2] * inv, oacc[dt][qt][grp * 4 + 3] * inv);
          *reinterpret_cast<u32x2*>(op + dt * 32 + grp * 8 + 4 * lg) = w;
        }
      if (lg == 0) lse[(int64_t)h * a.C + t] = lse_v;
    } else {
      const int64_t R = (int64_t)gi * CG + row[qt];
      const int64_t rows_total = (int64_t)a.n_kvh * CG;
      float* wp = ws_o + ((int64_t)sp * rows_total + R) * D;
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          f32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = oacc[dt][qt][grp * 4 + j] * inv;
          *reinterpret_cast<f32x4*>(wp + dt * 32 + grp * 8 + 4 * lg) = w;
        }
      if (lg == 0) ws_lse[(int64_t)sp * rows_total + R] = lse_v;
    }
  }
}

// Merge split partials: lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s.
// One thread per (row, 8 dims).
template <int D>
__global__ __launch_bounds__(256) void k_fwd_combine(AttnArgs a, int32_t splits, const float* __restrict__ ws_o,
                                                     const float* __restrict__ ws_lse, uint16_t* __restrict__ o,
                                                     float* __restrict__ lse) {
  const int32_t G = a.G, CG = a.C * G;
  const int64_t rows_total = (int64_t)a.n_kvh * CG;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows_total * (D / 8)) return;
  const int32_t dc = (int32_t)(idx % (D / 8));
  const int64_t R = idx / (D / 8);
  const int32_t gi = (int32_t)(R / CG), r = (int32_t)(R % CG);
  const int32_t t = r / G, h = (a.kvh0 + gi) * G + (r - (r / G) * G);
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, ws_lse[(int64_t)s * rows_total + R]);
  const float mu = (mx == -INFINITY) ? 0.f : mx;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float w = __expf(ws_lse[(int64_t)s * rows_total + R] - mu);
    wsum += w;
    const f32x4* src = reinterpret_cast<const f32x4*>(ws_o + ((int64_t)s * rows_total + R) * D + dc * 8);
    const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] += w * x0[j];
      acc[4 + j] += w * x1[j];
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = pack_bf16x2(acc[2 * j] * inv, acc[2 * j + 1] * inv);
  *reinterpret_cast<u32x4*>(o + ((int64_t)t * a.h_q + h) * D + dc * 8) = out;
  if (dc == 0) lse[(int64_t)h * a.C + t] = wsum > 0.f ? mu + __logf(wsum) : -INFINITY;
}

template <int D>
static hipError_t launch_fwd_d(const AttnArgs& a, const FwdPlan& plan, uint16_t* o, float* lse, void* ws,
                               hipStream_t s) {
  const int64_t rows_total = (int64_t)a.n_kvh * a.C * a.G;
  float* ws_o = (float*)ws;
  float* ws_lse = ws_o ? ws_o + (size_t)plan.splits * rows_total * D : nullptr;
  const int32_t n_units = a.n_kvh * plan.splits * plan.n_rb;
  {
    TimerScope ts_("k_attn_fwd", s);
    hipLaunchKernelGGL(k_attn_fwd<D>, dim3(n_units), dim3(256), 0, s, a, plan.n_rb, plan.splits, o, lse, ws_o, ws_lse);
  }
  if (plan.splits > 1) {
    const int64_t work = rows_total * (D / 8);
    {
      TimerScope ts_("k_fwd_combine", s);
      hipLaunchKernelGGL(k_fwd_combine<D>, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, a, plan.splits,
                         ws_o, ws_lse, o, lse);
    }
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const AttnArgs& a, const FwdPlan& plan, uint16_t* o, float* lse, void* ws, hipStream_t s) {
  if (a.d == 128) return launch_fwd_d<128>(a, plan, o, lse, ws, s);
  return launch_fwd_d<64>(a, plan, o, lse, ws, s);
}

}  // namespace pkv
