// Chunk attention forward over the paged KV cache, bf16 MFMA (gfx950), online softmax.
//
// "Out of the Memory Barrier" summaries: pt 2.A / es 2.A / it 2.A (one chunk attends to every
// earlier key and its own causal block), pt 2.B / es 2.B / it 2.B (keys and values read in place
// from non-contiguous pages through the block table), pt 2.C / es 2.B / it 2.D (sparse mode:
// only the selected pages plus the own block).
//
// Work decomposition. The G query heads sharing a KV head are packed into one row space:
// row r = t*G + hh (t = chunk token, hh = head within the group), so every K/V tile staged in LDS
// feeds every row of the workgroup. A workgroup = (KV head, key-range split, row block) with 8
// waves of 32 rows (256 rows, one workgroup per CU) or 4 (128 rows, two workgroups per CU; used
// when a 256-row block would be half empty). Either way two waves share each SIMD, so one wave's
// softmax overlaps the other's matrix work. With one page list per query page (pt 2.C) the row
// blocks are cut at query-page boundaries and each walks its query page's list. K/V tiles go
// straight from global memory into LDS. Splits > 1 write normalised partial outputs plus their
// log-sum-exp, merged by k_fwd_combine.
//
// Per wave and 64-key tile: S^T (keys x queries) = K Q^T as two 32x32 tiles (A = K rows from
// LDS, B = Q^T in registers), so each lane owns one query column and its softmax statistics
// (plus one exchange with lane l^32). P^T feeds O^T += V^T P^T directly as the B operand; the
// V^T operand is read from the row-major V tile with transposed LDS reads, in the key order the
// accumulator layout gives P^T (4 keys from each half-wave, twice per 16-key step).
// The running maximum is only moved (and O rescaled) when it grows by more than 2^8, so most
// tiles skip the rescale; probabilities then stay below 256 before normalisation.
#include <cstdlib>
#include <cstring>

#include "pkv_device.h"

namespace pkv {

template <int D, int NWAVES>
struct FwdCfg {
  static constexpr int NW = NWAVES;                 // waves per workgroup (32 rows each)
  static constexpr int BK = 64;                     // keys per tile
  static constexpr int KS = D / 16;                 // contraction steps over d
  static constexpr int DT = D / 32;                 // 32-row tiles of O^T
  static constexpr int CHR = D / 8;                 // 16-byte chunks per row
  static constexpr int TILE = BK * D;               // elements of one K or V tile
  static constexpr int SEG_PER_WAVE = TILE * 2 / 1024 / NW;  // 1 KiB direct-load segments per wave
  static constexpr int ROWS_PER_SEG = 1024 / (2 * D);
};

constexpr float kRescaleLog2 = 8.0f;

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_fwd(
    AttnArgs a, int32_t n_rb, int32_t splits, uint16_t* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_lse) {
  using T = FwdCfg<D, NW>;
  constexpr int BK = T::BK;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * 2 * T::TILE];  // [stage][K|V]

  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 5, l32 = lane & 31;
  // Wave-uniform, so the LDS destinations of the direct loads stay in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int tsh = (P == 128) ? 1 : 0;  // log2(tiles per page)
  const int32_t n_prior_tiles = list_prior(a) << tsh;
  const int32_t n_tiles = n_prior_tiles + t_max / BK + 1;
  const int32_t tb = (int32_t)((int64_t)n_tiles * sp / splits);
  const int32_t te = (int32_t)((int64_t)n_tiles * (sp + 1) / splits);

  // This lane's query row and its Q^T operand.
  const int32_t row = r0 + wave * 32 + l32;
  const bool rvalid = row < r_end;
  const int32_t rr = rvalid ? row : r_last;
  const int32_t tq = rr / G;
  const int32_t h = g * G + (rr - tq * G);
  bf16x8 qreg[T::KS];
  {
    const uint16_t* qp = a.q + ((int64_t)tq * a.h_q + h) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + ks * 16);
      if (!rvalid) v = (u32x4){0u, 0u, 0u, 0u};
      qreg[ks] = as_bf16x8(v);
    }
  }

  // Tiles of the key list in order, with their table reads issued a tile ahead.
  KeyWalk walk = walk_begin(a, g, li, tsh, tb, te);

  // Direct global->LDS staging: wave w fills 1 KiB segments w*SEG_PER_WAVE + j of the K and V
  // tiles; lane L lands at (row L / CHR of the segment, physical chunk L % CHR) and so fetches the
  // logical chunk the swizzle places there.
  uint32_t seg_off[T::SEG_PER_WAVE];  // byte offsets: unsigned 32-bit, added to a scalar base
#pragma unroll
  for (int j = 0; j < T::SEG_PER_WAVE; ++j) {
    const int rl = (wave * T::SEG_PER_WAVE + j) * T::ROWS_PER_SEG + lane / T::CHR;
    seg_off[j] = 2u * (uint32_t)(rl * D + (((lane % T::CHR) ^ swz<D>(rl)) << 3));
  }
  // Stage the walk's next tile (kp: its first key position, -1 when unreadable).
  auto load_tile = [&](int stage, int32_t& kp) {
    const uint16_t* src = walk_take<D>(a, walk, kp);
    if (src == nullptr) src = a.kv;  // unreadable page: any in-bounds bytes, the tile is masked
    uint16_t* kt = lds + stage * 2 * T::TILE;
    const char* ksrc = reinterpret_cast<const char*>(src);
    const char* vsrc = reinterpret_cast<const char*>(src + (int64_t)P * D);
#pragma unroll
    for (int j = 0; j < T::SEG_PER_WAVE; ++j) {
      const int seg = wave * T::SEG_PER_WAVE + j;
      g2lds16(ksrc + seg_off[j], kt + seg * 512);
      g2lds16(vsrc + seg_off[j], kt + T::TILE + seg * 512);
    }
  };

  // Loop-invariant LDS byte offsets of this lane's MFMA operands within a stage. The swizzle of a
  // tile row depends only on the row's low four bits, which the 32-key half (k2) and the 16-key
  // step (hf) never change, so every operand address is one of these plus a constant.
  uint32_t koff[T::KS];             // K rows l32, columns 16 ks + 8 lg
  uint32_t voff[T::DT][2];          // V^T: rows 4 lg + rr (+8), columns 32 dt + 16 b4 + 4 (lane%4)
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) koff[ks] = 2u * (uint32_t)toff<D>(l32, ks * 16 + 8 * lg);
  {
    const int rr = (lane & 15) >> 2, cb = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) voff[dt][kh] = 2u * (uint32_t)toff<D>(4 * lg + rr + 8 * kh, dt * 32 + cb);
  }

  const float sl2 = a.scale * kLog2e;
  float m = -INFINITY, l = 0.f;
  f32x16 oacc[T::DT];
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) oacc[dt] = (f32x16){};

  int32_t kpos_next = -1;
  if (tb < te) load_tile(0, kpos_next);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int32_t i = tb; i < te; ++i) {
    const int cur = (i - tb) & 1;
    const int32_t kpos0 = kpos_next;
    if (i + 1 < te) load_tile(cur ^ 1, kpos_next);
    const char* kt = reinterpret_cast<const char*>(lds + cur * 2 * T::TILE);
    const char* vt = kt + 2 * T::TILE;

    f32x16 sacc[2] = {(f32x16){}, (f32x16){}};
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + koff[ks] + k2 * 32 * D * 2));
        sacc[k2] = mfma32(ka, qreg[ks], sacc[k2]);
      }
    }
    __builtin_amdgcn_s_setprio(0);

    const bool bad = kpos0 < 0;
    if (bad || kpos0 + BK - 1 > q0 + t_min) {
      const int32_t lim = q0 + tq;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int32_t key = kpos0 + k2 * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
          if (bad || key > lim) sacc[k2][e] = -INFINITY;
        }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[k2][e]);
    mx = fmaxf(mx, wave_xor32(mx));
    const float m_new = fmaxf(m, mx);
    if (__any((m_new - m) * sl2 > kRescaleLog2)) {
      const float alpha = (m_new == m) ? 1.f : __builtin_amdgcn_exp2f((m - m_new) * sl2);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) oacc[dt] *= alpha;
      m = m_new;
    }
    const float mc = (m == -INFINITY) ? 0.f : m * sl2;
    bf16x8 pb[2][2];  // [k2][half]
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[k2][e], sl2, -mc));
        l += p[e];
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = cvt_pk_bf16(p[hf * 8 + 2 * j], p[hf * 8 + 2 * j + 1]);
        pb[k2][hf] = as_bf16x8(w);
      }
    }
    // O^T[dt] += V^T[dt rows][16 keys] P^T[16 keys]
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int rowb = (k2 * 32 + hf * 16) * D * 2;  // bytes
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
          const u32x2 lo = lds_tr16(reinterpret_cast<const uint16_t*>(vt + voff[dt][0] + rowb));
          const u32x2 hi = lds_tr16(reinterpret_cast<const uint16_t*>(vt + voff[dt][1] + rowb));
          const bf16x8 va = as_bf16x8((u32x4){lo[0], lo[1], hi[0], hi[1]});
          oacc[dt] = mfma32(va, pb[k2][hf], oacc[dt]);
        }
      }
    __builtin_amdgcn_s_setprio(0);

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Epilogue.
  const float lt = l + wave_xor32(l);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const float lse_v = lt > 0.f ? (m * sl2 + __log2f(lt)) * kLn2 : -INFINITY;
  if (!rvalid) return;
  if (splits == 1) {
    uint16_t* op = o + ((int64_t)tq * a.h_q + h) * D;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        u32x2 w;
        w[0] = cvt_pk_bf16(oacc[dt][grp * 4 + 0] * inv, oacc[dt][grp * 4 + 1] * inv);
        w[1] = cvt_pk_bf16(oacc[dt][grp * 4 + 2] * inv, oacc[dt][grp * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(op + dt * 32 + grp * 8 + 4 * lg) = w;
      }
    if (lg == 0) lse[(int64_t)h * a.C + tq] = lse_v;
  } else {
    const int64_t R = (int64_t)gi * CG + row;
    const int64_t rows_total = (int64_t)a.n_kvh * CG;
    float* wp = ws_o + ((int64_t)sp * rows_total + R) * D;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = oacc[dt][grp * 4 + j] * inv;
        *reinterpret_cast<f32x4*>(wp + dt * 32 + grp * 8 + 4 * lg) = w;
      }
    if (lg == 0) ws_lse[(int64_t)sp * rows_total + R] = lse_v;
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
  for (int j = 0; j < 4; ++j) out[j] = cvt_pk_bf16(acc[2 * j] * inv, acc[2 * j + 1] * inv);
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
    if (plan.nw == 8 && fwd_one_wave_per_simd()) {
      TimerScope ts_("k_attn_fwd64", s);
      launch_fwd64<D>(a, plan.n_rb, plan.splits, o, lse, ws_o, ws_lse, s);
    } else if (plan.nw == 8) {
      TimerScope ts_("k_attn_fwd", s);
      hipLaunchKernelGGL((k_attn_fwd<D, 8>), dim3(n_units), dim3(64 * 8), 0, s, a, plan.n_rb, plan.splits, o, lse,
                         ws_o, ws_lse);
    } else {
      TimerScope ts_("k_attn_fwd", s);
      hipLaunchKernelGGL((k_attn_fwd<D, 4>), dim3(n_units), dim3(64 * 4), 0, s, a, plan.n_rb, plan.splits, o, lse,
                         ws_o, ws_lse);
    }
  }
  if (plan.splits > 1) {
    const int64_t work = rows_total * (D / 8);
    TimerScope ts_("k_fwd_combine", s);
    hipLaunchKernelGGL(k_fwd_combine<D>, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, a, plan.splits,
                       ws_o, ws_lse, o, lse);
  }
  return hipGetLastError();
}

bool fwd_one_wave_per_simd() {
  static const bool v = [] {
    const char* e = getenv("PKV_FWD_KERNEL");
    return !(e && strcmp(e, "w8") == 0);
  }();
  return v;
}

hipError_t launch_fwd(const AttnArgs& a, const FwdPlan& plan, uint16_t* o, float* lse, void* ws, hipStream_t s) {
  if (a.d == 128) return launch_fwd_d<128>(a, plan, o, lse, ws, s);
  return launch_fwd_d<64>(a, plan, o, lse, ws, s);
}

}  // namespace pkv
