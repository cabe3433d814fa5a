// Chunk attention backward, key-major dK/dV pass, bf16 MFMA (gfx950).
//
// "Out of the Memory Barrier" summaries: pt 2.A / es 2.A / it 2.A (the probabilities dropped by
// the forward are recomputed in backward, here from the stored log-sum-exp), pt 2.B / es 2.B /
// it 2.B (custom kernels add the key/value gradients in place into gradient pages, outside
// autograd, with atomic adds).
//
// With one page list per query page (pt 2.C) a workgroup of listed keys takes one query page's
// rows and keys from that page's list, so every row block it streams sees all of its keys; the
// chunk's own keys, which every query page sees, run once over all rows.
//
// One workgroup = 4 waves, one per SIMD, each owning 64 keys (two 32-key tiles) of one KV head:
// K of its keys in VGPRs, V in LDS, dK and dV (2 x 64 x d fp32) in accumulation registers for the
// whole row range. The G query heads of the KV head are packed as rows r = t*G + hh and streamed
// in 32-row blocks (Q, dO, -LSE/scale, -D) through a 3-deep LDS ring filled by direct
// global->LDS loads. Per block a wave computes, with the chunk's own-block causal mask,
//   S' = Q K^T - LSE/scale and dP' = dO V^T - D (MFMAs accumulating onto the staged row values),
//   P = exp2(S' * scale * log2 e), dS = P * dP', dV += P^T dO, dK += dS^T Q.
// Rows past the end of the chunk read a padding entry (-inf, 0), so their P and dS are 0.
// Within a wave the blocks are pipelined: the dV/dK MFMAs of block b-1 and the P/dS VALU of
// block b, then the S/dP MFMAs of block b+1 (the two halves independent, so either pipe can run
// ahead). The finished dK/dV are added to the gradient pages with fp32 atomic adds, once per key
// per workgroup.
#include <type_traits>

#include "pkv_device.h"

namespace pkv {

template <int D>
struct DkvCfg {
  static constexpr int NW = 4;                    // waves per workgroup (one per SIMD)
  static constexpr int NKT = 2;                   // 32-key tiles per wave
  static constexpr int BQ = 32;                   // rows per staged block
  static constexpr int NS = 3;                    // staging ring depth
  static constexpr int KS = D / 16;               // MFMA k-steps over d
  static constexpr int DT = D / 32;               // 32-column tiles of d
  static constexpr int CHR = D / 8;               // 16-byte chunks per row
  static constexpr int TILE = BQ * D;             // elements of one staged Q or dO block
  static constexpr int SEG_PER_WAVE = TILE * 2 / 1024 / NW;
  static constexpr int ROWS_PER_SEG = 1024 / (2 * D);
  static constexpr int STAGE_BYTES = 2 * TILE * 2 + 2 * BQ * 4;  // Q, dO, [lse2 | -D]
  static constexpr int VROWS = NKT * 32;          // resident V rows per wave
};
static_assert(DkvCfg<128>::SEG_PER_WAVE == 2 && DkvCfg<64>::SEG_PER_WAVE == 1, "staging split");
static_assert(NKT_TILES_PER_WG == DkvCfg<128>::NW * DkvCfg<128>::NKT, "host plan and kernel disagree");

// x / G for 0 <= x < 2^24 from a float reciprocal, corrected to the exact quotient.
__device__ __forceinline__ int32_t div_small_kv(int32_t x, int32_t G, float invG) {
  int32_t q = (int32_t)((float)x * invG);
  q -= (q * G > x) ? 1 : 0;
  q += ((q + 1) * G <= x) ? 1 : 0;
  return q;
}

template <int D, bool HOST_SPLITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_bwd_dkdv(
    AttnArgs a, BwdExtra e, int32_t n_ku, int32_t row_splits, int32_t own_splits, RowSplits splits,
    const float* __restrict__ ndbuf, const float* __restrict__ nlsbuf, int32_t pad_row) {
  using T = DkvCfg<D>;
  constexpr int BQ = T::BQ;
  constexpr int NKT = T::NKT;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[T::NS * T::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint16_t vres[T::NW * T::VROWS * D];

  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 5, l32 = lane & 31;
  // Wave-uniform, so the LDS destinations of the direct loads stay in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t G = a.G, CG = a.C * G, P = a.page, H = a.h_kv;
  const float invG = 1.0f / (float)G;
  const int32_t q0 = a.n_prior * P;
  const int tsh = (P == 128) ? 2 : 1;  // log2(32-key tiles per page)
  // Units [0, n_full) hold a prior (or listed) key; the rest hold only the chunk's own keys.
  const int32_t prior_tiles = list_prior(a) << tsh, per_unit = T::NW * NKT;
  const int32_t n_full = min(n_ku, (prior_tiles + per_unit - 1) / per_unit);
  // With one page list per query page, a unit with a listed key runs once per query page: its row
  // splits are the query pages (the host plan sets row_splits = n_lists, whose row ranges start
  // and end on query-page boundaries), as a query page's rows see only its own list's pages. The
  // own-key units are seen alike by every query page from their causal diagonal on: with
  // own_splits > 0 they run once over all rows, in own_splits row splits of equal work, as the
  // first workgroups dispatched (the longest; consecutive workgroups go to different XCDs, so they
  // spread over all of them). Otherwise every unit runs in row_splits splits. Row splits vary
  // slowest within a family: the workgroups that run together on one XCD take neighbouring key
  // units of one (KV head, row split) and stream the same query rows through its L2.
  const bool split_own = a.n_lists > 1 && own_splits > 0 && n_full < n_ku;
  const int32_t n_own_wg = split_own ? a.n_kvh * (n_ku - n_full) * own_splits : 0;
  const int32_t n_fam = split_own ? n_full : n_ku;  // key units of the row-split family
  const bool own_family = (int32_t)blockIdx.x < n_own_wg;
  int32_t ku, gi, rs, n_rs;
  if (own_family) {
    const int32_t u = xcd_remap(blockIdx.x, n_own_wg), no = n_ku - n_full;
    ku = n_full + u % no;
    gi = (u / no) % a.n_kvh;
    rs = u / (no * a.n_kvh);
    n_rs = own_splits;
  } else {
    const int32_t u = xcd_remap(blockIdx.x - n_own_wg, a.n_kvh * n_fam * row_splits);
    ku = u % n_fam;
    gi = (u / n_fam) % a.n_kvh;
    rs = u / (n_fam * a.n_kvh);
    n_rs = row_splits;
  }
  const int32_t g = a.kvh0 + gi;
  const int32_t li = (a.n_lists > 1 && !own_family) ? rs : 0;
  const int32_t n_kt = (list_prior(a) + a.C / P) << tsh;
  const int32_t kt_first = ku * (T::NW * NKT);

  // First row any key of this workgroup can see (keys ascend along the list; only the chunk's own
  // pages start later than row 0).
  int32_t wg_kpos_min;
  {
    const int32_t pi0 = kt_first >> tsh;
    const int32_t lp0 = (pi0 < list_prior(a)) ? -1 : a.n_prior + (pi0 - list_prior(a));
    wg_kpos_min = (lp0 < 0) ? 0 : lp0 * P + ((kt_first - (pi0 << tsh)) * 32);
  }
  const int32_t n_blk = (CG + BQ - 1) / BQ;
  int32_t blk_b, blk_e;
  if ((a.n_lists > 1 && !own_family) || n_rs == 1) {
    blk_b = (int32_t)((int64_t)n_blk * rs / n_rs);
    blk_e = (int32_t)((int64_t)n_blk * (rs + 1) / n_rs);
  } else if constexpr (HOST_SPLITS) {
    // Row splits of equal work rather than equal rows (the own-key units start at their causal
    // diagonal, so later blocks carry more units): boundaries from the host plan, which counts
    // 32-row blocks. The search below finds the same boundaries in the kernel; it costs the
    // workgroup about 7 thousand cycles (64-bit arithmetic in a binary search).
    static_assert(BQ == 32, "the plan's row splits count 32-row blocks");
    blk_b = splits.b[rs];
    blk_e = splits.b[rs + 1];
  } else {
    // The same boundaries found in the kernel, in the instantiation launched with one row split,
    // where this branch does not run: with it in the code, the compiler schedules the block loop
    // below 0.7% faster than without. A unit with a prior key streams every row block; a unit of
    // own keys only starts at its causal diagonal, so later blocks carry more units. work(b)
    // counts the (unit, block) pairs of one KV head before block b (of the own-key units only,
    // for their own family), and split r starts at the first block where work reaches r/R of
    // the total, so the splits partition [0, n_blk) exactly. Own unit j >= n_full starts at block
    // G * (j * per_unit - prior_tiles) (32 keys per tile, 32 rows per block): an arithmetic
    // progression, so the sum over units has a closed form.
    static_assert(BQ == 32, "unit start blocks assume 32-row blocks");
    const int32_t s0 = G * (n_full * per_unit - prior_tiles), dlt = G * per_unit;
    auto work = [&](int32_t b) {
      int64_t w = own_family ? 0 : (int64_t)n_full * b;
      if (b > s0) {
        const int64_t k = min<int64_t>(n_ku - n_full, (b - s0 + dlt - 1) / dlt);  // units begun before b
        w += k * (b - s0) - (int64_t)dlt * k * (k - 1) / 2;
      }
      return w;
    };
    const int64_t total = work(n_blk);
    auto split_start = [&](int32_t r) {
      const int64_t target = total * r / n_rs;
      int32_t lo = 0, hi = n_blk;  // first b with work(b) >= target
      while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (work(mid) >= target) hi = mid;
        else lo = mid + 1;
      }
      return lo;
    };
    blk_b = split_start(rs);
    blk_e = rs + 1 == n_rs ? n_blk : split_start(rs + 1);
  }
  if (wg_kpos_min > q0) blk_b = max(blk_b, (G * (wg_kpos_min - q0)) / BQ);
  if (blk_b >= blk_e) return;  // no row of this split sees a key of the unit (uniform per workgroup)

  // Staging with direct global->LDS loads. Wave w fills 1 KiB segments w*SEG_PER_WAVE + j of the
  // Q and dO blocks; lane L lands at segment offset 16 L = (row L / CHR of the segment, physical
  // chunk L % CHR), so it fetches the logical chunk that the swizzle places there. Each lane
  // carries its row r, head hh = r mod G and element offset (t*H_q + hh)*D + chunk from block to
  // block. Rows past the end of the chunk re-read the last row; their row values come from the
  // padding entry. Wave 0 also fetches [-LSE/scale | -D] of the 32 rows.
  const char* qg = reinterpret_cast<const char*>(a.q + (int64_t)g * G * D);
  const char* dg = reinterpret_cast<const char*>(e.dout + (int64_t)g * G * D);
  const int32_t step_q = BQ / G, step_r = BQ - (BQ / G) * G;  // BQ = step_q * G + step_r
  const int32_t d_off = (step_q * a.h_q + step_r) * D, d_wrap = (a.h_q - G) * D;
  const int32_t off_last = ((a.C - 1) * a.h_q + G - 1) * D;
  int32_t st_r[T::SEG_PER_WAVE], st_h[T::SEG_PER_WAVE], st_o[T::SEG_PER_WAVE], st_c[T::SEG_PER_WAVE];
#pragma unroll
  for (int j = 0; j < T::SEG_PER_WAVE; ++j) {
    const int seg = wave * T::SEG_PER_WAVE + j;
    const int rl = seg * T::ROWS_PER_SEG + lane / T::CHR;
    st_r[j] = blk_b * BQ + rl;
    const int32_t t = div_small_kv(st_r[j], G, invG);
    st_h[j] = st_r[j] - t * G;
    st_c[j] = ((lane % T::CHR) ^ swz<D>(rl)) * 8;
    st_o[j] = (t * a.h_q + st_h[j]) * D + st_c[j];
  }
  const bool is_lse = lane < BQ;
  int32_t sl_r, sl_h, sl_i;  // row, head, index (g*G + hh)*C + t into the row arrays
  {
    sl_r = blk_b * BQ + (is_lse ? lane : lane - BQ);
    const int32_t t = div_small_kv(sl_r, G, invG);
    sl_h = sl_r - t * G;
    sl_i = (g * G + sl_h) * a.C + t;
  }
  const int32_t di_off = step_q + step_r * a.C, di_wrap = 1 - G * a.C;
  const float* rowsrc = is_lse ? nlsbuf : ndbuf;
  auto load_blk = [&](int stage) {
    unsigned char* bs = smem + stage * T::STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < T::SEG_PER_WAVE; ++j) {
      const int seg = wave * T::SEG_PER_WAVE + j;
      const uint32_t ob = 2u * (uint32_t)(st_r[j] < CG ? st_o[j] : off_last + st_c[j]);
      g2lds16(qg + ob, bs + seg * 1024);
      g2lds16(dg + ob, bs + T::TILE * 2 + seg * 1024);
      st_r[j] += BQ;
      st_h[j] += step_r;
      st_o[j] += d_off;
      if (st_h[j] >= G) {
        st_h[j] -= G;
        st_o[j] += d_wrap;
      }
    }
    if (wave == 0) g2lds4(rowsrc + (sl_r < CG ? sl_i : pad_row), bs + 2 * T::TILE * 2);
    sl_r += BQ;
    sl_h += step_r;
    sl_i += di_off;
    if (sl_h >= G) {
      sl_h -= G;
      sl_i += di_wrap;
    }
  };

  // The first block's rows do not depend on the key pages: stage them before the table walk and
  // the K/V loads below, so that their latencies overlap.
  load_blk(0);

  // This wave's two 32-key tiles: validity, first key position, gradient page, K/V base.
  bool kval[NKT];
  int32_t kpos[NKT], gph[NKT], tsub[NKT];
  const uint16_t* kbase[NKT];
#pragma unroll
  for (int j = 0; j < NKT; ++j) {
    const int32_t kt_idx = kt_first + wave * NKT + j;
    kval[j] = kt_idx < n_kt;
    kpos[j] = 0;
    gph[j] = -1;
    tsub[j] = 0;
    kbase[j] = nullptr;
    if (kval[j]) {
      const int32_t pi = kt_idx >> tsh;
      tsub[j] = kt_idx & ((1 << tsh) - 1);
      const int32_t lp = list_page(a, g, li, pi);
      const int32_t ph = phys_page(a.bt, a.n_bt, a.n_pool_pages, lp, a.err);
      gph[j] = phys_page(e.gbt, e.n_gbt, e.n_gpool_pages, lp, a.err);
      kval[j] = (ph >= 0) && (gph[j] >= 0);
      kpos[j] = (lp < 0 ? 0 : lp) * P + tsub[j] * 32;
      if (kval[j]) kbase[j] = a.kv + (((int64_t)ph * H + g) * 2) * P * D + (int64_t)tsub[j] * 32 * D;
    }
  }
  // Row r sees key k iff r >= G * (k - q0). Blocks before blk_m hold rows that some key of the
  // workgroup does not see (own pages only) and run the masked, unpipelined path.
  int32_t my_rmin[NKT];
#pragma unroll
  for (int j = 0; j < NKT; ++j) my_rmin[j] = G * (kpos[j] + l32 - q0);
  int32_t blk_m = blk_b;
  {
    const int32_t kt_last = min(kt_first + T::NW * NKT, n_kt) - 1;
    const int32_t pi = kt_last >> tsh;
    if (pi >= list_prior(a)) {
      const int32_t lp = a.n_prior + (pi - list_prior(a));
      const int32_t kpos_last = lp * P + (kt_last - (pi << tsh)) * 32 + 31;
      blk_m = min(blk_e, max(blk_b, (G * (kpos_last - q0) + BQ - 1) / BQ));
    }
  }

  // K of this wave's keys in registers (B operand of S^T = Q K^T); V rows in LDS (B operand of
  // dP^T = dO V^T), both tiles stacked as 64 swizzled rows.
  bf16x8 kreg[NKT][T::KS];
#pragma unroll
  for (int j = 0; j < NKT; ++j)
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      u32x4 x = (u32x4){0u, 0u, 0u, 0u};
      if (kval[j]) x = *reinterpret_cast<const u32x4*>(kbase[j] + (int64_t)l32 * D + ks * 16 + 8 * lg);
      kreg[j][ks] = as_bf16x8(x);
    }
  uint16_t* vmine = vres + wave * T::VROWS * D;
#pragma unroll
  for (int sg = 0; sg < T::VROWS * D * 2 / 1024; ++sg) {
    const int rl = sg * T::ROWS_PER_SEG + lane / T::CHR;
    const int j = rl >> 5;
    const uint16_t* vsrc = kval[j] ? kbase[j] + (int64_t)P * D : a.kv;  // invalid tiles: any bytes
    g2lds16(vsrc + (rl & 31) * D + (((lane % T::CHR) ^ swz<D>(rl)) << 3), vmine + sg * 512);
  }

  const float sl2 = a.scale * kLog2e;
  f32x16 dk[NKT][T::DT], dv[NKT][T::DT];
#pragma unroll
  for (int j = 0; j < NKT; ++j)
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
      dk[j][dt] = (f32x16){};
      dv[j][dt] = (f32x16){};
    }
  f32x16 sacc[NKT], pacc[NKT];
  bf16x8 pb[NKT][2], dsb[NKT][2];  // P and dS of the block whose dV/dK MFMAs run next

  // S' = S^T - LSE/scale and dP' = dP^T - D of the block staged in `stage` (accumulator element i
  // is row 8(i/4) + 4 lg + i%4 of the block, key l32 of tile j).
  auto s_dp = [&](int stage) {
    const uint16_t* qs = reinterpret_cast<const uint16_t*>(smem + stage * T::STAGE_BYTES);
    const uint16_t* dos = qs + T::TILE;
    const float* nl = reinterpret_cast<const float*>(smem + stage * T::STAGE_BYTES + 2 * T::TILE * 2);
    const float* nd = nl + BQ;
#pragma unroll
    for (int j = 0; j < NKT; ++j) {
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(nl + 8 * grp + 4 * lg);
        const f32x4 n4 = *reinterpret_cast<const f32x4*>(nd + 8 * grp + 4 * lg);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sacc[j][grp * 4 + i] = l4[i];
          pacc[j][grp * 4 + i] = n4[i];
        }
      }
    }
    // Operands of k-step ks + 1 are read from LDS while the MFMAs of k-step ks run, so the LDS
    // latency is not exposed before every k-step.
    bf16x8 opq[2], opd[2], opv[2][NKT];
    auto fetch = [&](int ks, int b) {
      const int off = toff<D>(l32, ks * 16 + 8 * lg);
      opq[b] = as_bf16x8(*reinterpret_cast<const u32x4*>(qs + off));
      opd[b] = as_bf16x8(*reinterpret_cast<const u32x4*>(dos + off));
#pragma unroll
      for (int j = 0; j < NKT; ++j) opv[b][j] = as_bf16x8(*reinterpret_cast<const u32x4*>(vmine + j * 32 * D + off));
    };
    fetch(0, 0);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      if (ks + 1 < T::KS) fetch(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int j = 0; j < NKT; ++j) {
        sacc[j] = mfma32(opq[ks & 1], kreg[j][ks], sacc[j]);
        pacc[j] = mfma32(opd[ks & 1], opv[ks & 1][j], pacc[j]);
      }
    }
  };

  // P and dS from sacc/pacc into pn/dn; with MASK, rows outside [my_rmin, CG) are zeroed (blocks
  // on the causal diagonal of the own pages).
  auto p_ds = [&](auto mask_c, int32_t blk, bf16x8 (&pn)[NKT][2], bf16x8 (&dn)[NKT][2]) {
    constexpr bool MASK = decltype(mask_c)::value;
#pragma unroll
    for (int j = 0; j < NKT; ++j) {
      float p[16];
#pragma unroll
      for (int el = 0; el < 16; ++el) p[el] = __builtin_amdgcn_exp2f(sacc[j][el] * sl2);
      if constexpr (MASK) {
        const int32_t rlim = CG - blk * BQ;
        const uint32_t lo = (uint32_t)(my_rmin[j] - blk * BQ), span = (uint32_t)(rlim - (my_rmin[j] - blk * BQ));
#pragma unroll
        for (int el = 0; el < 16; ++el) {
          const int rr = 8 * (el >> 2) + 4 * lg + (el & 3);
          if ((uint32_t)rr - lo >= span) p[el] = 0.f;
        }
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 w, x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int el = hf * 8 + 2 * i;
          w[i] = cvt_pk_bf16(p[el], p[el + 1]);
          x[i] = cvt_pk_bf16(p[el] * pacc[j][el], p[el + 1] * pacc[j][el + 1]);
        }
        pn[j][hf] = as_bf16x8(w);
        dn[j][hf] = as_bf16x8(x);
      }
    }
  };

  // dV[keys][d] += P^T[keys][rows] dO[rows][d] and dK += dS^T Q for the block in
  // `stage`, using pb/dsb. The B operands (rows along the contraction) come from transposed reads
  // of the staged blocks, in the row order of the accumulator layout.
  auto dv_dk = [&](int stage) {
    const uint16_t* qs = reinterpret_cast<const uint16_t*>(smem + stage * T::STAGE_BYTES);
    const uint16_t* dos = qs + T::TILE;
    // The transposed operands of step (hf, dt) + 1 are read while the MFMAs of (hf, dt) run.
    bf16x8 opo[2], opq[2];
    auto fetch = [&](int st, int b) {
      const int k_lo = (st / T::DT) * 16 + 4 * lg, dt = st % T::DT;
      opo[b] = tr_operand<D>(dos, k_lo, k_lo + 8, dt * 32, lane);
      opq[b] = tr_operand<D>(qs, k_lo, k_lo + 8, dt * 32, lane);
    };
    fetch(0, 0);
#pragma unroll
    for (int st = 0; st < 2 * T::DT; ++st) {
      if (st + 1 < 2 * T::DT) fetch(st + 1, (st + 1) & 1);
      const int hf = st / T::DT, dt = st % T::DT;
#pragma unroll
      for (int j = 0; j < NKT; ++j) {
        mfma32_agpr(dv[j][dt], pb[j][hf], opo[st & 1]);
        mfma32_agpr(dk[j][dt], dsb[j][hf], opq[st & 1]);
      }
    }
  };
  using Masked = std::integral_constant<bool, true>;
  using Plain = std::integral_constant<bool, false>;

  // Masked prefix: one block at a time, the next one staged while it runs (stages 0 and 1 in
  // turn; a wave has 2 SEG_PER_WAVE loads per block, wave 0 one more for the row values).
  for (int32_t blk = blk_b; blk < blk_m; ++blk) {
    const int st = (blk - blk_b) & 1;
    if (blk + 1 < blk_m) {
      load_blk(st ^ 1);  // its stage was last read before the barrier that ended the previous block
      if (wave == 0) wait_vmcnt<2 * T::SEG_PER_WAVE + 1>();
      else wait_vmcnt<2 * T::SEG_PER_WAVE>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    s_dp(st);
    p_ds(Masked{}, blk, pb, dsb);
    dv_dk(st);
    __syncthreads();
  }
  if (blk_m < blk_e) {
    // Pipelined part. Prologue: blocks blk_m and blk_m + 1 staged (blk_m already is when there is
    // no masked block), S/dP and P/dS of blk_m, S/dP of blk_m + 1.
    if (blk_m > blk_b) load_blk(0);
    if (blk_m + 1 < blk_e) load_blk(1);
    wait_vmcnt<0>();
    __syncthreads();
    s_dp(0);
    p_ds(Plain{}, blk_m, pb, dsb);
    wait_vmcnt<0>();
    __syncthreads();
    if (blk_m + 2 < blk_e) load_blk(2);
    s_dp(1);  // unused if blk_m is the last block
    int sp = 0, sc = 1;  // stages of blocks blk - 1 and blk
    for (int32_t blk = blk_m + 1; blk < blk_e; ++blk) {
      // dV/dK of blk - 1 on the MFMA pipe, P/dS of blk on the VALU.
      dv_dk(sp);
      p_ds(Plain{}, blk, pb, dsb);
      // The stage of blk - 1 is free once every wave is past this point; blk + 1 has landed.
      wait_vmcnt<0>();
      __syncthreads();
      const int sn = sc == 2 ? 0 : sc + 1;
      if (blk + 2 < blk_e) load_blk(sp);
      s_dp(sn);  // past the last block this reads a stale stage; the result is never used
      sp = sc;
      sc = sn;
    }
    dv_dk(sp);
  }

  // The accumulators are read back below by plain moves, which do not wait for the MFMA pipe.
#pragma unroll
  for (int j = 0; j < NKT; ++j)
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
      agpr_readback_fence(dk[j][dt]);
      agpr_readback_fence(dv[j][dt]);
    }

  // Accumulate into the gradient pages: element (key, d) of dK/dV goes to
  // grad[gphys][g][0/1][sub*32 + key][d]. Lanes of one instruction cover 32 consecutive d.
#pragma unroll
  for (int j = 0; j < NKT; ++j) {
    if (kval[j]) {
      float* gk = e.grad + (((int64_t)gph[j] * H + g) * 2) * P * D + (int64_t)tsub[j] * 32 * D;
      float* gv = gk + (int64_t)P * D;
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
        for (int el = 0; el < 16; ++el) {
          const int key = 8 * (el >> 2) + 4 * lg + (el & 3);
          const int64_t off = (int64_t)key * D + dt * 32 + l32;
          unsafeAtomicAdd(gk + off, dk[j][dt][el] * a.scale);
          unsafeAtomicAdd(gv + off, dv[j][dt][el]);
        }
    }
  }
}

// Workgroups of the dK/dV launch, from the same counts the kernel decodes its unit with.
static int32_t dkdv_workgroups(const AttnArgs& a, const BwdPlan& plan) {
  const int32_t tsh = a.page == 128 ? 2 : 1;
  const int32_t prior_tiles = (a.sel ? a.n_sel : a.n_prior) << tsh;
  const int32_t n_full = std::min(plan.n_ku, (prior_tiles + NKT_TILES_PER_WG - 1) / NKT_TILES_PER_WG);
  if (a.n_lists > 1 && plan.own_splits > 0 && n_full < plan.n_ku)
    return a.n_kvh * ((plan.n_ku - n_full) * plan.own_splits + n_full * plan.row_splits);
  return a.n_kvh * plan.n_ku * plan.row_splits;
}

template <int D>
hipError_t launch_dkdv(const AttnArgs& a, const BwdExtra& e, const BwdPlan& plan, const float* ndbuf,
                       const float* nlsbuf, int32_t pad_row, hipStream_t s) {
  TimerScope ts_("k_bwd_dkdv", s);
  // Equal-work row splits take their boundaries from the plan; a launch with one row split (the
  // dense pass) runs the instantiation whose block loop is scheduled faster.
  const bool host_splits = a.n_lists > 1 || plan.row_splits > 1;
  if (host_splits)
    hipLaunchKernelGGL((k_bwd_dkdv<D, true>), dim3(dkdv_workgroups(a, plan)), dim3(64 * DkvCfg<D>::NW), 0, s, a, e,
                       plan.n_ku, plan.row_splits, plan.own_splits, plan.work_splits, ndbuf, nlsbuf, pad_row);
  else
    hipLaunchKernelGGL((k_bwd_dkdv<D, false>), dim3(dkdv_workgroups(a, plan)), dim3(64 * DkvCfg<D>::NW), 0, s, a, e,
                       plan.n_ku, plan.row_splits, plan.own_splits, plan.work_splits, ndbuf, nlsbuf, pad_row);
  return hipGetLastError();
}

template hipError_t launch_dkdv<64>(const AttnArgs&, const BwdExtra&, const BwdPlan&, const float*, const float*,
                                    int32_t, hipStream_t);
template hipError_t launch_dkdv<128>(const AttnArgs&, const BwdExtra&, const BwdPlan&, const float*, const float*,
                                     int32_t, hipStream_t);

}  // namespace pkv
