// Chunk attention backward, query-major dQ pass with one wave per SIMD and 64 rows per wave.
//
// "Out of the Memory Barrier" summaries: pt 2.A / es 2.A / it 2.A (what the forward dropped is
// recomputed in backward: here the probabilities, from the stored log-sum-exp), pt 2.B / es 2.B /
// it 2.B (keys and values read in place from pages through the block table), pt 2.C / es 2.B /
// it 2.D (sparse mode: selected pages plus the own block).
//
// The work decomposition of k_bwd_dq with 8 waves (row r = t*G + hh; a workgroup = (KV head,
// key-range split, 256-row block); split partials summed by k_bwd_dq_reduce), but the 256 rows go
// to four waves of 64 rows, one wave per SIMD with the whole register file, as in k_attn_fwd64.
// Each wave keeps two 32-row blocks: their dQ^T accumulators and their Q^T and dO^T operands in
// AGPRs, their S^T and dP^T tiles in VGPRs. Every K, V and K^T operand read from LDS feeds both
// blocks, so LDS traffic per MFMA halves against one block per wave.
//
// Per 64-key tile and 32-key half h: S^T = K Q^T and dP^T = V dO^T of both blocks, then
// P^T = exp2(S^T scale log2 e - LSE log2 e), dS^T = P^T (dP^T - D), dQ^T += K^T dS^T. Each half
// runs as one part of three sections of MFMAs, each with VALU work between its MFMAs:
//   1. S^T(h) of both blocks, beside dS^T of the previous half (its P^T and dP^T held);
//   2. dP^T(h) of both blocks, beside P^T(h) of block 0 (exp2 in place of S^T);
//   3. dQ^T of the previous half (its dS^T from section 1), beside P^T(h) of block 1.
// So the held state between parts is one half's P^T and dP^T (64 VGPRs), and S^T of the next
// half is formed beside it. Tiles that need the causal mask (the chunk's own keys at and after
// the block's first row) run a plain loop with the mask; a tile of an unreadable page contributes
// nothing (in the pipelined loop its P^T is forced to 0, in the plain loop it is skipped).
#include "pkv_device.h"

namespace pkv {

template <int D>
struct Dq64Cfg {
  static constexpr int NW = 4;                     // waves per workgroup, one per SIMD
  static constexpr int BK = 64;                    // keys per tile
  static constexpr int KS = D / 16;                // contraction steps over d
  static constexpr int DT = D / 32;                // 32-row tiles of dQ^T
  static constexpr int CHR = D / 8;                // 16-byte chunks per row
  static constexpr int TILE = BK * D;              // elements of one K or V tile
  static constexpr int NS = 4;                     // staging stages (tiles i-1 .. i+2)
  static constexpr int SEG_PER_WAVE = TILE * 2 / 1024 / NW;  // 1 KiB direct-load segments per wave and tile
  static constexpr int ROWS_PER_SEG = 1024 / (2 * D);
};

namespace {

// The state of a section's software pipeline: four floats carried between its MFMAs (the dS^T
// products of section 1, or the scaled scores of sections 2 and 3). The written-out MFMAs pass it
// through unchanged ("+v", untouched by the instruction): work that updates it can neither issue
// before the MFMA it follows nor sink past the next one, which keeps each slot of VALU work between
// its two MFMAs (the instruction selector would otherwise cluster the arithmetic).
struct Pipe4 {
  float v[4];
};
#define PKV_PIPE4(p) "+v"(p.v[0]), "+v"(p.v[1]), "+v"(p.v[2]), "+v"(p.v[3])
// S^T or dP^T MFMA with the Q^T or dO^T operand in AGPRs (first step from 0, later steps in place).
__device__ __forceinline__ void mfma_sd_first(f32x16& d, const bf16x8& a, const bf16x8& b, Pipe4& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %5, %6, 0" : "=&v"(d), PKV_PIPE4(p) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_sd(f32x16& d, const bf16x8& a, const bf16x8& b, Pipe4& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %5, %6, %0" : "+v"(d), PKV_PIPE4(p) : "v"(a), "a"(b));
}
// dQ^T MFMA with its accumulator in AGPRs.
__device__ __forceinline__ void mfma_dq(f32x16& c, const bf16x8& a, const bf16x8& b, Pipe4& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %5, %6, %0" : "+a"(c), PKV_PIPE4(p) : "v"(a), "v"(b));
}
#undef PKV_PIPE4
// The forms without VALU work alongside (the plain loop).
__device__ __forceinline__ void mfma_sd_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_sd(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// An empty volatile statement that takes a value and gives it back (orders the work producing it).
template <typename V>
__device__ __forceinline__ void dq_pin(V& x) {
  asm volatile("" : "+v"(x));
}
// Operands of B loaded straight into AGPRs (KS 16-byte loads, 32 bytes apart), waiting for
// themselves inside the statement so that the registers are complete when it ends.
template <int KS>
__device__ __forceinline__ void load_agpr(bf16x8 (&q)[KS], const uint16_t* p) {
  if constexpr (KS == 8) {
    asm volatile(
        "global_load_dwordx4 %0, %8, off\n\tglobal_load_dwordx4 %1, %8, off offset:32\n\t"
        "global_load_dwordx4 %2, %8, off offset:64\n\tglobal_load_dwordx4 %3, %8, off offset:96\n\t"
        "global_load_dwordx4 %4, %8, off offset:128\n\tglobal_load_dwordx4 %5, %8, off offset:160\n\t"
        "global_load_dwordx4 %6, %8, off offset:192\n\tglobal_load_dwordx4 %7, %8, off offset:224\n\t"
        "s_waitcnt vmcnt(0)"
        : "=a"(q[0]), "=a"(q[1]), "=a"(q[2]), "=a"(q[3]), "=a"(q[4]), "=a"(q[5]), "=a"(q[6]), "=a"(q[7])
        : "v"(p)
        : "memory");
  } else {
    static_assert(KS == 4, "head_dim 64 or 128");
    asm volatile(
        "global_load_dwordx4 %0, %4, off\n\tglobal_load_dwordx4 %1, %4, off offset:32\n\t"
        "global_load_dwordx4 %2, %4, off offset:64\n\tglobal_load_dwordx4 %3, %4, off offset:96\n\t"
        "s_waitcnt vmcnt(0)"
        : "=a"(q[0]), "=a"(q[1]), "=a"(q[2]), "=a"(q[3])
        : "v"(p)
        : "memory");
  }
}
// XDL write of an S^T or dP^T pair, then VALU reads: the MFMA's pass count plus 2 wait states;
// three s_nop 7 give 24 and order every read of the tiles after the statement.
__device__ __forceinline__ void xdl_fence2(f32x16 (&s)[2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]));
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_bwd_dq64(
    AttnArgs a, BwdExtra e, int32_t n_rb, int32_t splits, const float* __restrict__ ndbuf,
    const float* __restrict__ lse2buf, float* __restrict__ ws_dq) {
  using T = Dq64Cfg<D>;
  constexpr int BK = T::BK;
  constexpr int KS = T::KS, DT = T::DT;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[T::NS * 2 * T::TILE];  // [stage][K|V]

  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t n_units = a.n_kvh * splits * n_rb;
  const int32_t u = xcd_remap(blockIdx.x, n_units);
  const int32_t rb = n_rb - 1 - u % n_rb;  // row blocks last to first (longest first), as k_bwd_dq
  const int32_t sp = (u / n_rb) % splits;
  const int32_t gi = u / (n_rb * splits);
  const int32_t g = a.kvh0 + gi;
  const int32_t G = a.G, CG = a.C * G, P = a.page;
  const int32_t RL = CG / a.n_lists;
  const int32_t bpl = (RL + 255) / 256;
  const int32_t li = rb / bpl;
  const int32_t r0 = li * RL + (rb - li * bpl) * 256;
  const int32_t r_end = min(r0 + 256, (li + 1) * RL);
  const int32_t r_last = r_end - 1;
  const int32_t t_min = r0 / G, t_max = r_last / G;
  const int32_t q0 = a.n_prior * P;
  const int tsh = (P == 128) ? 1 : 0;
  const int32_t n_prior_tiles = list_prior(a) << tsh;
  const int32_t n_tiles = n_prior_tiles + t_max / BK + 1;
  const int32_t tb = (int32_t)((int64_t)n_tiles * sp / splits);
  const int32_t te = (int32_t)((int64_t)n_tiles * (sp + 1) / splits);
  // Tiles whose every key is at or before the block's first row need no causal mask.
  const int32_t n_free = n_prior_tiles + (t_min + 1) / BK;
  const int32_t em = max(tb, min(te, n_free));  // pipelined tiles [tb, em), masked tiles [em, te)

  // This lane's two query rows (blocks c = 0, 1 of the wave): Q^T and dO^T operands, row values.
  int32_t tq[2], hh[2], lim[2];
  bool rvalid[2];
  float lse2[2], nd[2];
  bf16x8 qreg[2][KS], doreg[2][KS];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int32_t row = r0 + wave * 64 + c * 32 + l32;
    rvalid[c] = row < r_end;
    const int32_t rr = rvalid[c] ? row : r_last;
    tq[c] = rr / G;
    hh[c] = g * G + (rr - tq[c] * G);
    lim[c] = q0 + tq[c];
    // Rows past the block's end read the last row's values (in bounds); their dQ is dropped.
    const int64_t off = ((int64_t)tq[c] * a.h_q + hh[c]) * D + 8 * lg;
    load_agpr<KS>(qreg[c], a.q + off);
    load_agpr<KS>(doreg[c], e.dout + off);
    const int64_t si = (int64_t)hh[c] * a.C + tq[c];
    lse2[c] = lse2buf[si];
    nd[c] = ndbuf[si];
  }

  KeyWalk walk;  // the key-list walk of the loop being run (each loop starts its own)
  uint32_t seg_off[T::SEG_PER_WAVE];
#pragma unroll
  for (int j = 0; j < T::SEG_PER_WAVE; ++j) {
    const int rl = (wave * T::SEG_PER_WAVE + j) * T::ROWS_PER_SEG + lane / T::CHR;
    seg_off[j] = 2u * (uint32_t)(rl * D + (((lane % T::CHR) ^ swz<D>(rl)) << 3));
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)lds);
  struct TileSrc {
    const uint16_t* k;
    const uint16_t* v;
    uint32_t kb;
  };
  auto tile_src = [&](int stage, int32_t& kp) -> TileSrc {
    const uint16_t* src = walk_take<D>(a, walk, kp);
    if (src == nullptr) src = a.kv;  // unreadable page: any in-bounds bytes, the tile is skipped
    return TileSrc{src, src + (int64_t)P * D, lds_base + (uint32_t)stage * 4u * T::TILE};
  };
  auto tile_seg = [&](const TileSrc& ts, int kv, int j) {
    const uint32_t seg = (uint32_t)(wave * T::SEG_PER_WAVE + j) * 1024u;
    g2lds16_sbase(kv ? ts.v : ts.k, seg_off[j], ts.kb + (kv ? 2u * T::TILE : 0u) + seg);
  };
  auto load_tile = [&](int stage) -> int32_t {
    int32_t kp;
    const TileSrc ts = tile_src(stage, kp);
#pragma unroll
    for (int j = 0; j < T::SEG_PER_WAVE; ++j) {
      tile_seg(ts, 0, j);
      tile_seg(ts, 1, j);
    }
    return kp;
  };

  // LDS byte offsets of this lane's operands within a stage: the K or V operand of contraction
  // step ks (row l32 of a 32-key half, columns 16 ks + 8 lg), and half kh of the K^T operand of
  // d-tile dt (the layout of the forward's V^T operand); per-lane parts plus per-lane patterns
  // XORed with the step's chunk bits, as in k_attn_fwd64.
  uint32_t kA, kZ, vA[2], vZ[2];
  {
    const int sw = swz<D>(l32);
    kA = 2u * (uint32_t)(l32 * D) + 16u * (uint32_t)((lg ^ sw) & 1);
    kZ = 16u * (uint32_t)(sw & ~1);
    const int rr = (lane & 15) >> 2, cb = 16 * ((lane >> 4) & 1) + 4 * (lane & 3), c3 = cb >> 3;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int row = 4 * lg + rr + 8 * kh, swv = swz<D>(row);
      vA[kh] = 2u * (uint32_t)(row * D) + 16u * (uint32_t)((c3 ^ swv) & 3) + 2u * (uint32_t)(cb & 7);
      vZ[kh] = 16u * (uint32_t)(swv & ~3);
    }
  }
  auto koffs = [&](int ks) -> uint32_t { return (kZ ^ (32u * (uint32_t)ks)) + kA; };
  auto toffs = [&](int dt, int kh) -> uint32_t { return (vZ[kh] ^ (64u * (uint32_t)dt)) + vA[kh]; };
  auto stage_ptr = [&](int stage) { return reinterpret_cast<const char*>(lds + stage * 2 * T::TILE); };

  const float sl2 = a.scale * kLog2e;
  // dQ^T accumulators, zeroed here and made opaque, so that the zeros are not formed again right
  // before the first MFMA that accumulates onto them (a VALU write of an MFMA's C operand needs 2
  // wait states, which the compiler does not insert before inline assembly).
  f32x16 dq[2][DT];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dq[c][dt] = (f32x16){};
      asm volatile("" : "+a"(dq[c][dt]));
    }

  // K^T operand (dt, hf) of key half k2 of the tile at kt (two transposing LDS reads).
  auto ktop = [&](const char* kt, int k2, int hf, int dt) -> bf16x8 {
    const int rowb = (k2 * 32 + hf * 16) * D * 2;
    const u32x2 lo = lds_tr16(reinterpret_cast<const uint16_t*>(kt + toffs(dt, 0) + rowb));
    const u32x2 hi = lds_tr16(reinterpret_cast<const uint16_t*>(kt + toffs(dt, 1) + rowb));
    return as_bf16x8((u32x4){lo[0], lo[1], hi[0], hi[1]});
  };
  // K or V operand of contraction step ks of key half k2 of the tile at t.
  auto rowop = [&](const char* t, int k2, int ks) -> bf16x8 {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(t + koffs(ks) + (uint32_t)(k2 * 32 * D * 2)));
  };

  // Software pipeline of one part (one key half h of a tile): three sections of NM MFMAs each, one
  // slot of VALU work after every MFMA, fenced with sched_barrier so that the order written is the
  // order issued; the LDS operands of each section are read two MFMA groups ahead.
  constexpr int NM = 2 * KS;   // MFMAs per section
  constexpr int E1 = 32 / NM;  // dS^T elements per slot of section 1 (both blocks)
  constexpr int E2 = 16 / NM;  // P^T elements per slot of sections 2 and 3 (one block)
  static_assert(E1 * NM == 32 && E2 * NM == 16 && E1 <= 4 && (E1 & 1) == 0, "slot sizes");
  // Section-1 slot m: dS^T = P^T (dP^T - D) of elements m*E1.. of the held half (po, dp), packed.
  auto slot1 = [&](int m, const f32x16 (&po)[2], const f32x16 (&dp)[2], Pipe4& pp, u32x4 (&ds)[2][2]) {
#pragma unroll
    for (int q = 0; q < E1; ++q) {
      const int el = m * E1 + q, c = el >> 4, e = el & 15;
      pp.v[q] = po[c][e] * (dp[c][e] + nd[c]);
    }
#pragma unroll
    for (int q = 0; q < E1; q += 2) {
      const int el = m * E1 + q, c = el >> 4, e = el & 15;
      uint32_t w = cvt_pk_bf16(pp.v[q], pp.v[q + 1]);
      dq_pin(w);
      ds[c][e >> 3][(e & 7) >> 1] = w;
    }
  };
  // Section-2/3 slot m: P^T = exp2 of elements m*E2.. of block c, in place of S^T; then the scaled
  // and shifted scores of the next elements.
  auto slot2_first = [&](int c, const f32x16 (&sn)[2], const float (&sh)[2], Pipe4& pp) {
#pragma unroll
    for (int q = 0; q < E2; ++q) pp.v[q] = __builtin_fmaf(sn[c][q], sl2, -sh[c]);
  };
  auto slot2 = [&](int m, int c, f32x16 (&sn)[2], const float (&sh)[2], Pipe4& pp) {
#pragma unroll
    for (int q = 0; q < E2; ++q) {
      const int el = m * E2 + q;
      float x = __builtin_amdgcn_exp2f(pp.v[q]);
      dq_pin(x);
      sn[c][el] = x;
    }
    if ((m + 1) * E2 < 16) {
#pragma unroll
      for (int q = 0; q < E2; ++q) pp.v[q] = __builtin_fmaf(sn[c][(m + 1) * E2 + q], sl2, -sh[c]);
    }
  };
  // P^T of block c of a tile pair without MFMAs alongside.
  auto exp_plain = [&](int c, f32x16 (&sn)[2], const float (&sh)[2]) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sn[c][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sn[c][e], sl2, -sh[c]));
  };
  // One part: S^T(h) of both blocks into sn and dP^T(h) into dp for key half k2s of the tile in
  // stage ss, P^T(h) in place of sn (exp2 of S^T scale log2 e - sh: sh is LSE log2 e, or +inf
  // for a tile of an unreadable page, whose P^T and dS^T are then 0). With WD, the held previous
  // half (P^T po, dP^T dp) becomes dS^T in section 1 and its dQ^T MFMAs (key half k2q of the tile
  // in stage sq) run in section 3. With LD, the direct loads of tile source ts (K segments when
  // kv = 0, V when 1), spread over sections 1 and 2.
  auto part = [&](auto wd, auto ld, int ss, int k2s, const float (&sh)[2], f32x16 (&sn)[2], const f32x16 (&po)[2],
                  f32x16 (&dp)[2], int sq, int k2q, const TileSrc& ts, int kv) {
    constexpr bool WD = decltype(wd)::value, LD = decltype(ld)::value;
    constexpr int GPS = 2 * KS / T::SEG_PER_WAVE;  // groups per direct-load segment
    const char* kt = stage_ptr(ss);
    const char* vt = kt + 2 * T::TILE;
    Pipe4 pp;
#pragma unroll
    for (int q = 0; q < 4; ++q) pp.v[q] = 0.f;
    u32x4 ds[2][2];
    // Section 1: S^T(h) beside dS^T of the held half.
    {
      bf16x8 op[KS];
      op[0] = rowop(kt, k2s, 0);
      op[1] = rowop(kt, k2s, 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 2 < KS) op[ks + 2] = rowop(kt, k2s, ks + 2);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (ks == 0)
            mfma_sd_first(sn[c], op[ks], qreg[c][ks], pp);
          else
            mfma_sd(sn[c], op[ks], qreg[c][ks], pp);
          if constexpr (WD) slot1(2 * ks + c, po, dp, pp, ds);
        }
        if constexpr (LD) {
          if (ks % GPS == 1) tile_seg(ts, kv, ks / GPS);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    xdl_fence2(sn);
    // Section 2: dP^T(h) beside P^T(h) of block 0.
    {
      bf16x8 op[KS];
      op[0] = rowop(vt, k2s, 0);
      op[1] = rowop(vt, k2s, 1);
      slot2_first(0, sn, sh, pp);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 2 < KS) op[ks + 2] = rowop(vt, k2s, ks + 2);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (ks == 0)
            mfma_sd_first(dp[c], op[ks], doreg[c][ks], pp);
          else
            mfma_sd(dp[c], op[ks], doreg[c][ks], pp);
          slot2(2 * ks + c, 0, sn, sh, pp);
        }
        if constexpr (LD) {
          if (ks % GPS == 1) tile_seg(ts, kv, T::SEG_PER_WAVE / 2 + ks / GPS);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Section 3: dQ^T of the held half beside P^T(h) of block 1 (without a held half: P^T alone,
    // and a fence before the next part's VALU reads dP^T).
    if constexpr (WD) {
      const char* qt = stage_ptr(sq);
      bf16x8 top[2 * DT];
      top[0] = ktop(qt, k2q, 0, 0);
      top[1] = ktop(qt, k2q, 1 / DT, 1 % DT);
      slot2_first(1, sn, sh, pp);
#pragma unroll
      for (int j = 0; j < 2 * DT; ++j) {
        if (j + 2 < 2 * DT) top[j + 2] = ktop(qt, k2q, (j + 2) / DT, (j + 2) % DT);
        const int hf = j / DT, dt = j % DT;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          mfma_dq(dq[c][dt], top[j], as_bf16x8(ds[c][hf]), pp);
          slot2(2 * j + c, 1, sn, sh, pp);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (NM < 12) xdl_fence2(dp);  // fewer MFMAs than the XDL-to-VALU wait between
    } else {
      exp_plain(1, sn, sh);
      xdl_fence2(dp);
    }
  };
  // Plain forms (masked tiles): S^T and dP^T of key half k2 of both blocks, then dS^T with the
  // mask, then dQ^T.
  auto sdp_plain = [&](int stage, int k2, f32x16 (&sn)[2], f32x16 (&dp)[2]) {
    const char* kt = stage_ptr(stage);
    const char* vt = kt + 2 * T::TILE;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ko = rowop(kt, k2, ks), vo = rowop(vt, k2, ks);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (ks == 0) {
          mfma_sd_first(sn[c], ko, qreg[c][ks]);
          mfma_sd_first(dp[c], vo, doreg[c][ks]);
        } else {
          mfma_sd(sn[c], ko, qreg[c][ks]);
          mfma_sd(dp[c], vo, doreg[c][ks]);
        }
      }
    }
    xdl_fence2(sn);
    xdl_fence2(dp);
  };
  // dS^T of a half from its S^T (EXP: P^T computed here, with the mask when MASK) or from its P^T.
  auto ds_plain = [&](auto exp_c, auto mask_c, const f32x16 (&sn)[2], const f32x16 (&dp)[2], int32_t kpos0, int k2,
                      u32x4 (&ds)[2][2]) {
    constexpr bool EXP = decltype(exp_c)::value, MASK = decltype(mask_c)::value;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float y[16];
#pragma unroll
      for (int el = 0; el < 16; ++el) {
        float p = EXP ? __builtin_amdgcn_exp2f(__builtin_fmaf(sn[c][el], sl2, -lse2[c])) : sn[c][el];
        if constexpr (MASK) {
          const int32_t key = kpos0 + k2 * 32 + 8 * (el >> 2) + 4 * lg + (el & 3);
          if (key > lim[c]) p = 0.f;
        }
        y[el] = p * (dp[c][el] + nd[c]);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 4; ++j) ds[c][hf][j] = cvt_pk_bf16(y[hf * 8 + 2 * j], y[hf * 8 + 2 * j + 1]);
    }
  };
  auto dq_plain = [&](int stage, int k2, const u32x4 (&ds)[2][2]) {
    const char* kt = stage_ptr(stage);
#pragma unroll
    for (int j = 0; j < 2 * DT; ++j) {
      const int hf = j / DT, dt = j % DT;
      const bf16x8 to = ktop(kt, k2, hf, dt);
      mfma32_agpr(dq[0][dt], to, as_bf16x8(ds[0][hf]));
      mfma32_agpr(dq[1][dt], to, as_bf16x8(ds[1][hf]));
    }
  };
  auto tile_end = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // Tile boundary of the pipelined loop: this wave's direct loads of every staged tile but the
  // newest (when `newest_pending`) have landed and its LDS operations are complete; then the
  // workgroup barrier, without a memory fence, so the newest tile's loads stay in flight across it.
  // The waits are builtins, so the compiler's own count of pending LDS and scalar operations
  // restarts at zero after them. The direct loads are the only vector-memory operations in the
  // loop (table entries are scalar loads): the newest tile is 2 x SEG_PER_WAVE loads of this wave.
  auto tile_wait = [&](bool newest_pending) {
    constexpr int N = 2 * T::SEG_PER_WAVE;
    asm volatile("" ::: "memory");
    if (newest_pending)
      __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));  // vmcnt(N) lgkmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0x7 << 4);  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS read is moved above the barrier
  };
  using kOff = std::integral_constant<bool, false>;
  using kOn = std::integral_constant<bool, true>;
  const TileSrc no_src{a.kv, a.kv, lds_base};

  if (tb < em) {
    walk = walk_begin(a, g, li, tsh, tb, em);
    // Tile t of the range is staged in stage (t - tb) % 4, two tiles ahead of the one computed.
    // A tile of an unreadable page runs like any other with its P^T forced to 0 (no branch in the
    // loop: an exit would fork the accumulators' register assignment).
    auto shift = [&](int32_t kp, float (&sh)[2]) {
      sh[0] = kp < 0 ? INFINITY : lse2[0];
      sh[1] = kp < 0 ? INFINITY : lse2[1];
    };
    int32_t kpc = load_tile(0);
    int32_t kpn = load_tile(1);  // staged even past the range, like every later tile
    tile_wait(true);             // tile tb has landed
    // P^T (in place of S^T) of key half 0 (sa) and half 1 (sb) of the latest tiles; dP^T of the
    // latest half.
    f32x16 sa[2], sb[2], dp[2];
    float sh[2];
    shift(kpc, sh);
    part(kOff{}, kOff{}, 0, 0, sh, sa, sb, dp, 0, 0, no_src, 0);
    const int32_t kp2 = load_tile(2);
    part(kOn{}, kOff{}, 0, 1, sh, sb, sa, dp, 0, 0, no_src, 0);
    tile_wait(true);  // tile tb + 1 has landed
    kpc = kpn;
    kpn = kp2;
    for (int32_t i = tb + 1; i < em; ++i) {
      // Stage indices kept opaque, so that operand addresses are formed per use.
      int sc = (i - tb) & 3, sprev = (i - 1 - tb) & 3;
      asm("" : "+s"(sc), "+s"(sprev));
      int32_t kp2n;
      const TileSrc ts = tile_src((i + 2 - tb) & 3, kp2n);
      shift(kpc, sh);
      part(kOn{}, kOn{}, sc, 0, sh, sa, sb, dp, sprev, 1, ts, 0);  // with dQ^T of half 1 of tile i-1
      part(kOn{}, kOn{}, sc, 1, sh, sb, sa, dp, sc, 0, ts, 1);     // with dQ^T of half 0 of tile i
      tile_wait(true);  // tile i+1 has landed
      kpc = kpn;
      kpn = kp2n;
    }
    // Half 1 of the last tile.
    u32x4 ds[2][2];
    ds_plain(kOff{}, kOff{}, sb, dp, 0, 1, ds);
    dq_plain((em - 1 - tb) & 3, 1, ds);
    tile_end();
  }
  // Plain loop over [em, te): the tiles at the causal diagonal (masked; a tile of an unreadable page
  // is skipped), double-buffered through stages 0 and 1.
  if (em < te) {
    f32x16 sn[2], dp[2];
    u32x4 ds[2][2];
    walk = walk_begin(a, g, li, tsh, em, te);
    int32_t kp0 = load_tile(0);
    tile_end();
    for (int32_t i = em; i < te; ++i) {
      const int st = (i - em) & 1;
      const int32_t kp1 = (i + 1 < te) ? load_tile(st ^ 1) : -1;
      if (kp0 >= 0) {
        const bool masked = i >= n_free;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          sdp_plain(st, k2, sn, dp);
          if (masked)
            ds_plain(kOn{}, kOn{}, sn, dp, kp0, k2, ds);
          else
            ds_plain(kOn{}, kOff{}, sn, dp, kp0, k2, ds);
          dq_plain(st, k2, ds);
        }
      }
      tile_end();
      kp0 = kp1;
    }
  }

  // Epilogue: dQ of both row blocks (scaled to bf16, or fp32 partials of this split).
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) agpr_readback_fence(dq[c][dt]);
  const int64_t rows_total = (int64_t)a.n_kvh * CG;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (!rvalid[c]) continue;
    int32_t tqc = tq[c], hhc = hh[c];
    dq_pin(tqc);
    dq_pin(hhc);
    if (splits == 1) {
      uint16_t* dp = e.dq + ((int64_t)tqc * a.h_q + hhc) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          u32x2 w;
          w[0] = cvt_pk_bf16(dq[c][dt][grp * 4 + 0] * a.scale, dq[c][dt][grp * 4 + 1] * a.scale);
          w[1] = cvt_pk_bf16(dq[c][dt][grp * 4 + 2] * a.scale, dq[c][dt][grp * 4 + 3] * a.scale);
          *reinterpret_cast<u32x2*>(dp + dt * 32 + grp * 8 + 4 * lg) = w;
        }
    } else {
      const int64_t R = (int64_t)gi * CG + r0 + wave * 64 + c * 32 + l32;
      float* wp = ws_dq + ((int64_t)sp * rows_total + R) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          f32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = dq[c][dt][grp * 4 + j];
          *reinterpret_cast<f32x4*>(wp + dt * 32 + grp * 8 + 4 * lg) = w;
        }
    }
  }
}

template <int D>
hipError_t launch_dq64(const AttnArgs& a, const BwdExtra& e, int32_t n_rb, int32_t splits, const float* ndbuf,
                       const float* lse2buf, float* ws_dq, hipStream_t s) {
  const int32_t n_units = a.n_kvh * splits * n_rb;
  hipLaunchKernelGGL(k_bwd_dq64<D>, dim3(n_units), dim3(256), 0, s, a, e, n_rb, splits, ndbuf, lse2buf, ws_dq);
  return hipGetLastError();
}

template hipError_t launch_dq64<128>(const AttnArgs&, const BwdExtra&, int32_t, int32_t, const float*, const float*,
                                     float*, hipStream_t);
template hipError_t launch_dq64<64>(const AttnArgs&, const BwdExtra&, int32_t, int32_t, const float*, const float*,
                                    float*, hipStream_t);

}  // namespace pkv
