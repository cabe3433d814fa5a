// Chunk attention forward over the paged KV cache, one wave per SIMD with 64 rows per wave.
//
// "Out of the Memory Barrier" summaries: pt 2.A / es 2.A / it 2.A (a chunk attends to every earlier
// key and its own causal block), pt 2.B / es 2.B / it 2.B (keys and values read in place from pages
// through the block table), pt 2.C / es 2.B / it 2.D (sparse mode: selected pages plus the own block).
//
// The same work decomposition as k_attn_fwd (row r = t*G + hh; a workgroup = (KV head, key-range
// split, 256-row block); split partials merged by k_fwd_combine), but the 256 rows go to four waves
// of 64 rows, one wave per SIMD with the whole register file. Each wave keeps two 32-row blocks:
// their O^T accumulators (2 x d/32 32x32 tiles) sit in AGPRs, their Q^T operands and S^T tiles in
// VGPRs, and every K or V^T operand read from LDS feeds both blocks, so LDS traffic per MFMA halves.
//
// Overlap inside the wave instead of between waves: per 64-key tile the wave issues the S^T MFMAs
// of block 0, then those of block 1 among block 0's softmax VALU work (exp2, row sum, bf16 pack),
// then block 0's P^T V MFMAs among block 1's softmax, then block 1's P^T V MFMAs; each stretch is
// branch-free so the scheduler can interleave MFMA and VALU. To keep it so, the fast loop never
// touches O outside the MFMAs: each row's reference maximum is fixed by its first tile, and later
// tiles exponentiate against it. Values above the reference are fine up to p = 2^64 (fp32 and bf16
// keep their relative precision across the exponent range); a tile whose row sum exceeds that
// leaves the fast loop before its P^T V MFMAs for a general loop that moves the reference and
// rescales O (never met on ordinary data). The general loop also runs each range's first tile and
// the tiles at the causal diagonal (with the mask), and a tile of an unreadable page is skipped.
// K/V tiles are double-buffered in LDS by direct loads written out as assembly, so the compiler
// adds no wait for them before the transposed LDS reads of the other stage; each tile ends with an
// explicit wait and barrier.
#include "pkv_device.h"

namespace pkv {

template <int D>
struct Fwd64Cfg {
  static constexpr int NW = 4;                     // waves per workgroup, one per SIMD
  static constexpr int BK = 64;                    // keys per tile
  static constexpr int KS = D / 16;                // contraction steps over d
  static constexpr int DT = D / 32;                // 32-row tiles of O^T
  static constexpr int CHR = D / 8;                // 16-byte chunks per row
  static constexpr int TILE = BK * D;              // elements of one K or V tile
  static constexpr int NS = 4;                     // staging stages (fast loop: tiles i-1 .. i+2)
  static constexpr int SEG_PER_WAVE = TILE * 2 / 1024 / NW;  // 1 KiB direct-load segments per wave and tile
  static constexpr int ROWS_PER_SEG = 1024 / (2 * D);
};

constexpr float kRescaleLog2w = 8.0f;  // general loop: move the reference when a row grew by 2^8
constexpr float kFastSumLimit = 18446744073709551616.0f;  // 2^64: fast loop's bound on a lane's tile sum

// S^T MFMAs with the Q^T operand in AGPRs: the wave keeps Q^T and O^T in the AGPR half of its
// register file and the score tiles in the VGPR half. Written out because only assembly names an
// AGPR source operand; the hazard padding is that of mfma32_agpr (2 wait states after a VALU write
// of an operand). The first step of a chain starts from 0 and may not share a register with the
// VGPR operand (early clobber); later steps accumulate in place.
// The fast loop's forms also pass the softmax pipeline state (SoftPipe) through unchanged ("+v",
// untouched by the instruction): softmax work that uses the state cannot issue before the MFMA,
// and work that updates it cannot sink past the next one, which keeps the order written.
template <int EPS>
struct SoftPipe {
  float tok;     // the reference (scaled maximum) of the rows
  float f[EPS];  // fma results of the next element block
  float e[EPS];  // exp2 results of the current element block
  float ep;      // one element per block: the previous element's exp2 (first of its bf16 pair)
};
#define PKV_PIPE_OUT1(p) "+v"(p.tok), "+v"(p.f[0]), "+v"(p.e[0]), "+v"(p.ep)
#define PKV_PIPE_OUT2(p) "+v"(p.tok), "+v"(p.f[0]), "+v"(p.f[1]), "+v"(p.e[0]), "+v"(p.e[1])
__device__ __forceinline__ void mfma_s_first(f32x16& d, const bf16x8& a, const bf16x8& b, SoftPipe<1>& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %5, %6, 0" : "=&v"(d), PKV_PIPE_OUT1(p) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_s(f32x16& d, const bf16x8& a, const bf16x8& b, SoftPipe<1>& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %5, %6, %0" : "+v"(d), PKV_PIPE_OUT1(p) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_pv(f32x16& c, const bf16x8& a, const bf16x8& b, SoftPipe<1>& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %5, %6, %0" : "+a"(c), PKV_PIPE_OUT1(p) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_first(f32x16& d, const bf16x8& a, const bf16x8& b, SoftPipe<2>& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %6, %7, 0" : "=&v"(d), PKV_PIPE_OUT2(p) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_s(f32x16& d, const bf16x8& a, const bf16x8& b, SoftPipe<2>& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %6, %7, %0" : "+v"(d), PKV_PIPE_OUT2(p) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_pv(f32x16& c, const bf16x8& a, const bf16x8& b, SoftPipe<2>& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %6, %7, %0" : "+a"(c), PKV_PIPE_OUT2(p) : "v"(a), "v"(b));
}
#undef PKV_PIPE_OUT1
#undef PKV_PIPE_OUT2
// The forms without softmax alongside (first tile, last tile, general loop).
__device__ __forceinline__ void mfma32_qa_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma32_qa(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// An empty volatile statement that takes a value and gives it back: work that produced the value
// cannot sink past it, and volatile statements keep their written order. With the state passed
// through the MFMA statements this pins each softmax slot between two MFMAs (the instruction
// selector would otherwise cluster the arithmetic, which has no order of its own).
template <typename V>
__device__ __forceinline__ void issue_pin(V& x) {
  asm volatile("" : "+v"(x));
}

// Q^T operands of one row block loaded straight into AGPRs (KS 16-byte loads, 32 bytes apart), so
// that the register allocator never moves them through VGPRs. The loads are written out for the
// AGPR destinations and wait for themselves inside the statement (their registers are complete
// when it ends).
template <int KS>
__device__ __forceinline__ void load_q_agpr(bf16x8 (&q)[KS], const uint16_t* p) {
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

// The written-out MFMAs' results may be read by VALU only after the MFMA's pass count plus 2 wait
// states (the XDL-write / VALU-read rule); one fence after a block's last S^T MFMA gives 24 for its
// two accumulators (or both blocks'), and orders every read of them after it.
__device__ __forceinline__ void xdl_vgpr_fence(f32x16 (&s)[2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]));
}
__device__ __forceinline__ void xdl_vgpr_fence2(f32x16 (&s)[2], f32x16 (&t)[2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]), "+v"(t[0]), "+v"(t[1]));
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_attn_fwd64(
    AttnArgs a, int32_t n_rb, int32_t splits, uint16_t* __restrict__ o, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_lse) {
  using T = Fwd64Cfg<D>;
  constexpr int BK = T::BK;
  constexpr int KS = T::KS, DT = T::DT;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[T::NS * 2 * T::TILE];  // [stage][K|V]

  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t n_units = a.n_kvh * splits * n_rb;
  const int32_t u = xcd_remap(blockIdx.x, n_units);
  const int32_t rb = n_rb - 1 - u % n_rb;  // row blocks last to first (longest first), as k_attn_fwd
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

  // This lane's two query rows (blocks c = 0, 1 of the wave) and their Q^T operands.
  int32_t tq[2], hh[2];
  bool rvalid[2];
  bf16x8 qreg[2][KS];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int32_t row = r0 + wave * 64 + c * 32 + l32;
    rvalid[c] = row < r_end;
    const int32_t rr = rvalid[c] ? row : r_last;
    tq[c] = rr / G;
    hh[c] = g * G + (rr - tq[c] * G);
    // Rows past the block's end read the last row's queries (in bounds); their outputs are dropped.
    load_q_agpr<KS>(qreg[c], a.q + ((int64_t)tq[c] * a.h_q + hh[c]) * D + 8 * lg);
  }

  KeyWalk walk;  // the key-list walk of the loop being run (each loop starts its own)
  // Direct-load destinations: wave w fills 1 KiB segments w*SEG_PER_WAVE + j of the K and V tiles.
  uint32_t seg_off[T::SEG_PER_WAVE];
#pragma unroll
  for (int j = 0; j < T::SEG_PER_WAVE; ++j) {
    const int rl = (wave * T::SEG_PER_WAVE + j) * T::ROWS_PER_SEG + lane / T::CHR;
    seg_off[j] = 2u * (uint32_t)(rl * D + (((lane % T::CHR) ^ swz<D>(rl)) << 3));
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)lds);
  // The walk's next tile: its K and V sources and LDS stage, and its first key (-1: unreadable).
  struct TileSrc {
    const uint16_t* k;
    const uint16_t* v;
    uint32_t kb;
  };
  auto tile_src = [&](int stage, int32_t& kp) -> TileSrc {
    const uint16_t* src = walk_take<D>(a, walk, kp);
    if (src == nullptr) src = a.kv;  // unreadable page: any in-bounds bytes, the tile is masked
    return TileSrc{src, src + (int64_t)P * D, lds_base + (uint32_t)stage * 4u * T::TILE};
  };
  // Direct loads of segment j of a tile's K (kv = 0) or V (kv = 1) rows into its stage.
  auto tile_seg = [&](const TileSrc& ts, int kv, int j) {
    const uint32_t seg = (uint32_t)(wave * T::SEG_PER_WAVE + j) * 1024u;
    g2lds16_sbase(kv ? ts.v : ts.k, seg_off[j], ts.kb + (kv ? 2u * T::TILE : 0u) + seg);
  };
  // Stage the walk's next tile at once; returns its first key.
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

  // LDS byte offsets of this lane's operands within a stage, formed per use: the K operand of
  // contraction step ks (+ the key half's row offset), and half kh of the V^T operand of d-tile dt
  // (+ the 16-key group's row offset). The swizzle of a row leaves the step's chunk bits in place
  // up to an XOR, so each offset is a per-lane part (kA, vA) plus a per-lane pattern (kZ, vZ)
  // XORed with the step's chunk bits.
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
  auto voffs = [&](int dt, int kh) -> uint32_t { return (vZ[kh] ^ (64u * (uint32_t)dt)) + vA[kh]; };
  auto stage_ptr = [&](int stage) { return reinterpret_cast<const char*>(lds + stage * 2 * T::TILE); };

  const float sl2 = a.scale * kLog2e;
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x16 oacc[2][DT];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[c][dt] = (f32x16){};

  // S^T of row block c for the tile in `stage` (two 32-key halves).
  auto s_block = [&](int stage, int c, f32x16 (&s)[2]) {
    const char* kt = stage_ptr(stage);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + koffs(ks) + k2 * 32 * D * 2));
        if (ks == 0)
          mfma32_qa_first(s[k2], ka, qreg[c][ks]);
        else
          mfma32_qa(s[k2], ka, qreg[c][ks]);
      }
    xdl_vgpr_fence(s);
  };
  // P^T of block c in bf16 against a reference maximum (already scaled by log2 e and the softmax
  // scale) and this lane's part of the row sum.
  auto exp_block = [&](const f32x16 (&s)[2], float mc, u32x4 (&pb)[2][2]) {
    float lt = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[k2][e], sl2, -mc));
        lt += p[e];
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 4; ++j) pb[k2][hf][j] = cvt_pk_bf16(p[hf * 8 + 2 * j], p[hf * 8 + 2 * j + 1]);
    }
    return lt;
  };
  // General softmax of block c: each row moves its reference maximum to the tile's maximum when
  // that exceeds it by more than 2^8 (before exponentiating, so p <= 2^8), and O and the row sum
  // are rescaled with it.
  auto softmax_general = [&](const f32x16 (&s)[2], int c, u32x4 (&pb)[2][2]) {
    float x = s[0][0];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int e = 0; e < 16; ++e) x = fmaxf(x, s[k2][e]);
    const float mx = fmaxf(x, wave_xor32(x));
    const float mn = (mx - m[c]) * sl2 > kRescaleLog2w ? mx : m[c];
    const float al = (mn == m[c]) ? 1.f : __builtin_amdgcn_exp2f((m[c] - mn) * sl2);
    const float lt = exp_block(s, (mn == -INFINITY) ? 0.f : mn * sl2, pb);
    l[c] = l[c] * al + lt;
    m[c] = mn;
    if (__any(al != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        agpr_readback_fence(oacc[c][dt]);
        const f32x16 t = oacc[c][dt] * al;
        asm("" : "=a"(oacc[c][dt]) : "0"(t));  // straight back to the accumulator's AGPRs
      }
    }
  };
  // O^T[c][dt] += V^T[dt rows][16 keys] P^T[c][16 keys] for block c.
  auto pv_block = [&](int stage, int c, const u32x4 (&pb)[2][2]) {
    const char* vt = stage_ptr(stage) + 2 * T::TILE;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int rowb = (k2 * 32 + hf * 16) * D * 2;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x2 lo = lds_tr16(reinterpret_cast<const uint16_t*>(vt + voffs(dt, 0) + rowb));
          const u32x2 hi = lds_tr16(reinterpret_cast<const uint16_t*>(vt + voffs(dt, 1) + rowb));
          mfma32_agpr(oacc[c][dt], as_bf16x8((u32x4){lo[0], lo[1], hi[0], hi[1]}), as_bf16x8(pb[k2][hf]));
        }
      }
  };
  // Scores of keys after row block c's own rows become -inf (causal diagonal).
  auto mask_causal = [&](int32_t kpos0, int c, f32x16 (&s)[2]) {
    const int32_t lim = q0 + tq[c];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int32_t key = kpos0 + k2 * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
        if (key > lim) s[k2][e] = -INFINITY;
      }
  };
  auto tile_end = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // Fast-loop tile boundary: this wave's direct loads of every staged tile but the newest one
  // (when `newest_pending`) have landed and its LDS operations are complete; then the workgroup
  // barrier, without a memory fence, so the newest tile's loads stay in flight across it. The
  // direct loads are the only vector-memory operations in the loop (table entries are scalar
  // loads), so the count is exact: the newest tile is 2 x SEG_PER_WAVE loads of this wave.
  auto tile_wait = [&](bool newest_pending) {
    if (newest_pending)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * T::SEG_PER_WAVE) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS read is moved above the barrier
  };

  // Software pipeline of the fast loop. A part is a run of NSL MFMA slots in groups of two (one
  // LDS operand read two groups ahead, feeding one MFMA per row block), fenced with sched_barrier
  // so that the order written is the order issued. After each MFMA comes one softmax slot of a
  // held score tile: it adds the exp2 of element block m-1 into the row sums (two partial sums)
  // and packs finished bf16 pairs, takes the exp2 of block m, and forms the scaled and shifted
  // scores of block m+1, so that no instruction of a slot waits for another. The next tile's
  // direct loads are spread over the parts, one segment every four groups.
  constexpr int NSL = 4 * KS;     // MFMA slots per part (S^T of both blocks, or P^T V of both)
  constexpr int EPS = 32 / NSL;   // softmax elements per slot
  constexpr int GPS = (NSL / 2) / T::SEG_PER_WAVE;  // groups per direct-load segment
  using Pipe = SoftPipe<EPS>;
  auto soft_first = [&](const f32x16 (&sx)[2], Pipe& sp) {
#pragma unroll
    for (int q = 0; q < EPS; ++q) sp.f[q] = __builtin_fmaf(sx[0][q], sl2, -sp.tok);
  };
  auto soft_slot = [&](int m, const f32x16 (&sx)[2], Pipe& sp, float (&lt)[2], u32x4 (&px)[2][2]) {
    if (m >= 1) {
#pragma unroll
      for (int q = 0; q < EPS; ++q) {
        const int e = (m - 1) * EPS + q;
        lt[e & 1] += sp.e[q];
        if (e & 1) {
          uint32_t c = cvt_pk_bf16(EPS == 2 ? sp.e[0] : sp.ep, sp.e[q]);
          issue_pin(c);
          px[e >> 4][(e & 15) >> 3][(e & 7) >> 1] = c;
        }
      }
      if constexpr (EPS == 1) sp.ep = sp.e[0];
    }
    if (m < NSL) {
#pragma unroll
      for (int q = 0; q < EPS; ++q) sp.e[q] = __builtin_amdgcn_exp2f(sp.f[q]);
    }
    if (m + 1 < NSL) {
#pragma unroll
      for (int q = 0; q < EPS; ++q) {
        const int e = (m + 1) * EPS + q;
        sp.f[q] = __builtin_fmaf(sx[e >> 4][e & 15], sl2, -sp.tok);
      }
    }
    issue_pin(lt[0]);
    issue_pin(lt[1]);
  };
  // Part a: S^T of both blocks for the tile in `stage`; with the softmax (WE), P^T of a held score
  // tile sx is computed alongside; with a tile source (LD), its K segments are loaded.
  auto part_a = [&](auto we, auto ld, int stage, f32x16 (&sa)[2], f32x16 (&sb)[2], const f32x16 (&sx)[2],
                    float mc, u32x4 (&px)[2][2], const TileSrc& ts) -> float {
    constexpr bool WE = decltype(we)::value, LD = decltype(ld)::value;
    const char* kt = stage_ptr(stage);
    bf16x8 kop[2 * KS];
    auto kread = [&](int j) {
      kop[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + koffs(j >> 1) + (j & 1) * 32 * D * 2));
    };
    kread(0);
    kread(1);
    float lt[2] = {0.f, 0.f};
    Pipe sp;
    sp.tok = mc;
    sp.ep = 0.f;
    if constexpr (WE) soft_first(sx, sp);
#pragma unroll
    for (int j = 0; j < 2 * KS; ++j) {
      if (j + 2 < 2 * KS) kread(j + 2);
      const int ks = j >> 1, k2 = j & 1;
      if constexpr (WE) {
        if (ks == 0)
          mfma_s_first(sa[k2], kop[j], qreg[0][ks], sp);
        else
          mfma_s(sa[k2], kop[j], qreg[0][ks], sp);
        soft_slot(2 * j, sx, sp, lt, px);
        if (ks == 0)
          mfma_s_first(sb[k2], kop[j], qreg[1][ks], sp);
        else
          mfma_s(sb[k2], kop[j], qreg[1][ks], sp);
        soft_slot(2 * j + 1, sx, sp, lt, px);
      } else {
        if (ks == 0) {
          mfma32_qa_first(sa[k2], kop[j], qreg[0][ks]);
          mfma32_qa_first(sb[k2], kop[j], qreg[1][ks]);
        } else {
          mfma32_qa(sa[k2], kop[j], qreg[0][ks]);
          mfma32_qa(sb[k2], kop[j], qreg[1][ks]);
        }
      }
      if constexpr (LD) {
        if (j % GPS == GPS / 2) tile_seg(ts, 0, j / GPS);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (WE) soft_slot(NSL, sx, sp, lt, px);
    xdl_vgpr_fence2(sa, sb);
    return lt[0] + lt[1];
  };
  // Part b: O^T of both blocks += V^T P^T for the tile in `stage`; with the softmax (WE), P^T of a
  // held score tile sx alongside; with a tile source (LD), its V segments are loaded.
  auto part_b = [&](auto we, auto ld, int stage, const u32x4 (&p0)[2][2], const u32x4 (&p1)[2][2],
                    const f32x16 (&sx)[2], float mc, u32x4 (&px)[2][2], const TileSrc& ts) -> float {
    constexpr bool WE = decltype(we)::value, LD = decltype(ld)::value;
    const char* vt = stage_ptr(stage) + 2 * T::TILE;
    bf16x8 vop[4 * DT];
    auto vread = [&](int j) {
      const int k2 = j / (2 * DT), hf = (j / DT) & 1, dt = j % DT;
      const int rowb = (k2 * 32 + hf * 16) * D * 2;
      const u32x2 lo = lds_tr16(reinterpret_cast<const uint16_t*>(vt + voffs(dt, 0) + rowb));
      const u32x2 hi = lds_tr16(reinterpret_cast<const uint16_t*>(vt + voffs(dt, 1) + rowb));
      vop[j] = as_bf16x8((u32x4){lo[0], lo[1], hi[0], hi[1]});
    };
    vread(0);
    vread(1);
    float lt[2] = {0.f, 0.f};
    Pipe sp;
    sp.tok = mc;
    sp.ep = 0.f;
    if constexpr (WE) soft_first(sx, sp);
#pragma unroll
    for (int j = 0; j < 4 * DT; ++j) {
      if (j + 2 < 4 * DT) vread(j + 2);
      const int k2 = j / (2 * DT), hf = (j / DT) & 1, dt = j % DT;
      if constexpr (WE) {
        mfma_pv(oacc[0][dt], vop[j], as_bf16x8(p0[k2][hf]), sp);
        soft_slot(2 * j, sx, sp, lt, px);
        mfma_pv(oacc[1][dt], vop[j], as_bf16x8(p1[k2][hf]), sp);
        soft_slot(2 * j + 1, sx, sp, lt, px);
      } else {
        mfma32_agpr(oacc[0][dt], vop[j], as_bf16x8(p0[k2][hf]));
        mfma32_agpr(oacc[1][dt], vop[j], as_bf16x8(p1[k2][hf]));
      }
      if constexpr (LD) {
        if (j % GPS == GPS / 2) tile_seg(ts, 1, j / GPS);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (WE) soft_slot(NSL, sx, sp, lt, px);
    return lt[0] + lt[1];
  };
  using kNoExp = std::integral_constant<bool, false>;
  using kExp = std::integral_constant<bool, true>;
  using kNoLoad = std::integral_constant<bool, false>;
  using kLoad = std::integral_constant<bool, true>;
  const TileSrc no_src{a.kv, a.kv, lds_base};

  // Workgroup-wide control words: [0] the earliest fast-loop tile at which some wave had to leave
  // (every wave leaves after that tile's barrier), [1] the first tile of the general loop (the
  // minimum over waves of the first tile a wave still has to compute).
  __shared__ int32_t ctl[2];
  if (tid == 0) {
    ctl[0] = INT32_MAX;
    ctl[1] = INT32_MAX;
  }
  int32_t gs_b[2] = {tb, tb};  // per row block of this wave: the first tile it still has to compute
  int32_t gs = tb;    // first tile of the general loop (the same for every wave)
  if (tb < em) {
    walk = walk_begin(a, g, li, tsh, tb, em);
    // Tile t of the range is staged in stage (t - tb) % 4, two tiles ahead of the one computed.
    int32_t kpc = load_tile(0);
    int32_t kpn = load_tile(1);  // staged even past the range, like every later tile
    tile_wait(true);             // tile tb has landed; also publishes ctl
    f32x16 s0[2], s1a[2], s1b[2];
    u32x4 pb1[2][2], pb0a[2][2], pb0b[2][2];
    float lt0p = 0.f, m0r = 0.f, m1r = 0.f;
    bool ok = kpc >= 0;  // a first tile on an unreadable page leaves everything to the general loop
    if (ok) {
      // First tile: its row maxima become the reference maxima; block 0's softmax at once.
      part_a(kNoExp{}, kNoLoad{}, 0, s0, s1a, s0, 0.f, pb1, no_src);
      float x0 = s0[0][0], x1 = s1a[0][0];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          x0 = fmaxf(x0, s0[k2][e]);
          x1 = fmaxf(x1, s1a[k2][e]);
        }
      m[0] = fmaxf(x0, wave_xor32(x0));
      m[1] = fmaxf(x1, wave_xor32(x1));
      m0r = m[0] * sl2;
      m1r = m[1] * sl2;
      lt0p = exp_block(s0, m0r, pb0a);
      const int32_t kp2 = load_tile(2);
      tile_wait(true);  // tile tb + 1 has landed
      kpc = kpn;
      kpn = kp2;
    }
    // One pipelined tile i: S^T(i) with block 1's softmax of tile i-1, then P^T V of tile i-1 with
    // block 0's softmax of tile i; tile i+2 is staged meanwhile. P^T V always runs (a branch around
    // it would fork the accumulators' register assignment): when block 1's softmax of tile i-1
    // fails its check, its P^T is zeroed and the block redoes tile i-1 in the general loop.
    // Returns false when the wave leaves the loop (gs_b set).
    auto step = [&](int32_t i, const f32x16 (&s1p)[2], f32x16 (&s1n)[2], const u32x4 (&pb0p)[2][2],
                    u32x4 (&pb0n)[2][2]) -> bool {
      // Stage indices kept opaque (scalar values the compiler cannot enumerate), so that operand
      // addresses are formed per use instead of held per stage in registers.
      int sc = (i - tb) & 3, sprev = (i - 1 - tb) & 3;
      asm("" : "+s"(sc), "+s"(sprev));
      // Tile i+2 is staged even past the range (then from the pool's first bytes, into a stage
      // that is never read): one code path, and a constant count for the wait below.
      int32_t kp2;
      const TileSrc ts = tile_src((i + 2 - tb) & 3, kp2);
      if (kpc < 0) {  // unreadable page (the same for every wave): the general loop takes over
        gs_b[0] = gs_b[1] = i - 1;
        return false;
      }
      const float lt1 = part_a(kExp{}, kLoad{}, sc, s0, s1n, s1p, m1r, pb1, ts);
      const bool bad1 = __any(!(lt1 <= kFastSumLimit));  // a row of block 1 outgrew its reference
      if (bad1) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) pb1[k2][0] = pb1[k2][1] = (u32x4){};
      }
      const float lt0 = part_b(kExp{}, kLoad{}, sprev, pb0p, pb1, s0, m0r, pb0n, ts);
      l[0] += lt0p;
      l[1] += bad1 ? 0.f : lt1;
      lt0p = lt0;
      const bool left = bad1 || __any(!(lt0 <= kFastSumLimit));
      if (left) {
        gs_b[0] = i;
        gs_b[1] = bad1 ? i - 1 : i;
        if (lane == 0) atomicMin(&ctl[0], i);
      }
      tile_wait(true);  // tile i+1 has landed
      // Read as a wave-uniform value: a loop exit that looked divergent would move every value the
      // loop carries (the key walk's state) into vector registers.
      if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(&ctl[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) <=
          i) {
        if (!left) gs_b[0] = gs_b[1] = i;
        return false;
      }
      kpc = kpn;
      kpn = kp2;
      return true;
    };
    // The last tile's pending work: block 1's softmax, then P^T V of both blocks.
    auto finish = [&](const f32x16 (&s1p)[2], const u32x4 (&pb0p)[2][2]) {
      const float lt1 = exp_block(s1p, m1r, pb1);
      const bool bad1 = __any(!(lt1 <= kFastSumLimit));
      if (bad1) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) pb1[k2][0] = pb1[k2][1] = (u32x4){};
      }
      part_b(kNoExp{}, kNoLoad{}, (em - 1 - tb) & 3, pb0p, pb1, s0, 0.f, pb1, no_src);
      l[0] += lt0p;
      l[1] += bad1 ? 0.f : lt1;
      gs_b[0] = em;
      gs_b[1] = bad1 ? em - 1 : em;
    };
    if (ok) {
      // Unrolled by two so that the held tiles alternate between register sets without copies.
      bool fin = false;
      for (int32_t i = tb + 1;; i += 2) {
        if (i >= em) {
          fin = true;
          break;
        }
        if (!step(i, s1a, s1b, pb0a, pb0b)) break;
        if (i + 1 >= em) {
          fin = true;
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            s1a[k2] = s1b[k2];
            pb0a[k2][0] = pb0b[k2][0];
            pb0a[k2][1] = pb0b[k2][1];
          }
          break;
        }
        if (!step(i + 1, s1b, s1a, pb0b, pb0a)) break;
      }
      if (fin) finish(s1a, pb0a);
    }
    if (lane == 0) atomicMin(&ctl[1], min(gs_b[0], gs_b[1]));
    tile_end();
    gs = __builtin_amdgcn_readfirstlane(__hip_atomic_load(&ctl[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
  }
  // General loop over [gs, te): the tiles at the causal diagonal (masked), a range whose first
  // tile was unreadable, or the rest of the range after the fast loop met a row that outgrew its
  // reference; reference maxima move, and O is rescaled, as needed. Every wave stages every tile;
  // a row block is computed only from its own first pending tile (gs_b) on.
  if (gs < te) {
    f32x16 s0[2], s1[2];
    u32x4 pb0[2][2], pb1[2][2];
    walk = walk_begin(a, g, li, tsh, gs, te);
    int32_t kp0 = load_tile(0);
    tile_end();
    for (int32_t i = gs; i < te; ++i) {
      const int st = (i - gs) & 1;
      const int32_t kp1 = (i + 1 < te) ? load_tile(st ^ 1) : -1;
      if (kp0 >= 0) {
        const bool diag = i >= n_free;
        if (i >= gs_b[0]) {
          s_block(st, 0, s0);
          if (diag) mask_causal(kp0, 0, s0);
          softmax_general(s0, 0, pb0);
          pv_block(st, 0, pb0);
        }
        if (i >= gs_b[1]) {
          s_block(st, 1, s1);
          if (diag) mask_causal(kp0, 1, s1);
          softmax_general(s1, 1, pb1);
          pv_block(st, 1, pb1);
        }
      }
      tile_end();
      kp0 = kp1;
    }
  }

  // Epilogue: normalise and store both row blocks.
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) agpr_readback_fence(oacc[c][dt]);
  const int64_t rows_total = (int64_t)a.n_kvh * CG;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const float lt = l[c] + wave_xor32(l[c]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m[c] * sl2 + __log2f(lt)) * kLn2 : -INFINITY;
    if (!rvalid[c]) continue;
    // Row indices re-pinned: the output addresses are formed here, not kept from the Q loads.
    int32_t tqc = tq[c], hhc = hh[c];
    issue_pin(tqc);
    issue_pin(hhc);
    if (splits == 1) {
      uint16_t* op = o + ((int64_t)tqc * a.h_q + hhc) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          u32x2 w;
          w[0] = cvt_pk_bf16(oacc[c][dt][grp * 4 + 0] * inv, oacc[c][dt][grp * 4 + 1] * inv);
          w[1] = cvt_pk_bf16(oacc[c][dt][grp * 4 + 2] * inv, oacc[c][dt][grp * 4 + 3] * inv);
          *reinterpret_cast<u32x2*>(op + dt * 32 + grp * 8 + 4 * lg) = w;
        }
      if (lg == 0) lse[(int64_t)hhc * a.C + tqc] = lse_v;
    } else {
      const int64_t R = (int64_t)gi * CG + r0 + wave * 64 + c * 32 + l32;
      float* wp = ws_o + ((int64_t)sp * rows_total + R) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          f32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = oacc[c][dt][grp * 4 + j] * inv;
          *reinterpret_cast<f32x4*>(wp + dt * 32 + grp * 8 + 4 * lg) = w;
        }
      if (lg == 0) ws_lse[(int64_t)sp * rows_total + R] = lse_v;
    }
  }
}

template <int D>
hipError_t launch_fwd64(const AttnArgs& a, int32_t n_rb, int32_t splits, uint16_t* o, float* lse, float* ws_o,
                        float* ws_lse, hipStream_t s) {
  const int32_t n_units = a.n_kvh * splits * n_rb;
  hipLaunchKernelGGL((k_attn_fwd64<D>), dim3(n_units), dim3(256), 0, s, a, n_rb, splits, o, lse, ws_o, ws_lse);
  return hipGetLastError();
}

template hipError_t launch_fwd64<128>(const AttnArgs&, int32_t, int32_t, uint16_t*, float*, float*, float*,
                                      hipStream_t);
template hipError_t launch_fwd64<64>(const AttnArgs&, int32_t, int32_t, uint16_t*, float*, float*, float*,
                                     hipStream_t);

}  // namespace pkv
