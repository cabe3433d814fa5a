// Device helpers for the gfx950 kernels: vector types, bf16 packing, MFMA wrappers, page lookup.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round-to-nearest-even float -> bf16 (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// D(32x32, fp32) += A(32x16) * B(16x32), bf16 inputs. Lane l supplies A row l%32 and B column l%32,
// eight consecutive contraction indices from 8*(l/32). Accumulator element i of lane l holds row
// 8*(i/4) + 4*(l/32) + (i%4), column l%32.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// The same MFMA with its accumulator pinned to the AGPR file (kernels that keep S and dP in VGPRs
// for the softmax and their long-lived accumulators in AGPRs); the instruction is written out so
// that the accumulator stays there. The compiler's hazard recognizer does not see inline assembly
// as an MFMA, so the wait states it would insert are part of the statement: a VALU write of a VGPR
// (or a v_accvgpr_write of an AGPR) followed by an MFMA that reads it (the bf16 operands packed by
// VALU conversions, any VALU move assembling an operand) needs 2 wait states (CDNA3 instruction
// set reference, the MAI dependency-resolution table: "VALU write VGPR, V_MFMA* read of that VGPR";
// gfx950 keeps the rule), which s_nop 1 provides. Back-to-back MFMAs accumulating into the same
// registers need none.
__device__ __forceinline__ void mfma32_agpr(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Read-back fence for an AGPR accumulator: an XDL (MFMA) write of a register followed by a VALU
// read of it, v_accvgpr_read included, needs the MFMA's pass count plus 2 wait states (same table:
// "XDL write VGPR/AGPR, VALU read"; 18 for a 16-pass MFMA, fewer for 8 passes). The three s_nop 7
// give 24. The accumulator is an in/out operand, so the statement is ordered after every MFMA that
// writes it and before every read of it.
__device__ __forceinline__ void agpr_readback_fence(f32x16& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(c));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Two floats -> packed bf16 pair (round to nearest even; one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Row-major bf16 tiles in LDS are stored without padding; the 16-byte chunks of row r are
// XOR-permuted by swz(r) so that both access patterns used on them are free of bank conflicts:
// 16 lanes reading 16 consecutive rows at one chunk (MFMA operand along the row), and the
// transposed 8-byte reads below (4 consecutive rows x 4 chunks per 32 lanes).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
}
// Element offset of (row r, column c) in a swizzled tile with D columns; c % 4 == 0.
template <int D>
__device__ __forceinline__ int toff(int r, int c) {
  return r * D + (((c >> 3) ^ swz<D>(r)) << 3) + (c & 7);
}

// Transposed LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i receives column
// N0 + i of rows K0..K0+3 when lane L of the group addresses row K0 + L/4, column N0 + 4*(L%4).
__device__ __forceinline__ u32x2 lds_tr16(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// MFMA operand whose contraction index runs along the rows of a swizzled row-major tile: lane l
// gets column n0 + l%32 and rows k_lo..k_lo+3 (slots 0-3) and k_hi..k_hi+3 (slots 4-7).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* tile, int k_lo, int k_hi, int n0, int lane) {
  const int rr = (lane & 15) >> 2;
  const int cc = n0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const u32x2 a = lds_tr16(tile + toff<D>(k_lo + rr, cc));
  const u32x2 b = lds_tr16(tile + toff<D>(k_hi + rr, cc));
  u32x4 w;
  w[0] = a[0];
  w[1] = a[1];
  w[2] = b[0];
  w[3] = b[1];
  return as_bf16x8(w);
}

__device__ __forceinline__ float wave_xor32(float v) { return __shfl_xor(v, 32, 64); }

// Wait until at most N of this wave's vector-memory operations are outstanding (they complete in
// issue order); LDS and scalar counters are not waited on. gfx9 s_waitcnt encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Direct global -> LDS loads (global_load_lds_dwordx4 / _dword): lane L of the wave writes its 16
// (or 4) bytes to lds_base + 16 L (or 4 L). lds_base must be the same for every lane of the wave.
__device__ __forceinline__ void g2lds16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}
__device__ __forceinline__ void g2lds4(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)(lds_base), 4, 0, 0);
}

// The same 16-byte direct load written out, for loops that order their LDS ring with explicit
// waits: the compiler then does not know that it writes LDS and adds no wait for it before later
// LDS reads (it would add one before every transposed read, which need not wait: they read
// another stage of the ring). The load writes no register; M0 carries the wave-uniform LDS base
// and is set inside the statement. The caller waits for it (s_waitcnt vmcnt) before any wave reads
// the bytes, and keeps the source and LDS addresses in range as for g2lds16.
__device__ __forceinline__ void g2lds16_asm(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(lds_base)
               : "memory", "m0");
}

// The same direct load from a wave-uniform 64-bit base plus a per-lane 32-bit byte offset (the
// instruction's scalar-base form): no 64-bit per-lane address is formed or held.
__device__ __forceinline__ void g2lds16_sbase(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(lds_base)
               : "memory", "m0");
}

// Record an out-of-range table entry (first writer wins; the value is informational).
__device__ __forceinline__ void flag_error(int32_t* err, int32_t code) {
  if (err) atomicCAS(err, 0, code);
}

// Logical page of entry pi of a chunk's key-page list for KV head g and selection list li (the
// query page's list when there is one per query page, else 0): the prior part (all of
// [0, n_prior) when dense, else the selected pages) followed by the chunk's own pages.
// Returns -1 (and flags) for an out-of-range selection entry.
__device__ __forceinline__ int32_t list_page(const AttnArgs& a, int32_t g, int32_t li, int32_t pi) {
  if (a.sel == nullptr) return pi;
  if (pi < a.n_sel) {
    int32_t lp = a.sel[((size_t)g * a.n_lists + li) * a.n_sel + pi];
    if (lp < 0 || lp >= a.n_prior) {
      flag_error(a.err, 2);
      return -1;
    }
    return lp;
  }
  return a.n_prior + (pi - a.n_sel);
}

// Physical page of a logical page through the block table, -1 (flagged) if out of range.
__device__ __forceinline__ int32_t phys_page(const int32_t* bt, int32_t n_bt, int32_t n_pool, int32_t lp,
                                             int32_t* err) {
  if (lp < 0) return -1;
  if (lp >= n_bt) {
    flag_error(err, 3);
    return -1;
  }
  int32_t p = bt[lp];
  if (p < 0 || p >= n_pool) {
    flag_error(err, 1);
    return -1;
  }
  return p;
}

// Number of prior pages in the key list (selected count when sparse).
__device__ __forceinline__ int32_t list_prior(const AttnArgs& a) { return a.sel ? a.n_sel : a.n_prior; }

// Walk over the 64-key tiles of a chunk's key list with the table reads issued ahead of use.
// Tile i lies in list entry i >> tsh (tsh = log2 of tiles per page). Resolving it takes a
// selection read (prior entries of a sparse list) and then a block-table read, each a round trip
// to the L2; issued when the tile's K/V loads are due, they would stall every wave of the
// workgroup at the start of each tile. walk_take(i) instead uses the block-table entry of tile i
// read during the previous call and the selection entry of tile i + 1 read then too, and issues
// the reads for tiles i + 1 (block table) and i + 2 (selection). The kernels wait for all their
// memory operations at the end of each tile, so those values have landed by the next call.
// Every value is wave-uniform; validation and error flags are those of list_page / phys_page.
struct KeyWalk {
  int32_t g, li, tsh, te;
  int32_t t;     // tile the next walk_take resolves
  int32_t lp;    // its logical page (-1: unreadable or past the list)
  int32_t btv;   // block-table entry of lp (read ahead)
  int32_t selv;  // selection entry of tile t + 1 (read ahead; prior entries of sparse lists only)
};

// Logical page of tile t from the selection entry `selv` read for it (sparse prior entries) or
// directly (dense lists, the own block); -1 (flagged) when out of range or past the list.
__device__ __forceinline__ int32_t walk_page(const AttnArgs& a, const KeyWalk& w, int32_t t, int32_t selv) {
  if (t >= w.te) return -1;
  const int32_t pi = t >> w.tsh;
  int32_t lp;
  if (a.sel == nullptr) {
    lp = pi;
  } else if (pi >= a.n_sel) {
    lp = a.n_prior + (pi - a.n_sel);
  } else {
    lp = selv;  // a scalar load: already wave-uniform
    if (lp < 0 || lp >= a.n_prior) {
      flag_error(a.err, 2);
      return -1;
    }
  }
  if (lp >= a.n_bt) {
    flag_error(a.err, 3);
    return -1;
  }
  return lp;
}

__device__ __forceinline__ bool walk_needs_sel(const AttnArgs& a, const KeyWalk& w, int32_t t) {
  return a.sel != nullptr && t < w.te && (t >> w.tsh) < a.n_sel;
}

// Table entries are wave-uniform and the tables are not written while a kernel reads them, so
// they are read through the constant address space (scalar loads): they then count against the
// LDS/scalar counter, not the vector-memory counter that tracks a kernel's direct loads of K/V
// tiles, and a wait for a table entry never waits for tile data.
__device__ __forceinline__ int32_t table_read(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)(p);
}

__device__ __forceinline__ int32_t walk_sel_read(const AttnArgs& a, const KeyWalk& w, int32_t t) {
  return table_read(a.sel + ((size_t)w.g * a.n_lists + w.li) * a.n_sel + (t >> w.tsh));
}

// Start the walk at tile t0 (its reads complete before its walk_take returns).
__device__ __forceinline__ KeyWalk walk_begin(const AttnArgs& a, int32_t g, int32_t li, int32_t tsh, int32_t t0,
                                              int32_t te) {
  KeyWalk w;
  w.g = g;
  w.li = li;
  w.tsh = tsh;
  w.te = te;
  w.t = t0;
  w.btv = 0;
  w.selv = 0;
  const int32_t s0 = walk_needs_sel(a, w, t0) ? walk_sel_read(a, w, t0) : 0;
  w.lp = walk_page(a, w, t0, s0);
  if (w.lp >= 0) w.btv = table_read(a.bt + w.lp);
  if (walk_needs_sel(a, w, t0 + 1)) w.selv = walk_sel_read(a, w, t0 + 1);
  return w;
}

// K base of tile w.t (nullptr when unreadable; kpos0 = -1 then, else the tile's first key
// position) and the reads for the following tiles. D is the head dimension.
template <int D>
__device__ __forceinline__ const uint16_t* walk_take(const AttnArgs& a, KeyWalk& w, int32_t& kpos0) {
  const uint16_t* src = nullptr;
  kpos0 = -1;
  if (w.lp >= 0) {
    const int32_t ph = w.btv;  // a scalar load: already wave-uniform (no copy through a VGPR)
    if (ph < 0 || ph >= a.n_pool_pages) {
      flag_error(a.err, 1);
    } else {
      const int32_t sub = w.t & ((1 << w.tsh) - 1);
      kpos0 = w.lp * a.page + sub * 64;
      src = a.kv + (((int64_t)ph * a.h_kv + w.g) * 2) * a.page * D + (int64_t)sub * 64 * D;
    }
  }
  const int32_t t1 = w.t + 1;
  const int32_t lp1 = walk_page(a, w, t1, w.selv);
  if (lp1 >= 0) w.btv = table_read(a.bt + lp1);
  if (walk_needs_sel(a, w, t1 + 1)) w.selv = walk_sel_read(a, w, t1 + 1);
  w.lp = lp1;
  w.t = t1;
  return src;
}

// XCD-aware block ordering: workgroups are dispatched round-robin over 8 XCDs, so consecutive
// logical units are gathered onto one XCD (sharing its L2). Bijective on [0, n).
__device__ __forceinline__ int32_t xcd_remap(int32_t bid, int32_t n) {
  const int32_t x = bid & 7, k = bid >> 3;
  const int32_t q = n >> 3, r = n & 7;
  return x * q + (x < r ? x : r) + k;
}

}  // namespace pkv
