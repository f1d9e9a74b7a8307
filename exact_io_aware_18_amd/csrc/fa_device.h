// Device-side building blocks for the gfx950 attention kernels: MFMA
// wrappers, the lane/row permutation that keeps softmax rows in registers,
// the LDS tile swizzle, direct-to-LDS tile copies, operand reads and
// wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l supplies A[l % 32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l % 32];
// it receives C[8*(r/4) + 4*(l/32) + r%4][l % 32] in register r (0..15).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row permutation applied when an operand's rows are loaded, so that the
// accumulator rows a half-wave holds become contiguous: with A row x taken
// from source row perm32(x), register r of a lane in half h holds source
// row 16*(r/8) + 8*h + r%8.  Registers 0..7 and 8..15 then each cover eight
// consecutive source rows, which is exactly the k-slice (8*h .. 8*h+7) that
// lane feeds to the next MFMA, and eight consecutive elements of an output
// row for a 16-byte store.
__device__ __forceinline__ int perm32(int x) {
  const int a = x >> 3, hh = (x >> 2) & 1, b = x & 3;
  return ((a >> 1) << 4) | (hh << 3) | ((a & 1) << 2) | b;
}

// Source row held in register r by half-wave h after perm32-loaded rows.
__device__ __forceinline__ int acc_row(int r, int h) {
  return ((r >> 3) << 4) | (h << 3) | (r & 7);
}

// XOR swizzle of the 16-byte chunks of a natural [rows][D] bf16 LDS tile.
// The tiles are read two ways: ds_read_b128 of whole rows in perm32 order
// (MFMA operands that contract over d) and ds_read_b64_tr_b16 of 4-row by
// 32-byte blocks (operands that contract over the sequence).  Measured on
// gfx950, chunk ^ tswz(row) keeps both patterns free of bank conflicts for
// 128- and 256-byte rows.  It depends on row % 16 only.
template <int D>
__device__ __forceinline__ int tswz(int row) {
  return (((row & 1) << 3) | (((row >> 1) & 1) << 2) | ((row >> 2) & 3)) & (D / 8 - 1);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Transposed 8-byte LDS read (gfx950 ds_read_b64_tr_b16).  Within each group
// of 16 lanes, lane i receives element i % 4 of the 8-byte words addressed by
// lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4, in that order: if lane 4u + q
// addresses row u, columns 4q .. 4q+3 of a row-major bf16 block, lane i gets
// column i of rows 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr8(const __attribute__((address_space(3))) char* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// max over lane l and lane l ^ 32 (v_permlane32_swap)
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// sum over lane l and lane l ^ 32
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 lds_read16(const char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 gload16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Eight fp32 values -> eight bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3,
                                            float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

// Workgroups are dispatched round-robin over the eight XCDs (workgroup g
// runs on XCD g % 8), each with its own L2.  Give every XCD a contiguous
// range of logical tile ids so tiles that share K/V share an L2.
__device__ __forceinline__ int xcd_remap(int g, int total) {
  const int x = g & 7, s = g >> 3;
  const int q = total >> 3, r = total & 7;
  return (x < r) ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

// Causal tiles of a head differ in length (a query tile sees the keys up to
// its diagonal).  Workgroup g takes length rank g / BH (0 = longest) of head
// g % BH, so the grid runs longest first over all heads at once, the order
// that keeps the end of the launch balanced; ordering each head's tiles on
// its own left whole XCDs busy with the last heads' long tiles (GPT-2 shape:
// 70K against 48K cycles, simulated with the measured per-tile cost).  With
// BH a multiple of 8 the XCD of workgroup g (g % 8) still owns a fixed set of
// heads, whose tiles then share its L2.
__device__ __forceinline__ void causal_rank(int g, int BH, int& bh, int& rank) {
  rank = g / BH;
  bh = g - rank * BH;
}

// 16-byte direct-to-LDS copy (global_load_lds_dwordx4): lane l of the wave
// writes its 16 bytes at lds + 16*l; lds must be wave-uniform.  Issued
// through inline assembly so that the compiler does not track it: while it
// tracks a direct-to-LDS copy in flight, it turns every LDS-read wait into a
// full lgkmcnt(0) and every workgroup barrier into a wait for the copy.
// Users therefore wait for these copies themselves (s_waitcnt vmcnt(0), then
// a barrier) before any wave reads the destination; the compiler's own vmcnt
// waits for other loads can only become longer (completions are in order),
// never too short.  The LDS address goes in M0 as an input operand ("{m0}"),
// so the compiler writes M0 itself and knows the statement reads it and leaves
// it unchanged; the s_nop is the wait state between an M0 write and a copy
// that reads it.
__device__ __forceinline__ void lds_dma16_untracked(const void* src, char* lds) {
  const uint32_t m = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m) : "memory");
}

// Direct-to-LDS copy of ROWS consecutive rows of a [N][D] bf16 matrix into
// a natural LDS tile swizzled by tswz, by NT threads.  Wave w, round e fills
// LDS bytes [(e*NW + w) * 1024, +1024), lane l landing at +16*l; that slot
// holds tile row (e*NW + w) * (1024 / PITCH) + l / CPR, physical chunk
// l % CPR, i.e. logical chunk (l % CPR) ^ tswz(row).  The per-lane source
// offsets are the same for every tile.
template <int ROWS, int D, int NT>
struct TileCopy {
  static constexpr int NW = NT / 64;
  static constexpr int PITCH = 2 * D;
  static constexpr int CPR = PITCH / 16;
  static constexpr int ROUNDS = ROWS * PITCH / (NT * 16);
  static_assert(ROWS * PITCH % (NT * 16) == 0, "tile must be a whole number of rounds");
  uint32_t off[ROUNDS];  // byte offset of this lane's 16 bytes within the rows
  int row[ROUNDS];       // tile row of this lane's 16 bytes

  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int e = 0; e < ROUNDS; ++e) {
      row[e] = (e * NW + w) * (1024 / PITCH) + lane / CPR;
      off[e] = (uint32_t)(row[e] * PITCH + (((lane % CPR) ^ tswz<D>(row[e])) << 4));
    }
  }
  // rows [row0, row0 + ROWS) of src; rows past N re-read row N-1 (finite
  // data that the callers mask).  The copies are untracked: the caller waits
  // (s_waitcnt vmcnt(0) and a barrier) before the tile is read.
  __device__ __forceinline__ void issue(char* lds_tile, const __bf16* src, int row0, int N, int w) const {
    const char* base = reinterpret_cast<const char*>(src + (size_t)row0 * D);
    auto dma = [&](const char* g, char* l) { lds_dma16_untracked(g, l); };
    if (row0 + ROWS <= N) {
#pragma unroll
      for (int e = 0; e < ROUNDS; ++e) dma(base + off[e], lds_tile + (e * NW + w) * 1024);
    } else {
      const uint32_t last = (uint32_t)((N - 1 - row0) * PITCH);  // byte offset of row N-1
#pragma unroll
      for (int e = 0; e < ROUNDS; ++e) {
        const uint32_t o = (row0 + row[e] < N) ? off[e] : last + (off[e] - (uint32_t)(row[e] * PITCH));
        dma(base + o, lds_tile + (e * NW + w) * 1024);
      }
    }
  }
};

// Per-lane byte offsets of the MFMA operands in a tswz-swizzled natural tile.
// rows(): A operand rows perm32(li) (+32*t), 16-byte chunk 2kc + h: one
//   ds_read_b128 per k-step of a product that contracts over d.
// tr(): the A operand of a product that contracts over the tile's rows: for
//   read r of a 16-row k-step and 32-column group ct, lane l addresses tile
//   row 8h + 4r + (l%16)/4 (+16*kc) and columns 32ct + perm32(16*((l/16)%2) +
//   4*(l%4)) .. +3; two ds_read_b64_tr_b16 then give lane l column
//   32ct + perm32(l%32), rows 16kc + 8h .. +7.
template <int D>
struct TileOffsets {
  static constexpr int PITCH = 2 * D;
  int rows[D / 16];
  int tr[D / 32][2];
  __device__ __forceinline__ void init(int lane) {
    const int h = lane >> 5, li = lane & 31;
    const int rr = perm32(li);
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) rows[kc] = rr * PITCH + (((2 * kc + h) ^ tswz<D>(rr)) << 4);
    const int trow = 8 * h + ((lane & 15) >> 2);
    const int tcl = 2 * ((lane >> 4) & 1) + (lane & 1);
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = trow + 4 * r;
        tr[ct][r] = row * PITCH + (((4 * ct + tcl) ^ tswz<D>(row)) << 4) + ((lane >> 1) & 1) * 8;
      }
  }
  // A operand (transposed), rows 16*kc .. +15 of the tile, columns group ct
  __device__ __forceinline__ bf16x8 read_tr(const char* tile, int kc, int ct) const {
    const auto* base = (const __attribute__((address_space(3))) char*)(tile + 16 * kc * PITCH);
    return cat8(lds_read_tr8(base + tr[ct][0]), lds_read_tr8(base + tr[ct][1]));
  }
};

}  // namespace fa
