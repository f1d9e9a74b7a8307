// Device-side building blocks for the gfx950 attention kernels: MFMA
// wrappers, the lane/row permutation that keeps softmax rows in registers,
// LDS swizzles, tile staging and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// XOR swizzle of 16-byte chunks inside an LDS row.  Rows read together by
// eight (or sixteen) consecutive lanes through perm32 map to distinct
// chunks, so a ds_read_b128 wave touches distinct banks.
__device__ __forceinline__ int swz(int row, int chunk, int nchunk) {
  const int b3 = (row >> 3) & 1;
  const int f = ((row & 7) ^ (b3 << 2)) | (b3 << 3);
  return chunk ^ (f & (nchunk - 1));
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Sum of the eight bf16 values of v (as fp32) added to acc: four v_dot2 ops.
__device__ __forceinline__ float sum8(bf16x8 v, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  float a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, 0.f, false);
  a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, a0, false);
  a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, a1, false);
  return a0 + a1;
}

__device__ __forceinline__ bf16x8 lds_read16(const char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void lds_write16(char* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ void lds_write8(char* p, u32x2 v) {
  *reinterpret_cast<u32x2*>(p) = v;
}

__device__ __forceinline__ u32x4 gload16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x2 gload8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// Eight fp32 values -> eight bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3,
                                            float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// Registers r0 .. r0+7 of an accumulator as bf16x8.
__device__ __forceinline__ bf16x8 acc_to_bf16(const f32x16& c, int r0) {
  return to_bf16x8(c[r0 + 0], c[r0 + 1], c[r0 + 2], c[r0 + 3],
                   c[r0 + 4], c[r0 + 5], c[r0 + 6], c[r0 + 7]);
}

// Value held by lane l ^ 32.
__device__ __forceinline__ float xhalf(float x) { return __shfl_xor(x, 32); }

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

// ---- 4x4 bf16 block transpose ----------------------------------------------
// rows[e] holds elements (row e, cols 0..3) of a 4x4 block; returns in
// out[t] the elements (rows 0..3, col t).
__device__ __forceinline__ void transpose4x4(const u32x2 rows[4], u32x2 out[4]) {
  out[0] = u32x2{(rows[0].x & 0xffffu) | (rows[1].x << 16), (rows[2].x & 0xffffu) | (rows[3].x << 16)};
  out[1] = u32x2{(rows[0].x >> 16) | (rows[1].x & 0xffff0000u), (rows[2].x >> 16) | (rows[3].x & 0xffff0000u)};
  out[2] = u32x2{(rows[0].y & 0xffffu) | (rows[1].y << 16), (rows[2].y & 0xffffu) | (rows[3].y << 16)};
  out[3] = u32x2{(rows[0].y >> 16) | (rows[1].y & 0xffff0000u), (rows[2].y >> 16) | (rows[3].y & 0xffff0000u)};
}

// ---- tile staging -----------------------------------------------------------
// A tile of ROWS consecutive sequence rows x D columns (bf16) is staged by
// NT threads.  Natural layout in LDS: [ROWS][D], pitch 2*D bytes, 16-byte
// chunks swizzled by swz(row, .).  Transposed layout: [D][ROWS], pitch
// 2*ROWS bytes, chunks swizzled by swz(col, .).  Rows at or beyond `nvalid`
// are staged as zeros.

// Natural layout only, 16-byte pieces.
template <int ROWS, int D, int NT>
struct StageRows16 {
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int NCHUNK = ROWS * CH;
  static constexpr int PER = (NCHUNK + NT - 1) / NT;   // chunks per thread
  static_assert(NCHUNK % NT == 0 || NCHUNK < NT, "tile must divide evenly");
  u32x4 r[PER];

  __device__ __forceinline__ void load(const __bf16* src, int row0, int nvalid, int tid) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int u = tid + NT * e;
      const int row = u / CH, ch = u % CH;
      if (u < NCHUNK && row0 + row < nvalid)
        r[e] = gload16(src + (size_t)(row0 + row) * D + ch * 8);
      else
        r[e] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int u = tid + NT * e;
      const int row = u / CH, ch = u % CH;
      if (u < NCHUNK) lds_write16(lds + row * (2 * D) + swz(row, ch, CH) * 16, r[e]);
    }
  }
};

// 4x4 blocks, written in natural and/or transposed layout.
template <int ROWS, int D, int NT>
struct StageBlocks4 {
  static constexpr int CG = D / 4;                 // 4-column groups per row
  static constexpr int NBLK = (ROWS / 4) * CG;
  static constexpr int PER = (NBLK + NT - 1) / NT;
  static_assert(NBLK % NT == 0 || NBLK < NT, "tile must divide evenly");
  u32x2 r[PER][4];

  __device__ __forceinline__ void load(const __bf16* src, int row0, int nvalid, int tid) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int blk = tid + NT * e;
      const int c0 = 4 * (blk % CG), j0 = 4 * (blk / CG);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (blk < NBLK && row0 + j0 + t < nvalid)
          r[e][t] = gload8(src + (size_t)(row0 + j0 + t) * D + c0);
        else
          r[e][t] = u32x2{0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store_nat(char* lds, int tid) const {
    constexpr int CH = D / 8;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int blk = tid + NT * e;
      if (blk >= NBLK) continue;
      const int c0 = 4 * (blk % CG), j0 = 4 * (blk / CG);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = j0 + t;
        lds_write8(lds + row * (2 * D) + swz(row, c0 >> 3, CH) * 16 + ((c0 >> 2) & 1) * 8, r[e][t]);
      }
    }
  }
  __device__ __forceinline__ void store_tr(char* lds, int tid) const {
    constexpr int CH = ROWS / 8;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int blk = tid + NT * e;
      if (blk >= NBLK) continue;
      const int c0 = 4 * (blk % CG), j0 = 4 * (blk / CG);
      u32x2 t4[4];
      transpose4x4(r[e], t4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = c0 + t;
        lds_write8(lds + row * (2 * ROWS) + swz(row, j0 >> 3, CH) * 16 + ((j0 >> 2) & 1) * 8, t4[t]);
      }
    }
  }
};

// Read the 16-byte MFMA operand slice (row, logical chunk) of a swizzled tile.
template <int PITCH_BYTES>
__device__ __forceinline__ bf16x8 tile_read(const char* lds, int row, int chunk) {
  constexpr int CH = PITCH_BYTES / 16;
  return lds_read16(lds + row * PITCH_BYTES + swz(row, chunk, CH) * 16);
}

// 16-byte direct-to-LDS copy (global_load_lds_dwordx4): lane l of the wave
// writes its 16 bytes at lds + 16*l; lds must be wave-uniform.
__device__ __forceinline__ void lds_dma16(const void* src, char* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
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
  // data that the callers mask)
  __device__ __forceinline__ void issue(char* lds_tile, const __bf16* src, int row0, int N, int w) const {
    const char* base = reinterpret_cast<const char*>(src + (size_t)row0 * D);
    if (row0 + ROWS <= N) {
#pragma unroll
      for (int e = 0; e < ROUNDS; ++e) lds_dma16(base + off[e], lds_tile + (e * NW + w) * 1024);
    } else {
      const uint32_t last = (uint32_t)((N - 1 - row0) * PITCH);  // byte offset of row N-1
#pragma unroll
      for (int e = 0; e < ROUNDS; ++e) {
        const uint32_t o = (row0 + row[e] < N) ? off[e] : last + (off[e] - (uint32_t)(row[e] * PITCH));
        lds_dma16(base + o, lds_tile + (e * NW + w) * 1024);
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
