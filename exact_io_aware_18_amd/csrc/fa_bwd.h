// Backward attention kernels for gfx950, bf16 inputs, fp32 gradients.
//
// The backward pass never reads an N x N matrix: P is recomputed on-chip
// from Q, K and the stored per-row logsumexp ("Softmax rescaling /
// recomputation", summary page of "FlashAttention: Fast and Memory-Efficient
// Exact Attention with IO-Awareness", §3 Method).  The gradients are those of
// O = softmax(scale * Q K^T) V:
//   dV = P^T dO,  dP = dO V^T,  D_i = rowsum(dO o O)_i,
//   dS = P o (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Three launches, no atomics, bitwise repeatable:
//   bwd_pre   D_i = sum_c dO_ic O_ic                          (HBM-bound)
//   bwd_dkdv  one workgroup per 128 keys, loop over query tiles, dK and dV
//             accumulated in registers (keys outer, queries inner, the loop
//             order of the Figure 1 caption of "No More Quadratic Complexity
//             for Transformers: Discover the Power of Flash Attention!");
//             one wave per 32 keys at d = 64, a wave pair per 32 keys at
//             d = 128 (bwd_dkdv_pair_kernel)
//   bwd_dq    one workgroup per 128 queries, loop over key tiles, dQ
//             accumulated in registers (recomputes S and dP a second time
//             instead of accumulating dQ with atomics)
#pragma once

#include <type_traits>

#include "fa_device.h"
#include "fa_fwd.h"
#include "fa_sched.h"

namespace fa {

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* Dw;            // workspace: D_i, [B*H*N]
  const uint8_t* mask;  // nb x nb or nullptr
  int N;
  int nb;
  int ntile;            // workgroups per head
  int total;            // workgroups in the grid
  float c;              // scale * log2(e) (signed)
  float scale;
  DropArgs drop;        // used by the dropout instantiations only
};

// Keep bits, for the lane's key kj, of the four queries i0 .. i0+3 held by
// accumulator rows of the S = Q K^T layout (lane = key): the four lanes of a
// quad share the queries and hold four consecutive keys, so each computes
// one generator call (query i0 + t, keys kj & ~3 ..) and the quad exchanges
// the bits.
__device__ __forceinline__ uint32_t keep4_keylane(const DropArgs& dp, int bh, int i0, int kj,
                                                  int lane) {
  const int t = lane & 3;
  return quad_transpose4(keep4(dp, bh, i0 + t, kj & ~3), t);
}

// ---- D_i = sum_c dO_ic * O_ic ------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* __restrict__ o,
                                                      const __bf16* __restrict__ dout,
                                                      float* __restrict__ Dw, long rows) {
  constexpr int LPR = D / 8;  // lanes per row, 16 bytes each
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gid / LPR;
  const int part = (int)(gid % LPR);
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, gload16(o + row * D + part * 8));
    const bf16x8 y = __builtin_bit_cast(bf16x8, gload16(dout + row * D + part * 8));
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)x[e], (float)y[e], acc);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (part == 0 && row < rows) Dw[row] = acc;
}

// ---- dK, dV: keys outer (d = 64) -------------------------------------------
// One workgroup owns 128 keys (one mask block); each wave keeps the K and V
// rows of its 32 keys in registers and accumulates dK^T and dV^T in
// registers.  Query tiles of 64 rows (Q, dO, and per query lse*log2(e) and
// D) stream through two LDS buffers; Q and dO are read as rows for S = Q K^T
// and dP = dO V^T and through transposed reads for dK^T += Q^T dS and
// dV^T += dO^T P.
template <int D>
struct DkdvTile {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BK = 32 * NW;  // 128 keys per workgroup
  static constexpr int BQ = 64;       // queries per tile
  static constexpr int PITCH = 2 * D;
  static constexpr int T_BYTES = BQ * PITCH;
  static constexpr int LIST_CAP = 1024;
  static constexpr int MIN_WG = 2;  // two waves per SIMD
};

template <int D, bool CAUSAL, bool MASK, bool DROP>
__global__ __launch_bounds__(256, DkdvTile<D>::MIN_WG) void bwd_dkdv_kernel(BwdArgs a) {
  using T = DkdvTile<D>;
  constexpr int NT = T::NT, BQ = T::BQ, BK = T::BK, PITCH = T::PITCH;
  constexpr int NKC = D / 16, NCT = D / 32;
  constexpr int TPB = 128 / BQ;  // query tiles per mask block
  __shared__ __attribute__((aligned(1024))) char qb0[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char qb1[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char db0[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char db1[T::T_BYTES];
  __shared__ __attribute__((aligned(16))) float lb0[BQ], lb1[BQ], eb0[BQ], eb1[BQ];
  __shared__ int blist[MASK ? T::LIST_CAP : 1];
  __shared__ int wcount[T::NW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  int bh, kt;
  if (CAUSAL) {  // low key tiles see the most queries: they go first, over all heads
    causal_rank(blockIdx.x, a.total / a.ntile, bh, kt);
  } else {
    const int g = xcd_remap(blockIdx.x, a.total);
    bh = g / a.ntile;
    kt = g - bh * a.ntile;
  }
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const int k0 = kt * BK;
  const int kw0 = k0 + 32 * w;
  const int kj = kw0 + li;  // this lane's key

  // K and V rows (B operands): lane supplies row kj, columns 16kc+8h..+7.
  bf16x8 kf[NKC], vf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    u32x4 x = u32x4{0u, 0u, 0u, 0u}, y = x;
    if (kj < N) {
      x = gload16(a.k + head + (size_t)kj * D + 16 * kc + 8 * h);
      y = gload16(a.v + head + (size_t)kj * D + 16 * kc + 8 * h);
    }
    kf[kc] = __builtin_bit_cast(bf16x8, x);
    vf[kc] = __builtin_bit_cast(bf16x8, y);
  }
  f32x16 dk[NCT], dv[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) { dk[ct] = f32x16{}; dv[ct] = f32x16{}; }

  const __bf16* Qh = a.q + head;
  const __bf16* dOh = a.dout + head;
  const float* Lh = a.lse + (size_t)bh * N;
  const float* Dh = a.Dw + (size_t)bh * N;
  const float c = a.c;
  TileOffsets<D> toff;
  toff.init(lane);
  TileCopy<BQ, D, NT> cp;  // Q and dO tiles have the same shape
  cp.init(w, lane);

  // raw lse (wave 0) or D (wave 1) of query q0 + lane, loaded a step ahead
  // and converted only when stored, so that nothing waits for the load early
  auto load_vec = [&] __device__ (int q0) -> float {
    const int i = q0 + lane;
    float x = 0.f;
    if (w < 2 && i < N) x = (w == 0 ? Lh : Dh)[i];
    return x;
  };
  auto store_vec = [&] __device__ (float* lb, float* eb, float x) {
    if (w == 0) {
      const float l = x * kLog2e;
      lb[lane] = (l == -INFINITY) ? INFINITY : l;  // empty row: P = 0
    } else if (w == 1) {
      eb[lane] = x;
    }
  };

  // One 64-query tile: two 32-query sub-blocks, overlapped inside the wave.
  // The S and dP products of sub-block 1 go between the softmax steps of
  // sub-block 0 (four elements each), and the dV and dK products of
  // sub-block 0 between those of sub-block 1, so that the wave's own products
  // run while it issues VALU work; dK and dV sum sub-block 0, then 1.  Causal
  // and range masks apply per element, behind a uniform branch per
  // sub-block; with dropout each step of four queries makes the one generator
  // call that covers them.  A sub-block whose queries all precede the wave's
  // keys is not skipped: with P = dS = 0 its products add exact zeros to
  // accumulators that are never -0.  One path for every tile keeps the
  // accumulators in the same registers from tile to tile.
  static_assert(BQ == 64, "the overlapped tile has two 32-query sub-blocks");
  auto compute_pipe = [&] __device__ (const char* qt, const char* dt, const float* lt, const float* et, int q0) {
    auto rowop = [&] __device__ (int sb, int m) -> bf16x8 {
      return lds_read16(((m & 1) ? dt : qt) + 32 * sb * PITCH + toff.rows[m >> 1]);
    };
    auto trop = [&] __device__ (int sb, int m) -> bf16x8 {
      return toff.read_tr(((m & 2) ? qt : dt) + 32 * sb * PITCH, m & 1, m >> 2);
    };
    constexpr int NM1 = 2 * NKC, NM2 = 4 * NCT;  // products per sub-block
    f32x16 S[2], dP[2];
    // sub-block 0: S and dP
    {
      bf16x8 ring[4];
#pragma unroll
      for (int m = 0; m < 3; ++m) ring[m] = rowop(0, m);
      S[0] = f32x16{};
      dP[0] = f32x16{};
#pragma unroll
      for (int m = 0; m < NM1; ++m) {
        if (m + 3 < NM1) ring[(m + 3) & 3] = rowop(0, m + 3);
        if (m & 1) dP[0] = mfma32(ring[m & 3], vf[m >> 1], dP[0]);
        else S[0] = mfma32(ring[m & 3], kf[m >> 1], S[0]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // softmax step of sub-block sb, elements 4u .. 4u+3 (group u of lse and
    // D), straight into the bf16 P and dS operands (k-step u / 2); causal and
    // range masks only on the tiles that need them
    bool edge[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int qs0 = q0 + 32 * sb;
      edge[sb] = (CAUSAL && qs0 < kw0 + 31) || (qs0 + 32 > N);
    }
    bf16x8 pb[2][2], sbv[2][2];
    auto soft4 = [&] __device__ (int sb, int u, const f32x4& l4, const f32x4& e4) __attribute__((always_inline)) {
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[sb][4 * u + e], c, -l4[e]));
      if (edge[sb]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qq = q0 + 32 * sb + acc_row(4 * u + e, h);
          if ((CAUSAL && kj > qq) || qq >= N) pv[e] = 0.f;
        }
      }
      uint32_t kbits = 0xFu;  // keep bits of queries q0 + 32 sb + 16 (u / 2) + 8h + 4 (u % 2) + e
      if constexpr (DROP)
        kbits = keep4_keylane(a.drop, bh, q0 + 32 * sb + 16 * (u >> 1) + 8 * h + 4 * (u & 1), kj, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * u + e;
        if constexpr (DROP) {
          const bool kept = (kbits >> e) & 1u;
          pb[sb][u >> 1][r & 7] = (__bf16)(kept ? pv[e] : 0.f);
          sbv[sb][u >> 1][r & 7] = (__bf16)(pv[e] * ((kept ? dP[sb][r] * a.drop.keep_scale : 0.f) - e4[e]));
        } else {
          pb[sb][u >> 1][r & 7] = (__bf16)pv[e];
          sbv[sb][u >> 1][r & 7] = (__bf16)(pv[e] * (dP[sb][r] - e4[e]));
        }
      }
    };
    auto lvec = [&] __device__ (const float* v, int sb, int u) -> f32x4 {
      return *reinterpret_cast<const f32x4*>(v + 32 * sb + 16 * (u >> 1) + 8 * h + 4 * (u & 1));
    };
    // sub-block 1's S and dP products between sub-block 0's softmax steps
    {
      f32x4 l4 = lvec(lt, 0, 0), e4 = lvec(et, 0, 0);  // one group ahead
      bf16x8 ring[3];  // two products ahead: the softmax steps cover the reads
#pragma unroll
      for (int m = 0; m < 2; ++m) ring[m] = rowop(1, m);
      S[1] = f32x16{};
      dP[1] = f32x16{};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int j = 0; j < NM1 / 4; ++j) {
          const int m = (NM1 / 4) * u + j;
          if (m + 2 < NM1) ring[(m + 2) % 3] = rowop(1, m + 2);
          if (m & 1) dP[1] = mfma32(ring[m % 3], vf[m >> 1], dP[1]);
          else S[1] = mfma32(ring[m % 3], kf[m >> 1], S[1]);
        }
        const f32x4 lc = l4, ec = e4;
        if (u + 1 < 4) { l4 = lvec(lt, 0, u + 1); e4 = lvec(et, 0, u + 1); }
        soft4(0, u, lc, ec);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // sub-block 0's dV and dK products between sub-block 1's softmax steps
    {
      f32x4 l4 = lvec(lt, 1, 0), e4 = lvec(et, 1, 0);
      bf16x8 ring[3];
#pragma unroll
      for (int m = 0; m < 2; ++m) ring[m] = trop(0, m);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int j = 0; j < NM2 / 4; ++j) {
          const int m = (NM2 / 4) * u + j;
          if (m + 2 < NM2) ring[(m + 2) % 3] = trop(0, m + 2);
          const int ct = m >> 2;
          if (m & 2) dk[ct] = mfma32(ring[m % 3], sbv[0][m & 1], dk[ct]);
          else dv[ct] = mfma32(ring[m % 3], pb[0][m & 1], dv[ct]);
        }
        const f32x4 lc = l4, ec = e4;
        if (u + 1 < 4) { l4 = lvec(lt, 1, u + 1); e4 = lvec(et, 1, u + 1); }
        soft4(1, u, lc, ec);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // sub-block 1's dV and dK products
    {
      bf16x8 ring[4];
#pragma unroll
      for (int m = 0; m < 3; ++m) ring[m] = trop(1, m);
#pragma unroll
      for (int m = 0; m < NM2; ++m) {
        if (m + 3 < NM2) ring[(m + 3) & 3] = trop(1, m + 3);
        const int ct = m >> 2;
        if (m & 2) dk[ct] = mfma32(ring[m & 3], sbv[1][m & 1], dk[ct]);
        else dv[ct] = mfma32(ring[m & 3], pb[1][m & 1], dv[ct]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  const int kb = k0 >> 7;  // mask column (BK == 128)
  const int nqt_all = (N + BQ - 1) / BQ;
  const int qb_lo = CAUSAL ? kb : 0;
  for (int cb0 = qb_lo; cb0 < (MASK ? a.nb : qb_lo + 1); cb0 += T::LIST_CAP) {
    int ntiles, first = 0;
    if (!MASK) {
      first = CAUSAL ? k0 / BQ : 0;
      ntiles = nqt_all - first;
    } else {
      const int cb1 = min(a.nb, cb0 + T::LIST_CAP);
      const int cnt = compact_mask_run<NT>(a.mask, (size_t)kb, (size_t)a.nb, cb0, cb1, blist, wcount);
      ntiles = cnt * TPB;
      if (cnt > 0 && blist[cnt - 1] * TPB + TPB > nqt_all) ntiles -= blist[cnt - 1] * TPB + TPB - nqt_all;
    }
    auto tile_of = [&] __device__ (int t) -> int { return MASK ? blist[t / TPB] * TPB + (t % TPB) : first + t; };
    if (ntiles == 0) continue;

    {
      const int q0 = tile_of(0) * BQ;
      cp.issue(qb0, Qh, q0, N, w);
      cp.issue(db0, dOh, q0, N, w);
      store_vec(lb0, eb0, load_vec(q0));
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    auto step = [&] __device__ (int t, const char* qc, const char* dc, const float* lc, const float* ec,
                                char* qn, char* dn, float* ln, float* en) {
      float nv = 0.f;
      if (t + 1 < ntiles) {
        const int q1 = tile_of(t + 1) * BQ;
        cp.issue(qn, Qh, q1, N, w);
        cp.issue(dn, dOh, q1, N, w);
        nv = load_vec(q1);
      }
      const int q0 = tile_of(t) * BQ;
      if (kw0 < N) compute_pipe(qc, dc, lc, ec, q0);
      if (t + 1 < ntiles) store_vec(ln, en, nv);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
      step(t, qb0, db0, lb0, eb0, qb1, db1, lb1, eb1);
      if (t + 1 < ntiles) step(t + 1, qb1, db1, lb1, eb1, qb0, db0, lb0, eb0);
    }
  }

  if (kj < N) {
    float* dKrow = a.dk + head + (size_t)kj * D;
    float* dVrow = a.dv + head + (size_t)kj * D;
    const float sc = a.scale;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int col = 32 * ct + 16 * hh + 8 * h;
        const int r0 = 8 * hh;
        f32x4* pk = reinterpret_cast<f32x4*>(dKrow + col);
        f32x4* pv = reinterpret_cast<f32x4*>(dVrow + col);
        pk[0] = f32x4{dk[ct][r0] * sc, dk[ct][r0 + 1] * sc, dk[ct][r0 + 2] * sc, dk[ct][r0 + 3] * sc};
        pk[1] = f32x4{dk[ct][r0 + 4] * sc, dk[ct][r0 + 5] * sc, dk[ct][r0 + 6] * sc, dk[ct][r0 + 7] * sc};
        const float vs = DROP ? a.drop.keep_scale : 1.f;  // dV = (P o Z)^T dO / (1 - p)
        pv[0] = f32x4{dv[ct][r0] * vs, dv[ct][r0 + 1] * vs, dv[ct][r0 + 2] * vs, dv[ct][r0 + 3] * vs};
        pv[1] = f32x4{dv[ct][r0 + 4] * vs, dv[ct][r0 + 5] * vs, dv[ct][r0 + 6] * vs, dv[ct][r0 + 7] * vs};
      }
  }
}

// ---- dK, dV with a wave pair per 32 keys --------------------------------------
// A wave issues an LDS read only every ~23-31 cycles whatever its width
// (measured on gfx950), and the kernel above issues 1.5 of them per MFMA; at
// d = 128 it runs one wave per SIMD and is bound by that issue rate.  Here
// the work of each 32-key group is split between two waves on one SIMD:
//   the P-wave holds K, computes S = Q K^T and P, hands P to its partner
//   through LDS and accumulates dV^T += dO^T P;
//   the dS-wave holds V, computes dP = dO V^T, takes P and forms
//   dS = P o (dP - D), and accumulates dK^T += Q^T dS.
// Each wave needs about half the registers of the single-wave kernel, so two
// share a SIMD and the LDS reads of one overlap the MFMAs of the other.  P
// crosses in fp32 with the dropout decision in its sign bit, so every value
// is computed exactly as in the single-wave kernel.
template <int D>
struct DkdvPairTile {
  static constexpr int NW = 8;
  static constexpr int NT = 64 * NW;
  static constexpr int NPAIR = NW / 2;
  static constexpr int BK = 32 * NPAIR;  // 128 keys per workgroup
  static constexpr int BQ = 64;          // queries per tile
  static constexpr int PITCH = 2 * D;
  static constexpr int T_BYTES = BQ * PITCH;
  static constexpr int P_BYTES = BQ * 32 * 4;  // one pair's P of a tile, fp32
  static constexpr int LIST_CAP = 1024;
};

// Workgroup barrier for LDS written by the waves themselves: the
// direct-to-LDS tile copies still in flight (vmcnt) are not waited for.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D, bool CAUSAL, bool MASK, bool DROP>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_pair_kernel(BwdArgs a) {
  using T = DkdvPairTile<D>;
  constexpr int NT = T::NT, BQ = T::BQ, BK = T::BK, PITCH = T::PITCH;
  constexpr int NKC = D / 16, NCT = D / 32;
  constexpr int TPB = 128 / BQ;  // query tiles per mask block
  __shared__ __attribute__((aligned(1024))) char qb0[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char qb1[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char db0[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char db1[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char pbuf[T::NPAIR * T::P_BYTES];
  __shared__ __attribute__((aligned(16))) float lb0[BQ], lb1[BQ], eb0[BQ], eb1[BQ];
  __shared__ int blist[MASK ? T::LIST_CAP : 1];
  __shared__ int wcount[T::NW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = w & (T::NPAIR - 1);
  const bool ds_wave = w >= T::NPAIR;  // waves w and w + 4 share a SIMD
  const int h = lane >> 5, li = lane & 31;
  int bh, kt;
  if (CAUSAL) {  // low key tiles see the most queries: they go first, over all heads
    causal_rank(blockIdx.x, a.total / a.ntile, bh, kt);
  } else {
    const int g = xcd_remap(blockIdx.x, a.total);
    bh = g / a.ntile;
    kt = g - bh * a.ntile;
  }
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const int k0 = kt * BK;
  const int kw0 = k0 + 32 * pair;
  const int kj = kw0 + li;  // this lane's key

  // B operand rows: K (P-wave) or V (dS-wave), row kj, columns 16kc+8h..+7
  bf16x8 bop[NKC];
  {
    const __bf16* src = (ds_wave ? a.v : a.k) + head + (size_t)kj * D;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (kj < N) x = gload16(src + 16 * kc + 8 * h);
      bop[kc] = __builtin_bit_cast(bf16x8, x);
    }
  }
  f32x16 acc[NCT];  // dV^T (P-wave) or dK^T (dS-wave)
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x16{};

  const __bf16* Qh = a.q + head;
  const __bf16* dOh = a.dout + head;
  const float* Lh = a.lse + (size_t)bh * N;
  const float* Dh = a.Dw + (size_t)bh * N;
  const float c = a.c;
  TileOffsets<D> toff;
  toff.init(lane);
  // the four dS-waves copy the Q tiles, the four P-waves the dO tiles
  TileCopy<BQ, D, NT / 2> cp;
  cp.init(pair, lane);
  // this lane's 16-byte slots of the pair's P: + 1024 * (4 * sb + j)
  char* const pslot = pbuf + pair * T::P_BYTES + 16 * lane;

  // raw lse (wave 0) or D (wave 1) of query q0 + lane, loaded a step ahead
  // and converted only when stored, so that nothing waits for the load early
  auto load_vec = [&] __device__ (int q0) -> float {
    const int i = q0 + lane;
    float x = 0.f;
    if (w < 2 && i < N) x = (w == 0 ? Lh : Dh)[i];
    return x;
  };
  auto store_vec = [&] __device__ (float* lb, float* eb, float x) {
    if (w == 0) {
      const float l = x * kLog2e;
      lb[lane] = (l == -INFINITY) ? INFINITY : l;  // empty row: P = 0
    } else if (w == 1) {
      eb[lane] = x;
    }
  };

  // Phase 1: X = S (P-wave, rows of Q) or dP (dS-wave, rows of dO) for the
  // two 32-query sub-blocks; the P-wave turns S into P, keeps it as bf16 B
  // operands and writes it (fp32) for its partner.
  auto phase1 = [&] __device__ (auto role_c, auto edge_c, const char* qt, const char* dt, const float* lt,
                                const float* et, int q0, f32x16* X, bf16x8* pb) __attribute__((always_inline)) {
    constexpr bool DS = decltype(role_c)::value;
    constexpr bool EDGE = decltype(edge_c)::value;
    const char* src = DS ? dt : qt;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      bf16x8 av[NKC];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) av[kc] = lds_read16(src + 32 * sb * PITCH + toff.rows[kc]);
      X[sb] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) X[sb] = mfma32(av[kc], bop[kc], X[sb]);
    }
    if constexpr (DS) {
      // dP - D here, where the dS-wave would otherwise wait for P
      if constexpr (!DROP) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const f32x4 e0 = *reinterpret_cast<const f32x4*>(et + 32 * sb + 16 * hf + 8 * h);
            const f32x4 e1 = *reinterpret_cast<const f32x4*>(et + 32 * sb + 16 * hf + 8 * h + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) X[sb][8 * hf + e] -= e < 4 ? e0[e] : e1[e - 4];
          }
      }
      return;
    }
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int qs0 = q0 + 32 * sb;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(lt + 32 * sb + 16 * hf + 8 * h);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(lt + 32 * sb + 16 * hf + 8 * h + 4);
        uint32_t kbits = 0xFFu;  // keep bits of rows 8hf .. 8hf+7
        if constexpr (DROP) {
          const int i0 = qs0 + 16 * hf + 8 * h;
          kbits = keep4_keylane(a.drop, bh, i0, kj, lane) | (keep4_keylane(a.drop, bh, i0 + 4, kj, lane) << 4);
        }
        float p[8], x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * hf + e;
          const float lv = e < 4 ? l0[e] : l1[e - 4];
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(X[sb][r], c, -lv));
          if (EDGE) {
            const int qq = qs0 + acc_row(r, h);
            if ((CAUSAL && kj > qq) || qq >= N) pv = 0.f;
          }
          if constexpr (DROP) {
            const bool kept = (kbits >> e) & 1u;
            p[e] = kept ? pv : 0.f;
            x[e] = kept ? pv : -pv;
          } else {
            p[e] = pv;
            x[e] = pv;
          }
        }
        pb[2 * sb + hf] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        f32x4* dst = reinterpret_cast<f32x4*>(pslot + 1024 * (4 * sb + 2 * hf));
        dst[0] = f32x4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32x4*>(pslot + 1024 * (4 * sb + 2 * hf + 1)) = f32x4{x[4], x[5], x[6], x[7]};
      }
    }
  };

  // Phase 2: the dS-wave forms dS = P o (dP - D) from its partner's P; both
  // accumulate over the tile's queries through transposed reads: dV^T +=
  // dO^T P (P-wave), dK^T += Q^T dS (dS-wave).
  auto phase2 = [&] __device__ (auto role_c, const char* qt, const char* dt, const float* et, const f32x16* X,
                                bf16x8* pb) __attribute__((always_inline)) {
    constexpr bool DS = decltype(role_c)::value;
    if constexpr (DS) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(pslot + 1024 * (4 * sb + 2 * hf));
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(pslot + 1024 * (4 * sb + 2 * hf + 1));
          float dsv[8];
          if constexpr (DROP) {
            const f32x4 e0 = *reinterpret_cast<const f32x4*>(et + 32 * sb + 16 * hf + 8 * h);
            const f32x4 e1 = *reinterpret_cast<const f32x4*>(et + 32 * sb + 16 * hf + 8 * h + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 8 * hf + e;
              const float x = e < 4 ? x0[e] : x1[e - 4];
              const float dvv = e < 4 ? e0[e] : e1[e - 4];
              const bool kept = (__float_as_uint(x) >> 31) == 0u;
              dsv[e] = __builtin_fabsf(x) * ((kept ? X[sb][r] * a.drop.keep_scale : 0.f) - dvv);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) dsv[e] = (e < 4 ? x0[e] : x1[e - 4]) * X[sb][8 * hf + e];  // X = dP - D
          }
          pb[2 * sb + hf] = to_bf16x8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
        }
    }
    const char* src = DS ? qt : dt;
    // MFMA m = 2 NCT sb + 2 ct + hf in the order of the sums; its transposed
    // operand is read three MFMAs ahead into a ring of four, one scheduling
    // step per MFMA, so each wait covers exactly the operand it needs
    constexpr int NM = 4 * NCT;
    auto opnd = [&] __device__ (int m) -> bf16x8 {
      return toff.read_tr(src + 32 * (m / (2 * NCT)) * PITCH, m & 1, (m >> 1) % NCT);
    };
    bf16x8 ring[4];
#pragma unroll
    for (int m = 0; m < 3; ++m) ring[m] = opnd(m);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m + 3 < NM) ring[(m + 3) & 3] = opnd(m + 3);
      const int ct = (m >> 1) % NCT;
      acc[ct] = mfma32(ring[m & 3], pb[2 * (m / (2 * NCT)) + (m & 1)], acc[ct]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // the whole tile loop in one copy per role, so that each role's
  // registers are allocated for that role alone (the barriers match)
  auto run = [&] __device__ (auto role_c) __attribute__((always_inline)) {
  const int kb = k0 >> 7;  // mask column (BK == 128)
  const int nqt_all = (N + BQ - 1) / BQ;
  const int qb_lo = CAUSAL ? kb : 0;
  for (int cb0 = qb_lo; cb0 < (MASK ? a.nb : qb_lo + 1); cb0 += T::LIST_CAP) {
    int ntiles, first = 0;
    if (!MASK) {
      first = CAUSAL ? k0 / BQ : 0;
      ntiles = nqt_all - first;
    } else {
      const int cb1 = min(a.nb, cb0 + T::LIST_CAP);
      const int cnt = compact_mask_run<NT>(a.mask, (size_t)kb, (size_t)a.nb, cb0, cb1, blist, wcount);
      ntiles = cnt * TPB;
      if (cnt > 0 && blist[cnt - 1] * TPB + TPB > nqt_all) ntiles -= blist[cnt - 1] * TPB + TPB - nqt_all;
    }
    auto tile_of = [&] __device__ (int t) -> int { return MASK ? blist[t / TPB] * TPB + (t % TPB) : first + t; };
    if (ntiles == 0) continue;

    {
      const int q0 = tile_of(0) * BQ;
      if constexpr (decltype(role_c)::value) cp.issue(qb0, Qh, q0, N, pair);
      else cp.issue(db0, dOh, q0, N, pair);
      store_vec(lb0, eb0, load_vec(q0));
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    auto step = [&] __device__ (int t, const char* qc, const char* dc, const float* lc, const float* ec,
                                char* qn, char* dn, float* ln, float* en) __attribute__((always_inline)) {
      constexpr bool DS = decltype(role_c)::value;
      float nv = 0.f;
      const int q1 = (t + 1 < ntiles) ? tile_of(t + 1) * BQ : 0;
      if (t + 1 < ntiles) {
        if constexpr (DS) cp.issue(qn, Qh, q1, N, pair);  // the dS-wave waits for P in phase 1 anyway
        nv = load_vec(q1);
      }
      const int q0 = tile_of(t) * BQ;
      // the pair has work unless its keys are past the end or follow every query
      const bool live = kw0 < N && !(CAUSAL && q0 + BQ - 1 < kw0);
      f32x16 X[2];
      bf16x8 pb[4];
      if (live) {
        if ((CAUSAL && q0 < kw0 + 31) || (q0 + BQ > N))
          phase1(role_c, std::true_type{}, qc, dc, lc, ec, q0, X, pb);
        else
          phase1(role_c, std::false_type{}, qc, dc, lc, ec, q0, X, pb);
      }
      lds_barrier();  // P of the tile is in LDS
      if constexpr (!DS) {  // and the P-wave has the shorter phase 2
        if (t + 1 < ntiles) cp.issue(dn, dOh, q1, N, pair);
      }
      if (live) phase2(role_c, qc, dc, ec, X, pb);
      if (t + 1 < ntiles) store_vec(ln, en, nv);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // next tile landed; this tile's buffers and P are free
    };
    for (int t = 0; t < ntiles; t += 2) {
      step(t, qb0, db0, lb0, eb0, qb1, db1, lb1, eb1);
      if (t + 1 < ntiles) step(t + 1, qb1, db1, lb1, eb1, qb0, db0, lb0, eb0);
    }
  }
  };
  if (ds_wave) run(std::true_type{});
  else run(std::false_type{});

  if (kj < N) {
    // dK = scale * dS^T Q; dV = (P o Z)^T dO / (1 - p) under dropout
    float* row = (ds_wave ? a.dk : a.dv) + head + (size_t)kj * D;
    const float sc = ds_wave ? a.scale : (DROP ? a.drop.keep_scale : 1.f);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int col = 32 * ct + 16 * hh + 8 * h;
        const int r0 = 8 * hh;
        f32x4* pr = reinterpret_cast<f32x4*>(row + col);
        pr[0] = f32x4{acc[ct][r0] * sc, acc[ct][r0 + 1] * sc, acc[ct][r0 + 2] * sc, acc[ct][r0 + 3] * sc};
        pr[1] = f32x4{acc[ct][r0 + 4] * sc, acc[ct][r0 + 5] * sc, acc[ct][r0 + 6] * sc, acc[ct][r0 + 7] * sc};
      }
  }
}

// ---- dQ: queries outer -------------------------------------------------------
// One workgroup owns 128 queries; each wave keeps Q and dO of its 32 queries
// in registers and accumulates dQ^T in registers.  K/V tiles of 64 keys
// stream through two LDS buffers; K is read as rows for S^T = K Q^T and
// through transposed reads for dQ^T += K^T dS^T; V as rows for dP^T = V dO^T.
template <int D>
struct DqTile {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;  // 128 queries per workgroup
  static constexpr int BC = 64;       // keys per tile
  static constexpr int PITCH = 2 * D;
  static constexpr int T_BYTES = BC * PITCH;
  static constexpr int LIST_CAP = 1024;
  static constexpr int MIN_WG = 2;
};

template <int D, bool CAUSAL, bool MASK, bool DROP>
__global__ __launch_bounds__(256, DqTile<D>::MIN_WG) void bwd_dq_kernel(BwdArgs a) {
  using T = DqTile<D>;
  constexpr int NT = T::NT, BR = T::BR, BC = T::BC, PITCH = T::PITCH;
  constexpr int NKC = D / 16, NCT = D / 32;
  __shared__ __attribute__((aligned(1024))) char kb0[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char kb1[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb0[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb1[T::T_BYTES];
  __shared__ int blist[MASK ? T::LIST_CAP : 1];
  __shared__ int wcount[T::NW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  int bh, qt;
  if (CAUSAL) {  // longest rows first, over all heads
    causal_rank(blockIdx.x, a.total / a.ntile, bh, qt);
    qt = a.ntile - 1 - qt;
  } else {
    const int g = xcd_remap(blockIdx.x, a.total);
    bh = g / a.ntile;
    qt = g - bh * a.ntile;
  }
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const int q0 = qt * BR;
  const int qw0 = q0 + 32 * w;
  const int qi = qw0 + li;

  bf16x8 qf[NKC], df[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    u32x4 x = u32x4{0u, 0u, 0u, 0u}, y = x;
    if (qi < N) {
      x = gload16(a.q + head + (size_t)qi * D + 16 * kc + 8 * h);
      y = gload16(a.dout + head + (size_t)qi * D + 16 * kc + 8 * h);
    }
    qf[kc] = __builtin_bit_cast(bf16x8, x);
    df[kc] = __builtin_bit_cast(bf16x8, y);
  }
  float lse2 = (qi < N) ? a.lse[(size_t)bh * N + qi] * kLog2e : 0.f;
  if (lse2 == -INFINITY) lse2 = INFINITY;  // empty row: P = 0
  const float Di = (qi < N) ? a.Dw[(size_t)bh * N + qi] : 0.f;
  f32x16 dq[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) dq[ct] = f32x16{};

  const __bf16* Kh = a.k + head;
  const __bf16* Vh = a.v + head;
  const float c = a.c;
  TileOffsets<D> toff;
  toff.init(lane);
  TileCopy<BC, D, NT> cp;
  cp.init(w, lane);

  auto compute = [&] __device__ (const char* kt, const char* vt, int k0) {
    const bool edge = (CAUSAL && k0 + BC - 1 > qw0) || (k0 + BC > N);
    bf16x8 dsb[4];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      // S^T and dP^T: MFMA m takes K (m even) or V (m odd) rows of k-step
      // m/2, read three MFMAs ahead into a ring of four, one scheduling step
      // per MFMA, so each wait covers exactly the operand it needs
      auto rowop = [&] __device__ (int m) -> bf16x8 {
        return lds_read16(((m & 1) ? vt : kt) + toff.rows[m >> 1] + 32 * t2 * PITCH);
      };
      f32x16 S = f32x16{}, dP = f32x16{};
      {
        bf16x8 ring[4];
#pragma unroll
        for (int m = 0; m < 3; ++m) ring[m] = rowop(m);
#pragma unroll
        for (int m = 0; m < 2 * NKC; ++m) {
          if (m + 3 < 2 * NKC) ring[(m + 3) & 3] = rowop(m + 3);
          if (m & 1) dP = mfma32(ring[m & 3], df[m >> 1], dP);
          else S = mfma32(ring[m & 3], qf[m >> 1], S);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      float dsv[16];
      uint32_t kbits = 0xFFFFu;  // keep bits of rows 0..15 (keys k0 + 32 t2 + acc_row(r, h))
      if constexpr (DROP) {
        const int j0 = k0 + 32 * t2 + 8 * h;
        kbits = keep4(a.drop, bh, qi, j0) | (keep4(a.drop, bh, qi, j0 + 4) << 4) |
                (keep4(a.drop, bh, qi, j0 + 16) << 8) | (keep4(a.drop, bh, qi, j0 + 20) << 12);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], c, -lse2));
        if (edge) {
          const int key = k0 + 32 * t2 + acc_row(r, h);
          if ((CAUSAL && key > qi) || key >= N) pv = 0.f;
        }
        if constexpr (DROP) {
          const bool kept = (kbits >> r) & 1u;
          dsv[r] = pv * ((kept ? dP[r] * a.drop.keep_scale : 0.f) - Di);
        } else {
          dsv[r] = pv * (dP[r] - Di);
        }
      }
      dsb[2 * t2 + 0] = to_bf16x8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
      dsb[2 * t2 + 1] = to_bf16x8(dsv[8], dsv[9], dsv[10], dsv[11], dsv[12], dsv[13], dsv[14], dsv[15]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // dQ^T += K^T dS^T: MFMA m = (BC/16) ct + kc, transposed K operands
    // three MFMAs ahead as above
    {
      constexpr int KS = BC / 16, NM = NCT * KS;
      bf16x8 ring[4];
#pragma unroll
      for (int m = 0; m < 3; ++m) ring[m] = toff.read_tr(kt, m % KS, m / KS);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (m + 3 < NM) ring[(m + 3) & 3] = toff.read_tr(kt, (m + 3) % KS, (m + 3) / KS);
        dq[m / KS] = mfma32(ring[m & 3], dsb[m % KS], dq[m / KS]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // At d = 64, the tile's two 32-key halves overlapped inside the wave: half
  // 1's S and dP products go between half 0's exp and dS steps, the dQ
  // products over half 0's keys between half 1's, and those over half 1's
  // keys last.  Each dQ accumulator still sums the tile's k-steps in order
  // and every value is computed as in compute (with dropout, each step of
  // four keys makes the one generator call that covers them), so the results
  // are the same bit for bit.  It serves every tile, masked ones included, so
  // that the accumulators stay in the same registers.
  auto compute_pipe = [&] __device__ (const char* kt, const char* vt, int k0) {
    constexpr int NM1 = 2 * NKC;
    auto rowop = [&] __device__ (int t2, int m) -> bf16x8 {
      return lds_read16(((m & 1) ? vt : kt) + toff.rows[m >> 1] + 32 * t2 * PITCH);
    };
    f32x16 S[2], dP[2];
    bf16x8 dsb[4];
    {
      bf16x8 ring[4];
#pragma unroll
      for (int m = 0; m < 3; ++m) ring[m] = rowop(0, m);
      S[0] = f32x16{};
      dP[0] = f32x16{};
#pragma unroll
      for (int m = 0; m < NM1; ++m) {
        if (m + 3 < NM1) ring[(m + 3) & 3] = rowop(0, m + 3);
        if (m & 1) dP[0] = mfma32(ring[m & 3], df[m >> 1], dP[0]);
        else S[0] = mfma32(ring[m & 3], qf[m >> 1], S[0]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // exp and dS of half t2, rows 4u .. 4u+3, straight into its bf16
    // operands; causal and range masks only on the halves that need them
    bool edge[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int ks0 = k0 + 32 * t2;
      edge[t2] = (CAUSAL && ks0 + 31 > qw0) || (ks0 + 32 > N);
    }
    auto soft4 = [&] __device__ (int t2, int u) __attribute__((always_inline)) {
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[t2][4 * u + e], c, -lse2));
      if (edge[t2]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = k0 + 32 * t2 + acc_row(4 * u + e, h);
          if ((CAUSAL && key > qi) || key >= N) pv[e] = 0.f;
        }
      }
      uint32_t kbits = 0xFu;  // keep bits of the four keys k0 + 32 t2 + acc_row(4u + e, h)
      if constexpr (DROP) kbits = keep4(a.drop, bh, qi, k0 + 32 * t2 + 16 * (u >> 1) + 8 * h + 4 * (u & 1));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * u + e;
        float dsv;
        if constexpr (DROP) {
          const bool kept = (kbits >> e) & 1u;
          dsv = pv[e] * ((kept ? dP[t2][r] * a.drop.keep_scale : 0.f) - Di);
        } else {
          dsv = pv[e] * (dP[t2][r] - Di);
        }
        dsb[2 * t2 + (r >> 3)][r & 7] = (__bf16)dsv;
      }
    };
    // half 1's S and dP between half 0's steps
    {
      bf16x8 ring[3];
#pragma unroll
      for (int m = 0; m < 2; ++m) ring[m] = rowop(1, m);
      S[1] = f32x16{};
      dP[1] = f32x16{};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int j = 0; j < NM1 / 4; ++j) {
          const int m = (NM1 / 4) * u + j;
          if (m + 2 < NM1) ring[(m + 2) % 3] = rowop(1, m + 2);
          if (m & 1) dP[1] = mfma32(ring[m % 3], df[m >> 1], dP[1]);
          else S[1] = mfma32(ring[m % 3], qf[m >> 1], S[1]);
        }
        soft4(0, u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // dQ^T += K^T dS^T over half 0's k-steps (kc = 0, 1) between half 1's
    // steps, then over half 1's (kc = 2, 3); MFMA m of a half: ct = m / 2
    auto kop = [&] __device__ (int hk, int m) -> bf16x8 { return toff.read_tr(kt, 2 * hk + (m & 1), m >> 1); };
    {
      constexpr int NM = 2 * NCT;
      bf16x8 ring[3];
#pragma unroll
      for (int m = 0; m < 2; ++m) ring[m] = kop(0, m);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int j = 0; j < NM / 4; ++j) {
          const int m = (NM / 4) * u + j;
          if (m + 2 < NM) ring[(m + 2) % 3] = kop(0, m + 2);
          dq[m >> 1] = mfma32(ring[m % 3], dsb[m & 1], dq[m >> 1]);
        }
        soft4(1, u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    {
      constexpr int NM = 2 * NCT;
      bf16x8 ring[4];
#pragma unroll
      for (int m = 0; m < 3; ++m) ring[m] = kop(1, m);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (m + 3 < NM) ring[(m + 3) & 3] = kop(1, m + 3);
        dq[m >> 1] = mfma32(ring[m & 3], dsb[2 + (m & 1)], dq[m >> 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  const int ntiles_all = (N + BC - 1) / BC;
  const int qb = q0 >> 7;
  int kend_blocks = a.nb;
  if (MASK && CAUSAL) kend_blocks = min(a.nb, qb + 1);
  for (int cb0 = 0; cb0 < (MASK ? kend_blocks : 1); cb0 += T::LIST_CAP) {
    int ntiles;
    if (!MASK) {
      const int kend = CAUSAL ? min(N, q0 + BR) : N;
      ntiles = (kend + BC - 1) / BC;
    } else {
      const int cb1 = min(kend_blocks, cb0 + T::LIST_CAP);
      const int cnt = compact_mask_run<NT>(a.mask, (size_t)qb * a.nb, 1, cb0, cb1, blist, wcount);
      ntiles = 2 * cnt;
      if (cnt > 0 && 2 * blist[cnt - 1] + 1 >= ntiles_all) ntiles -= 1;
    }
    auto tile_of = [&] __device__ (int t) -> int { return MASK ? 2 * blist[t >> 1] + (t & 1) : t; };
    auto active = [&] __device__ (int k0) -> bool { return qw0 < N && !(CAUSAL && k0 > qw0 + 31); };
    if (ntiles == 0) continue;

    cp.issue(kb0, Kh, tile_of(0) * BC, N, w);
    cp.issue(vb0, Vh, tile_of(0) * BC, N, w);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    auto step = [&] __device__ (int t, const char* kc_, const char* vc_, char* kn, char* vn) {
      if (t + 1 < ntiles) {
        const int k1 = tile_of(t + 1) * BC;
        cp.issue(kn, Kh, k1, N, w);
        cp.issue(vn, Vh, k1, N, w);
      }
      const int k0 = tile_of(t) * BC;
      if (active(k0)) {
        if constexpr (D == 64) compute_pipe(kc_, vc_, k0);
        else compute(kc_, vc_, k0);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
      step(t, kb0, vb0, kb1, vb1);
      if (t + 1 < ntiles) step(t + 1, kb1, vb1, kb0, vb0);
    }
  }

  if (qi < N) {
    float* dQrow = a.dq + head + (size_t)qi * D;
    const float sc = a.scale;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int col = 32 * ct + 16 * hh + 8 * h;
        const int r0 = 8 * hh;
        f32x4* pq = reinterpret_cast<f32x4*>(dQrow + col);
        pq[0] = f32x4{dq[ct][r0] * sc, dq[ct][r0 + 1] * sc, dq[ct][r0 + 2] * sc, dq[ct][r0 + 3] * sc};
        pq[1] = f32x4{dq[ct][r0 + 4] * sc, dq[ct][r0 + 5] * sc, dq[ct][r0 + 6] * sc, dq[ct][r0 + 7] * sc};
      }
  }
}

}  // namespace fa
