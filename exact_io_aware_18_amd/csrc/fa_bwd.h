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
//             for Transformers: Discover the Power of Flash Attention!")
//   bwd_dq    one workgroup per 128 queries, loop over key tiles, dQ
//             accumulated in registers (recomputes S and dP a second time
//             instead of accumulating dQ with atomics)
#pragma once

#include "fa_device.h"
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
};

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

// ---- dK, dV: keys outer ----------------------------------------------------
template <int D>
struct DkdvTile {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BK = 32 * NW;            // 128 keys per workgroup
  static constexpr int BQ = (D == 64) ? 64 : 32;  // queries per tile
  static constexpr int T_BYTES = BQ * D * 2;
  // stage: Q, Q^T, dO, dO^T, lse*log2e, D
  static constexpr int OFF_Q = 0, OFF_QT = T_BYTES, OFF_DO = 2 * T_BYTES, OFF_DOT = 3 * T_BYTES;
  static constexpr int OFF_L = 4 * T_BYTES, OFF_D = 4 * T_BYTES + BQ * 4;
  static constexpr int STAGE = 4 * T_BYTES + 2 * BQ * 4;
  static constexpr int LIST_CAP = 1024;
  static constexpr int MIN_WG = (D == 64) ? 2 : 1;
};

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256, DkdvTile<D>::MIN_WG) void bwd_dkdv_kernel(BwdArgs a) {
  using T = DkdvTile<D>;
  constexpr int NT = T::NT, BQ = T::BQ, BK = T::BK;
  constexpr int TPB = 128 / BQ;  // query tiles per mask block
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];
  __shared__ int blist[MASK ? T::LIST_CAP : 1];
  __shared__ int wcount[T::NW];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, li = lane & 31;
  const int g = xcd_remap(blockIdx.x, a.total);
  const int bh = g / a.ntile;
  const int kt = g - bh * a.ntile;  // causal: low key tiles see the most queries, so they go first
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const int k0 = kt * BK;
  const int kw0 = k0 + 32 * w;
  const int kj = kw0 + li;  // this lane's key

  // K and V fragments (B operands): lane supplies row kj, columns 16kc+8h..+7.
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    u32x4 x = u32x4{0u, 0u, 0u, 0u}, y = x;
    if (kj < N) {
      x = gload16(a.k + head + (size_t)kj * D + 16 * kc + 8 * h);
      y = gload16(a.v + head + (size_t)kj * D + 16 * kc + 8 * h);
    }
    kf[kc] = __builtin_bit_cast(bf16x8, x);
    vf[kc] = __builtin_bit_cast(bf16x8, y);
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) { dk[ct] = f32x16{}; dv[ct] = f32x16{}; }

  const __bf16* Qh = a.q + head;
  const __bf16* dOh = a.dout + head;
  const float* Lh = a.lse + (size_t)bh * N;
  const float* Dh = a.Dw + (size_t)bh * N;
  const float c = a.c;

  StageBlocks4<BQ, D, NT> qs, ds;
  float lval = 0.f, dval = 0.f;
  auto load_tile = [&](int q0) {
    qs.load(Qh, q0, N, tid);
    ds.load(dOh, q0, N, tid);
    if (tid < BQ) {
      const int i = q0 + tid;
      // an empty row (lse = -inf) must give P = 0, not 2^inf
      lval = (i < N) ? Lh[i] * kLog2e : 0.f;
      if (lval == -INFINITY) lval = INFINITY;
    } else if (tid < 2 * BQ) {
      const int i = q0 + tid - BQ;
      dval = (i < N) ? Dh[i] : 0.f;
    }
  };
  auto store_tile = [&](char* st) {
    qs.store_nat(st + T::OFF_Q, tid);
    qs.store_tr(st + T::OFF_QT, tid);
    ds.store_nat(st + T::OFF_DO, tid);
    ds.store_tr(st + T::OFF_DOT, tid);
    if (tid < BQ) reinterpret_cast<float*>(st + T::OFF_L)[tid] = lval;
    else if (tid < 2 * BQ) reinterpret_cast<float*>(st + T::OFF_D)[tid - BQ] = dval;
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
    auto tile_of = [&](int t) -> int { return MASK ? blist[t / TPB] * TPB + (t % TPB) : first + t; };

    if (ntiles > 0) { load_tile(tile_of(0) * BQ); store_tile(smem); }
    if (ntiles > 1) load_tile(tile_of(1) * BQ);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
      const char* st = smem + (t & 1) * T::STAGE;
      const int q0 = tile_of(t) * BQ;
      if (kw0 < N) {
#pragma unroll
        for (int sb = 0; sb < BQ / 32; ++sb) {
          const int qs0 = q0 + 32 * sb;
          if (CAUSAL && qs0 + 31 < kw0) continue;  // every query precedes every key
          f32x16 S = f32x16{}, dP = f32x16{};
          const int row = 32 * sb + perm32(li);
#pragma unroll
          for (int kc = 0; kc < D / 16; ++kc) {
            S = mfma32(tile_read<2 * D>(st + T::OFF_Q, row, 2 * kc + h), kf[kc], S);
            dP = mfma32(tile_read<2 * D>(st + T::OFF_DO, row, 2 * kc + h), vf[kc], dP);
          }
          const float* Ls = reinterpret_cast<const float*>(st + T::OFF_L) + 32 * sb + 8 * h;
          const float* Ds = reinterpret_cast<const float*>(st + T::OFF_D) + 32 * sb + 8 * h;
          const bool edge = (CAUSAL && qs0 < kw0 + 31) || (qs0 + 32 > N);
          float p[16], dsv[16];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const f32x4 l0 = *reinterpret_cast<const f32x4*>(Ls + 16 * half);
            const f32x4 l1 = *reinterpret_cast<const f32x4*>(Ls + 16 * half + 4);
            const f32x4 d0 = *reinterpret_cast<const f32x4*>(Ds + 16 * half);
            const f32x4 d1 = *reinterpret_cast<const f32x4*>(Ds + 16 * half + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 8 * half + e;
              const float lv = e < 4 ? l0[e] : l1[e - 4];
              const float dvv = e < 4 ? d0[e] : d1[e - 4];
              float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], c, -lv));
              if (edge) {
                const int qq = qs0 + acc_row(r, h);
                if ((CAUSAL && kj > qq) || qq >= N) pv = 0.f;
              }
              p[r] = pv;
              dsv[r] = pv * (dP[r] - dvv);
            }
          }
          const bf16x8 pb0 = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
          const bf16x8 pb1 = to_bf16x8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
          const bf16x8 sb0 = to_bf16x8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
          const bf16x8 sb1 = to_bf16x8(dsv[8], dsv[9], dsv[10], dsv[11], dsv[12], dsv[13], dsv[14], dsv[15]);
#pragma unroll
          for (int ct = 0; ct < D / 32; ++ct) {
            const int crow = 32 * ct + perm32(li);
            dv[ct] = mfma32(tile_read<2 * BQ>(st + T::OFF_DOT, crow, 4 * sb + 0 + h), pb0, dv[ct]);
            dv[ct] = mfma32(tile_read<2 * BQ>(st + T::OFF_DOT, crow, 4 * sb + 2 + h), pb1, dv[ct]);
            dk[ct] = mfma32(tile_read<2 * BQ>(st + T::OFF_QT, crow, 4 * sb + 0 + h), sb0, dk[ct]);
            dk[ct] = mfma32(tile_read<2 * BQ>(st + T::OFF_QT, crow, 4 * sb + 2 + h), sb1, dk[ct]);
          }
        }
      }
      if (t + 1 < ntiles) store_tile(smem + ((t + 1) & 1) * T::STAGE);
      if (t + 2 < ntiles) load_tile(tile_of(t + 2) * BQ);
      __syncthreads();
    }
  }

  if (kj < N) {
    float* dKrow = a.dk + head + (size_t)kj * D;
    float* dVrow = a.dv + head + (size_t)kj * D;
    const float sc = a.scale;
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int col = 32 * ct + 16 * hh + 8 * h;
        const int r0 = 8 * hh;
        f32x4* pk = reinterpret_cast<f32x4*>(dKrow + col);
        f32x4* pv = reinterpret_cast<f32x4*>(dVrow + col);
        pk[0] = f32x4{dk[ct][r0] * sc, dk[ct][r0 + 1] * sc, dk[ct][r0 + 2] * sc, dk[ct][r0 + 3] * sc};
        pk[1] = f32x4{dk[ct][r0 + 4] * sc, dk[ct][r0 + 5] * sc, dk[ct][r0 + 6] * sc, dk[ct][r0 + 7] * sc};
        pv[0] = f32x4{dv[ct][r0], dv[ct][r0 + 1], dv[ct][r0 + 2], dv[ct][r0 + 3]};
        pv[1] = f32x4{dv[ct][r0 + 4], dv[ct][r0 + 5], dv[ct][r0 + 6], dv[ct][r0 + 7]};
      }
  }
}

// ---- dQ: queries outer -------------------------------------------------------
template <int D>
struct DqTile {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;  // 128 queries per workgroup
  static constexpr int BC = 64;       // keys per tile
  static constexpr int T_BYTES = BC * D * 2;
  static constexpr int OFF_K = 0, OFF_KT = T_BYTES, OFF_V = 2 * T_BYTES;
  static constexpr int STAGE = 3 * T_BYTES;
  static constexpr int LIST_CAP = 1024;
  static constexpr int MIN_WG = (D == 64) ? 2 : 1;
};

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256, DqTile<D>::MIN_WG) void bwd_dq_kernel(BwdArgs a) {
  using T = DqTile<D>;
  constexpr int NT = T::NT, BR = T::BR, BC = T::BC;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];
  __shared__ int blist[MASK ? T::LIST_CAP : 1];
  __shared__ int wcount[T::NW];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, li = lane & 31;
  const int g = xcd_remap(blockIdx.x, a.total);
  const int bh = g / a.ntile;
  int qt = g - bh * a.ntile;
  if (CAUSAL) qt = a.ntile - 1 - qt;
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const int q0 = qt * BR;
  const int qw0 = q0 + 32 * w;
  const int qi = qw0 + li;

  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
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
  f32x16 dq[D / 32];
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) dq[ct] = f32x16{};

  const __bf16* Kh = a.k + head;
  const __bf16* Vh = a.v + head;
  const float c = a.c;
  StageBlocks4<BC, D, NT> ks;
  StageRows16<BC, D, NT> vs;

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
    auto tile_of = [&](int t) -> int { return MASK ? 2 * blist[t >> 1] + (t & 1) : t; };
    auto store_tile = [&](char* st) {
      ks.store_nat(st + T::OFF_K, tid);
      ks.store_tr(st + T::OFF_KT, tid);
      vs.store(st + T::OFF_V, tid);
    };

    if (ntiles > 0) {
      const int k0 = tile_of(0) * BC;
      ks.load(Kh, k0, N, tid);
      vs.load(Vh, k0, N, tid);
      store_tile(smem);
    }
    if (ntiles > 1) {
      const int k0 = tile_of(1) * BC;
      ks.load(Kh, k0, N, tid);
      vs.load(Vh, k0, N, tid);
    }
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
      const char* st = smem + (t & 1) * T::STAGE;
      const int k0 = tile_of(t) * BC;
      const bool active = qw0 < N && !(CAUSAL && k0 > qw0 + 31);
      if (active) {
        const bool edge = (CAUSAL && k0 + BC - 1 > qw0) || (k0 + BC > N);
        bf16x8 dsb[4];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          f32x16 S = f32x16{}, dP = f32x16{};
          const int row = 32 * t2 + perm32(li);
#pragma unroll
          for (int kc = 0; kc < D / 16; ++kc) {
            S = mfma32(tile_read<2 * D>(st + T::OFF_K, row, 2 * kc + h), qf[kc], S);
            dP = mfma32(tile_read<2 * D>(st + T::OFF_V, row, 2 * kc + h), df[kc], dP);
          }
          float dsv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], c, -lse2));
            if (edge) {
              const int key = k0 + 32 * t2 + acc_row(r, h);
              if ((CAUSAL && key > qi) || key >= N) pv = 0.f;
            }
            dsv[r] = pv * (dP[r] - Di);
          }
          dsb[2 * t2 + 0] = to_bf16x8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
          dsb[2 * t2 + 1] = to_bf16x8(dsv[8], dsv[9], dsv[10], dsv[11], dsv[12], dsv[13], dsv[14], dsv[15]);
        }
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct) {
          const int crow = 32 * ct + perm32(li);
#pragma unroll
          for (int kc = 0; kc < BC / 16; ++kc)
            dq[ct] = mfma32(tile_read<2 * BC>(st + T::OFF_KT, crow, 2 * kc + h), dsb[kc], dq[ct]);
        }
      }
      if (t + 1 < ntiles) store_tile(smem + ((t + 1) & 1) * T::STAGE);
      if (t + 2 < ntiles) {
        const int k2 = tile_of(t + 2) * BC;
        ks.load(Kh, k2, N, tid);
        vs.load(Vh, k2, N, tid);
      }
      __syncthreads();
    }
  }

  if (qi < N) {
    float* dQrow = a.dq + head + (size_t)qi * D;
    const float sc = a.scale;
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
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
