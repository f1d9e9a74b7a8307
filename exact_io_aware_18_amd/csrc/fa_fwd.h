// Forward attention kernel for gfx950, bf16 inputs, fp32 accumulation.
//
// One workgroup owns 128 query rows of one (batch, head); each of its four
// waves owns 32 of them and keeps its Q fragment in registers for the whole
// kernel.  K/V tiles of 64 keys are streamed HBM -> registers -> LDS with
// one tile of prefetch and two LDS buffers, so each iteration needs a single
// barrier ("Tiling": blocks of Q, K, V are loaded from HBM to on-chip memory
// and the output is accumulated block by block, "FlashAttention: Fast and
// Memory-Efficient Exact Attention with IO-Awareness", summary page, §3
// Method).
//
// Per key tile and wave:
//   S^T = K Q^T on MFMA 32x32x16 bf16 (keys are accumulator rows, the
//         wave's 32 queries are accumulator columns, so a lane holds 16
//         scores of one query row per 32 keys and the row max / row sum are
//         register reductions plus one exchange with lane l^32);
//   online softmax in the log2 domain with a lazily updated reference max
//         (the running max is replaced, and O and l rescaled, only when a new
//         row max exceeds it by more than kLazyTau; the final O / l uses the
//         same reference, so the result is unchanged) ("Softmax rescaling":
//         the normalisation is computed incrementally across blocks, §3);
//   O^T += V^T P^T on MFMA, with P converted to bf16 straight from the score
//         registers (perm32 row order makes the score registers the MFMA
//         B operand as they stand).
// Only O (bf16) and lse (fp32, natural log) are written (Figure 1 caption
// of "No More Quadratic Complexity for Transformers: Discover the Power of
// Flash Attention!": the N x N matrix never goes to HBM).
#pragma once

#include "fa_device.h"
#include "fa_sched.h"

namespace fa {

constexpr float kLazyTau = 8.0f;  // log2 units: P values stay below 2^8

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  const uint8_t* mask;  // nb x nb or nullptr
  int N;
  int nqt;              // query tiles per head
  int total;            // workgroups in the grid
  int nb;               // mask blocks per side
  float c;              // |scale| * log2(e)
  int negate_q;         // scale < 0: scores computed with -Q and |scale|
};

template <int D>
struct FwdTile {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;     // 128 query rows per workgroup
  static constexpr int BC = 64;          // keys per tile
  static constexpr int K_BYTES = BC * D * 2;
  static constexpr int VT_BYTES = D * BC * 2;
  static constexpr int STAGE = K_BYTES + VT_BYTES;
  static constexpr int LIST_CAP = 1024;  // mask blocks listed per pass
};

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a) {
  using T = FwdTile<D>;
  constexpr int BC = T::BC, BR = T::BR, NT = T::NT;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];
  __shared__ int blist[MASK ? T::LIST_CAP : 1];
  __shared__ int wcount[T::NW];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, li = lane & 31;

  const int g = xcd_remap(blockIdx.x, a.total);
  const int bh = g / a.nqt;
  int qt = g - bh * a.nqt;
  if (CAUSAL) qt = a.nqt - 1 - qt;  // longest rows first
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const __bf16* Qh = a.q + head;
  const __bf16* Kh = a.k + head;
  const __bf16* Vh = a.v + head;
  const int q0 = qt * BR;
  const int qw0 = q0 + 32 * w;       // first query of this wave
  const int qi = qw0 + li;           // this lane's query row

  // Q^T fragments (B operand): lane supplies Q[qi][16kc + 8h .. +7].
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    if (qi < N) x = gload16(Qh + (size_t)qi * D + 16 * kc + 8 * h);
    if (a.negate_q) x ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    qf[kc] = __builtin_bit_cast(bf16x8, x);
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) o[ct] = f32x16{};
  float Mref = -INFINITY;  // reference max (log2 units), identical in both halves
  float L = 0.f;           // partial row sum over this lane's keys

  const int ntiles_all = (N + BC - 1) / BC;
  const float c = a.c;

  StageRows16<BC, D, NT> ks;
  StageBlocks4<BC, D, NT> vs;

  // Key-tile schedule: a list pass covers mask blocks [cb0, cb1).
  const int qb = q0 >> 7;  // mask row (BR == 128)
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
      if (cnt > 0 && 2 * blist[cnt - 1] + 1 >= ntiles_all) ntiles -= 1;  // short last block
    }
    auto tile_of = [&](int t) -> int { return MASK ? 2 * blist[t >> 1] + (t & 1) : t; };

    if (ntiles > 0) {
      const int k0 = tile_of(0) * BC;
      ks.load(Kh, k0, N, tid);
      vs.load(Vh, k0, N, tid);
      ks.store(smem, tid);
      vs.store_tr(smem + T::K_BYTES, tid);
    }
    if (ntiles > 1) {
      const int k0 = tile_of(1) * BC;
      ks.load(Kh, k0, N, tid);
      vs.load(Vh, k0, N, tid);
    }
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
      const char* Ks = smem + (t & 1) * T::STAGE;
      const char* Vt = Ks + T::K_BYTES;
      const int k0 = tile_of(t) * BC;
      const bool active = qw0 < N && !(CAUSAL && k0 > qw0 + 31);
      if (active) {
        // ---- S^T = K Q^T for two 32-key halves of the tile
        f32x16 s[2];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          s[t2] = f32x16{};
          const int row = 32 * t2 + perm32(li);
#pragma unroll
          for (int kc = 0; kc < D / 16; ++kc)
            s[t2] = mfma32(tile_read<2 * D>(Ks, row, 2 * kc + h), qf[kc], s[t2]);
        }
        // ---- mask (only tiles that cross the diagonal or the sequence end)
        const bool edge = (CAUSAL && k0 + BC - 1 > qw0) || (k0 + BC > N);
        if (edge) {
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + 32 * t2 + acc_row(r, h);
              if ((CAUSAL && key > qi) || key >= N) s[t2][r] = -INFINITY;
            }
        }
        // ---- row max over the tile, shared by both halves
        float mx = -INFINITY;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t2][r]);
        mx = fmaxf(mx, xhalf(mx));
        const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
        const bool need = mt > Mref + kLazyTau;
        if (wave_any(need)) {
          const float Mn = need ? mt : Mref;
          const float alpha = need ? __builtin_amdgcn_exp2f(Mref - Mn) : 1.f;
          L *= alpha;
#pragma unroll
          for (int ct = 0; ct < D / 32; ++ct) o[ct] *= alpha;
          Mref = Mn;
        }
        const float mb = (Mref == -INFINITY) ? 0.f : Mref;
        // ---- P = 2^(S*c - Mref) as bf16; l accumulates the same values
        bf16x8 pb[4];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          float p[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t2][r], c, -mb));
            if (edge) x = (s[t2][r] == -INFINITY) ? 0.f : x;
            p[r] = x;
            L += x;
          }
          pb[2 * t2 + 0] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
          pb[2 * t2 + 1] = to_bf16x8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
        }
        // ---- O^T += V^T P^T
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct) {
          const int row = 32 * ct + perm32(li);
#pragma unroll
          for (int kc = 0; kc < BC / 16; ++kc)
            o[ct] = mfma32(tile_read<2 * BC>(Vt, row, 2 * kc + h), pb[kc], o[ct]);
        }
      }
      // ---- stage tile t+1 into the other buffer, prefetch tile t+2
      if (t + 1 < ntiles) {
        char* nb = smem + ((t + 1) & 1) * T::STAGE;
        ks.store(nb, tid);
        vs.store_tr(nb + T::K_BYTES, tid);
      }
      if (t + 2 < ntiles) {
        const int k2 = tile_of(t + 2) * BC;
        ks.load(Kh, k2, N, tid);
        vs.load(Vh, k2, N, tid);
      }
      __syncthreads();
    }
  }

  // ---- epilogue: O = O / l, lse = (Mref + log2 l) * ln 2
  const float Lt = L + xhalf(L);
  if (qi < N) {
    const bool empty = !(Lt > 0.f);
    const float inv = empty ? 0.f : 1.f / Lt;
    __bf16* Orow = a.o + head + (size_t)qi * D;
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int col = 32 * ct + 16 * hh + 8 * h;
        const f32x16& x = o[ct];
        const int r0 = 8 * hh;
        bf16x8 v = to_bf16x8(x[r0] * inv, x[r0 + 1] * inv, x[r0 + 2] * inv, x[r0 + 3] * inv,
                             x[r0 + 4] * inv, x[r0 + 5] * inv, x[r0 + 6] * inv, x[r0 + 7] * inv);
        *reinterpret_cast<bf16x8*>(Orow + col) = v;
      }
    if (h == 0)
      a.lse[(size_t)bh * N + qi] = empty ? -INFINITY : (Mref + __log2f(Lt)) * kLn2;
  }
}

}  // namespace fa
