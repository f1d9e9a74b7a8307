// Forward attention kernels for gfx950, bf16 inputs, fp32 accumulation.
//
// fwd_pp_kernel (dense and causal): 256 query rows per workgroup, eight
// waves in two groups that alternate matrix and vector phases (described at
// the kernel).  fwd_bf16_kernel (block mask): one workgroup owns 128 query
// rows of one (batch, head), one mask row; each of its four
// waves owns 32 of them and keeps its Q fragment in registers for the whole
// kernel.  K/V tiles of 64 keys are copied HBM -> LDS by direct-to-LDS loads
// (global_load_lds_dwordx4) into two buffers, so the copy of tile t+1 runs
// behind the arithmetic of tile t and each tile costs a single barrier
// ("Tiling": blocks of Q, K, V are loaded from HBM to on-chip memory and the
// output is accumulated block by block, "FlashAttention: Fast and
// Memory-Efficient Exact Attention with IO-Awareness", summary page, §3
// Method).
//
// Per key tile and wave:
//   S^T = K Q^T on MFMA 32x32x16 bf16.  Keys are accumulator rows and the
//         wave's 32 queries are accumulator columns, so a lane holds 16
//         scores of one query row per 32 keys: the row max and row sum are
//         register reductions plus one exchange with lane l^32.
//   online softmax in the log2 domain with a lazily updated reference max:
//         the reference (and O and l with it) moves only when a new row max
//         exceeds it by more than kLazyTau; O / l uses the same reference, so
//         the result is unchanged ("Softmax rescaling": the normalisation is
//         computed incrementally across blocks, §3).
//   O^T += V^T P^T on MFMA.  P goes to bf16 straight from the score
//         registers (perm32 row order makes them the B operand as they
//         stand); V^T comes from the natural V tile through transposed LDS
//         reads.
// Only O (bf16) and lse (fp32, natural log) are written (Figure 1 caption of
// "No More Quadratic Complexity for Transformers: Discover the Power of Flash
// Attention!": the N x N matrix never goes to HBM).
#pragma once

#include "fa_device.h"
#include "fa_dropout.h"
#include "fa_sched.h"

namespace fa {

constexpr float kLazyTau = 8.0f;  // log2 units: P values stay below 2^8
// A tile whose probabilities against the current reference sum (per lane,
// 32 keys) to at most this needs no row max (P then stays below 2^14).
constexpr float kSkipSum = 16384.0f;

// instruction classes for __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

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
  float c;              // max(|scale| * log2(e), FLT_MIN): masked scores stay -inf
  int negate_q;         // scale < 0: scores computed with -Q and |scale|
  DropArgs drop;        // used by the dropout instantiations only
};

// Zero the dropped entries of the 8 probabilities p[0..7] that a lane holds
// for query i and keys j0 .. j0+7 (j0 a multiple of 8).
__device__ __forceinline__ void drop8(const DropArgs& dp, int bh, int i, int j0, float* p) {
  const uint32_t lo = keep4(dp, bh, i, j0), hi = keep4(dp, bh, i, j0 + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[e] = ((lo >> e) & 1u) ? p[e] : 0.f;
    p[4 + e] = ((hi >> e) & 1u) ? p[4 + e] : 0.f;
  }
}

template <int D>
struct FwdTile {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;     // 128 query rows per workgroup
  static constexpr int BC = 64;          // keys per tile
  static constexpr int PITCH = 2 * D;    // bytes per K or V row in LDS
  static constexpr int T_BYTES = BC * PITCH;
  static constexpr int STAGE = 2 * T_BYTES;  // K tile then V tile
  static constexpr int LIST_CAP = 1024;  // mask blocks listed per pass
  // Two workgroups per CU (two waves per SIMD): one wave's softmax overlaps
  // the other's products.  At d=64 a wave also keeps the scores of the next
  // tile in flight (PIPE); at d=128 that does not fit in the 256 registers a
  // wave has at this occupancy.
  static constexpr int MIN_WG = 2;
  static constexpr bool PIPE = (D == 64);
};

template <int D, bool CAUSAL, bool MASK, bool DROP>
__global__ __launch_bounds__(256, FwdTile<D>::MIN_WG) void fwd_bf16_kernel(FwdArgs a) {
  using T = FwdTile<D>;
  constexpr int BC = T::BC, BR = T::BR, NT = T::NT, PITCH = T::PITCH;
  constexpr int NKC = D / 16;  // k-steps of S^T = K Q^T
  constexpr int NCT = D / 32;  // 32-row tiles of O^T
  // K runs one tile ahead of V: while tile t is normalised and multiplied
  // with V(t), S(t+1) = K(t+1) Q^T is already in the matrix pipe.  Four
  // separate buffers (not arrays indexed by t & 1) let the compiler prove
  // that a copy into one does not alias reads of another.
  __shared__ __attribute__((aligned(1024))) char kb0[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char kb1[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb0[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb1[T::T_BYTES];
  __shared__ int blist[MASK ? T::LIST_CAP : 1];
  __shared__ int wcount[T::NW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in an SGPR
  const int h = lane >> 5, li = lane & 31;

  int bh, qt;
  if (CAUSAL) {  // longest rows first, over all heads
    causal_rank(blockIdx.x, a.total / a.nqt, bh, qt);
    qt = a.nqt - 1 - qt;
  } else {
    const int g = xcd_remap(blockIdx.x, a.total);
    bh = g / a.nqt;
    qt = g - bh * a.nqt;
  }
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const __bf16* Qh = a.q + head;
  const __bf16* Kh = a.k + head;
  const __bf16* Vh = a.v + head;
  const int q0 = qt * BR;
  const int qw0 = q0 + 32 * w;  // first query of this wave
  const int qi = qw0 + li;      // this lane's query row

  // Q^T fragments (B operand): lane supplies Q[qi][16kc + 8h .. +7].
  bf16x8 qf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    if (qi < N) x = gload16(Qh + (size_t)qi * D + 16 * kc + 8 * h);
    if (a.negate_q) x ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    qf[kc] = __builtin_bit_cast(bf16x8, x);
  }

  // Per-lane LDS offsets of the K (rows) and V^T (transposed) operands.
  TileOffsets<D> toff;
  toff.init(lane);

  f32x16 o[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o[ct] = f32x16{};
  float Mref = -INFINITY;  // reference max (log2 units), identical in both halves
  float L = 0.f;           // partial row sum over this lane's keys

  const int ntiles_all = (N + BC - 1) / BC;
  const float c = a.c;
  TileCopy<BC, D, NT> kcopy;
  TileCopy<BC, D, NT> vcopy;
  kcopy.init(w, lane);
  vcopy.init(w, lane);

  // S^T = K Q^T for the two 32-key halves of the tile in `kt`.
  auto scores = [&] __device__ (const char* kt, f32x16& s0, f32x16& s1) {
    bf16x8 ka0[NKC], ka1[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      ka0[kc] = lds_read16(kt + toff.rows[kc]);
      ka1[kc] = lds_read16(kt + toff.rows[kc] + 32 * PITCH);
    }
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      s0 = mfma32(ka0[kc], qf[kc], s0);
      s1 = mfma32(ka1[kc], qf[kc], s1);
    }
    // K reads run three k-steps ahead of their products
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 0);
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
      if (kc + 3 < NKC) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
  };

  // One pipelined step on the tile at key k0, whose scores are in s0/s1:
  // mask, row max and (rarely) the rescale of O and l first; then, in one
  // scheduling region, the products S(next) = K(next) Q^T go to the matrix
  // pipe interleaved with P = 2^(S*c - Mref), its bf16 copy and its fp32 row
  // sum on the VALU; finally O^T += V^T P^T with V from `vt`.
  auto softmax_pv = [&] __device__ (f32x16 s0, f32x16 s1, const char* vt, int k0,
                                    const char* knext, f32x16& n0, f32x16& n1) {
    // ---- mask (only tiles that cross the diagonal or the sequence end)
    const bool edge = (CAUSAL && k0 + BC - 1 > qw0) || (k0 + BC > N);
    if (edge) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key0 = k0 + acc_row(r, h), key1 = key0 + 32;
        if ((CAUSAL && key0 > qi) || key0 >= N) s0[r] = -INFINITY;
        if ((CAUSAL && key1 > qi) || key1 >= N) s1[r] = -INFINITY;
      }
    }
    // ---- P = 2^(S*c - Mref) against the current reference, its fp32 row
    // sum and its bf16 copy for the product.  The row max is taken only when
    // a row has no reference yet or a P of this tile would exceed 2^14 (the
    // tile is then recomputed after the max, below).
    bf16x8 pb[4];
    auto make_p = [&] __device__ (float mb) __attribute__((always_inline)) -> float {
      float lsum[4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float p0[8], p1[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p0[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[8 * hh + e], c, -mb));
          p1[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[8 * hh + e], c, -mb));
        }
        // l sums the undropped probabilities; the product takes the kept ones
        lsum[hh] = ((p0[0] + p0[1]) + (p0[2] + p0[3])) + ((p0[4] + p0[5]) + (p0[6] + p0[7]));
        lsum[2 + hh] = ((p1[0] + p1[1]) + (p1[2] + p1[3])) + ((p1[4] + p1[5]) + (p1[6] + p1[7]));
        if constexpr (DROP) {
          drop8(a.drop, bh, qi, k0 + 16 * hh + 8 * h, p0);
          drop8(a.drop, bh, qi, k0 + 32 + 16 * hh + 8 * h, p1);
        }
        pb[hh] = to_bf16x8(p0[0], p0[1], p0[2], p0[3], p0[4], p0[5], p0[6], p0[7]);
        pb[2 + hh] = to_bf16x8(p1[0], p1[1], p1[2], p1[3], p1[4], p1[5], p1[6], p1[7]);
      }
      return (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    };
    const bool noref = wave_any(Mref == -INFINITY);
    // ---- S(next) on the matrix pipe ...
    if constexpr (T::PIPE) {
      bf16x8 ka0[NKC], ka1[NKC];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        ka0[kc] = lds_read16(knext + toff.rows[kc]);
        ka1[kc] = lds_read16(knext + toff.rows[kc] + 32 * PITCH);
      }
      n0 = f32x16{};
      n1 = f32x16{};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        n0 = mfma32(ka0[kc], qf[kc], n0);
        n1 = mfma32(ka1[kc], qf[kc], n1);
      }
    }
    // ---- ... while P runs on the VALU (discarded below when noref).  The
    // reference is opaque to the compiler: otherwise it specialises P for
    // noref into a second block, and the products and the exponentials can
    // no longer share one scheduling region.
    float mb = noref ? 0.f : Mref;
    asm volatile("" : "+v"(mb));
    float lt = make_p(mb);
    if constexpr (T::PIPE) {
      // interleave: K reads three k-steps ahead, one MFMA per ~7 VALU ops
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 1);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 112 / (2 * NKC), 1);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 112 / (2 * NKC), 1);
        if (kc + 3 < NKC) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- rare: row max over the tile (v_max3 chains, both halves), lazy
    // move of the reference with the rescale of O and l, P again.  One
    // ballot over both conditions, so that P above is computed on every path
    // and stays in the scheduling region of the products.
    if (wave_any(Mref == -INFINITY || !(lt <= kSkipSum))) {
      float m0 = fmaxf(s0[0], s0[1]), m1 = fmaxf(s1[0], s1[1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) {
        m0 = fmaxf(fmaxf(m0, s0[r]), s0[r + 1]);
        m1 = fmaxf(fmaxf(m1, s1[r]), s1[r + 1]);
      }
      const float mx = xhalf_max(fmaxf(m0, m1));
      const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
      const bool need = mt > Mref + kLazyTau;
      if (wave_any(need)) {
        const float Mn = need ? mt : Mref;
        const float alpha = need ? __builtin_amdgcn_exp2f(Mref - Mn) : 1.f;
        L *= alpha;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) o[ct] *= alpha;
        Mref = Mn;
      }
      lt = make_p((Mref == -INFINITY) ? 0.f : Mref);
    }
    L += lt;
    // ---- O^T += V^T P^T, V reads two products ahead
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int kc = 0; kc < BC / 16; ++kc) {
        o[ct] = mfma32(toff.read_tr(vt, kc, ct), pb[kc], o[ct]);
      }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 2);
#pragma unroll
    for (int m = 0; m < NCT * BC / 16; ++m) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 2);
      if (m + 2 < NCT * BC / 16) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 2);
    }
  };

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
    auto tile_of = [&] __device__ (int t) -> int { return MASK ? 2 * blist[t >> 1] + (t & 1) : t; };
    auto active = [&] __device__ (int k0) -> bool { return qw0 < N && !(CAUSAL && k0 > qw0 + 31); };
    if (ntiles == 0) continue;

    // prologue: K(0), V(0) (and with PIPE K(1) and S(0))
    kcopy.issue(kb0, Kh, tile_of(0) * BC, N, w);
    vcopy.issue(vb0, Vh, tile_of(0) * BC, N, w);
    if (T::PIPE && ntiles > 1) kcopy.issue(kb1, Kh, tile_of(1) * BC, N, w);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 sa0, sa1, sb0, sb1;  // scores of the even / odd tiles
    if (T::PIPE && active(tile_of(0) * BC)) scores(kb0, sa0, sa1);

    // Iteration t: K(t+1) and V(t) have landed (barrier); copy K(t+2) into
    // the buffer S(t) was read from and V(t+1) into the one PV(t-1) read;
    // S(t+1) goes to the matrix pipe, then softmax(t) and PV(t).
    auto step = [&] __device__ (int t, char* kcur, const char* knext, const char* vcur, char* vnext,
                                f32x16& scur0, f32x16& scur1, f32x16& snext0, f32x16& snext1) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (T::PIPE) {
        if (t + 2 < ntiles) kcopy.issue(kcur, Kh, tile_of(t + 2) * BC, N, w);
      } else {
        if (t + 1 < ntiles) kcopy.issue(const_cast<char*>(knext), Kh, tile_of(t + 1) * BC, N, w);
      }
      if (t + 1 < ntiles) vcopy.issue(vnext, Vh, tile_of(t + 1) * BC, N, w);
      // a wave with no visible key in tile t has none in later tiles either;
      // at the last tile S(next) reads a stale buffer and is never used
      const int k0 = tile_of(t) * BC;
      if (active(k0)) {
        if (!T::PIPE) scores(kcur, scur0, scur1);
        softmax_pv(scur0, scur1, vcur, k0, knext, snext0, snext1);
      }
    };
    for (int t = 0; t < ntiles; t += 2) {
      step(t, kb0, kb1, vb0, vb1, sa0, sa1, sb0, sb1);
      if (t + 1 < ntiles) step(t + 1, kb1, kb0, vb1, vb0, sb0, sb1, sa0, sa1);
    }
    // all reads of this pass are done before the next pass (or nothing) reuses the buffers
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: O = O / l, lse = (Mref + log2 l) * ln 2
  const float Lt = xhalf_sum(L);
  if (qi < N) {
    const bool empty = !(Lt > 0.f);
    const float inv = empty ? 0.f : (DROP ? a.drop.keep_scale : 1.f) / Lt;
    __bf16* Orow = a.o + head + (size_t)qi * D;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
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

// ---- phased forward (dense and causal) --------------------------------------
// One workgroup of G groups of four waves owns 128 G query rows: group g
// (waves 4g .. 4g+3) owns rows 128 g .. +127 of the tile, and wave w runs on
// SIMD w % 4, so every SIMD holds one wave of each group.  Per key tile a
// wave does a matrix phase M (O^T += V^T P^T of the previous tile, then
// S^T = K Q^T of this tile) and a vector phase (softmax of this tile's
// scores).  The groups run one phase apart, so in every phase one wave per
// SIMD issues products while the others run softmax.
//
// G = 2 (ping-pong): the vector phase is one step V.
//   round r, phase 1:  A: M(r)      B: V(r-1)
//   round r, phase 2:  A: V(r)      B: M(r)
// Only the barrier at the end of a round (the copies have landed, the
// buffers are free) holds the groups together: within a round the opposite
// phase orders keep them apart, and a barrier between the two phases made
// the round ~1.6% longer.
// G = 3: the softmax is split into two steps V1 (mask, P and bf16 P of the
// tile's first 32 keys) and V2 (the other 32 keys, the max check and the slow
// path when it is needed), and two waves per SIMD run softmax while the
// third runs its products.  This does not raise the exponential rate: one
// wave's exponentials already keep a SIMD's VALU nearly busy (plain VALU
// instructions it issues at about half the SIMD's rate).  The three groups
// were chosen on measured time: at d = 64 a round takes ~1310 cycles per
// tile against ~1600 with two groups.
//   round r, phase 1:  A: M(r)      B: V2(r-1)   C: V1(r-1)
//   round r, phase 2:  A: V1(r)     B: M(r)      C: V2(r-1)
//   round r, phase 3:  A: V2(r)     B: V1(r)     C: M(r)
// One barrier inside the round (between phases 2 and 3) and the one at its
// end hold the groups: with a barrier between phases 1 and 2 as well the
// forward was ~3% slower, and with none inside the round ~1.6% slower.
// Round r reads K(r) and V(r-1); K(r+1) and V(r) are copied meanwhile into
// the buffers round r-1 finished with.  Direct-to-LDS copies queue for the
// CU's address unit and a wave stalls while its copies issue, so issuing
// them from every wave at the start of a round lengthened that round's first
// phase by ~300 cycles for all groups.  Group 0 issues V inside its matrix
// phase (between the PV and score products).  With G = 3 it also issues K,
// before its PV products; with G = 2 group 1 issues K at the start of its
// round, ahead of its vector phase (1-2% faster than group 0 issuing both).
template <int D, int G = 2>
struct FwdPPTile {
  static constexpr int NW = 4 * G;
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 128 * G;  // query rows per workgroup
  static constexpr int BC = 64;       // keys per tile
  static constexpr int PITCH = 2 * D;
  static constexpr int T_BYTES = BC * PITCH;
  static constexpr int CPT = 256;     // threads that copy the K/V tiles (group 0)
};

template <int D, int G, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(256 * G, 1) void fwd_pp_kernel(FwdArgs a) {
  using T = FwdPPTile<D, G>;
  static_assert(G == 2 || G == 3, "two or three wave groups");
  constexpr int BC = T::BC, BR = T::BR, PITCH = T::PITCH;
  constexpr int NKC = D / 16, NCT = D / 32;
  __shared__ __attribute__((aligned(1024))) char kb0[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char kb1[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb0[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb1[T::T_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2;
  const int h = lane >> 5, li = lane & 31;

  int bh, qt;
  if (CAUSAL) {  // longest rows first, over all heads
    causal_rank(blockIdx.x, a.total / a.nqt, bh, qt);
    qt = a.nqt - 1 - qt;
  } else {
    const int g = xcd_remap(blockIdx.x, a.total);
    bh = g / a.nqt;
    qt = g - bh * a.nqt;
  }
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const __bf16* Qh = a.q + head;
  const __bf16* Kh = a.k + head;
  const __bf16* Vh = a.v + head;
  const int q0 = qt * BR;
  const int qw0 = q0 + 32 * w;  // first query of this wave
  const int qi = qw0 + li;

  bf16x8 qf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    if (qi < N) x = gload16(Qh + (size_t)qi * D + 16 * kc + 8 * h);
    if (a.negate_q) x ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    qf[kc] = __builtin_bit_cast(bf16x8, x);
  }
  TileOffsets<D> toff;
  toff.init(lane);
  TileCopy<BC, D, T::CPT> cp;
  cp.init(w & 3, lane);
  const bool copier = grp == 0;

  f32x16 o[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o[ct] = f32x16{};
  float Mref = -INFINITY, L = 0.f;
  const float c = a.c;
  const int kend = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kend + BC - 1) / BC;
  // tiles this wave has visible keys in: [0, wtiles)
  const int wtiles = (qw0 >= N) ? 0 : (CAUSAL ? min(ntiles, (qw0 + 31) / BC + 1) : ntiles);

  f32x16 s0, s1;  // scores of the current tile
  bf16x8 pb[4];   // P of the previous tile (bf16)

  // matrix phase of round r: O^T += V^T P^T for tile r-1, then S^T of tile r
  auto mphase = [&] __device__ (int r, const char* kt, const char* vprev, auto&& mid) __attribute__((always_inline)) {
    if (r >= 1 && r - 1 < wtiles) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int kc = 0; kc < BC / 16; ++kc) o[ct] = mfma32(toff.read_tr(vprev, kc, ct), pb[kc], o[ct]);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 13);
#pragma unroll
      for (int m = 0; m < NCT * BC / 16; ++m) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 13);
        if (m + 2 < NCT * BC / 16) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 13);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    mid();
    if (r < wtiles) {
      bf16x8 ka0[NKC], ka1[NKC];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        ka0[kc] = lds_read16(kt + toff.rows[kc]);
        ka1[kc] = lds_read16(kt + toff.rows[kc] + 32 * PITCH);
      }
      s0 = f32x16{};
      s1 = f32x16{};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        s0 = mfma32(ka0[kc], qf[kc], s0);
        s1 = mfma32(ka1[kc], qf[kc], s1);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 14);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 14);
        if (kc + 2 < NKC) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 14);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // vector phase: softmax of the scores of tile r into pb, in two steps.
  // P = 2^(S*c - Mref) against the current reference.  The row max is
  // needed only when a row has no reference yet or some P of this tile
  // would exceed 2^kSkipLog2: then the reference moves (lazily, as in the
  // other kernel) and P is recomputed.  Either way O / l and lse use the
  // same reference, so the result does not depend on which path ran.
  // Step 1 masks the tile and takes P (and its bf16 copy) of the first 32
  // keys; step 2 the other 32, the check, and the slow path if needed, which
  // recomputes both halves.  Run back to back, the steps are the single
  // vector phase of the two-group schedule; each element is computed the
  // same way in both, so the two schedules give bitwise identical results.
  float p0[16], p1[16];
  float lt0 = 0.f;
  auto exps0 = [&] __device__ (float mb) __attribute__((always_inline)) -> float {
    float ls[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int e = 0; e < 8; ++e) p0[8 * hh + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[8 * hh + e], c, -mb));
      const float* a0 = p0 + 8 * hh;
      ls[hh] = ((a0[0] + a0[1]) + (a0[2] + a0[3])) + ((a0[4] + a0[5]) + (a0[6] + a0[7]));
    }
    return ls[0] + ls[1];
  };
  auto exps1 = [&] __device__ (float mb) __attribute__((always_inline)) -> float {
    float ls[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int e = 0; e < 8; ++e) p1[8 * hh + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[8 * hh + e], c, -mb));
      const float* a1 = p1 + 8 * hh;
      ls[hh] = ((a1[0] + a1[1]) + (a1[2] + a1[3])) + ((a1[4] + a1[5]) + (a1[6] + a1[7]));
    }
    return ls[0] + ls[1];
  };
  // bf16 P of the first / last 32 keys of the tile (after the dropout mask)
  auto conv0 = [&] __device__ (int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if constexpr (DROP) drop8(a.drop, bh, qi, k0 + 16 * hh + 8 * h, p0 + 8 * hh);
      const float* a0 = p0 + 8 * hh;
      pb[hh] = to_bf16x8(a0[0], a0[1], a0[2], a0[3], a0[4], a0[5], a0[6], a0[7]);
    }
  };
  auto conv1 = [&] __device__ (int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if constexpr (DROP) drop8(a.drop, bh, qi, k0 + 32 + 16 * hh + 8 * h, p1 + 8 * hh);
      const float* a1 = p1 + 8 * hh;
      pb[2 + hh] = to_bf16x8(a1[0], a1[1], a1[2], a1[3], a1[4], a1[5], a1[6], a1[7]);
    }
  };
  auto vstep1 = [&] __device__ (int r) __attribute__((always_inline)) {
    if (r < 0 || r >= wtiles) return;
    const int k0 = r * BC;
    const bool edge = (CAUSAL && k0 + BC - 1 > qw0) || (k0 + BC > N);
    if (edge) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key0 = k0 + acc_row(e, h), key1 = key0 + 32;
        if ((CAUSAL && key0 > qi) || key0 >= N) s0[e] = -INFINITY;
        if ((CAUSAL && key1 > qi) || key1 >= N) s1[e] = -INFINITY;
      }
    }
    if (Mref != -INFINITY) {
      lt0 = exps0(Mref);
      conv0(k0);
    }
  };
  auto vstep2 = [&] __device__ (int r) __attribute__((always_inline)) {
    if (r < 0 || r >= wtiles) return;
    const int k0 = r * BC;
    bool slow = wave_any(Mref == -INFINITY);
    float lt = 0.f;
    if (!slow) {
      lt = lt0 + exps1(Mref);
      slow = wave_any(!(lt <= kSkipSum));  // also catches inf / NaN
    }
    if (slow) {
      float m0 = fmaxf(s0[0], s0[1]), m1 = fmaxf(s1[0], s1[1]);
#pragma unroll
      for (int e = 2; e < 16; e += 2) {
        m0 = fmaxf(fmaxf(m0, s0[e]), s0[e + 1]);
        m1 = fmaxf(fmaxf(m1, s1[e]), s1[e + 1]);
      }
      const float mx = xhalf_max(fmaxf(m0, m1));
      const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
      const bool need = mt > Mref + kLazyTau;
      if (wave_any(need)) {
        const float Mn = need ? mt : Mref;
        const float alpha = need ? __builtin_amdgcn_exp2f(Mref - Mn) : 1.f;
        L *= alpha;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) o[ct] *= alpha;
        Mref = Mn;
      }
      const float mb = (Mref == -INFINITY) ? 0.f : Mref;
      lt = exps0(mb);
      conv0(k0);
      lt = lt + exps1(mb);
    }
    L += lt;
    conv1(k0);
  };

  // prologue: K(0) into kb0
  if (ntiles > 0 && copier) cp.issue(kb0, Kh, 0, N, w);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // round r (r = 0 .. ntiles): K(r) in kb[r&1], V(r-1) in vb[(r-1)&1].
  // Each group runs its own loop (the phase order differs); all execute the
  // same barriers per round (one with G = 2, two with G = 3), the last
  // after waiting for the copies.
  // mphase runs its last argument between the PV and the score products.
  // copies: see the schedule above; TileCopy covers 256 threads, so a
  // wave copies as wave w & 3 of its group
  auto copyk = [&] __device__ (int r, char* knext) __attribute__((always_inline)) {
    if (copier && r + 1 < ntiles) cp.issue(knext, Kh, (r + 1) * BC, N, w);
  };
  auto copyv = [&] __device__ (int r, char* vcur) __attribute__((always_inline)) {
    if (copier && r < ntiles) cp.issue(vcur, Vh, r * BC, N, w);
  };
  auto nomid = [] __device__ () {};
  auto endround = [&] __device__ () __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  auto rounds = [&] __device__ (auto&& round) __attribute__((always_inline)) {
    for (int r = 0; r <= ntiles; r += 2) {
      round(r, kb0, kb1, vb1, vb0);
      if (r + 1 <= ntiles) round(r + 1, kb1, kb0, vb0, vb1);
    }
  };
  if constexpr (G == 2) {
    if (grp == 0) {
      rounds([&] __device__ (int r, const char* kcur, char* knext, const char* vprev, char* vcur) __attribute__((always_inline)) {
        mphase(r, kcur, vprev, [&] __device__ () { copyv(r, vcur); });
        vstep1(r);
        vstep2(r);
        endround();
      });
    } else {
      rounds([&] __device__ (int r, const char* kcur, char* knext, const char* vprev, char* vcur) __attribute__((always_inline)) {
        if (r + 1 < ntiles) cp.issue(knext, Kh, (r + 1) * BC, N, w & 3);  // K(r+1)
        vstep1(r - 1);
        vstep2(r - 1);
        mphase(r, kcur, vprev, nomid);
        endround();
      });
    }
  } else {
    if (grp == 0) {
      rounds([&] __device__ (int r, const char* kcur, char* knext, const char* vprev, char* vcur) __attribute__((always_inline)) {
        copyk(r, knext);
        mphase(r, kcur, vprev, [&] __device__ () { copyv(r, vcur); });
        vstep1(r);
        __syncthreads();
        vstep2(r);
        endround();
      });
    } else if (grp == 1) {
      rounds([&] __device__ (int r, const char* kcur, char* knext, const char* vprev, char* vcur) __attribute__((always_inline)) {
        vstep2(r - 1);
        mphase(r, kcur, vprev, nomid);
        __syncthreads();
        vstep1(r);
        endround();
      });
    } else {
      rounds([&] __device__ (int r, const char* kcur, char* knext, const char* vprev, char* vcur) __attribute__((always_inline)) {
        vstep1(r - 1);
        vstep2(r - 1);
        __syncthreads();
        mphase(r, kcur, vprev, nomid);
        endround();
      });
    }
  }

  const float Lt = xhalf_sum(L);
  if (qi < N) {
    const bool empty = !(Lt > 0.f);
    const float inv = empty ? 0.f : (DROP ? a.drop.keep_scale : 1.f) / Lt;
    __bf16* Orow = a.o + head + (size_t)qi * D;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int col = 32 * ct + 16 * hh + 8 * h;
        const f32x16& x = o[ct];
        const int r0 = 8 * hh;
        bf16x8 v = to_bf16x8(x[r0] * inv, x[r0 + 1] * inv, x[r0 + 2] * inv, x[r0 + 3] * inv,
                             x[r0 + 4] * inv, x[r0 + 5] * inv, x[r0 + 6] * inv, x[r0 + 7] * inv);
        *reinterpret_cast<bf16x8*>(Orow + col) = v;
      }
    if (h == 0) a.lse[(size_t)bh * N + qi] = empty ? -INFINITY : (Mref + __log2f(Lt)) * kLn2;
  }
}

}  // namespace fa
