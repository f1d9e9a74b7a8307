// Decode: a few new queries (Nq <= a few tens) against a long key/value cache
// (Nk up to millions), the inference case the aggregator page "Flashattention
// fast and memory efficient exact attention with io awareness" names as
// Flash-Decoding.  With so few queries the query-tile loop of the forward has
// almost no parallelism, so the keys are split instead:
//
//   decode_split_kernel  one single-wave workgroup per (batch*head, group of
//                        32 queries, key chunk): online softmax over its chunk
//                        exactly as in the forward, written as a partial
//                        (O_s normalised, lse_s) in fp32;
//   decode_merge_kernel  per query, the exact merge of the partials:
//                        lse = log sum_s exp(lse_s),
//                        O = sum_s exp(lse_s - lse) O_s.
//
// The work is a stream over K and V, each read once: the path is HBM-bound
// (4d bytes per key per head against 4d flops per (query, key) pair).
// Causal: query i is the sequence position i + Nk - Nq and sees keys
// j <= i + Nk - Nq.
#pragma once

#include "fa_device.h"
#include "fa_fwd.h"

namespace fa {

struct DecArgs {
  const __bf16* q;  // [BH, Nq, D]
  const __bf16* k;  // [BH, Nk, D]
  const __bf16* v;  // [BH, Nk, D]
  __bf16* o;        // [BH, Nq, D]
  float* lse;       // [BH, Nq]
  float* part_o;    // [BH, Nq, nsplit, D]
  float* part_lse;  // [BH, Nq, nsplit]
  int Nq;
  int Nk;
  int nqg;          // groups of 32 queries
  int nsplit;       // key chunks
  int chunk;        // keys per chunk (a multiple of the tile)
  int off;          // Nk - Nq: causal position of query 0
  float c;          // max(|scale| * log2(e), FLT_MIN)
  int negate_q;     // scale < 0
};

template <int D>
struct DecTile {
  static constexpr int BC = (D == 64) ? 64 : 32;  // keys per tile: 32 KB of LDS per workgroup
  static constexpr int NH = BC / 32;              // 32-key halves per tile
  static constexpr int PITCH = 2 * D;
  static constexpr int T_BYTES = BC * PITCH;
};

// Keys per chunk and number of chunks: enough workgroups to fill the chip
// several times over, chunks no shorter than 256 keys.
inline void decode_split(int BH, int Nq, int Nk, int D, int* nsplit, int* chunk) {
  const int bc = (D == 64) ? 64 : 32;
  const long base = (long)BH * ((Nq + 31) / 32);
  long want = (2048 + base - 1) / base;
  const long max_split = (Nk + 255) / 256;
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  long ch = (Nk + want - 1) / want;
  ch = (ch + bc - 1) / bc * bc;
  *chunk = (int)ch;
  *nsplit = (int)((Nk + ch - 1) / ch);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void decode_split_kernel(DecArgs a) {
  using T = DecTile<D>;
  constexpr int BC = T::BC, NH = T::NH, PITCH = T::PITCH;
  constexpr int NKC = D / 16, NCT = D / 32;
  __shared__ __attribute__((aligned(1024))) char kb0[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char kb1[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb0[T::T_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb1[T::T_BYTES];

  const int lane = threadIdx.x;
  const int h = lane >> 5, li = lane & 31;
  const int s = blockIdx.x % a.nsplit;
  const int t0 = blockIdx.x / a.nsplit;
  const int g = t0 % a.nqg;
  const int bh = t0 / a.nqg;
  const int Nq = a.Nq, Nk = a.Nk;
  const int qi = 32 * g + li;  // this lane's query
  const __bf16* Kh = a.k + (size_t)bh * Nk * D;
  const __bf16* Vh = a.v + (size_t)bh * Nk * D;

  // keys of this chunk that any query of the group can see
  const int k_lo = s * a.chunk;
  int k_hi = min(Nk, k_lo + a.chunk);
  if (CAUSAL) k_hi = min(k_hi, min(Nq - 1, 32 * g + 31) + a.off + 1);
  const int ntiles = (k_hi > k_lo) ? (k_hi - k_lo + BC - 1) / BC : 0;

  bf16x8 qf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    if (qi < Nq) x = gload16(a.q + ((size_t)bh * Nq + qi) * D + 16 * kc + 8 * h);
    if (a.negate_q) x ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    qf[kc] = __builtin_bit_cast(bf16x8, x);
  }
  TileOffsets<D> toff;
  toff.init(lane);
  TileCopy<BC, D, 64> cp;
  cp.init(0, lane);

  f32x16 o[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o[ct] = f32x16{};
  float Mref = -INFINITY, L = 0.f;
  const float c = a.c;
  const int qlim = CAUSAL ? qi + a.off : Nk - 1;  // last key this query sees

  auto tile = [&] __device__ (int t, const char* kt, const char* vt) __attribute__((always_inline)) {
    const int k0 = k_lo + t * BC;
    f32x16 sc[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      bf16x8 ka[NKC];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) ka[kc] = lds_read16(kt + toff.rows[kc] + 32 * hf * PITCH);
      sc[hf] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) sc[hf] = mfma32(ka[kc], qf[kc], sc[hf]);
    }
    // mask: keys past the chunk end, the cache end or the query's position
    if (k0 + BC > k_hi || (CAUSAL && k0 + BC - 1 > 32 * g + a.off)) {
#pragma unroll
      for (int hf = 0; hf < NH; ++hf)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * hf + acc_row(r, h);
          if (key >= k_hi || key > qlim) sc[hf][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int hf = 0; hf < NH; ++hf)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[hf][r]);
    mx = xhalf_max(mx);
    const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
    if (mt > Mref + kLazyTau) {  // per lane: this wave has one query per lane
      const float alpha = __builtin_amdgcn_exp2f(Mref - mt);
      L *= alpha;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) o[ct] *= alpha;
      Mref = mt;
    }
    const float mb = (Mref == -INFINITY) ? 0.f : Mref;
    bf16x8 pb[2 * NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[hf][8 * hh + e], c, -mb));
        L += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        pb[2 * hf + hh] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int kc = 0; kc < BC / 16; ++kc) o[ct] = mfma32(toff.read_tr(vt, kc, ct), pb[kc], o[ct]);
  };

  if (ntiles > 0) {
    cp.issue(kb0, Kh, k_lo, Nk, 0);
    cp.issue(vb0, Vh, k_lo, Nk, 0);
  }
  for (int t = 0; t < ntiles; t += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntiles) {
      cp.issue(kb1, Kh, k_lo + (t + 1) * BC, Nk, 0);
      cp.issue(vb1, Vh, k_lo + (t + 1) * BC, Nk, 0);
    }
    tile(t, kb0, vb0);
    if (t + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t + 2 < ntiles) {
        cp.issue(kb0, Kh, k_lo + (t + 2) * BC, Nk, 0);
        cp.issue(vb0, Vh, k_lo + (t + 2) * BC, Nk, 0);
      }
      tile(t + 1, kb1, vb1);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  // partial: O_s = O / l (fp32), lse_s = (Mref + log2 l) ln 2, or empty
  const float Lt = xhalf_sum(L);
  if (qi < Nq) {
    const bool empty = !(Lt > 0.f);
    const float inv = empty ? 0.f : 1.f / Lt;
    const size_t row = ((size_t)bh * Nq + qi) * a.nsplit + s;
    float* dst = a.part_o + row * D;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int col = 32 * ct + 16 * hh + 8 * h;
        const int r0 = 8 * hh;
        f32x4* pd = reinterpret_cast<f32x4*>(dst + col);
        pd[0] = f32x4{o[ct][r0] * inv, o[ct][r0 + 1] * inv, o[ct][r0 + 2] * inv, o[ct][r0 + 3] * inv};
        pd[1] = f32x4{o[ct][r0 + 4] * inv, o[ct][r0 + 5] * inv, o[ct][r0 + 6] * inv, o[ct][r0 + 7] * inv};
      }
    if (h == 0) a.part_lse[row] = empty ? -INFINITY : (Mref + __log2f(Lt)) * kLn2;
  }
}

// One group of D/4 threads per query: each thread owns four columns.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecArgs a, long rows) {
  constexpr int TPR = D / 4;
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gid / TPR;  // bh * Nq + qi
  const int part = (int)(gid % TPR);
  if (row >= rows) return;
  const int S = a.nsplit;
  const float* pl = a.part_lse + row * S;
  float m = -INFINITY;
  for (int s = 0; s < S; ++s) m = fmaxf(m, pl[s]);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float w = __expf(pl[s] - m);
      l += w;
      const f32x4 x = *reinterpret_cast<const f32x4*>(a.part_o + (row * S + s) * D + 4 * part);
      acc += w * x;
    }
  }
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  __bf16* dst = a.o + row * D + 4 * part;
  dst[0] = (__bf16)(acc[0] * inv);
  dst[1] = (__bf16)(acc[1] * inv);
  dst[2] = (__bf16)(acc[2] * inv);
  dst[3] = (__bf16)(acc[3] * inv);
  if (part == 0) a.lse[row] = (l > 0.f) ? m + __logf(l) : -INFINITY;
}

}  // namespace fa
