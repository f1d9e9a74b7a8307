// fp32 path: the same tiled, online-softmax attention in fp32 arithmetic
// throughout, for callers that need fp32 accuracy (no bf16 rounding of
// inputs, P or outputs).  Four threads share one sequence row, each owning
// every fourth column; K/V (or Q/dO) tiles of 64 rows are staged in LDS.
// Scores use the accurate expf/logf rather than the hardware exp2.
#pragma once

#include "fa_device.h"

namespace fa {

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* o;     // backward only
  const float* lse;   // backward input / forward output
  float* out_lse;     // forward only
  const float* dout;  // backward only
  float* dst0;        // fwd: O;  bwd: dQ (dq kernel) or dK (dkdv kernel)
  float* dst1;        // bwd dkdv: dV
  float* Dw;          // bwd: D_i workspace
  const uint8_t* mask;
  int N;
  int nb;
  int causal;
  float scale;
};

constexpr int kF32Rows = 64;  // rows per workgroup and per staged tile

__device__ __forceinline__ bool f32_allowed(const F32Args& a, int i, int j) {
  if (j >= a.N || i >= a.N) return false;
  if (a.causal && j > i) return false;
  if (a.mask && a.mask[(size_t)(i >> 7) * a.nb + (j >> 7)] == 0) return false;
  return true;
}

// Sum over the four threads that share a row.
__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

// Stage rows [r0, r0+64) of a [N][D] fp32 matrix into LDS, zero past N.
template <int D>
__device__ __forceinline__ void f32_stage(float* dst, const float* src, int r0, int N) {
  for (int u = threadIdx.x; u < kF32Rows * D / 4; u += 256) {
    const int row = u / (D / 4), c4 = u % (D / 4);
    f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
    if (r0 + row < N) x = *reinterpret_cast<const f32x4*>(src + (size_t)(r0 + row) * D + 4 * c4);
    *reinterpret_cast<f32x4*>(dst + row * D + 4 * c4) = x;
  }
}

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(F32Args a) {
  constexpr int E = D / 4;
  __shared__ float Ks[kF32Rows * D], Vs[kF32Rows * D];
  const int bh = blockIdx.y, part = threadIdx.x & 3;
  const int i = blockIdx.x * kF32Rows + (threadIdx.x >> 2);
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  float q[E], o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = (i < N) ? a.q[head + (size_t)i * D + 4 * e + part] : 0.f;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int last_row = min(N, (int)(blockIdx.x + 1) * kF32Rows) - 1;
  const int kend = a.causal ? last_row + 1 : N;
  for (int k0 = 0; k0 < kend; k0 += kF32Rows) {
    __syncthreads();
    f32_stage<D>(Ks, a.k + head, k0, N);
    f32_stage<D>(Vs, a.v + head, k0, N);
    __syncthreads();
    float s[kF32Rows];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32Rows; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc = __builtin_fmaf(q[e], Ks[j * D + 4 * e + part], acc);
      acc = a.scale * quad_sum(acc);
      s[j] = f32_allowed(a, i, k0 + j) ? acc : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float mn = fmaxf(m, mt);
    if (mn == -INFINITY) continue;  // nothing visible yet (uniform per row)
    const float alpha = expf(m - mn);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kF32Rows; ++j) {
      const float p = expf(s[j] - mn);
      l += p;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = __builtin_fmaf(p, Vs[j * D + 4 * e + part], o[e]);
    }
    m = mn;
  }
  if (i < N) {
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
#pragma unroll
    for (int e = 0; e < E; ++e) a.dst0[head + (size_t)i * D + 4 * e + part] = o[e] * inv;
    if (part == 0) a.out_lse[(size_t)bh * N + i] = empty ? -INFINITY : m + logf(l);
  }
}

// D_i = sum_c dO_ic O_ic in fp32.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_f32_kernel(F32Args a, long rows) {
  const long r = (long)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  float acc = 0.f;
  if (r < rows) {
#pragma unroll
    for (int e = 0; e < D / 4; ++e)
      acc = __builtin_fmaf(a.dout[r * D + 4 * e + part], a.o[r * D + 4 * e + part], acc);
  }
  acc = quad_sum(acc);
  if (r < rows && part == 0) a.Dw[r] = acc;
}

// dQ_i = scale * sum_j P_ij (dP_ij - D_i) K_j, one row i per four threads.
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(F32Args a) {
  constexpr int E = D / 4;
  __shared__ float Ks[kF32Rows * D], Vs[kF32Rows * D];
  const int bh = blockIdx.y, part = threadIdx.x & 3;
  const int i = blockIdx.x * kF32Rows + (threadIdx.x >> 2);
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  float q[E], dO[E], dq[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = (i < N) ? a.q[head + (size_t)i * D + 4 * e + part] : 0.f;
    dO[e] = (i < N) ? a.dout[head + (size_t)i * D + 4 * e + part] : 0.f;
    dq[e] = 0.f;
  }
  const float lse = (i < N) ? a.lse[(size_t)bh * N + i] : 0.f;
  const float Di = (i < N) ? a.Dw[(size_t)bh * N + i] : 0.f;
  const int last_row = min(N, (int)(blockIdx.x + 1) * kF32Rows) - 1;
  const int kend = a.causal ? last_row + 1 : N;
  for (int k0 = 0; k0 < kend; k0 += kF32Rows) {
    __syncthreads();
    f32_stage<D>(Ks, a.k + head, k0, N);
    f32_stage<D>(Vs, a.v + head, k0, N);
    __syncthreads();
    for (int j = 0; j < kF32Rows; ++j) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        s = __builtin_fmaf(q[e], Ks[j * D + 4 * e + part], s);
        dp = __builtin_fmaf(dO[e], Vs[j * D + 4 * e + part], dp);
      }
      s = a.scale * quad_sum(s);
      dp = quad_sum(dp);
      const float p = f32_allowed(a, i, k0 + j) ? expf(s - lse) : 0.f;
      const float ds = p * (dp - Di);
#pragma unroll
      for (int e = 0; e < E; ++e) dq[e] = __builtin_fmaf(ds, Ks[j * D + 4 * e + part], dq[e]);
    }
  }
  if (i < N) {
#pragma unroll
    for (int e = 0; e < E; ++e) a.dst0[head + (size_t)i * D + 4 * e + part] = a.scale * dq[e];
  }
}

// dV_j = sum_i P_ij dO_i and dK_j = scale * sum_i P_ij (dP_ij - D_i) Q_i,
// one key row j per four threads.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(F32Args a) {
  constexpr int E = D / 4;
  __shared__ float Qs[kF32Rows * D], dOs[kF32Rows * D], Ls[kF32Rows], Ds[kF32Rows];
  const int bh = blockIdx.y, part = threadIdx.x & 3;
  const int j = blockIdx.x * kF32Rows + (threadIdx.x >> 2);
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  float k[E], v[E], dk[E], dv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k[e] = (j < N) ? a.k[head + (size_t)j * D + 4 * e + part] : 0.f;
    v[e] = (j < N) ? a.v[head + (size_t)j * D + 4 * e + part] : 0.f;
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  const int q_first = a.causal ? (int)blockIdx.x * kF32Rows : 0;
  for (int q0 = q_first; q0 < N; q0 += kF32Rows) {
    __syncthreads();
    f32_stage<D>(Qs, a.q + head, q0, N);
    f32_stage<D>(dOs, a.dout + head, q0, N);
    if (threadIdx.x < kF32Rows) {
      const int r = q0 + threadIdx.x;
      Ls[threadIdx.x] = (r < N) ? a.lse[(size_t)bh * N + r] : 0.f;
      Ds[threadIdx.x] = (r < N) ? a.Dw[(size_t)bh * N + r] : 0.f;
    }
    __syncthreads();
    for (int ii = 0; ii < kF32Rows; ++ii) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        s = __builtin_fmaf(Qs[ii * D + 4 * e + part], k[e], s);
        dp = __builtin_fmaf(dOs[ii * D + 4 * e + part], v[e], dp);
      }
      s = a.scale * quad_sum(s);
      dp = quad_sum(dp);
      const float p = f32_allowed(a, q0 + ii, j) ? expf(s - Ls[ii]) : 0.f;
      const float ds = p * (dp - Ds[ii]);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        dv[e] = __builtin_fmaf(p, dOs[ii * D + 4 * e + part], dv[e]);
        dk[e] = __builtin_fmaf(ds, Qs[ii * D + 4 * e + part], dk[e]);
      }
    }
  }
  if (j < N) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      a.dst0[head + (size_t)j * D + 4 * e + part] = a.scale * dk[e];
      a.dst1[head + (size_t)j * D + 4 * e + part] = dv[e];
    }
  }
}

}  // namespace fa
