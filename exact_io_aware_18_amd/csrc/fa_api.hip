// C ABI of the attention library: argument checks, variant dispatch and
// launches.  Every check runs before the first HIP call, so an invalid call
// enqueues nothing and is testable without a GPU.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa.h"
#include "fa_bwd.h"
#include "fa_decode.h"
#include "fa_f32.h"
#include "fa_fwd.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + bytes};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void* p, size_t al) { return (reinterpret_cast<uintptr_t>(p) % al) == 0; }

int nblocks(int N) { return (N + 127) / 128; }

// Shape limits shared by every call.
int check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if ((long long)N * d >= (1LL << 31)) return FA_ERR_SHAPE;
  const long long bh = (long long)B * H;
  if (bh * nblocks(N) >= (1LL << 24)) return FA_ERR_SHAPE;
  if (bh * N * d >= (1LL << 46)) return FA_ERR_SHAPE;
  return FA_OK;
}

int check_flags(float scale, int causal) {
  if (causal != 0 && causal != 1) return FA_ERR_FLAG;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  return FA_OK;
}

// Outputs must not overlap inputs or each other.
int check_alias(const Span* outs, int nout, const Span* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

size_t workspace_bytes(int B, int H, int N) {
  const size_t n = (size_t)B * H * N * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

int launched() {
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// ---- bf16 forward -----------------------------------------------------------
template <int D, bool CAUSAL, bool MASK, bool DROP>
void launch_fwd_t(const fa::FwdArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((fa::fwd_bf16_kernel<D, CAUSAL, MASK, DROP>), dim3(grid), dim3(256), 0, s, a);
}

template <int D, int G, bool CAUSAL, bool DROP>
void launch_fwd_pp(fa::FwdArgs a, int BH, hipStream_t s) {
  using T = fa::FwdPPTile<D, G>;
  a.nqt = (a.N + T::BR - 1) / T::BR;
  a.total = BH * a.nqt;
  hipLaunchKernelGGL((fa::fwd_pp_kernel<D, G, CAUSAL, DROP>), dim3(a.total), dim3(T::NT), 0, s, a);
}

template <int D, int G>
long pp_workgroups(int BH, int N) {
  return (long)BH * ((N + fa::FwdPPTile<D, G>::BR - 1) / fa::FwdPPTile<D, G>::BR);
}

// Dense and causal use the phased kernel (one workgroup per CU) when it gets
// at least two workgroups per CU; smaller grids go to the 128-row kernel
// (two workgroups per CU), which fills the chip with more workgroups
// (measured: +10-18% at B*H*N = 96K-100K, 8-18% slower than the two-group
// kernel from 512 of its workgroups up).  The three-group kernel (384 rows,
// d=64 without dropout, whose generator does not fit beside it in 168
// registers per wave) runs from N = 4096 up: there its per-tile rounds are
// ~18% shorter (+11% on a dense grid of 16 workgroups per CU), while at
// short N its 384-row tiles leave ragged tails.  A block mask needs 128-row
// workgroups (one mask row each).
constexpr long kPingPongMinWorkgroups = 512;
constexpr int kThreeGroupMinN = 4096;

// Query rows per workgroup of the bf16 forward kernel a call takes: 128
// (block mask, or a small grid), 256 (two groups) or 384 (three groups).
// The launch below and fa_fwd_query_rows both decide through this function.
int fwd_rows(int BH, int N, int d, bool mask, bool drop) {
  if (mask) return 128;
  const bool g3 = d == 64 && !drop && N >= kThreeGroupMinN &&
                  pp_workgroups<64, 3>(BH, N) >= kPingPongMinWorkgroups;
  if (g3) return fa::FwdPPTile<64, 3>::BR;
  const long g2 = d == 64 ? pp_workgroups<64, 2>(BH, N) : pp_workgroups<128, 2>(BH, N);
  return g2 >= kPingPongMinWorkgroups ? fa::FwdPPTile<64, 2>::BR : fa::FwdTile<64>::BR;
}

template <int D, bool DROP>
void launch_fwd_dd(const fa::FwdArgs& a, int BH, bool causal, bool mask, hipStream_t s) {
  const int rows = fwd_rows(BH, a.N, D, mask, DROP);
  if (rows == 128) {
    if (mask) {
      if (causal) launch_fwd_t<D, true, true, DROP>(a, a.total, s);
      else launch_fwd_t<D, false, true, DROP>(a, a.total, s);
    } else {
      if (causal) launch_fwd_t<D, true, false, DROP>(a, a.total, s);
      else launch_fwd_t<D, false, false, DROP>(a, a.total, s);
    }
    return;
  }
  if constexpr (D == 64 && !DROP) {
    if (rows == fa::FwdPPTile<D, 3>::BR) {
      if (causal) launch_fwd_pp<D, 3, true, DROP>(a, BH, s);
      else launch_fwd_pp<D, 3, false, DROP>(a, BH, s);
      return;
    }
  }
  if (causal) launch_fwd_pp<D, 2, true, DROP>(a, BH, s);
  else launch_fwd_pp<D, 2, false, DROP>(a, BH, s);
}

template <int D>
void launch_fwd_d(const fa::FwdArgs& a, int BH, bool causal, bool mask, bool drop, hipStream_t s) {
  if (drop) launch_fwd_dd<D, true>(a, BH, causal, mask, s);
  else launch_fwd_dd<D, false>(a, BH, causal, mask, s);
}

// ---- bf16 backward ----------------------------------------------------------
enum BwdStage { kPre = 1, kDkdv = 2, kDq = 4 };

template <int D, bool CAUSAL, bool MASK, bool DROP>
void launch_bwd_t(fa::BwdArgs a, int BH, int stages, hipStream_t s) {
  a.total = BH * a.ntile;
  if (stages & kDkdv) {
    if constexpr (D == 128)
      hipLaunchKernelGGL((fa::bwd_dkdv_pair_kernel<D, CAUSAL, MASK, DROP>), dim3(a.total),
                         dim3(fa::DkdvPairTile<D>::NT), 0, s, a);
    else
      hipLaunchKernelGGL((fa::bwd_dkdv_kernel<D, CAUSAL, MASK, DROP>), dim3(a.total), dim3(256), 0, s, a);
  }
  if (stages & kDq)
    hipLaunchKernelGGL((fa::bwd_dq_kernel<D, CAUSAL, MASK, DROP>), dim3(a.total), dim3(256), 0, s, a);
}

template <int D, bool DROP>
void launch_bwd_dd(const fa::BwdArgs& a, int BH, bool causal, bool mask, int stages, hipStream_t s) {
  if (causal) {
    if (mask) launch_bwd_t<D, true, true, DROP>(a, BH, stages, s);
    else launch_bwd_t<D, true, false, DROP>(a, BH, stages, s);
  } else {
    if (mask) launch_bwd_t<D, false, true, DROP>(a, BH, stages, s);
    else launch_bwd_t<D, false, false, DROP>(a, BH, stages, s);
  }
}

template <int D>
void launch_bwd_d(const fa::BwdArgs& a, int BH, bool causal, bool mask, bool drop, int stages,
                  hipStream_t s) {
  if (stages & kPre) {
    const long rows = (long)BH * a.N;
    const int pre_grid = (int)((rows * (D / 8) + 255) / 256);
    hipLaunchKernelGGL((fa::bwd_pre_kernel<D>), dim3(pre_grid), dim3(256), 0, s, a.o, a.dout, a.Dw, rows);
  }
  if (drop) launch_bwd_dd<D, true>(a, BH, causal, mask, stages, s);
  else launch_bwd_dd<D, false>(a, BH, causal, mask, stages, s);
}

int run_bwd(const fa::BwdArgs& a, int BH, int d, int causal, bool mask, int stages, void* stream,
            bool drop = false) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (d == 64) launch_bwd_d<64>(a, BH, causal, mask, drop, stages, s);
  else launch_bwd_d<128>(a, BH, causal, mask, drop, stages, s);
  return launched();
}

// Dropout parameters: T = floor(p * 2^32) (the float p widened exactly to
// double), keep scale 1 / (1 - p).
int check_dropout(float p) {
  if (!(p >= 0.f && p < 1.f)) return FA_ERR_DROPOUT;  // NaN fails both
  return FA_OK;
}

fa::DropArgs drop_args(float p, unsigned long long seed) {
  fa::DropArgs dp;
  const double t = std::floor((double)p * 4294967296.0);
  dp.thresh = t >= 4294967295.0 ? 0xFFFFFFFFu : (uint32_t)t;
  dp.seed_lo = (uint32_t)(seed & 0xFFFFFFFFull);
  dp.seed_hi = (uint32_t)(seed >> 32);
  dp.keep_scale = (float)(1.0 / (1.0 - (double)p));
  return dp;
}

// ---- fp32 -------------------------------------------------------------------
template <int D>
void launch_fwd_f32_d(const fa::F32Args& a, int BH, hipStream_t s) {
  dim3 grid((a.N + fa::kF32Rows - 1) / fa::kF32Rows, BH);
  hipLaunchKernelGGL((fa::fwd_f32_kernel<D>), grid, dim3(256), 0, s, a);
}

template <int D>
void launch_bwd_f32_d(fa::F32Args a, int BH, float* dq, float* dk, float* dv, hipStream_t s) {
  const long rows = (long)BH * a.N;
  hipLaunchKernelGGL((fa::bwd_pre_f32_kernel<D>), dim3((unsigned)((rows + 63) / 64)), dim3(256), 0, s, a, rows);
  dim3 grid((a.N + fa::kF32Rows - 1) / fa::kF32Rows, BH);
  a.dst0 = dq;
  hipLaunchKernelGGL((fa::bwd_dq_f32_kernel<D>), grid, dim3(256), 0, s, a);
  a.dst0 = dk;
  a.dst1 = dv;
  hipLaunchKernelGGL((fa::bwd_dkdv_f32_kernel<D>), grid, dim3(256), 0, s, a);
}

// A tensor argument: address, extent in bytes, required alignment.
struct Buf {
  const void* p;
  size_t bytes;
  size_t align;
};

// Null, alignment and overlap checks over the inputs and outputs of a call.
// `ins` may hold entries with p == nullptr that are optional (the mask).
int check_bufs(const Buf* ins, int nin, const Buf* outs, int nout) {
  for (int i = 0; i < nout; ++i)
    if (!outs[i].p) return FA_ERR_NULL;
  for (int i = 0; i < nin; ++i)
    if (ins[i].p && !aligned(ins[i].p, ins[i].align)) return FA_ERR_ALIGN;
  for (int i = 0; i < nout; ++i)
    if (!aligned(outs[i].p, outs[i].align)) return FA_ERR_ALIGN;
  Span si[8], so[8];
  int ni = 0;
  for (int i = 0; i < nin; ++i)
    if (ins[i].p) si[ni++] = span(ins[i].p, ins[i].bytes);
  for (int i = 0; i < nout; ++i) so[i] = span(outs[i].p, outs[i].bytes);
  return check_alias(so, nout, si, ni);
}

struct Sizes {
  size_t t;   // one [B,H,N,d] input tensor
  size_t g;   // one fp32 [B,H,N,d] gradient
  size_t l;   // one fp32 [B,H,N] vector
  size_t m;   // block mask
  size_t ws;  // workspace
};

Sizes sizes(int B, int H, int N, int d, size_t esz) {
  const size_t rows = (size_t)B * H * N;
  const size_t nb = (size_t)nblocks(N);
  return Sizes{rows * d * esz, rows * d * sizeof(float), rows * sizeof(float), nb * nb,
               workspace_bytes(B, H, N)};
}

int check_common(int B, int H, int N, int d, float scale, int causal) {
  int st = check_shape(B, H, N, d);
  if (st) return st;
  return check_flags(scale, causal);
}

int check_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
              int B, int H, int N, int d, float scale, int causal, const unsigned char* mask,
              size_t esz) {
  if (!q || !k || !v) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale, causal);
  if (st) return st;
  const Sizes z = sizes(B, H, N, d, esz);
  const Buf ins[4] = {{q, z.t, 16}, {k, z.t, 16}, {v, z.t, 16}, {mask, z.m, 1}};
  const Buf outs[2] = {{o, z.t, 16}, {lse, z.l, 4}};
  return check_bufs(ins, 4, outs, 2);
}

int check_ws(const void* ws, size_t ws_bytes, int B, int H, int N) {
  if (!ws || ws_bytes < workspace_bytes(B, H, N)) return FA_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return FA_ERR_ALIGN;
  return FA_OK;
}

int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, const float* dq, const float* dk, const float* dv, int B, int H,
              int N, int d, float scale, int causal, const unsigned char* mask,
              const void* ws, size_t ws_bytes, size_t esz) {
  if (!q || !k || !v || !o || !lse || !dout) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale, causal);
  if (st) return st;
  if ((st = check_ws(ws, ws_bytes, B, H, N))) return st;
  const Sizes z = sizes(B, H, N, d, esz);
  const Buf ins[7] = {{q, z.t, 16}, {k, z.t, 16}, {v, z.t, 16}, {o, z.t, 16},
                      {dout, z.t, 16}, {lse, z.l, 4}, {mask, z.m, 1}};
  const Buf outs[4] = {{dq, z.g, 16}, {dk, z.g, 16}, {dv, z.g, 16}, {ws, z.ws, 16}};
  return check_bufs(ins, 7, outs, 4);
}

// ---- decode ------------------------------------------------------------------
int check_decode_shape(int B, int H, int Nq, int Nk, int d) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if ((long long)Nk * d >= (1LL << 31) || (long long)Nq * d >= (1LL << 31)) return FA_ERR_SHAPE;
  const long long bh = (long long)B * H;
  if (bh * ((Nq + 31) / 32) * ((Nk + 255) / 256) >= (1LL << 31)) return FA_ERR_SHAPE;
  if (bh * Nk * d >= (1LL << 46)) return FA_ERR_SHAPE;
  return FA_OK;
}

size_t decode_ws_bytes(int B, int H, int Nq, int Nk, int d) {
  int nsplit, chunk;
  fa::decode_split(B * H, Nq, Nk, d, &nsplit, &chunk);
  const size_t rows = (size_t)B * H * Nq * nsplit;
  const size_t lse_bytes = (rows * sizeof(float) + 255) & ~(size_t)255;
  return lse_bytes + rows * d * sizeof(float);
}

template <int D>
void launch_decode_d(const fa::DecArgs& a, int BH, bool causal, hipStream_t s) {
  const unsigned grid = (unsigned)((long)BH * a.nqg * a.nsplit);
  if (causal) hipLaunchKernelGGL((fa::decode_split_kernel<D, true>), dim3(grid), dim3(64), 0, s, a);
  else hipLaunchKernelGGL((fa::decode_split_kernel<D, false>), dim3(grid), dim3(64), 0, s, a);
  const long rows = (long)BH * a.Nq;
  const unsigned mgrid = (unsigned)((rows * (D / 4) + 255) / 256);
  hipLaunchKernelGGL((fa::decode_merge_kernel<D>), dim3(mgrid), dim3(256), 0, s, a, rows);
}

fa::BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, float* dq, float* dk, float* dv,
                     int N, float scale, const unsigned char* mask, void* ws) {
  fa::BwdArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<const __bf16*>(o);
  a.dout = static_cast<const __bf16*>(dout);
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.Dw = static_cast<float*>(ws);
  a.mask = mask;
  a.N = N;
  a.nb = nblocks(N);
  a.ntile = (N + 127) / 128;  // dK/dV and dQ workgroups each own 128 rows
  a.total = 0;
  a.c = scale * fa::kLog2e;
  a.scale = scale;
  a.drop = fa::DropArgs{0u, 0u, 0u, 1.f};
  return a;
}

int run_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
            int d, float scale, int causal, const unsigned char* blockmask, const fa::DropArgs* drop,
            void* stream) {
  fa::FwdArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.mask = blockmask;
  a.N = N;
  a.nqt = (N + 127) / 128;
  a.total = B * H * a.nqt;
  a.nb = nblocks(N);
  // c > 0 even for scale == 0, so masked scores (-inf) stay -inf after the
  // scaling; FLT_MIN times a finite score rounds 2^(score) to exactly 1.
  a.c = std::fmax(std::fabs(scale) * fa::kLog2e, FLT_MIN);
  a.negate_q = scale < 0.f;
  a.drop = drop ? *drop : fa::DropArgs{0u, 0u, 0u, 1.f};
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (d == 64) launch_fwd_d<64>(a, B * H, causal, blockmask != nullptr, drop != nullptr, s);
  else launch_fwd_d<128>(a, B * H, causal, blockmask != nullptr, drop != nullptr, s);
  return launched();
}

// ---- backward without a caller workspace ------------------------------------
// fa_bwd_noalloc keeps the per-row D of the backward in this file-scope device
// array instead of a caller workspace.  Every GPU the library runs on holds
// its own copy, from the first use until the process ends.  Host code must
// not pass `scratch` itself to a kernel (on the host it names a stand-in, not
// the device array): the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and is kept below.
constexpr size_t kScratchFloats = size_t(1) << 22;  // 16 MiB: B * H * N <= 4,194,304
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the GPU that runs stream s (the current GPU
// for the default stream), looked up on the first call on that GPU with that
// GPU current; the caller's current device is restored.
int scratch_for_stream(hipStream_t s, float** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_LAUNCH;
  int dev = cur;
  if (s && hipStreamGetDevice(s, &dev) != hipSuccess) return FA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return FA_ERR_LAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return FA_ERR_LAUNCH;
    if (e != hipSuccess || !p) return FA_ERR_LAUNCH;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int causal, const unsigned char* blockmask, void* stream) {
  int st = check_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, 2);
  if (st) return st;
  return run_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, nullptr, stream);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int N, int d, float scale, int causal, const unsigned char* blockmask,
                   float p_drop, unsigned long long seed, void* stream) {
  int st = check_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, 2);
  if (st) return st;
  if ((st = check_dropout(p_drop))) return st;
  if (p_drop == 0.f)  // every element kept: the plain kernels, bit for bit
    return run_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, nullptr, stream);
  const fa::DropArgs dp = drop_args(p_drop, seed);
  return run_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, &dp, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, float* dq, float* dk, float* dv, int B, int H, int N, int d,
           float scale, int causal, const unsigned char* blockmask, void* workspace,
           size_t workspace_bytes_, void* stream) {
  int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, blockmask,
                     workspace, workspace_bytes_, 2);
  if (st) return st;
  const fa::BwdArgs a = bwd_args(q, k, v, o, lse, dout, dq, dk, dv, N, scale, blockmask, workspace);
  return run_bwd(a, B * H, d, causal, blockmask != nullptr, kPre | kDkdv | kDq, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                   float scale, int causal, const unsigned char* blockmask, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale, causal);
  if (st) return st;
  if ((size_t)B * H * N > kScratchFloats) return FA_ERR_SCRATCH;
  const Sizes z = sizes(B, H, N, d, 2);
  const Buf ins[7] = {{q, z.t, 16}, {k, z.t, 16}, {v, z.t, 16}, {o, z.t, 16},
                      {dout, z.t, 16}, {lse, z.l, 4}, {blockmask, z.m, 1}};
  const Buf outs[3] = {{dq, z.g, 16}, {dk, z.g, 16}, {dv, z.g, 16}};
  if ((st = check_bufs(ins, 7, outs, 3))) return st;
  float* ws = nullptr;
  if ((st = scratch_for_stream(static_cast<hipStream_t>(stream), &ws))) return st;
  const fa::BwdArgs a = bwd_args(q, k, v, o, lse, dout, dq, dk, dv, N, scale, blockmask, ws);
  return run_bwd(a, B * H, d, causal, blockmask != nullptr, kPre | kDkdv | kDq, stream);
}

size_t fa_bwd_noalloc_max_rows(void) { return kScratchFloats; }

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                   float scale, int causal, const unsigned char* blockmask, float p_drop,
                   unsigned long long seed, void* workspace, size_t workspace_bytes_,
                   void* stream) {
  int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, blockmask,
                     workspace, workspace_bytes_, 2);
  if (st) return st;
  if ((st = check_dropout(p_drop))) return st;
  fa::BwdArgs a = bwd_args(q, k, v, o, lse, dout, dq, dk, dv, N, scale, blockmask, workspace);
  a.drop = drop_args(p_drop, seed);
  return run_bwd(a, B * H, d, causal, blockmask != nullptr, kPre | kDkdv | kDq, stream, p_drop != 0.f);
}

int fa_bwd_preprocess(const void* o, const void* dout, int B, int H, int N, int d,
                      void* workspace, size_t workspace_bytes_, void* stream) {
  if (!o || !dout) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st) return st;
  if ((st = check_ws(workspace, workspace_bytes_, B, H, N))) return st;
  const Sizes z = sizes(B, H, N, d, 2);
  const Buf ins[2] = {{o, z.t, 16}, {dout, z.t, 16}};
  const Buf outs[1] = {{workspace, z.ws, 16}};
  if ((st = check_bufs(ins, 2, outs, 1))) return st;
  const fa::BwdArgs a = bwd_args(nullptr, nullptr, nullptr, o, nullptr, dout, nullptr, nullptr,
                                 nullptr, N, 1.f, nullptr, workspace);
  return run_bwd(a, B * H, d, 0, false, kPre, stream);
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                float* dk, float* dv, int B, int H, int N, int d, float scale, int causal,
                const unsigned char* blockmask, const void* workspace, size_t workspace_bytes_,
                void* stream) {
  if (!q || !k || !v || !lse || !dout) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale, causal);
  if (st) return st;
  if ((st = check_ws(workspace, workspace_bytes_, B, H, N))) return st;
  const Sizes z = sizes(B, H, N, d, 2);
  const Buf ins[7] = {{q, z.t, 16}, {k, z.t, 16}, {v, z.t, 16}, {dout, z.t, 16},
                      {lse, z.l, 4}, {workspace, z.ws, 16}, {blockmask, z.m, 1}};
  const Buf outs[2] = {{dk, z.g, 16}, {dv, z.g, 16}};
  if ((st = check_bufs(ins, 7, outs, 2))) return st;
  const fa::BwdArgs a = bwd_args(q, k, v, nullptr, lse, dout, nullptr, dk, dv, N, scale, blockmask,
                                 const_cast<void*>(workspace));
  return run_bwd(a, B * H, d, causal, blockmask != nullptr, kDkdv, stream);
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dout,
              float* dq, int B, int H, int N, int d, float scale, int causal,
              const unsigned char* blockmask, const void* workspace, size_t workspace_bytes_,
              void* stream) {
  if (!q || !k || !v || !lse || !dout) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale, causal);
  if (st) return st;
  if ((st = check_ws(workspace, workspace_bytes_, B, H, N))) return st;
  const Sizes z = sizes(B, H, N, d, 2);
  const Buf ins[7] = {{q, z.t, 16}, {k, z.t, 16}, {v, z.t, 16}, {dout, z.t, 16},
                      {lse, z.l, 4}, {workspace, z.ws, 16}, {blockmask, z.m, 1}};
  const Buf outs[1] = {{dq, z.g, 16}};
  if ((st = check_bufs(ins, 7, outs, 1))) return st;
  const fa::BwdArgs a = bwd_args(q, k, v, nullptr, lse, dout, dq, nullptr, nullptr, N, scale,
                                 blockmask, const_cast<void*>(workspace));
  return run_bwd(a, B * H, d, causal, blockmask != nullptr, kDq, stream);
}

int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int Nq, int Nk, int d, float scale, int causal, void* workspace,
                  size_t workspace_bytes_, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_decode_shape(B, H, Nq, Nk, d);
  if (st) return st;
  if ((st = check_flags(scale, causal))) return st;
  const size_t need = decode_ws_bytes(B, H, Nq, Nk, d);
  if (!workspace || workspace_bytes_ < need) return FA_ERR_WORKSPACE;
  const size_t tq = (size_t)B * H * Nq * d * 2, tk = (size_t)B * H * Nk * d * 2;
  const Buf ins[3] = {{q, tq, 16}, {k, tk, 16}, {v, tk, 16}};
  const Buf outs[3] = {{o, tq, 16}, {lse, (size_t)B * H * Nq * 4, 4}, {workspace, need, 16}};
  if ((st = check_bufs(ins, 3, outs, 3))) return st;
  fa::DecArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.Nq = Nq;
  a.Nk = Nk;
  a.nqg = (Nq + 31) / 32;
  fa::decode_split(B * H, Nq, Nk, d, &a.nsplit, &a.chunk);
  const size_t rows = (size_t)B * H * Nq * a.nsplit;
  a.part_lse = static_cast<float*>(workspace);
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      ((rows * sizeof(float) + 255) & ~(size_t)255));
  a.off = Nk - Nq;
  a.c = std::fmax(std::fabs(scale) * fa::kLog2e, FLT_MIN);
  a.negate_q = scale < 0.f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (d == 64) launch_decode_d<64>(a, B * H, causal != 0, s);
  else launch_decode_d<128>(a, B * H, causal != 0, s);
  return launched();
}

size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  if (check_decode_shape(B, H, Nq, Nk, d) != FA_OK) return 0;
  return decode_ws_bytes(B, H, Nq, Nk, d);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d) != FA_OK) return 0;
  return workspace_bytes(B, H, N);
}

int fa_fwd_query_rows(int B, int H, int N, int d, int causal, int has_blockmask, int dropout) {
  if (check_shape(B, H, N, d) != FA_OK) return 0;
  if ((causal != 0 && causal != 1) || (has_blockmask != 0 && has_blockmask != 1) ||
      (dropout != 0 && dropout != 1))
    return 0;
  return fwd_rows(B * H, N, d, has_blockmask != 0, dropout != 0);
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, const unsigned char* blockmask,
               void* stream) {
  int st = check_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, 4);
  if (st) return st;
  if ((long long)B * H >= 65536) return FA_ERR_UNSUPPORTED;  // grid.y limit
  fa::F32Args a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dst0 = o;
  a.out_lse = lse;
  a.mask = blockmask;
  a.N = N;
  a.nb = nblocks(N);
  a.causal = causal;
  a.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (d == 64) launch_fwd_f32_d<64>(a, B * H, s);
  else launch_fwd_f32_d<128>(a, B * H, s);
  return launched();
}

int fa_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* lse,
               const float* dout, float* dq, float* dk, float* dv, int B, int H, int N, int d,
               float scale, int causal, const unsigned char* blockmask, void* workspace,
               size_t workspace_bytes_, void* stream) {
  int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, blockmask,
                     workspace, workspace_bytes_, 4);
  if (st) return st;
  if ((long long)B * H >= 65536) return FA_ERR_UNSUPPORTED;
  fa::F32Args a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.Dw = static_cast<float*>(workspace);
  a.mask = blockmask;
  a.N = N;
  a.nb = nblocks(N);
  a.causal = causal;
  a.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (d == 64) launch_bwd_f32_d<64>(a, B * H, dq, dk, dv, s);
  else launch_bwd_f32_d<128>(a, B * H, dq, dk, dv, s);
  return launched();
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H or N is below 1 or a size limit is exceeded";
    case FA_ERR_HEADDIM: return "head dimension d must be 64 or 128";
    case FA_ERR_ALIGN: return "tensor pointers must be 16-byte aligned (lse 4-byte)";
    case FA_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA_ERR_WORKSPACE: return "workspace is NULL or smaller than fa_bwd_workspace_bytes()";
    case FA_ERR_FLAG: return "causal must be 0 or 1";
    case FA_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch or a runtime query";
    case FA_ERR_UNSUPPORTED: return "arguments are valid but not supported by this build";
    case FA_ERR_SCALE: return "scale must be finite";
    case FA_ERR_DROPOUT: return "dropout probability must be in [0, 1)";
    case FA_ERR_SCRATCH: return "B * H * N exceeds fa_bwd_noalloc_max_rows()";
    default: return "unknown status";
  }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
