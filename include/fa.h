/*
 * fa.h - C ABI of an exact, tile-by-tile attention library for MI355X (gfx950).
 *
 * What the calls compute.  Standard scaled-dot-product attention per
 * (batch, head): S = scale * Q K^T, P = softmax(S) row-wise, O = P V
 * ("FlashAttention: Fast and Memory-Efficient Exact Attention with
 * IO-Awareness", summary page, §2 Background), computed without ever writing
 * S or P to HBM: Q/K/V are split into tiles staged on-chip, the softmax is
 * normalised incrementally across key tiles, and only O plus one per-row
 * statistic (the logsumexp) go back to memory (same page, §3 Method:
 * "Tiling" and "Softmax rescaling / recomputation").  The backward pass
 * recomputes P on-chip from that statistic (same section) and returns the
 * exact gradients of O with respect to Q, K and V.  Block-sparse attention
 * skips the key blocks a block mask zeroes (abstract on the same pages:
 * "We also extend FlashAttention to block-sparse attention").
 *
 * Conventions shared by every call
 *   - Tensors are [B, H, N, d], contiguous, d fastest.  Q, K and V have the
 *     same N (self-attention shape).  lse and the backward workspace are
 *     [B, H, N] fp32.
 *   - lse[b,h,i] = ln sum_j exp(S_ij) over allowed j (natural log of the
 *     scaled scores).  A row with no allowed key gets O = 0 and lse = -inf,
 *     and contributes nothing to the gradients.
 *   - causal != 0 keeps key j for query i only when j <= i.
 *   - blockmask: NULL for dense, else a device array of nb*nb bytes with
 *     nb = ceil(N/128); entry [qb*nb + kb] != 0 lets query rows of block qb
 *     see key rows of block kb.  One mask serves every (b, h).  The last
 *     block covers the remainder when N % 128 != 0.  causal and blockmask
 *     combine by AND.
 *   - Ownership: every pointer is caller-owned device memory.  The library
 *     allocates nothing and frees nothing.  Apart from fa_bwd_noalloc (a
 *     fixed per-GPU device array, see there) it keeps no state, so concurrent
 *     calls on different streams are safe.  Inputs are only read; outputs
 *     are fully overwritten.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t, NULL = the
 *     null stream) and the call returns without waiting.  A call only
 *     launches kernels on that stream: it allocates nothing, records no
 *     memset or copy and never synchronises, so calls can be captured into
 *     a HIP graph (stream capture) and replayed.
 *   - Errors: arguments are checked before any HIP call, so a bad call
 *     returns a negative fa_status and enqueues nothing.  A failed launch
 *     returns FA_ERR_LAUNCH.  Faults inside a kernel surface at the caller's
 *     next synchronisation.  No C++ exception crosses this interface.
 *   - Supported: d in {64, 128}; B, H, N >= 1; N * d < 2^31;
 *     B * H * ceil(N/128) < 2^24; scale finite.
 *     Tensor pointers must be 16-byte aligned, lse 4-byte aligned.
 *     No output may overlap an input or another output.
 *   - Accuracy.  Any finite scale is accepted; the error is that of the
 *     arithmetic's precision, not of the scale.  bf16 path: products take
 *     bf16 operands with fp32 accumulation; P (in O = P V and dV = P^T dO),
 *     dS (in dQ and dK) and the returned O are rounded to bf16 (unit
 *     roundoff 2^-8), and the backward's D = rowsum(dO o O) uses that bf16
 *     O.  Errors therefore scale with the outputs: measured max-abs error of
 *     O, dQ, dK and dV is at most 0.85% of the largest |element| of the same
 *     tensor (N(0,1) inputs, |scale| up to 0.5, rows with 40-unit score
 *     spreads), which is within 2e-2 absolute while |O|, |dQ|, |dK|, |dV|
 *     stay below ~2.5 (N(0,1) inputs at scale 1/sqrt(d)).  lse is fp32
 *     (error ~1e-6 of |lse|).  fp32 path: fp32 throughout, measured max-abs
 *     error at most 3.2e-6 of the largest |element| (|scale| up to 1).
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = -1,        /* a required pointer is NULL */
    FA_ERR_SHAPE = -2,       /* B, H or N < 1, or a size limit exceeded */
    FA_ERR_HEADDIM = -3,     /* d is not 64 or 128 */
    FA_ERR_ALIGN = -4,       /* a pointer is not aligned as required */
    FA_ERR_ALIAS = -5,       /* an output overlaps an input or another output */
    FA_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than fa_bwd_workspace_bytes() */
    FA_ERR_FLAG = -7,        /* causal is not 0 or 1 */
    FA_ERR_LAUNCH = -8,      /* the HIP runtime rejected a launch or a query */
    FA_ERR_UNSUPPORTED = -9, /* valid arguments this build does not handle */
    FA_ERR_SCALE = -10,      /* scale is NaN or infinite */
    FA_ERR_DROPOUT = -11,    /* p_drop is NaN or outside [0, 1) */
    FA_ERR_SCRATCH = -12     /* B*H*N exceeds fa_bwd_noalloc_max_rows() */
} fa_status;

/*
 * Forward, bf16.  q, k, v: bf16 [B,H,N,d] (uint16 storage).  o: bf16
 * [B,H,N,d], rounded to nearest even from the fp32 accumulator.  lse: fp32
 * [B,H,N].  Computes O = softmax(scale * Q K^T, masked) V row by row with an
 * online softmax over key tiles (§3 Method, "Tiling", "Softmax rescaling").
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal,
           const unsigned char* blockmask, void* stream);

/*
 * Backward, bf16 inputs, fp32 gradients.  q, k, v, o, dout: bf16 [B,H,N,d];
 * o and lse must be the outputs of fa_fwd on the same q, k, v, scale, causal
 * and blockmask.  dq, dk, dv: fp32 [B,H,N,d], fully overwritten.  P is
 * recomputed from lse instead of being read from memory (§3 Method,
 * "recomputation").  workspace: device memory of at least
 * fa_bwd_workspace_bytes(B,H,N,d) bytes, 16-byte aligned; its contents on
 * entry are ignored and on exit are unspecified.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, float* dq, float* dk, float* dv,
           int B, int H, int N, int d, float scale, int causal,
           const unsigned char* blockmask, void* workspace,
           size_t workspace_bytes, void* stream);

/*
 * fa_bwd without the workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that
 * forbid hipMalloc).  The per-row D that fa_bwd keeps in the caller's
 * workspace lives instead in a fixed device array inside the library, one
 * per GPU, held from the first call on that GPU until the process ends
 * (16 MiB: B * H * N <= fa_bwd_noalloc_max_rows() = 4,194,304, else
 * FA_ERR_SCRATCH before any HIP call).  The call allocates and frees nothing.
 * Every call on one GPU shares that array: calls on one GPU that overlap in
 * time (different streams, or host threads without ordering) race on it and
 * must be serialised by the caller.  The array used is that of the GPU that
 * runs `stream` (the current GPU for the default stream, NULL).  Other
 * arguments, results and errors as for fa_bwd; the first call on a GPU also
 * queries the array's address there, with that GPU made current for the
 * query and the caller's current GPU restored (FA_ERR_LAUNCH if the runtime
 * refuses).  Under HIP graph capture, make the first call on a GPU outside
 * the capture, so that the query is not recorded.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, float* dq, float* dk, float* dv,
                   int B, int H, int N, int d, float scale, int causal,
                   const unsigned char* blockmask, void* stream);

/* Largest B * H * N fa_bwd_noalloc accepts. */
size_t fa_bwd_noalloc_max_rows(void);

/*
 * The three stages fa_bwd runs, in this order, as separate calls (bf16 path)
 * for callers that schedule or time them one by one.  Arguments mean what
 * they mean for fa_bwd; each call checks only the arguments it uses.
 *   fa_bwd_preprocess  D_i = sum_c dout_ic * o_ic into the workspace
 *   fa_bwd_dkdv        dk and dv (needs the preprocess result)
 *   fa_bwd_dq          dq (needs the preprocess result)
 */
int fa_bwd_preprocess(const void* o, const void* dout, int B, int H, int N, int d,
                      void* workspace, size_t workspace_bytes, void* stream);
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                const void* dout, float* dk, float* dv, int B, int H, int N, int d,
                float scale, int causal, const unsigned char* blockmask,
                const void* workspace, size_t workspace_bytes, void* stream);
int fa_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
              const void* dout, float* dq, int B, int H, int N, int d, float scale,
              int causal, const unsigned char* blockmask, const void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * Forward and backward with dropout on the attention probabilities, bf16
 * (the dropout stage of the fused kernel in the figure of "Flashattention
 * fast and memory efficient exact attention with io awareness"):
 *   O = (P o Z) V / (1 - p_drop),  P = softmax(scale * Q K^T, masked),
 * lse = the logsumexp of the undropped scores (as for fa_fwd).  Z_ij is 1
 * (kept) when word (j mod 4) of Philox-4x32-10 (Salmon et al., "Parallel
 * random numbers: as easy as 1, 2, 3", SC 2011) at counter
 * (j / 4, i, b*H + h, 0) and key (seed mod 2^32, seed / 2^32) is at least
 * floor(p_drop * 2^32); i is the query and j the key index within the head.
 * The mask is regenerated, never stored: fa_bwd_dropout must get the same
 * p_drop and seed as the forward that produced o and lse, and computes the
 * exact gradient for that mask (dV = (P o Z)^T dO / (1 - p),
 * dP = (dO V^T) o Z / (1 - p), dS = P o (dP - D)).  Other arguments,
 * layouts, ownership and errors as for fa_fwd / fa_bwd; p_drop must lie in
 * [0, 1) (else FA_ERR_DROPOUT).  p_drop = 0 gives exactly fa_fwd / fa_bwd.
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   const unsigned char* blockmask, float p_drop,
                   unsigned long long seed, void* stream);
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, float* dq, float* dk, float* dv,
                   int B, int H, int N, int d, float scale, int causal,
                   const unsigned char* blockmask, float p_drop, unsigned long long seed,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode: Nq new queries per (batch, head) against a cache of Nk keys and
 * values (Flash-Decoding, named on the aggregator page "Flashattention fast
 * and memory efficient exact attention with io awareness").  q: bf16
 * [B,H,Nq,d]; k, v: bf16 [B,H,Nk,d]; o: bf16 [B,H,Nq,d]; lse: fp32 [B,H,Nq].
 * Computes O = softmax(scale * Q K^T) V.  With causal = 1, query i is
 * sequence position i + Nk - Nq and sees keys j <= i + Nk - Nq (a query
 * with no visible key gets O = 0, lse = -inf).  The keys are split into
 * chunks processed in parallel and the partial results merged exactly
 * (lse = log sum exp of the parts).  workspace: device memory of at least
 * fa_decode_workspace_bytes(B,H,Nq,Nk,d) bytes, 16-byte aligned, holding
 * the fp32 partials; contents on entry ignored, on exit unspecified.  No
 * block mask.  Any Nq, Nk >= 1; errors as for fa_fwd, plus FA_ERR_WORKSPACE.
 */
int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Nq, int Nk, int d, float scale, int causal,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace fa_fwd_decode needs (0 for invalid sizes). */
size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d);

/* Bytes of workspace fa_bwd and fa_bwd_f32 need (0 for invalid sizes). */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/* Query rows per workgroup (the outer tile height Br) of the kernel that
 * fa_fwd (dropout = 0) or fa_fwd_dropout with p_drop > 0 (dropout = 1)
 * launches for these sizes: 128, 256 or 384.  The tiled algorithm reads K
 * and V once per query tile of Br rows ("Tiling", FlashAttention summary
 * page, §3 Method), so this fixes the no-reuse IO term of a call.  Host
 * only: no HIP call, no state.  Returns 0 for sizes or flags fa_fwd rejects
 * (flags must be 0 or 1). */
int fa_fwd_query_rows(int B, int H, int N, int d, int causal, int has_blockmask, int dropout);

/* Forward with fp32 tensors throughout (fp32 arithmetic, fp32 O and lse). */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o,
               float* lse, int B, int H, int N, int d, float scale,
               int causal, const unsigned char* blockmask, void* stream);

/* Backward with fp32 tensors throughout.  Arguments as for fa_bwd. */
int fa_bwd_f32(const float* q, const float* k, const float* v,
               const float* o, const float* lse, const float* dout,
               float* dq, float* dk, float* dv, int B, int H, int N, int d,
               float scale, int causal, const unsigned char* blockmask,
               void* workspace, size_t workspace_bytes, void* stream);

/* Static English text for a status code (never NULL). */
const char* fa_strerror(int status);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
