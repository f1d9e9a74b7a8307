"""Attention with dropout on the attention probabilities: float64 CPU oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Shares no code with the
HIP path.

The fused kernel of the aggregator page "Flashattention fast and memory
efficient exact attention with io awareness" includes dropout between the
softmax and the second product (its figure: "Matmul Mask Softmax Dropout
Matmul" fused into one kernel), and its memory note says the footprint is the
same with or without dropout.  The pages give no formula; the plainest reading,
and the one written out here, is inverted dropout applied to the normalised
probabilities:

  P    = softmax(S)            (as in oracle/attention.py, lse unchanged)
  Z_ij in {0, 1}, kept with probability 1 - p
  O    = (P o Z) V / (1 - p)

Backward, the exact gradient of that function for a fixed Z:

  dV   = (P o Z)^T dO / (1 - p)
  dP   = (dO V^T) o Z / (1 - p)
  D_i  = sum_j P_ij dP_ij            (= dO_i . O_i)
  dS   = P o (dP - D 1^T)
  dQ   = scale * dS K,   dK = scale * dS^T Q

Z is a pure function of (seed, batch*H + head, i, j), so the backward
regenerates it instead of storing it.  The generator is Philox-4x32 with 10
rounds (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC 2011), written here from that definition:

  round: (hi0, lo0) = M0 * c0, (hi1, lo1) = M1 * c2   (32x32 -> 64-bit)
         c' = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
  key schedule between rounds: k0 += W0, k1 += W1
  M0 = 0xD2511F53, M1 = 0xCD9E8D57, W0 = 0x9E3779B9, W1 = 0xBB67AE85

Keep rule (a choice of this library, the same on both sides):
  key     = (seed mod 2^32, seed div 2^32)
  counter = (j div 4, i, b*H + h, 0)
  word    = output word (j mod 4) of Philox(counter, key)
  T       = floor(p * 2^32) with p the float32 value passed, clamped to 2^32-1
  Z_ij    = 1 if word >= T else 0
so p = 0 keeps everything.
"""
from __future__ import annotations

import numpy as np

from .attention import _as64, _check_shapes, _probs, _row_groups

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Philox-4x32-10 of uint32 counters [..., 4] under key (k0, k1)."""
    c = np.asarray(counter, dtype=np.uint64) & _MASK32
    c0, c1, c2, c3 = (c[..., t].copy() for t in range(4))
    k0, k1 = int(key[0]) & _MASK32, int(key[1]) & _MASK32
    for r in range(10):
        if r > 0:
            k0 = (k0 + PHILOX_W0) & _MASK32
            k1 = (k1 + PHILOX_W1) & _MASK32
        p0 = c0 * np.uint64(PHILOX_M0)
        p1 = c2 * np.uint64(PHILOX_M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(_MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(_MASK32)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0)
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def drop_threshold(p) -> int:
    """T = floor(p * 2^32) for the float32 value of p, clamped to 2^32 - 1."""
    pf = float(np.float32(p))
    if not (0.0 <= pf < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min(int(np.floor(pf * 4294967296.0)), _MASK32)


def keep_mask(bh: int, rows, cols, p, seed: int) -> np.ndarray:
    """Z for query rows x key cols of head bh (= b*H + h)."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    T = drop_threshold(p)
    if rows.size == 0 or cols.size == 0:
        return np.ones((rows.size, cols.size), dtype=bool)
    groups = np.unique(cols // 4)
    ctr = np.zeros((rows.size, groups.size, 4), dtype=np.uint64)
    ctr[..., 0] = groups[None, :]
    ctr[..., 1] = rows[:, None]
    ctr[..., 2] = bh
    words = philox4x32_10(ctr, (seed & _MASK32, (seed >> 32) & _MASK32))
    gi = np.searchsorted(groups, cols // 4)
    w = words[:, gi, cols % 4]
    return w >= np.uint32(T) if T > 0 else np.ones(w.shape, dtype=bool)


def _keep_scale(p) -> float:
    return 1.0 / (1.0 - float(np.float32(p)))


def attention_fwd_dropout(q, k, v, scale, causal, mask, p, seed):
    """O [B,H,N,dv] and lse [B,H,N] with dropout on P."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    _check_shapes(q, k, v)
    B, H, N = q.shape[:3]
    mask = None if mask is None else np.asarray(mask)
    ks = _keep_scale(p)
    o = np.zeros((B, H, N, v.shape[3]))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for g in _row_groups(np.arange(N), mask):
                P, l_, cols = _probs(q[b, h], k[b, h], scale, g, causal, mask)
                Z = keep_mask(b * H + h, g, cols, p, seed)
                o[b, h, g] = ks * ((P * Z) @ v[b, h, cols])
                lse[b, h, g] = l_
    return o, lse


def attention_bwd_dropout(q, k, v, do, scale, causal, mask, p, seed):
    """dQ, dK, dV [B,H,N,d] of L = sum(dO * O) for the dropout forward."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    _check_shapes(q, k, v)
    B, H, N, d = q.shape
    mask = None if mask is None else np.asarray(mask)
    ks = _keep_scale(p)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = q[b, h], k[b, h], v[b, h], do[b, h]
            for g in _row_groups(np.arange(N), mask):
                P, _, cols = _probs(qh, kh, scale, g, causal, mask)
                Z = keep_mask(b * H + h, g, cols, p, seed)
                dP = ks * Z * (doh[g] @ vh[cols].T)
                Dg = (P * dP).sum(axis=1)
                dS = P * (dP - Dg[:, None])
                dq[b, h, g] = scale * (dS @ kh[cols])
                dk[b, h, cols] += scale * (dS.T @ qh[g])
                dv[b, h, cols] += ks * ((P * Z).T @ doh[g])
    return dq, dk, dv
