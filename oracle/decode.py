"""Attention of a few new queries against a long key/value cache: float64 CPU
oracle for the decode path.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Shares no code with the
HIP path.

The aggregator page "Flashattention fast and memory efficient exact attention
with io awareness" names Flash-Decoding for long-context inference; the
result it computes is plain attention with Nq queries and Nk >= 1 keys per
head, which is what is written out here:

  S = scale * Q K^T              (Nq x Nk)
  causal: query i sits at sequence position i + (Nk - Nq), the last Nq
          positions of the cache, and sees key j iff j <= i + (Nk - Nq)
  P = softmax over the allowed keys,  lse_i = ln sum_j exp(S_ij)
  O = P V

A query with no allowed key (causal with Nq > Nk) gets O = 0, lse = -inf.
How the keys are split among workgroups and merged back is not part of the
result (the merge is exact: lse = logsumexp of the parts, O = sum of the
parts weighted by exp(lse_part - lse)).
"""
from __future__ import annotations

import numpy as np

_ROWS = 64


def attention_fwd_decode(q, k, v, scale, causal=False):
    """O [B,H,Nq,dv] and lse [B,H,Nq] for q [B,H,Nq,d], k [B,H,Nk,d], v [B,H,Nk,dv]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3] or v.shape[:3] != k.shape[:3]:
        raise ValueError("q [B,H,Nq,d], k [B,H,Nk,d], v [B,H,Nk,dv] expected")
    B, H, Nq, _ = q.shape
    Nk = k.shape[2]
    off = Nk - Nq
    o = np.zeros((B, H, Nq, v.shape[3]))
    lse = np.full((B, H, Nq), -np.inf)
    cols = np.arange(Nk)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, _ROWS):
                rows = np.arange(r0, min(Nq, r0 + _ROWS))
                S = scale * (q[b, h, rows] @ k[b, h].T)
                if causal:
                    S = np.where(cols[None, :] <= rows[:, None] + off, S, -np.inf)
                m = S.max(axis=1)
                ok = np.isfinite(m)
                if not ok.any():
                    continue
                E = np.exp(S[ok] - m[ok, None])
                l = E.sum(axis=1)
                o[b, h, rows[ok]] = (E / l[:, None]) @ v[b, h]
                lse[b, h, rows[ok]] = m[ok] + np.log(l)
    return o, lse
