"""Plain float64 attention on the CPU: the oracle for the HIP library.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP path
and imports nothing from it.

What it computes is the plain definition of scaled-dot-product attention,
written out without tiling or online softmax.  FlashAttention's claim is that
its tiled algorithm reaches exactly this result ("exact attention", abstract of
"FlashAttention: Fast and Memory-Efficient Exact Attention with
IO-Awareness"; "numerically exact", §5 Conclusion of the same paper's
summary page), so the definition itself is the thing to compare against.

Per head, with 0-based indices and the same input values the GPU receives
(bf16 -> float64 and fp32 -> float64 are exact):

  S   = scale * Q K^T                          (§2 Background: standard
                                                attention materialises S and P)
  A_ij = [causal => j <= i] and [mask => M[i // 128][j // 128] != 0]
  S_ij = -inf where A_ij is false
  m_i = max_j S_ij,  l_i = sum_j exp(S_ij - m_i)
  P   = exp(S - m) / l,   lse_i = m_i + ln l_i   (the per-row statistic the
                                                backward keeps, §3 Method,
                                                "Softmax rescaling /
                                                recomputation")
  O   = P V

Backward (the exact gradient of the same function; the pages state only that
the backward recomputes P from the stored statistics, §3 Method):

  dV = P^T dO
  dP = dO V^T
  D_i = sum_j P_ij dP_ij
  dS = P o (dP - D 1^T)
  dQ = scale * dS K
  dK = scale * dS^T Q

Readings where the pages are silent (each listed in the design notes):
  * lse uses the natural log of the scaled scores.
  * causal keeps the diagonal (j <= i).
  * causal and a block mask combine by AND.
  * the block mask is uint8 [ceil(N/128)]^2, row = query block, shared by all
    (batch, head); the last block covers the remainder when N % 128 != 0.
  * a row with no allowed key has O = 0, lse = -inf and zero gradients.

Masked entries contribute exp(-inf) = 0, so the code evaluates each row only
over the key columns whose 128-block the mask allows; this is the definition,
not a reordering of it.
"""
from __future__ import annotations

import numpy as np

MASK_BLOCK = 128
_ROW_CHUNK = 256


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _candidate_cols(rows: np.ndarray, N: int, causal: bool, mask) -> np.ndarray:
    """Key columns that may be allowed for any row of `rows` (block level)."""
    hi = N
    if causal:
        hi = int(rows.max()) + 1
    if mask is None:
        return np.arange(hi)
    blocks = np.unique(rows // MASK_BLOCK)
    allowed_blocks = np.nonzero(np.any(mask[blocks] != 0, axis=0))[0]
    if allowed_blocks.size == 0:
        return np.zeros(0, dtype=np.int64)
    cols = (allowed_blocks[:, None] * MASK_BLOCK + np.arange(MASK_BLOCK)[None, :]).reshape(-1)
    return cols[cols < hi]


def allowed(rows: np.ndarray, cols: np.ndarray, causal: bool, mask) -> np.ndarray:
    """A_ij for the given row and column index vectors."""
    a = np.ones((rows.size, cols.size), dtype=bool)
    if causal:
        a &= cols[None, :] <= rows[:, None]
    if mask is not None:
        a &= mask[(rows // MASK_BLOCK)[:, None], (cols // MASK_BLOCK)[None, :]] != 0
    return a


def _row_groups(rows: np.ndarray, mask):
    """Split sorted row indices into groups evaluated together."""
    if rows.size == 0:
        return
    if mask is not None:
        blk = rows // MASK_BLOCK
        cuts = np.nonzero(np.diff(blk))[0] + 1
        for g in np.split(rows, cuts):
            yield g
    else:
        for s in range(0, rows.size, _ROW_CHUNK):
            yield rows[s:s + _ROW_CHUNK]


def _probs(q, k, scale, rows, causal, mask):
    """P (normalised), lse and the column set for one group of rows of a head."""
    N = k.shape[0]
    cols = _candidate_cols(rows, N, causal, mask)
    S = scale * (q[rows] @ k[cols].T)
    A = allowed(rows, cols, causal, mask)
    S = np.where(A, S, -np.inf)
    if cols.size:
        m = S.max(axis=1)
    else:
        m = np.full(rows.size, -np.inf)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    E = np.exp(S - m_safe[:, None])
    l = E.sum(axis=1)
    P = E / np.where(empty, 1.0, l)[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return P, lse, cols


def _check_shapes(q, k, v):
    """q [B,H,Nq,d], k [B,H,Nk,d], v [B,H,Nk,dv]."""
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3] or k.shape[:3] != v.shape[:3]:
        raise ValueError("q, k, v shapes disagree")


def attention_fwd(q, k, v, scale, causal=False, mask=None):
    """O [B,H,N,d] and lse [B,H,N] for every row."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    _check_shapes(q, k, v)
    B, H, N = q.shape[:3]
    mask = None if mask is None else np.asarray(mask)
    o = np.zeros((B, H, N, v.shape[3]))
    lse = np.zeros((B, H, N))
    rows_all = np.arange(N)
    for b in range(B):
        for h in range(H):
            for g in _row_groups(rows_all, mask):
                P, l_, cols = _probs(q[b, h], k[b, h], scale, g, causal, mask)
                o[b, h, g] = P @ v[b, h, cols]
                lse[b, h, g] = l_
    return o, lse


def attention_bwd(q, k, v, do, scale, causal=False, mask=None):
    """dQ, dK, dV [B,H,N,d] for L = sum(dO * O)."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    _check_shapes(q, k, v)
    B, H, N, d = q.shape
    mask = None if mask is None else np.asarray(mask)
    dq = np.zeros_like(q)
    dk = np.zeros_like(q)
    dv = np.zeros_like(q)
    rows_all = np.arange(N)
    for b in range(B):
        for h in range(H):
            qh, kh, vh, doh = q[b, h], k[b, h], v[b, h], do[b, h]
            for g in _row_groups(rows_all, mask):
                P, _, cols = _probs(qh, kh, scale, g, causal, mask)
                dP = doh[g] @ vh[cols].T
                Dg = (P * dP).sum(axis=1)
                dS = P * (dP - Dg[:, None])
                dq[b, h, g] = scale * (dS @ kh[cols])
                dk[b, h, cols] += scale * (dS.T @ qh[g])
                dv[b, h, cols] += P.T @ doh[g]
    return dq, dk, dv


def attention_fwd_rows(q, k, v, scale, causal, mask, b_idx, h_idx, i_idx):
    """O rows and lse at the given (b, h, i) query positions."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    mask = None if mask is None else np.asarray(mask)
    n = len(i_idx)
    o = np.zeros((n, q.shape[-1]))
    lse = np.zeros(n)
    for t in range(n):
        b, h, i = int(b_idx[t]), int(h_idx[t]), int(i_idx[t])
        rows = np.array([i])
        P, l_, cols = _probs(q[b, h], k[b, h], scale, rows, causal, mask)
        o[t] = (P @ v[b, h, cols])[0]
        lse[t] = l_[0]
    return o, lse


def attention_dq_rows(q, k, v, do, scale, causal, mask, b_idx, h_idx, i_idx):
    """dQ rows at the given (b, h, i) query positions (row-local)."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    mask = None if mask is None else np.asarray(mask)
    out = np.zeros((len(i_idx), q.shape[-1]))
    for t in range(len(i_idx)):
        b, h, i = int(b_idx[t]), int(h_idx[t]), int(i_idx[t])
        rows = np.array([i])
        P, _, cols = _probs(q[b, h], k[b, h], scale, rows, causal, mask)
        dP = do[b, h, rows] @ v[b, h, cols].T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        out[t] = scale * (dS @ k[b, h, cols])[0]
    return out


def attention_dkdv_rows(q, k, v, do, scale, causal, mask, b_idx, h_idx, j_idx):
    """dK and dV rows at the given (b, h, j) key positions.

    dK_j and dV_j sum over every query row i that attends to key j, so each
    such row's full softmax (its lse and D_i) is evaluated here.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    mask = None if mask is None else np.asarray(mask)
    B, H, N, d = q.shape
    n = len(j_idx)
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    b_idx = np.asarray(b_idx)
    h_idx = np.asarray(h_idx)
    j_idx = np.asarray(j_idx)
    for bh in sorted(set(zip(b_idx.tolist(), h_idx.tolist()))):
        b, h = bh
        sel = np.nonzero((b_idx == b) & (h_idx == h))[0]
        keys = j_idx[sel]
        # query rows that may attend to any of these keys
        rows = np.arange(N)
        if causal:
            rows = rows[rows >= keys.min()]
        if mask is not None:
            kb = np.unique(keys // MASK_BLOCK)
            qb_ok = np.any(mask[:, kb] != 0, axis=1)
            rows = rows[qb_ok[rows // MASK_BLOCK]]
        qh, kh, vh, doh = q[b, h], k[b, h], v[b, h], do[b, h]
        for g in _row_groups(rows, mask):
            P, _, cols = _probs(qh, kh, scale, g, causal, mask)
            if cols.size == 0:
                continue
            dP = doh[g] @ vh[cols].T
            Dg = (P * dP).sum(axis=1)
            dS = P * (dP - Dg[:, None])
            pos = np.searchsorted(cols, keys)
            hit = (pos < cols.size) & (cols[np.minimum(pos, cols.size - 1)] == keys)
            for s_local, (t, ok) in enumerate(zip(sel, hit)):
                if not ok:
                    continue
                c = pos[s_local]
                dv[t] += P[:, c] @ doh[g]
                dk[t] += scale * (dS[:, c] @ qh[g])
    return dk, dv
