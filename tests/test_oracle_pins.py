"""Pins for the fp64 oracle: every check here comes from something other than
the oracle's own formulas (closed forms, hand-derived values, brute force,
finite differences, an independent library implementation, invariants).

Each pin is chosen so that a plausible mistake in the oracle fails it:
a dropped D term or a transposed operand fails the finite differences, a
wrong causal convention fails the brute force and row-0 checks, a transposed
block mask fails the asymmetric-mask reduction, a wrong lse base fails the
identical-keys closed form.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (
    attention_bwd,
    attention_dkdv_rows,
    attention_dq_rows,
    attention_fwd,
    attention_fwd_rows,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def rnd(*shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- golden ----
@pytest.mark.parametrize("variant", ["dense", "causal"])
def test_hand_derived_two_keys(variant):
    g = json.load(open(os.path.join(GOLDEN, "hand_two_keys.json")))
    inp = g["inputs"]
    q, k, v, do = (np.array(inp[n])[None, None] for n in ("q", "k", "v", "do"))
    causal = variant == "causal"
    o, lse = attention_fwd(q, k, v, inp["scale"], causal)
    dq, dk, dv = attention_bwd(q, k, v, do, inp["scale"], causal)
    exp = g[variant]
    np.testing.assert_allclose(o[0, 0], exp["o"], atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], exp["lse"], atol=1e-14)
    np.testing.assert_allclose(dq[0, 0], exp["dq"], atol=1e-14)
    np.testing.assert_allclose(dk[0, 0], exp["dk"], atol=1e-14)
    np.testing.assert_allclose(dv[0, 0], exp["dv"], atol=1e-14)


# ------------------------------------------------------- closed forms (fwd) --
@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(causal):
    N, d, scale = 37, 8, 0.3
    q = rnd(1, 2, N, d)
    kvec = rnd(d)
    k = np.broadcast_to(kvec, (1, 2, N, d)).copy()
    v = rnd(1, 2, N, d)
    o, lse = attention_fwd(q, k, v, scale, causal)
    for i in range(N):
        n_vis = i + 1 if causal else N
        np.testing.assert_allclose(o[:, :, i], v[:, :, :n_vis].mean(axis=2), atol=1e-12)
        np.testing.assert_allclose(lse[:, :, i], scale * q[:, :, i] @ kvec + math.log(n_vis), atol=1e-12)


def test_identical_keys_with_block_mask():
    # rows of block 1 see key blocks {0, 1}; rows of block 0 see only block 0
    N, d, scale = 200, 4, 0.5
    mask = np.array([[1, 0], [1, 1]], dtype=np.uint8)
    q = rnd(1, 1, N, d)
    kvec = rnd(d)
    k = np.broadcast_to(kvec, (1, 1, N, d)).copy()
    v = rnd(1, 1, N, d)
    o, lse = attention_fwd(q, k, v, scale, False, mask)
    np.testing.assert_allclose(o[0, 0, :128], np.broadcast_to(v[0, 0, :128].mean(0), (128, d)), atol=1e-12)
    np.testing.assert_allclose(o[0, 0, 128:], np.broadcast_to(v[0, 0].mean(0), (72, d)), atol=1e-12)
    np.testing.assert_allclose(lse[0, 0, :128], scale * q[0, 0, :128] @ kvec + math.log(128), atol=1e-12)
    np.testing.assert_allclose(lse[0, 0, 128:], scale * q[0, 0, 128:] @ kvec + math.log(200), atol=1e-12)


def test_dominant_logit_selects_its_row():
    N, d = 16, 4
    q = np.zeros((1, 1, N, d))
    q[..., 0] = 10.0
    k = 0.01 * rnd(1, 1, N, d)
    jstar = 5
    k[0, 0, jstar] = [10.0, 0, 0, 0]
    v = rnd(1, 1, N, d)
    o, lse = attention_fwd(q, k, v, 1.0, False)
    s = q[0, 0] @ k[0, 0].T
    gap = 100.0 - np.sort(s[0])[-2]
    assert gap > 50
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, jstar], (N, d)), atol=N * math.exp(-gap) * 10)
    np.testing.assert_allclose(lse[0, 0], 100.0, atol=N * math.exp(-gap))


@pytest.mark.parametrize("causal,masked", [(False, False), (True, False), (False, True)])
def test_probabilities_are_a_distribution(causal, masked):
    # With V = I (d = N) the output row is the probability row itself.
    N = 160
    q = rnd(1, 1, N, 6)
    k = rnd(1, 1, N, 6)
    v = np.eye(N)[None, None]
    mask = np.array([[1, 0], [1, 1]], dtype=np.uint8) if masked else None
    # pad q/k to width N so shapes agree; extra columns are zero
    qp = np.zeros((1, 1, N, N)); qp[..., :6] = q
    kp = np.zeros((1, 1, N, N)); kp[..., :6] = k
    o, _ = attention_fwd(qp, kp, v, 0.7, causal, mask)
    P = o[0, 0]
    assert (P >= 0).all()
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-13)
    i, j = np.meshgrid(np.arange(N), np.arange(N), indexing="ij")
    forbidden = np.zeros((N, N), dtype=bool)
    if causal:
        forbidden |= j > i
    if masked:
        forbidden |= (i < 128) & (j >= 128)
    assert (P[forbidden] == 0).all()


def test_row_constant_shift():
    # Adding c_i to every score of row i leaves O unchanged and adds c_i to lse.
    N, d, scale = 50, 8, 0.25
    q = rnd(1, 1, N, d)
    k = rnd(1, 1, N, d)
    v = rnd(1, 1, N, d)
    c = 3.0 * rnd(N)
    qa = np.concatenate([q, (c / scale)[None, None, :, None]], axis=-1)
    ka = np.concatenate([k, np.ones((1, 1, N, 1))], axis=-1)
    for causal in (False, True):
        o0, l0 = attention_fwd(q, k, v, scale, causal)
        va = np.concatenate([v, np.zeros((1, 1, N, 1))], axis=-1)
        o1, l1 = attention_fwd(qa, ka, va, scale, causal)
        np.testing.assert_allclose(o1[..., :d], o0, atol=1e-12)
        np.testing.assert_allclose(l1, l0 + c, atol=1e-12)


def test_single_key():
    q, k, v, do = rnd(1, 3, 1, 5), rnd(1, 3, 1, 5), rnd(1, 3, 1, 5), rnd(1, 3, 1, 5)
    o, lse = attention_fwd(q, k, v, 0.4)
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse, 0.4 * (q * k).sum(-1), atol=1e-14)
    dq, dk, dv = attention_bwd(q, k, v, do, 0.4)
    np.testing.assert_allclose(dq, 0, atol=1e-15)
    np.testing.assert_allclose(dk, 0, atol=1e-15)
    np.testing.assert_allclose(dv, do, atol=1e-15)


def test_causal_row_zero_and_constant_v():
    N, d = 20, 4
    q, k, v, do = rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d)
    o, lse = attention_fwd(q, k, v, 0.5, True)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 0], 0.5 * q[0, 0, 0] @ k[0, 0, 0], atol=1e-14)
    vc = np.broadcast_to(rnd(d), (1, 1, N, d)).copy()
    for causal in (False, True):
        o, _ = attention_fwd(q, k, vc, 0.5, causal)
        np.testing.assert_allclose(o, vc, atol=1e-13)
        dq, dk, dv = attention_bwd(q, k, vc, do, 0.5, causal)
        np.testing.assert_allclose(dq, 0, atol=1e-13)
        np.testing.assert_allclose(dk, 0, atol=1e-13)


def test_all_ones_mask_is_dense_and_diagonal_mask_is_blockwise():
    N, d = 300, 4
    q, k, v, do = rnd(2, 1, N, d), rnd(2, 1, N, d), rnd(2, 1, N, d), rnd(2, 1, N, d)
    ones = np.ones((3, 3), dtype=np.uint8)
    for causal in (False, True):
        a = attention_fwd(q, k, v, 0.5, causal)
        b = attention_fwd(q, k, v, 0.5, causal, ones)
        np.testing.assert_allclose(a[0], b[0], atol=1e-14)
        np.testing.assert_allclose(a[1], b[1], atol=1e-14)
        ga = attention_bwd(q, k, v, do, 0.5, causal)
        gb = attention_bwd(q, k, v, do, 0.5, causal, ones)
        for x, y in zip(ga, gb):
            np.testing.assert_allclose(x, y, atol=1e-13)
    diag = np.eye(3, dtype=np.uint8)
    o, lse = attention_fwd(q, k, v, 0.5, False, diag)
    dq, dk, dv = attention_bwd(q, k, v, do, 0.5, False, diag)
    for s in range(0, N, 128):
        e = min(N, s + 128)
        ob, lb = attention_fwd(q[:, :, s:e], k[:, :, s:e], v[:, :, s:e], 0.5)
        np.testing.assert_allclose(o[:, :, s:e], ob, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, s:e], lb, atol=1e-14)
        gq, gk, gv = attention_bwd(q[:, :, s:e], k[:, :, s:e], v[:, :, s:e], do[:, :, s:e], 0.5)
        np.testing.assert_allclose(dq[:, :, s:e], gq, atol=1e-13)
        np.testing.assert_allclose(dk[:, :, s:e], gk, atol=1e-13)
        np.testing.assert_allclose(dv[:, :, s:e], gv, atol=1e-13)


def test_asymmetric_mask_reduces_to_prefix_attention():
    # mask [[1,0],[1,1]]: block-0 rows attend keys [0,128); block-1 rows
    # attend every key.  A transposed mask would swap these.
    N, d = 256, 3
    q, k, v, do = rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d)
    mask = np.array([[1, 0], [1, 1]], dtype=np.uint8)
    o, lse = attention_fwd(q, k, v, 0.6, False, mask)
    o0, l0 = attention_fwd(q[:, :, :128], k[:, :, :128], v[:, :, :128], 0.6)
    np.testing.assert_allclose(o[:, :, :128], o0, atol=1e-14)
    np.testing.assert_allclose(lse[:, :, :128], l0, atol=1e-14)
    o1, l1 = attention_fwd(q, k, v, 0.6, False)
    np.testing.assert_allclose(o[:, :, 128:], o1[:, :, 128:], atol=1e-14)
    np.testing.assert_allclose(lse[:, :, 128:], l1[:, :, 128:], atol=1e-14)


def test_empty_rows_are_zero_not_nan():
    N, d = 200, 4
    q, k, v, do = rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d)
    mask = np.array([[0, 0], [1, 1]], dtype=np.uint8)  # block-0 rows see nothing
    o, lse = attention_fwd(q, k, v, 0.5, False, mask)
    assert np.all(o[:, :, :128] == 0) and np.all(np.isneginf(lse[:, :, :128]))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse[:, :, 128:]))
    dq, dk, dv = attention_bwd(q, k, v, do, 0.5, False, mask)
    assert np.all(dq[:, :, :128] == 0)
    assert all(np.all(np.isfinite(x)) for x in (dq, dk, dv))


# ------------------------------------------------------------ brute force ----
def _brute_fwd(q, k, v, scale, causal, mask):
    """Scalar loops with math.exp, tiny inputs only."""
    N, d = len(q), len(q[0])
    o = [[0.0] * d for _ in range(N)]
    lse = [0.0] * N
    for i in range(N):
        s = []
        for j in range(N):
            ok = (not causal or j <= i) and (mask is None or mask[i // 128][j // 128])
            if ok:
                s.append((j, scale * sum(q[i][c] * k[j][c] for c in range(d))))
        if not s:
            lse[i] = -math.inf
            continue
        m = max(x for _, x in s)
        den = sum(math.exp(x - m) for _, x in s)
        lse[i] = m + math.log(den)
        for j, x in s:
            p = math.exp(x - m) / den
            for c in range(d):
                o[i][c] += p * v[j][c]
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_with_block_mask(causal):
    N, d = 260, 2
    q, k, v = rnd(N, d), rnd(N, d), rnd(N, d)
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    ob, lb = _brute_fwd(q.tolist(), k.tolist(), v.tolist(), 0.8, causal, mask.tolist())
    o, lse = attention_fwd(q[None, None], k[None, None], v[None, None], 0.8, causal, mask)
    np.testing.assert_allclose(o[0, 0], ob, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], lb, atol=1e-12)


# ------------------------------------------------------ finite differences --
def _loss(q, k, v, do, scale, causal, mask):
    o, _ = attention_fwd(q, k, v, scale, causal, mask)
    return float((o * do).sum())


def _fd_grad(x, f, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        xp = x.copy(); xp[idx] += h
        xm = x.copy(); xm[idx] -= h
        g[idx] = (f(xp) - f(xm)) / (2 * h)
    return g


CASES = [(N, d, c) for N in (1, 2, 3, 5, 8) for d in (1, 2, 4) for c in (False, True)]


@pytest.mark.parametrize("N,d,causal", CASES)
def test_finite_differences(N, d, causal):
    q, k, v, do = rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d)
    scale = 0.9
    dq, dk, dv = attention_bwd(q, k, v, do, scale, causal)
    fq = _fd_grad(q, lambda x: _loss(x, k, v, do, scale, causal, None))
    fk = _fd_grad(k, lambda x: _loss(q, x, v, do, scale, causal, None))
    fv = _fd_grad(v, lambda x: _loss(q, k, x, do, scale, causal, None))
    for a, f in ((dq, fq), (dk, fk), (dv, fv)):
        err = np.abs(a - f).max()
        ref = max(1.0, np.abs(f).max())
        assert err <= 1e-6 * ref, err


def test_finite_differences_block_mask():
    N, d = 200, 2
    q, k, v, do = rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d)
    mask = np.array([[1, 1], [0, 1]], dtype=np.uint8)
    scale = 0.7
    dq, dk, dv = attention_bwd(q, k, v, do, scale, True, mask)
    # a subset of coordinates keeps the cost bounded
    sel = [0, 1, 63, 127, 128, 129, 150, 199]
    for name, x, a in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for i in sel:
            for c in range(d):
                xp = x.copy(); xp[0, 0, i, c] += 1e-6
                xm = x.copy(); xm[0, 0, i, c] -= 1e-6
                args = {"q": q, "k": k, "v": v}
                fp = _loss(*(xp if n == name else args[n] for n in "qkv"), do, scale, True, mask)
                fm = _loss(*(xm if n == name else args[n] for n in "qkv"), do, scale, True, mask)
                fd = (fp - fm) / 2e-6
                assert abs(fd - a[0, 0, i, c]) <= 1e-6 * max(1.0, abs(fd)), (name, i, c)


# ------------------------------------------------- independent library ------
@pytest.mark.parametrize("causal,masked", [(False, False), (True, False), (False, True), (True, True)])
def test_torch_sdpa_fp64_cross_check(causal, masked):
    B, H, N, d = 2, 2, 200, 8
    q, k, v, do = rnd(B, H, N, d), rnd(B, H, N, d), rnd(B, H, N, d), rnd(B, H, N, d)
    scale = 0.35
    mask = np.array([[1, 0], [1, 1]], dtype=np.uint8) if masked else None
    o, lse = attention_fwd(q, k, v, scale, causal, mask)
    dq, dk, dv = attention_bwd(q, k, v, do, scale, causal, mask)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    am = torch.ones(N, N, dtype=torch.bool)
    if causal:
        am &= torch.tril(torch.ones(N, N, dtype=torch.bool))
    if masked:
        bm = torch.tensor(mask, dtype=torch.bool)
        idx = torch.arange(N) // 128
        am &= bm[idx[:, None], idx[None, :]]
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, scale=scale)
    to.backward(torch.tensor(do))
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)
    # lse against torch.logsumexp over the masked score matrix
    s = scale * torch.tensor(q) @ torch.tensor(k).transpose(-1, -2)
    s = s.masked_fill(~am, -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


# -------------------------------------------------------------- invariants --
@pytest.mark.parametrize("causal,masked", [(False, False), (True, False), (False, True)])
def test_gradient_invariants(causal, masked):
    B, H, N, d = 1, 2, 300, 8
    q, k, v, do = rnd(B, H, N, d), rnd(B, H, N, d), rnd(B, H, N, d), rnd(B, H, N, d)
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8) if masked else None
    dq, dk, dv = attention_bwd(q, k, v, do, 0.5, causal, mask)
    np.testing.assert_allclose(dk.sum(axis=2), 0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    np.testing.assert_allclose((q * dq).sum(axis=(2, 3)), (k * dk).sum(axis=(2, 3)), atol=1e-11)


def test_forward_bounds_and_permutation():
    B, H, N, d = 1, 1, 150, 5
    q, k, v = rnd(B, H, N, d), rnd(B, H, N, d), rnd(B, H, N, d)
    o, lse = attention_fwd(q, k, v, 0.5, True)
    S = 0.5 * q[0, 0] @ k[0, 0].T
    for i in range(N):
        vis = v[0, 0, : i + 1]
        assert np.all(o[0, 0, i] >= vis.min(0) - 1e-12) and np.all(o[0, 0, i] <= vis.max(0) + 1e-12)
        smax = S[i, : i + 1].max()
        assert smax - 1e-12 <= lse[0, 0, i] <= smax + math.log(i + 1) + 1e-12
    perm = rng.permutation(N)
    o1, l1 = attention_fwd(q, k, v, 0.5, False)
    o2, l2 = attention_fwd(q, k[:, :, perm], v[:, :, perm], 0.5, False)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    o3, l3 = attention_fwd(q[:, :, perm], k, v, 0.5, False)
    np.testing.assert_allclose(o3, o1[:, :, perm], atol=1e-13)


def test_causal_row_is_prefix_attention():
    N, d = 40, 3
    q, k, v = rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d)
    o, lse = attention_fwd(q, k, v, 0.5, True)
    for i in (0, 1, 7, 39):
        op, lp = attention_fwd(q[:, :, i:i + 1], k[:, :, : i + 1], v[:, :, : i + 1], 0.5, False)
        np.testing.assert_allclose(o[:, :, i], op[:, :, 0], atol=1e-14)
        np.testing.assert_allclose(lse[:, :, i], lp[:, :, 0], atol=1e-14)


# ------------------------------------------ sampled-row variants agree ------
@pytest.mark.parametrize("causal,masked", [(False, False), (True, False), (False, True), (True, True)])
def test_row_variants_match_full(causal, masked):
    B, H, N, d = 2, 2, 300, 4
    q, k, v, do = rnd(B, H, N, d), rnd(B, H, N, d), rnd(B, H, N, d), rnd(B, H, N, d)
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8) if masked else None
    o, lse = attention_fwd(q, k, v, 0.5, causal, mask)
    dq, dk, dv = attention_bwd(q, k, v, do, 0.5, causal, mask)
    b = np.array([0, 0, 1, 1, 1, 0])
    h = np.array([0, 1, 0, 1, 1, 1])
    i = np.array([0, 299, 128, 127, 5, 200])
    o_r, l_r = attention_fwd_rows(q, k, v, 0.5, causal, mask, b, h, i)
    np.testing.assert_allclose(o_r, o[b, h, i], atol=1e-13)
    np.testing.assert_allclose(l_r, lse[b, h, i], atol=1e-13)
    dq_r = attention_dq_rows(q, k, v, do, 0.5, causal, mask, b, h, i)
    np.testing.assert_allclose(dq_r, dq[b, h, i], atol=1e-12)
    dk_r, dv_r = attention_dkdv_rows(q, k, v, do, 0.5, causal, mask, b, h, i)
    np.testing.assert_allclose(dk_r, dk[b, h, i], atol=1e-12)
    np.testing.assert_allclose(dv_r, dv[b, h, i], atol=1e-12)
