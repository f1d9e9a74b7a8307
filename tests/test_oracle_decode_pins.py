"""Pins for the decode oracle (oracle/decode.py): it must agree with the
pinned full-attention oracle where the two overlap (Nq = Nk; the last Nq rows
of a causal prefill), with PyTorch's float64 scaled_dot_product_attention
under an explicit mask, and with closed forms (one key; identical keys)."""
import numpy as np
import pytest
import torch

from oracle import attention_fwd
from oracle.decode import attention_fwd_decode

rng = np.random.default_rng(99)


def rnd(*shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_full_attention(causal):
    q, k, v = rnd(2, 3, 40, 8), rnd(2, 3, 40, 8), rnd(2, 3, 40, 8)
    o, lse = attention_fwd_decode(q, k, v, 0.3, causal)
    o2, lse2 = attention_fwd(q, k, v, 0.3, causal)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)


@pytest.mark.parametrize("nq", [1, 3, 17])
def test_causal_decode_is_the_tail_of_a_causal_prefill(nq):
    nk = 50
    k, v = rnd(1, 2, nk, 8), rnd(1, 2, nk, 8)
    qfull = rnd(1, 2, nk, 8)
    o, lse = attention_fwd_decode(qfull[:, :, nk - nq:], k, v, 0.4, True)
    of, lsef = attention_fwd(qfull, k, v, 0.4, True)
    np.testing.assert_allclose(o, of[:, :, nk - nq:], atol=1e-13)
    np.testing.assert_allclose(lse, lsef[:, :, nk - nq:], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_with_explicit_mask(causal):
    nq, nk, d = 5, 37, 16
    q, k, v = rnd(2, 2, nq, d), rnd(2, 2, nk, d), rnd(2, 2, nk, d)
    o, _ = attention_fwd_decode(q, k, v, 0.25, causal)
    mask = None
    if causal:
        i = torch.arange(nq)[:, None]
        j = torch.arange(nk)[None, :]
        mask = j <= i + (nk - nq)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask, scale=0.25)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)


def test_single_key_and_identical_keys():
    q, v = rnd(1, 1, 4, 6), rnd(1, 1, 1, 6)
    k = rnd(1, 1, 1, 6)
    o, lse = attention_fwd_decode(q, k, v, 0.7, False)
    np.testing.assert_allclose(o[0, 0], np.repeat(v[0, 0], 4, axis=0), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], 0.7 * q[0, 0] @ k[0, 0, 0], atol=1e-13)
    kk = np.broadcast_to(rnd(6), (1, 1, 30, 6)).copy()
    vv = rnd(1, 1, 30, 6)
    o, lse = attention_fwd_decode(q, kk, vv, 0.7, False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(vv[0, 0].mean(axis=0), (4, 6)), atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], 0.7 * q[0, 0] @ kk[0, 0, 0] + np.log(30), atol=1e-12)


def test_more_queries_than_keys_gives_empty_rows():
    q, k, v = rnd(1, 1, 6, 4), rnd(1, 1, 3, 4), rnd(1, 1, 3, 4)
    o, lse = attention_fwd_decode(q, k, v, 0.5, True)
    # queries 0..2 sit before the first key
    assert np.all(o[0, 0, :3] == 0) and np.all(np.isneginf(lse[0, 0, :3]))
    of, lsef = attention_fwd(q[:, :, 3:], k, v, 0.5, True)
    np.testing.assert_allclose(o[0, 0, 3:], of[0, 0], atol=1e-13)
