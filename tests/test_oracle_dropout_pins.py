"""Pins for the dropout oracle (oracle/dropout.py).

The generator is pinned by the published known-answer vectors of
Philox-4x32-10.  The keep rule is pinned by the first vector too: at seed 0
the words Philox returns for counter (0, 0, 0, 0) are the ones compared with
the threshold for query 0, keys 0..3 of head 0, so three thresholds between
those four words fix which word serves which key.  The placement of the key
group, query and head in the counter is checked against the layout the C
header documents, at coordinates where a transposed (i, j), or head and query
exchanged, gives a different mask.  Then the threshold arithmetic, the
binomial statistics of the mask, p = 0 reducing to plain attention,
unbiasedness over seeds (inverted dropout has E[O] equal to the dropout-free
O), central finite differences of L = sum(dO * O) at a fixed seed and the dK
column-sum invariant pin the rest.  A dropped 1/(1-p) factor, a mask applied
to the wrong operand, a mask missing from dP, a permuted word order or a
transposed (i, j) in the counter each fail one of these.
"""
import json
import os

import numpy as np
import pytest

from oracle import attention_bwd, attention_fwd
from oracle.dropout import (
    attention_bwd_dropout,
    attention_fwd_dropout,
    drop_threshold,
    keep_mask,
    philox4x32_10,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(4321)


def rnd(*shape):
    return rng.standard_normal(shape)


def test_philox_known_answers():
    g = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for vec in g["vectors"]:
        ctr = np.array([int(x, 16) for x in vec["counter"]], dtype=np.uint64)
        key = tuple(int(x, 16) for x in vec["key"])
        out = philox4x32_10(ctr, key)
        assert [int(x) for x in out] == [int(x, 16) for x in vec["out"]]


def _kat():
    g = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    return g["vectors"]


def test_keep_rule_known_answers():
    """Query 0, keys 0..3, head 0, seed 0 use counter (0, 0, 0, 0) under key
    (0, 0), the first published vector: key j takes word j, kept when the
    word is at least floor(p * 2^32).  The four words lie in the order
    w0 < w3 < w2 < w1, and p = 0.5, 0.7, 0.85 put a threshold in each gap, so
    the three patterns fix the word of every key."""
    vec = _kat()[0]
    assert vec["counter"] == ["00000000"] * 4 and vec["key"] == ["00000000"] * 2
    words = [int(x, 16) for x in vec["out"]]
    patterns = {}
    for p in (0.5, 0.7, 0.85):
        T = int(np.floor(float(np.float32(p)) * 2.0**32))
        expected = [w >= T for w in words]
        got = keep_mask(0, np.array([0]), np.arange(4), p, seed=0)[0].tolist()
        assert got == expected, (p, got, expected)
        patterns[p] = tuple(expected)
    assert patterns == {0.5: (False, True, True, True), 0.7: (False, True, True, False),
                        0.85: (False, True, False, False)}


def _documented_keep(bh, i, j, p, seed):
    """The layout the C header states: word (j mod 4) of Philox-4x32-10 at
    counter (j / 4, i, b*H + h, 0) and key (seed mod 2^32, seed / 2^32)."""
    w = philox4x32_10(np.array([j // 4, i, bh, 0], dtype=np.uint64),
                      (seed & 0xFFFFFFFF, seed >> 32))[j % 4]
    return int(w) >= drop_threshold(p)


def test_keep_rule_counter_layout():
    """keep_mask against the documented layout at random coordinates, and the
    same coordinates distinguish that layout from a transposed (i, j) and from
    head and query exchanged."""
    r = np.random.default_rng(77)
    p, seed = 0.5, (3 << 32) + 12345
    n_transposed = n_swapped = 0
    for _ in range(300):
        bh, i, j = (int(x) for x in r.integers(0, 5000, size=3))
        z = keep_mask(bh, np.array([i]), np.array([j]), p, seed)[0, 0]
        assert bool(z) == _documented_keep(bh, i, j, p, seed), (bh, i, j)
        n_transposed += bool(z) != _documented_keep(bh, j, i, p, seed)
        w = philox4x32_10(np.array([j // 4, bh, i, 0], dtype=np.uint64),
                          (seed & 0xFFFFFFFF, seed >> 32))[j % 4]
        n_swapped += bool(z) != (int(w) >= drop_threshold(p))
    # independent fair coins disagree about half the time
    assert 100 < n_transposed < 200 and 100 < n_swapped < 200


def test_philox_batched_equals_single():
    ctr = rng.integers(0, 2**32, size=(5, 3, 4), dtype=np.uint64)
    key = (0x12345678, 0x9ABCDEF0)
    batched = philox4x32_10(ctr, key)
    for a in range(5):
        for b in range(3):
            assert np.array_equal(batched[a, b], philox4x32_10(ctr[a, b], key))


def test_threshold_arithmetic():
    assert drop_threshold(0.0) == 0
    assert drop_threshold(0.5) == 2**31
    assert drop_threshold(0.25) == 2**30
    # float32(0.1) = 0.100000001490116119384765625, times 2^32 = 429496736 exactly
    assert drop_threshold(0.1) == 429496736
    for bad in (1.0, -0.1, float("nan"), 2.0):
        with pytest.raises(ValueError):
            drop_threshold(bad)


def test_zero_probability_keeps_everything():
    z = keep_mask(3, np.arange(50), np.arange(70), 0.0, seed=99)
    assert z.all()


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_fraction_is_binomial(p):
    n_rows, n_cols = 300, 300
    z = np.concatenate([keep_mask(bh, np.arange(n_rows), np.arange(n_cols), p, seed=2024)
                        for bh in range(4)])
    n = z.size
    frac = z.mean()
    sigma = np.sqrt(p * (1 - p) / n)
    assert abs(frac - (1 - p)) < 6 * sigma


def test_mask_depends_on_every_coordinate():
    base = keep_mask(0, np.arange(64), np.arange(64), 0.5, seed=7)
    for other in (keep_mask(1, np.arange(64), np.arange(64), 0.5, seed=7),
                  keep_mask(0, np.arange(64), np.arange(64), 0.5, seed=8),
                  keep_mask(0, np.arange(64) + 64, np.arange(64), 0.5, seed=7),
                  keep_mask(0, np.arange(64), np.arange(64) + 64, 0.5, seed=7),
                  keep_mask(0, np.arange(64), np.arange(64), 0.5, seed=7 + (1 << 32))):
        agree = (base == other).mean()
        assert 0.4 < agree < 0.6  # independent fair coins agree half the time
    # the mask is not symmetric in (i, j)
    assert 0.4 < (base == base.T).mean() < 0.6


def test_mask_is_a_function_of_coordinates():
    full = keep_mask(5, np.arange(40), np.arange(90), 0.3, seed=11)
    rows = np.array([3, 17, 39])
    cols = np.array([0, 5, 6, 7, 44, 89])
    assert np.array_equal(keep_mask(5, rows, cols, 0.3, seed=11), full[np.ix_(rows, cols)])


@pytest.mark.parametrize("causal", [False, True])
def test_zero_probability_reduces_to_attention(causal):
    q, k, v, do = rnd(1, 2, 33, 8), rnd(1, 2, 33, 8), rnd(1, 2, 33, 8), rnd(1, 2, 33, 8)
    o, lse = attention_fwd(q, k, v, 0.4, causal)
    od, lsed = attention_fwd_dropout(q, k, v, 0.4, causal, None, 0.0, seed=5)
    assert np.array_equal(o, od) and np.array_equal(lse, lsed)
    g = attention_bwd(q, k, v, do, 0.4, causal)
    gd = attention_bwd_dropout(q, k, v, do, 0.4, causal, None, 0.0, seed=5)
    for a, b in zip(g, gd):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_lse_does_not_see_dropout():
    q, k, v = rnd(1, 1, 20, 4), rnd(1, 1, 20, 4), rnd(1, 1, 20, 4)
    _, lse = attention_fwd(q, k, v, 0.5, True)
    _, lsed = attention_fwd_dropout(q, k, v, 0.5, True, None, 0.3, seed=1)
    assert np.array_equal(lse, lsed)


def test_forward_is_unbiased_over_seeds():
    N, d, p = 12, 4, 0.3
    q, k, v = rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d)
    o, _ = attention_fwd(q, k, v, 0.5, False)
    samples = np.stack([attention_fwd_dropout(q, k, v, 0.5, False, None, p, seed=s)[0]
                        for s in range(1500)])
    mean = samples.mean(axis=0)
    sem = samples.std(axis=0) / np.sqrt(samples.shape[0])
    assert np.all(np.abs(mean - o) < 6 * sem + 1e-12)


def _fd_grads(q, k, v, do, scale, causal, mask, p, seed, h=1e-6):
    def loss(q_, k_, v_):
        o, _ = attention_fwd_dropout(q_, k_, v_, scale, causal, mask, p, seed)
        return float((o * do).sum())

    out = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        out.append(g)
    return out


@pytest.mark.parametrize("N,d", [(1, 2), (3, 2), (5, 4), (8, 1), (8, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(N, d, causal):
    q, k, v, do = rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d), rnd(1, 1, N, d)
    p, seed, scale = 0.35, 31337, 0.7
    dq, dk, dv = attention_bwd_dropout(q, k, v, do, scale, causal, None, p, seed)
    fq, fk, fv = _fd_grads(q, k, v, do, scale, causal, None, p, seed)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        denom = max(1.0, np.abs(b).max())
        assert np.abs(a - b).max() / denom < 1e-6


def test_backward_with_block_mask_matches_finite_differences():
    N, d = 130, 2  # two mask blocks, the second of 2 rows
    mask = np.array([[1, 0], [1, 1]], dtype=np.uint8)
    q, k, v, do = (0.5 * rnd(1, 1, N, d) for _ in range(4))
    p, seed, scale = 0.2, 77, 0.9
    dq, dk, dv = attention_bwd_dropout(q, k, v, do, scale, False, mask, p, seed)
    # spot-check a few coordinates of each gradient by central differences
    h = 1e-6

    def loss(q_, k_, v_):
        o, _ = attention_fwd_dropout(q_, k_, v_, scale, False, mask, p, seed)
        return float((o * do).sum())

    for which, g in ((0, dq), (1, dk), (2, dv)):
        for idx in ((0, 0, 0, 0), (0, 0, 127, 1), (0, 0, 128, 0), (0, 0, 129, 1)):
            args = [q, k, v]
            plus = [x.copy() for x in args]
            minus = [x.copy() for x in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(g[idx] - fd) < 1e-6 * max(1.0, abs(fd))


@pytest.mark.parametrize("causal", [False, True])
def test_dk_columns_sum_to_zero(causal):
    q, k, v, do = rnd(2, 2, 40, 8), rnd(2, 2, 40, 8), rnd(2, 2, 40, 8), rnd(2, 2, 40, 8)
    _, dk, _ = attention_bwd_dropout(q, k, v, do, 0.3, causal, None, 0.25, seed=3)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)


def test_heads_get_independent_masks():
    # the same inputs in two heads: the outputs differ because the masks do
    q1, k1, v1 = rnd(1, 1, 16, 4), rnd(1, 1, 16, 4), rnd(1, 1, 16, 4)
    q, k, v = (np.concatenate([x, x], axis=1) for x in (q1, k1, v1))
    o, _ = attention_fwd_dropout(q, k, v, 0.5, False, None, 0.5, seed=9)
    assert not np.allclose(o[0, 0], o[0, 1])
    ob, _ = attention_fwd_dropout(np.concatenate([q, q]), np.concatenate([k, k]),
                                  np.concatenate([v, v]), 0.5, False, None, 0.5, seed=9)
    # batch index enters through b*H + h: batch 1 head 0 is counter head 2
    assert np.array_equal(ob[0], o[0])
    assert not np.allclose(ob[1, 0], o[0, 0])
