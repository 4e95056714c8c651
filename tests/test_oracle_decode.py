"""Pins of the oracle's address decoder against things other than itself.

* indices: a full stable sort of every slot's key (brute force), with heavy
  ties, for flat (U = 1) and factorised (U = 2, 3) addresses;
* weights: scipy's softmax / logsumexp (the slot probability is the product of
  the digit softmaxes, paper App. B.1 "Order U of Product Softmax");
* the Top-K prefix-tree search of paper §3.2 / §4 "Efficient Address
  Decoding" returns exactly the exhaustive top-K (the paper's exactness claim);
* renormalisation (ramnet-ops "Arguments", top_k_re_norm);
* CAPE: the first cape_heads heads shift the chosen slot by the absolute token
  position (ramnet-ops "Quick start").
"""
import itertools

import numpy as np
import pytest
from scipy.special import logsumexp, softmax


def flat_keys_f32(row, U, P):
    """Key of every flat slot: float32 sum of its digit logits, u ascending."""
    digits = np.asarray(row, dtype=np.float32).reshape(U, P)
    key = np.zeros(P ** U, dtype=np.float32)
    for a in range(P ** U):
        acc = np.float32(0.0)
        rem = a
        for u in range(U):
            stride = P ** (U - 1 - u)
            acc = np.float32(acc + digits[u, rem // stride])
            rem %= stride
        key[a] = acc
    return key


def brute_topk(keys, k):
    """Full stable sort: key descending, then index ascending."""
    order = np.lexsort((np.arange(keys.size), -keys.astype(np.float64)))
    return order[:k]


def prefix_tree_topk(row, U, P, k):
    """Top-K prefix-tree search: level by level keep the K best prefixes by
    (float32 prefix key desc, prefix index asc); each level extends every kept
    prefix by all P digits."""
    digits = np.asarray(row, dtype=np.float32).reshape(U, P)
    beams = [(np.float32(0.0), 0)]
    for u in range(U):
        cand = [(np.float32(key + digits[u, d]), pre * P + d) for key, pre in beams for d in range(P)]
        cand.sort(key=lambda c: (-float(c[0]), c[1]))
        beams = cand[:k]
    return np.array([c[1] for c in beams])


def rows_of(rng, shape, ties):
    if ties:
        return rng.integers(-3, 4, size=shape).astype(np.float64)
    return rng.standard_normal(shape).astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("S,k", [(1, 1), (5, 2), (5, 5), (64, 2), (100, 7), (257, 8)])
@pytest.mark.parametrize("ties", [True, False])
def test_flat_indices_match_full_sort(orc, S, k, ties):
    rng = np.random.default_rng(1000 * S + k + ties)
    B, T, H = 2, 9, 3
    wl = rows_of(rng, (B, T, H, S), ties)
    p = orc.problem(B, H, T, S, k_w=k, k_r=k, d_v=1)
    idx, w, lse = orc.decode(p, 0, wl)
    for b, t, h in itertools.product(range(B), range(T), range(H)):
        row = wl[b, t, h]
        np.testing.assert_array_equal(idx[b, t, h], brute_topk(row, k))
        ref_lse = logsumexp(row)
        assert abs(lse[b, t, h, 0] - ref_lse) <= 1e-13 * max(1.0, abs(ref_lse))
        ref_w = softmax(row)[idx[b, t, h]]
        np.testing.assert_allclose(w[b, t, h], ref_w, rtol=1e-13, atol=0)


def test_signed_zero_ties_break_by_index(orc):
    # -0.0 and +0.0 are the same number: the lower index wins
    row = np.array([-1.0, -0.0, 0.0, -0.0, -2.0])
    p = orc.problem(1, 1, 1, 5, k_w=3, k_r=3, d_v=1)
    idx, _, _ = orc.decode(p, 0, row.reshape(1, 1, 1, 5))
    np.testing.assert_array_equal(idx[0, 0, 0], [1, 2, 3])


@pytest.mark.parametrize("U,P,k", [(2, 3, 2), (2, 4, 5), (3, 3, 4), (3, 4, 8), (2, 5, 25)])
def test_factorised_indices_and_weights(orc, U, P, k):
    rng = np.random.default_rng(U * 100 + P * 10 + k)
    B, T, H = 1, 12, 2
    for ties in (True, False):
        wl = rows_of(rng, (B, T, H, U, P), ties)
        p = orc.problem(B, H, T, U=U, P=P, k_w=k, k_r=k, d_v=1)
        idx, w, lse = orc.decode(p, 1, wl)
        for t, h in itertools.product(range(T), range(H)):
            row = wl[0, t, h]
            keys = flat_keys_f32(row, U, P)
            np.testing.assert_array_equal(idx[0, t, h], brute_topk(keys, k))
            # slot probability = Kronecker product of the digit softmaxes
            prob = softmax(row[0])
            for u in range(1, U):
                prob = np.kron(prob, softmax(row[u]))
            np.testing.assert_allclose(w[0, t, h], prob[idx[0, t, h]], rtol=1e-12, atol=0)
            np.testing.assert_allclose(lse[0, t, h], [logsumexp(row[u]) for u in range(U)],
                                       rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("U,P,k", [(2, 2, 1), (2, 3, 3), (2, 4, 4), (3, 2, 3), (3, 3, 5),
                                   (3, 4, 8), (4, 3, 6)])
def test_prefix_tree_search_is_exact(orc, U, P, k):
    # integer logits: every float32 partial sum is exact and ties are frequent
    rng = np.random.default_rng(7 * U + 11 * P + k)
    T = 300
    wl = rng.integers(-2, 3, size=(1, T, 1, U, P)).astype(np.float64)
    p = orc.problem(1, 1, T, U=U, P=P, k_w=k, k_r=k, d_v=1)
    idx, _, _ = orc.decode(p, 0, wl)
    for t in range(T):
        np.testing.assert_array_equal(idx[0, t, 0], prefix_tree_topk(wl[0, t, 0], U, P, k))


def test_renormalisation(orc):
    rng = np.random.default_rng(5)
    B, T, H, S, k = 2, 7, 2, 33, 5
    wl = rng.standard_normal((B, T, H, S))
    p0 = orc.problem(B, H, T, S, k_w=k, k_r=3, d_v=1)
    p1 = orc.problem(B, H, T, S, k_w=k, k_r=3, d_v=1, renorm=(True, False))
    i0, w0, _ = orc.decode(p0, 0, wl)
    i1, w1, _ = orc.decode(p1, 0, wl)
    np.testing.assert_array_equal(i0, i1)
    np.testing.assert_allclose(w1, w0 / w0.sum(-1, keepdims=True), rtol=1e-14)
    np.testing.assert_allclose(w1.sum(-1), 1.0, rtol=1e-14)
    # the read side keeps its own (off) setting
    _, r1, _ = orc.decode(p1, 1, wl[..., :S])
    _, r0, _ = orc.decode(p0, 1, wl[..., :S])
    np.testing.assert_array_equal(r0, r1)


def test_cape_shift(orc):
    rng = np.random.default_rng(9)
    B, T, H, S, k, t0 = 2, 11, 4, 16, 3, 37
    wl = rng.standard_normal((B, T, H, S))
    plain = orc.problem(B, H, T, S, k_w=k, k_r=k, d_v=1)
    cape = orc.problem(B, H, T, S, k_w=k, k_r=k, d_v=1, cape_heads=2, t0=t0)
    i0, w0, _ = orc.decode(plain, 0, wl)
    i1, w1, _ = orc.decode(cape, 0, wl)
    np.testing.assert_array_equal(w0, w1)
    for t in range(T):
        for h in range(H):
            want = (i0[:, t, h] + t0 + t) % S if h < 2 else i0[:, t, h]
            np.testing.assert_array_equal(i1[:, t, h], want)
