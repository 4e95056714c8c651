"""Pins of the oracle's Gated Sparse Update, read-out and forward loop.

Each test compares the oracle with something it does not share code with:

* the stated properties of GSU (paper §3.4): (i) exact sparsity, writes of
  different tokens interact only at jointly addressed slots; (ii) bounded
  content; (iii) the two limits of the forgetting strength: gamma -> -inf
  gives a cumulative average of the writes, gamma -> +inf overwrites;
* a dense O(T^2) brute force in log-space (numpy/scipy) of the same
  recurrence: o_t = sum_{tau<=t} A[t,tau] v_tau + (initial-state term), built
  from closed forms of the mass and of the content weights, with its own
  decoder (full sort + scipy softmax) and its own retention (scipy expit of
  logit(1-w) - gamma);
* read-out after write (paper §3.4 "Read-out": o_t = r_t S_t).
"""
import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

from linear_attention_ram_amd import synth


def dense_weights(logits, k, renorm=False):
    """(T,S) logits -> (T,S) sparse weights: top-k by (value desc, idx asc)."""
    T, S = logits.shape
    out = np.zeros((T, S))
    for t in range(T):
        order = np.lexsort((np.arange(S), -logits[t]))[:k]
        p = softmax(logits[t])
        out[t, order] = p[order]
        if renorm:
            out[t] /= out[t].sum()
    return out


def brute_force_bh(wl, rl, v, gamma, k_w, k_r, eps, s0=None, m0=None):
    """Dense O(T^2 S) evaluation for one (b, h).  wl, rl (T,S); v (T,d);
    gamma (T,)."""
    T, S = wl.shape
    d = v.shape[1]
    W = dense_weights(wl, k_w)
    R = dense_weights(rl, k_r)
    s0 = np.zeros((S, d)) if s0 is None else s0
    m0 = np.zeros(S) if m0 is None else m0
    addressed = W > 0
    Wc = np.where(addressed, W, 0.5)
    lam = np.where(addressed, expit(np.log1p(-Wc) - np.log(Wc) - gamma[:, None]), 1.0)
    # mass: m_tau = exp(L_tau) m0 + sum_{sig<=tau} W_sig exp(L_tau - L_sig),
    # L_tau = sum_{rho<=tau} log lambda_rho
    L = np.cumsum(np.log(lam), axis=0)                            # (T,S)
    decay = np.exp(L[:, None, :] - L[None, :, :])                  # [tau, sig, a]
    causal = np.tril(np.ones((T, T)))[:, :, None]
    m = np.exp(L) * m0[None, :] + np.sum(causal * decay * W[None, :, :], axis=1)
    eta = np.where(addressed, W / (m + eps), 0.0)                  # (T,S)
    # content: s_t = exp(Q_t) s0 + sum_{tau<=t} eta_tau exp(Q_t - Q_tau) v_tau,
    # Q_t = sum_{sig<=t} log(1 - eta_sig)
    Q = np.cumsum(np.log1p(-eta), axis=0)
    keep = np.exp(Q[:, None, :] - Q[None, :, :]) * causal          # [t, tau, a]
    A = np.einsum("ta,tua,ua->tu", R, keep, eta)                   # (T,T)
    init = (R * np.exp(Q)) @ s0                                    # (T,d)
    o = A @ v + init
    s_T = np.exp(Q[-1])[:, None] * s0 + (eta * np.exp(Q[-1][None, :] - Q)).T @ v
    return o, s_T, m[-1]


def as_np(x):
    return x.double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, np.float64)


def test_tiny_matches_quadratic_brute_force(orc):
    cfg = synth.CONFIGS["tiny"]
    x = synth.layer_inputs(cfg, seed=0)
    p = orc.problem(cfg.B, cfg.H, cfg.T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, eps=cfg.eps)
    o, s1, m1 = orc.forward(p, as_np(x["wl"]), as_np(x["rl"]), as_np(x["v"]), as_np(x["gamma"]))
    bo, bs, bm = brute_force_bh(as_np(x["wl"])[0, :, 0], as_np(x["rl"])[0, :, 0],
                                as_np(x["v"])[0, :, 0], as_np(x["gamma"])[0, :, 0],
                                cfg.k_w, cfg.k_r, cfg.eps)
    assert np.max(np.abs(o[0, :, 0] - bo)) <= 1e-10 * np.max(np.abs(bo))
    assert np.max(np.abs(s1[0, 0] - bs)) <= 1e-10 * np.max(np.abs(bs))
    np.testing.assert_allclose(m1[0, 0], bm, rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("seed", [1, 2])
def test_random_state_matches_quadratic_brute_force(orc, seed):
    rng = np.random.default_rng(seed)
    B, H, T, S, kw, kr, d = 1, 2, 40, 9, 3, 2, 5
    wl = rng.standard_normal((B, T, H, S)) * 2
    rl = rng.standard_normal((B, T, H, S)) * 2
    v = rng.standard_normal((B, T, H, d))
    gam = rng.normal(np.log(9), 1.5, (B, T, H))
    s0 = rng.standard_normal((B, H, S, d))
    m0 = rng.uniform(0, 1, (B, H, S))
    p = orc.problem(B, H, T, S, kw, kr, d, eps=1e-3)
    o, s1, m1 = orc.forward(p, wl, rl, v, gam, s0, m0)
    for h in range(H):
        bo, bs, bm = brute_force_bh(wl[0, :, h], rl[0, :, h], v[0, :, h], gam[0, :, h], kw, kr,
                                    1e-3, s0[0, h], m0[0, h])
        np.testing.assert_allclose(o[0, :, h], bo, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(s1[0, h], bs, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(m1[0, h], bm, rtol=1e-10, atol=1e-14)


def random_case(rng, B=2, H=3, T=30, S=12, kw=3, kr=2, d=4):
    wl = rng.standard_normal((B, T, H, S))
    rl = rng.standard_normal((B, T, H, S))
    v = rng.standard_normal((B, T, H, d))
    gam = rng.normal(np.log(9), 1.0, (B, T, H))
    s0 = rng.standard_normal((B, H, S, d))
    m0 = rng.uniform(0, 1, (B, H, S))
    return wl, rl, v, gam, s0, m0


def test_exact_sparsity_untouched_slots_bit_identical(orc):
    rng = np.random.default_rng(3)
    B, H, T, S, kw, kr, d = 2, 3, 30, 40, 2, 3, 4
    wl, rl, v, gam, s0, m0 = random_case(rng, B, H, T, S, kw, kr, d)
    p = orc.problem(B, H, T, S, kw, kr, d)
    _, s1, m1 = orc.forward(p, wl, rl, v, gam, s0, m0)
    iw, _, _ = orc.decode(p, 0, wl)
    n_untouched = 0
    for b in range(B):
        for h in range(H):
            written = set(iw[b, :, h].ravel().tolist())
            for a in range(S):
                if a not in written:
                    n_untouched += 1
                    assert np.array_equal(s1[b, h, a], s0[b, h, a])
                    assert m1[b, h, a] == m0[b, h, a]
                else:
                    assert not np.array_equal(s1[b, h, a], s0[b, h, a])
    assert n_untouched > 0


def test_disjoint_addresses_do_not_interact(orc):
    rng = np.random.default_rng(4)
    B, H, T, S, kw, kr, d = 1, 2, 25, 20, 2, 2, 3
    wl, rl, v, gam, s0, m0 = random_case(rng, B, H, T, S, kw, kr, d)
    p = orc.problem(B, H, T, S, kw, kr, d)
    o, _, _ = orc.forward(p, wl, rl, v, gam, s0, m0)
    iw, _, _ = orc.decode(p, 0, wl)
    ir, _, _ = orc.decode(p, 1, rl)
    total_changed = 0
    for tau in (0, 7, 19):
        v2 = v.copy()
        v2[0, tau, 1] += 1.0
        o2, _, _ = orc.forward(p, wl, rl, v2, gam, s0, m0)
        assert np.array_equal(o2[0, :, 0], o[0, :, 0])     # other head: untouched
        changed = 0
        for t in range(T):
            linked = t >= tau and set(ir[0, t, 1]) & set(iw[0, tau, 1])
            if not linked:
                assert np.array_equal(o2[0, t, 1], o[0, t, 1]), (tau, t)
            else:
                changed += int(not np.array_equal(o2[0, t, 1], o[0, t, 1]))
        total_changed += changed
    assert total_changed > 0


def test_bounded_content(orc):
    rng = np.random.default_rng(6)
    B, H, T, S, kw, kr, d = 1, 2, 60, 8, 3, 2, 4
    wl, rl, v, gam, s0, m0 = random_case(rng, B, H, T, S, kw, kr, d)
    p = orc.problem(B, H, T, S, kw, kr, d)
    _, s1, m1 = orc.forward(p, wl, rl, v, gam, s0, m0)
    iw, _, _ = orc.decode(p, 0, wl)
    for h in range(H):
        for a in range(S):
            writers = [t for t in range(T) if a in iw[0, t, h]]
            vals = np.vstack([s0[0, h, a][None]] + [v[0, t, h][None] for t in writers])
            assert np.all(s1[0, h, a] >= vals.min(0) - 1e-12)
            assert np.all(s1[0, h, a] <= vals.max(0) + 1e-12)
            assert m1[0, h, a] >= 0


def test_overwrite_limit_is_last_writer_wins_bitwise(orc):
    # gamma -> +inf, eps = 0: lambda = 0, eta = 1, each write replaces the slot
    rng = np.random.default_rng(8)
    B, H, T, S, kw, kr, d = 1, 2, 50, 10, 3, 3, 4
    wl, rl, v, _, s0, m0 = random_case(rng, B, H, T, S, kw, kr, d)
    gam = np.full((B, T, H), 1e4)
    p = orc.problem(B, H, T, S, kw, kr, d, eps=0.0)
    o, s1, m1 = orc.forward(p, wl, rl, v, gam, s0, m0)
    iw, ww, _ = orc.decode(p, 0, wl)
    ir, wr, _ = orc.decode(p, 1, rl)
    for h in range(H):
        state = s0[0, h].copy()
        mass = m0[0, h].copy()
        for t in range(T):
            for j in range(kw):
                state[iw[0, t, h, j]] = v[0, t, h]
                mass[iw[0, t, h, j]] = ww[0, t, h, j]
            acc = np.zeros(d)
            for j in range(kr):
                acc = acc + wr[0, t, h, j] * state[ir[0, t, h, j]]
            assert np.array_equal(o[0, t, h], acc)
        assert np.array_equal(s1[0, h], state)
        assert np.array_equal(m1[0, h], mass)


def test_history_limit_is_cumulative_average(orc):
    # gamma -> -inf, eps = 0: lambda = 1, the slot is the mass-weighted mean
    # of its initial content and every value written to it
    rng = np.random.default_rng(10)
    B, H, T, S, kw, kr, d = 1, 2, 50, 10, 3, 2, 4
    wl, rl, v, _, s0, m0 = random_case(rng, B, H, T, S, kw, kr, d)
    gam = np.full((B, T, H), -1e4)
    p = orc.problem(B, H, T, S, kw, kr, d, eps=0.0)
    _, s1, m1 = orc.forward(p, wl, rl, v, gam, s0, m0)
    iw, ww, _ = orc.decode(p, 0, wl)
    for h in range(H):
        num = m0[0, h][:, None] * s0[0, h]
        den = m0[0, h].copy()
        for t in range(T):
            for j in range(kw):
                a = iw[0, t, h, j]
                num[a] += ww[0, t, h, j] * v[0, t, h]
                den[a] += ww[0, t, h, j]
        np.testing.assert_allclose(m1[0, h], den, rtol=1e-12)
        np.testing.assert_allclose(s1[0, h], num / den[:, None], rtol=1e-12, atol=1e-12)


def test_step_size_shrinks_with_mass(orc):
    # property (iii): repeated writes of the same weight to one slot take
    # ever smaller steps; with one value the step is visible as the distance
    # still to travel
    S, d, T = 4, 1, 12
    wl = np.full((1, T, 1, S), -50.0)
    wl[0, :, 0, 2] = 0.0                       # always write slot 2, weight ~1
    wl[0, :, 0, 1] = -1.0
    rl = wl.copy()
    v = np.zeros((1, T, 1, d))
    v[0, :, 0, 0] = 1.0
    gam = np.full((1, T, 1), -3.0)
    s0 = np.zeros((1, 1, S, d))
    m0 = np.zeros((1, 1, S))
    p = orc.problem(1, 1, T, S, 1, 1, d, eps=1e-6)
    o, _, _ = orc.forward(p, wl, rl, v, gam, s0, m0)
    # reads of slot 2 give s_t = 1 - prod(1 - eta): eta_t decreasing
    s = o[0, :, 0, 0] / softmax(wl[0, 0, 0])[2]
    eta = [s[0]] + [(s[t] - s[t - 1]) / (1 - s[t - 1]) for t in range(1, T)]
    assert all(e2 < e1 for e1, e2 in zip(eta, eta[1:]))
    assert all(0 <= e < 1 for e in eta)
