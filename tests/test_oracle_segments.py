"""Pins of the oracle's event / segment view and of state continuation.

* segments: every selected read or write is one event, grouped by
  (batch, head, slot) and kept in time order (paper §4 "Slot-Parallel
  Execution"; ramnet-ops "CUDA execution").  Checked against numpy's lexsort
  of the (segment, t, side) tuples; each token contributes exactly
  k_w + k_r events (ramnet-ops: event capacity B*H*T*(write_k+read_k)).
* continuation (ramnet-ops "Arguments", init_ram): a forward split into
  chunks that pass their final (slot, mass) on is bitwise the unsplit one.
* autoregressive mode (ramnet-ops "CUDA execution"): T one-token steps
  reproduce the parallel forward bitwise.
* the page's quick-start example (golden shapes, tests/golden/).
"""
import json
import os

import numpy as np
import pytest


@pytest.mark.parametrize("B,H,T,S,kw,kr", [(1, 1, 50, 8, 2, 3), (2, 3, 37, 16, 4, 1),
                                           (1, 2, 64, 5, 5, 5), (2, 1, 1, 3, 1, 2)])
def test_bucket_matches_lexsort(orc, B, H, T, S, kw, kr):
    rng = np.random.default_rng(B * 1000 + T)
    wl = rng.integers(-2, 3, size=(B, T, H, S)).astype(np.float64)
    rl = rng.integers(-2, 3, size=(B, T, H, S)).astype(np.float64)
    p = orc.problem(B, H, T, S, kw, kr, 1)
    iw, _, _ = orc.decode(p, 0, wl)
    ir, _, _ = orc.decode(p, 1, rl)
    seg, ev_t, ev_s, ev_j = orc.bucket(p, iw, ir)
    # brute force: list every event, sort by (segment, t, side)
    g, tt, ss, jj = [], [], [], []
    for b in range(B):
        for t in range(T):
            for h in range(H):
                for side, idx, k in ((0, iw, kw), (1, ir, kr)):
                    for j in range(k):
                        g.append((b * H + h) * S + idx[b, t, h, j])
                        tt.append(t)
                        ss.append(side)
                        jj.append(j)
    g, tt, ss, jj = map(np.array, (g, tt, ss, jj))
    order = np.lexsort((ss, tt, g))
    np.testing.assert_array_equal(ev_t, tt[order])
    np.testing.assert_array_equal(ev_s, ss[order])
    np.testing.assert_array_equal(ev_j, jj[order])
    counts = np.bincount(g, minlength=B * H * S)
    np.testing.assert_array_equal(np.diff(seg), counts)
    assert seg[0] == 0 and seg[-1] == B * H * T * (kw + kr)
    # every (b, h) holds exactly T * (k_w + k_r) events
    per_bh = counts.reshape(B * H, S).sum(1)
    np.testing.assert_array_equal(per_bh, T * (kw + kr))


def inputs(rng, B, H, T, S, d):
    return (rng.standard_normal((B, T, H, S)), rng.standard_normal((B, T, H, S)),
            rng.standard_normal((B, T, H, d)), rng.normal(np.log(9), 1, (B, T, H)))


@pytest.mark.parametrize("cape", [0, 2])
def test_chunked_forward_is_bitwise_unchunked(orc, cape):
    rng = np.random.default_rng(21)
    B, H, T, S, kw, kr, d = 2, 3, 48, 10, 3, 2, 4
    wl, rl, v, gam = inputs(rng, B, H, T, S, d)
    p = orc.problem(B, H, T, S, kw, kr, d, cape_heads=cape, t0=3)
    o, s1, m1 = orc.forward(p, wl, rl, v, gam)
    s, m = None, None
    outs = []
    for lo, hi in ((0, 5), (5, 21), (21, 22), (22, 48)):
        pc = orc.problem(B, H, hi - lo, S, kw, kr, d, cape_heads=cape, t0=3 + lo)
        oc, s, m = orc.forward(pc, wl[:, lo:hi], rl[:, lo:hi], v[:, lo:hi], gam[:, lo:hi], s, m)
        outs.append(oc)
    assert np.array_equal(np.concatenate(outs, axis=1), o)
    assert np.array_equal(s, s1)
    assert np.array_equal(m, m1)


def test_decode_steps_reproduce_forward(orc):
    rng = np.random.default_rng(22)
    B, H, T, S, kw, kr, d = 3, 2, 20, 12, 2, 3, 5
    wl, rl, v, gam = inputs(rng, B, H, T, S, d)
    s0 = rng.standard_normal((B, H, S, d)) * 0.02
    m0 = np.zeros((B, H, S))
    p = orc.problem(B, H, T, S, kw, kr, d, cape_heads=1, t0=7)
    o, s1, m1 = orc.forward(p, wl, rl, v, gam, s0, m0)
    slot, mass = s0.copy(), m0.copy()
    for t in range(T):
        ps = orc.problem(B, H, 1, S, kw, kr, d, cape_heads=1, t0=7 + t)
        ot = orc.decode_step(ps, wl[:, t:t + 1], rl[:, t:t + 1], v[:, t:t + 1], gam[:, t:t + 1],
                             slot, mass)
        assert np.array_equal(ot[:, 0], o[:, t])
    assert np.array_equal(slot, s1)
    assert np.array_equal(mass, m1)


def test_quickstart_example_shapes(orc):
    """The op page's quick-start example: shapes it prints for y, slot, mass."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "quickstart_shapes.json")) as f:
        gold = json.load(f)
    c = gold["example"]
    B, T, H, U, P, C, K, E = c["B"], c["T"], c["H"], c["U"], c["P"], c["C"], c["top_k"], c["embed_num"]
    env = {"B": B, "T": T, "H": H, "C": C, "P ** U": P ** U}
    rng = np.random.default_rng(0)
    wl = rng.standard_normal((B, T, H, U, P))
    rl = rng.standard_normal((B, T, H, U, P))
    v = rng.standard_normal((B, T, H, C))
    gam = rng.standard_normal((B, T, H))
    p = orc.problem(B, H, T, U=U, P=P, k_w=K, k_r=K, d_v=C, cape_heads=E)
    y, slot, mass = orc.forward(p, wl, rl, v, gam)
    assert y.shape == tuple(env[n] for n in gold["y_shape"])
    assert slot.shape == tuple(env[n] for n in gold["slot_shape"])
    assert mass.shape == tuple(env[n] for n in gold["mass_shape"])
    # the example's loss uses y, slot and mass; its backward runs
    n_y, n_s, n_m = y.size, slot.size, mass.size
    g = orc.backward(p, wl, rl, v, gam, None, None, 2 * y / n_y, 2 * slot / n_s, 2 * mass / n_m)
    assert g["d_wlogits"].shape == wl.shape and np.all(np.isfinite(g["d_wlogits"]))
    assert g["d_v"].shape == v.shape and np.all(np.isfinite(g["d_v"]))
