"""Pins of the oracle's token mask (ramnet-ops "Arguments", mask: masked
tokens are not written and their outputs are to be ignored; reading R21: a
masked token is absent).  The pin is the definition itself: with a mask, the
result for the valid tokens and the final state equal, bit for bit, those of
the same call on the sequence with the masked tokens removed; masked tokens
get output 0 and zero gradients."""
import numpy as np
import pytest

B, H, T, S, KW, KR, D = 3, 2, 40, 16, 3, 2, 4


def inputs(seed):
    rng = np.random.default_rng(seed)
    x = {
        "wl": rng.standard_normal((B, T, H, S)),
        "rl": rng.standard_normal((B, T, H, S)),
        "v": rng.standard_normal((B, T, H, D)),
        "gamma": rng.standard_normal((B, T, H)) + np.log(9.0),
        "d_o": rng.standard_normal((B, T, H, D)),
        "slot0": rng.standard_normal((B, H, S, D)),
        "mass0": rng.uniform(0, 1, (B, H, S)),
        "d_slot1": rng.standard_normal((B, H, S, D)),
        "d_mass1": rng.standard_normal((B, H, S)),
    }
    mask = rng.uniform(size=(B, T)) < 0.7
    mask[0, :5] = False          # leading and trailing runs of masked tokens
    mask[1, -4:] = False
    return x, mask


def compact(x, b, keep):
    per_tok = {k: x[k][b:b + 1][:, keep] for k in ("wl", "rl", "v", "gamma", "d_o")}
    per_tok.update({k: x[k][b:b + 1] for k in ("slot0", "mass0", "d_slot1", "d_mass1")})
    return per_tok


@pytest.mark.parametrize("with_state", [False, True])
def test_forward_is_the_compacted_forward(orc, with_state):
    x, mask = inputs(1)
    p = orc.problem(B, H, T, S, KW, KR, D)
    s0 = x["slot0"] if with_state else None
    m0 = x["mass0"] if with_state else None
    o, s1, m1 = orc.forward(p, x["wl"], x["rl"], x["v"], x["gamma"], s0, m0, mask=mask)
    for b in range(B):
        keep = np.nonzero(mask[b])[0]
        c = compact(x, b, keep)
        pc = orc.problem(1, H, len(keep), S, KW, KR, D)
        oc, sc, mc = orc.forward(pc, c["wl"], c["rl"], c["v"], c["gamma"],
                                 c["slot0"] if with_state else None,
                                 c["mass0"] if with_state else None)
        np.testing.assert_array_equal(s1[b:b + 1], sc)
        np.testing.assert_array_equal(m1[b:b + 1], mc)
        np.testing.assert_array_equal(o[b:b + 1][:, keep], oc)
        assert not np.any(o[b][~mask[b]])


def test_backward_is_the_compacted_backward(orc):
    x, mask = inputs(2)
    p = orc.problem(B, H, T, S, KW, KR, D)
    g = orc.backward(p, x["wl"], x["rl"], x["v"], x["gamma"], x["slot0"], x["mass0"], x["d_o"],
                     x["d_slot1"], x["d_mass1"], mask=mask)
    for b in range(B):
        keep = np.nonzero(mask[b])[0]
        c = compact(x, b, keep)
        pc = orc.problem(1, H, len(keep), S, KW, KR, D)
        gc = orc.backward(pc, c["wl"], c["rl"], c["v"], c["gamma"], c["slot0"], c["mass0"],
                          c["d_o"], c["d_slot1"], c["d_mass1"])
        for name in ("d_wlogits", "d_rlogits", "d_v", "d_gamma", "dw", "dr"):
            np.testing.assert_array_equal(g[name][b:b + 1][:, keep], gc[name], err_msg=name)
            assert not np.any(g[name][b][~mask[b]]), name
        np.testing.assert_array_equal(g["d_slot0"][b:b + 1], gc["d_slot0"])
        np.testing.assert_array_equal(g["d_mass0"][b:b + 1], gc["d_mass0"])


def test_all_masked_keeps_the_state(orc):
    x, _ = inputs(3)
    p = orc.problem(B, H, T, S, KW, KR, D)
    mask = np.zeros((B, T), bool)
    o, s1, m1 = orc.forward(p, x["wl"], x["rl"], x["v"], x["gamma"], x["slot0"], x["mass0"],
                            mask=mask)
    np.testing.assert_array_equal(s1, x["slot0"])
    np.testing.assert_array_equal(m1, x["mass0"])
    assert not np.any(o)


def test_masked_decode_step_leaves_its_sequence(orc):
    x, _ = inputs(4)
    p = orc.problem(B, H, 1, S, KW, KR, D)
    step = {k: x[k][:, :1] for k in ("wl", "rl", "v", "gamma")}
    mask = np.array([1, 0, 1], np.uint8)
    slot, mass = x["slot0"].copy(), x["mass0"].copy()
    o = orc.decode_step(p, step["wl"], step["rl"], step["v"], step["gamma"], slot, mass, mask=mask)
    slot_u, mass_u = x["slot0"].copy(), x["mass0"].copy()
    o_u = orc.decode_step(p, step["wl"], step["rl"], step["v"], step["gamma"], slot_u, mass_u)
    np.testing.assert_array_equal(slot[1], x["slot0"][1])
    np.testing.assert_array_equal(mass[1], x["mass0"][1])
    assert not np.any(o[1])
    for b in (0, 2):
        np.testing.assert_array_equal(slot[b], slot_u[b])
        np.testing.assert_array_equal(o[b], o_u[b])
