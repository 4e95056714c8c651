"""GPU parity over seeded random shapes of the decode step and the gated
read-out.

Decode step: product addresses of U = 1, 2 or 3 digits, CAPE heads with the
position advancing one per step, renormalised sides, masked sequences, a
random nonzero starting mass; several steps in a row, o at every step and the
final state against the oracle's steps.

Gated read-out (y = sigmoid(gate) * RMSNorm(o) * gain): the same features
plus T, the initial state, the gain and the RMSNorm epsilon.  Three kinds of
problem are left out on purpose because their exact gradients are
ill-conditioned in o, so fp32 rounding of o moves even the oracle's own
gradients far past any bar: d_v = 1 (RMSNorm of one value is sign(o) with a
transition of width sqrt(eps)); one token with no initial state (then o is a
multiple of v, RMSNorm cancels the write's step size and its exact gradient is
zero); and one read slot (o is then the read weight times one slot's value,
and RMSNorm cancels the read weight the same way)."""
import random

import numpy as np
import pytest
import torch

import linear_attention_ram_amd as ram
import oracle
from gpu_util import TOL, check_grads, host, oracle_problem, say
from linear_attention_ram_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FLOOR = 1e-9


def frel(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), FLOOR))


def draw_shape(rng, widths):
    U = rng.choice([1, 1, 2, 2, 3])
    if U == 1:
        P = rng.choice([16, 64, 256, 1024])
    elif U == 2:
        P = rng.choice([8, 16, 32, 64])
    else:
        P = rng.choice([8, 16])
    S = P ** U
    return dict(U=U, P=P, S=S, io=rng.choice(["f32", "bf16"]), B=rng.randint(1, 6),
                H=rng.randint(1, 4), kw=rng.randint(1, min(S, 16)), kr=rng.randint(1, min(S, 16)),
                d=rng.choice(widths), rn=(rng.random() < 0.3, rng.random() < 0.3),
                eps=rng.choice([1e-6, 1e-3]), cape_draw=rng.random(), t0=rng.randint(0, 5000))


def cape_heads(c, rng):
    return rng.randint(0, c["H"]) if c.pop("cape_draw") < 0.5 else 0


def decode_cases(seed, n):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        c = draw_shape(rng, [1, 16, 33, 64, 128])
        c["cape"] = cape_heads(c, rng)
        c["steps"] = rng.choice([3, 10, 30])
        c["masked"] = rng.random() < 0.5
        out.append(c)
    return out


def gated_cases(seed, n):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        c = draw_shape(rng, [16, 33, 64, 128])
        c["cape"] = cape_heads(c, rng)
        c["B"] = min(c["B"], 3)
        c["kr"] = max(c["kr"], 2)
        c["T"] = rng.choice([1, 3, 40, 300])
        c["masked"] = rng.random() < 0.5
        c["state"] = c["T"] == 1 or rng.random() < 0.5
        c["gain"] = rng.random() < 0.7
        c["rms_eps"] = rng.choice([1e-6, 1e-5, 0.25])
        out.append(c)
    return out


def problem_of(c, T):
    return ram.problem(c["B"], c["H"], T, None if c["U"] > 1 else c["S"], c["kw"], c["kr"], c["d"],
                       io=c["io"], eps=c["eps"], renorm=c["rn"], cape_heads=c["cape"],
                       t0=c["t0"], U=c["U"], P=c["P"])


DECODE = decode_cases(3, 24)
GATED = gated_cases(4, 16)


@pytest.mark.parametrize("case", range(len(DECODE)))
def test_random_decode_steps(case):
    c = dict(DECODE[case])
    say("random decode steps", case, c)
    B, H, S, d = c["B"], c["H"], c["S"], c["d"]
    cfg = synth.Config("steps", B, H, 1, S, c["kw"], c["kr"], d, c["io"], U=c["U"])
    slot, mass = synth.decode_state(cfg, device=DEV, seed=case)
    gen = torch.Generator(device="cpu").manual_seed(5000 + case)
    mass.copy_((3.0 * torch.rand((B, H, S), generator=gen)).to(DEV))
    o_slot, o_mass = np.ascontiguousarray(host(slot)), np.ascontiguousarray(host(mass))
    o = torch.empty((B, 1, H, d), dtype=cfg.dtype, device=DEV)
    tol = TOL[c["io"]]
    for step in range(c["steps"]):
        x = synth.decode_step_inputs(cfg, step, device=DEV, seed=case)
        mask = None
        if c["masked"]:
            mask = (torch.rand((B,), generator=gen) > 0.3).to(torch.uint8).to(DEV)
        p = problem_of(dict(c, t0=c["t0"] + step), 1)
        ram.ram_decode_step(p, x["wl"], x["rl"], x["v"], x["gamma"], slot, mass, o, mask=mask)
        torch.cuda.synchronize()
        h = {k: host(v) for k, v in x.items()}
        hm = None if mask is None else mask.cpu().numpy()
        ref = oracle.decode_step(oracle_problem(p), h["wl"], h["rl"], h["v"], h["gamma"], o_slot,
                                 o_mass, mask=hm)
        got = host(o)
        assert frel(got, ref) <= tol, step
        if hm is not None:
            assert np.all(got[hm == 0] == 0), step
    assert frel(host(slot), o_slot) <= tol
    assert frel(host(mass), o_mass) <= tol


@pytest.mark.parametrize("case", range(len(GATED)))
def test_random_gated_readout(case):
    c = GATED[case]
    say("random gated read-out", case, c)
    B, H, T, S, d = c["B"], c["H"], c["T"], c["S"], c["d"]
    cfg = synth.Config("gated", B, H, T, S, c["kw"], c["kr"], d, c["io"], U=c["U"])
    x = synth.layer_inputs(cfg, device=DEV, seed=700 + case, with_state=True)
    gx = synth.gate_inputs(cfg, device=DEV, seed=700 + case)
    p = problem_of(c, T)
    gen = torch.Generator(device="cpu").manual_seed(case)
    mask = (torch.rand((B, T), generator=gen) > 0.2).to(torch.uint8).to(DEV) if c["masked"] else None
    gain = gx["gain"] if c["gain"] else None
    ep = ram.epilogue(p, gx["gate"], gain, c["rms_eps"])
    s0, m0 = (x["slot0"], x["mass0"]) if c["state"] else (None, None)
    ws = ram.workspace(p, True, DEV)
    y = torch.empty_like(x["v"])
    s1 = torch.empty((B, H, S, d), device=DEV)
    m1 = torch.empty((B, H, S), device=DEV)
    ram.ram_forward_gated(p, ep, x["wl"], x["rl"], x["v"], x["gamma"], s0, m0, y, s1, m1, ws,
                          mask=mask)
    g = {"d_wlogits": torch.empty_like(x["wl"]), "d_rlogits": torch.empty_like(x["rl"]),
         "d_v": torch.empty_like(x["v"]), "d_gamma": torch.empty_like(x["gamma"]),
         "d_gate": torch.empty_like(gx["gate"]),
         "d_gain": torch.empty((d,), dtype=torch.float32, device=DEV)}
    ram.ram_backward_gated(p, ep, ws, x["wl"], x["rl"], x["v"], x["gamma"], s0, m0, gx["d_y"],
                           None, None, g["d_wlogits"], g["d_rlogits"], g["d_v"], g["d_gamma"],
                           g["d_gate"], g["d_gain"] if c["gain"] else None, mask=mask)
    torch.cuda.synchronize()
    h = {k: host(v) for k, v in x.items()}
    hg = {k: host(v) for k, v in gx.items()}
    op = oracle_problem(p)
    hm = mask.cpu().numpy() if c["masked"] else None
    h_gain = hg["gain"] if c["gain"] else None
    hs0, hm0 = (h["slot0"], h["mass0"]) if c["state"] else (None, None)
    oo, os_, om = oracle.forward(op, h["wl"], h["rl"], h["v"], h["gamma"], hs0, hm0, mask=hm)
    yy = oracle.epilogue_forward(oo, hg["gate"], h_gain, c["rms_eps"])
    d_o, d_gate, d_gain = oracle.epilogue_backward(oo, hg["gate"], hg["d_y"], h_gain, c["rms_eps"])
    if hm is not None:
        # a masked token is absent: no gradient reaches its gate
        d_gate = d_gate * np.asarray(hm, np.float64)[:, :, None, None]
    rg = oracle.backward(op, h["wl"], h["rl"], h["v"], h["gamma"], hs0, hm0, d_o, None, None,
                         mask=hm)
    tol = TOL[c["io"]]
    checks = [("y", y, yy), ("slot1", s1, os_), ("mass1", m1, om), ("d_v", g["d_v"], rg["d_v"]),
              ("d_gamma", g["d_gamma"], rg["d_gamma"]), ("d_gate", g["d_gate"], d_gate)]
    if c["gain"]:
        checks.append(("d_gain", g["d_gain"], d_gain))
    for name, got, ref in checks:
        assert frel(host(got), ref) <= tol, name
    check_grads(g, rg, op, h, tol, ("d_wlogits", "d_rlogits"))
