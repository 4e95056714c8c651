"""GPU parity over seeded random shapes of the other paths: product
addresses of U = 1, 2 or 3 digits, token masks, CAPE heads at random
positions, renormalised sides, with and without the initial state; forward
and backward against the oracle with the bars of the other parity tests
(relative errors floored at 1e-9 where an exact gradient is zero)."""
import random

import numpy as np
import pytest
import torch

import linear_attention_ram_amd as ram
import oracle
import parity
from gpu_util import TOL, host, oracle_problem, say
from linear_attention_ram_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FLOOR = 1e-9


def frel(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), FLOOR))


def cases(seed, n):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        U = rng.choice([1, 1, 2, 2, 3])
        if U == 1:
            P = rng.choice([16, 64, 256, 1024])
        elif U == 2:
            P = rng.choice([8, 16, 32, 64])
        else:
            P = rng.choice([8, 16])
        S = P ** U
        io = rng.choice(["f32", "bf16"])
        B, H = rng.randint(1, 3), rng.randint(1, 4)
        T = rng.choice([1, 3, 40, 300])
        kw, kr = rng.randint(1, min(S, 12)), rng.randint(1, min(S, 12))
        d = rng.choice([1, 16, 33, 64, 128])
        rn = (rng.random() < 0.3, rng.random() < 0.3)
        eps = rng.choice([1e-6, 1e-3])
        cape = rng.randint(0, H) if rng.random() < 0.5 else 0
        t0 = rng.randint(0, 5000)
        out.append((B, H, T, U, P, kw, kr, d, io, rn, eps, cape, t0, rng.random() < 0.5,
                    rng.random() < 0.5))
    return out


@pytest.mark.parametrize("case", range(24))
def test_random_features(case):
    B, H, T, U, P, kw, kr, d, io, rn, eps, cape, t0, masked, state = cases(1, 24)[case]
    say("random features", case, cases(1, 24)[case])
    S = P ** U
    cfg = synth.Config("features", B, H, T, S, kw, kr, d, io, U=U)
    x = synth.layer_inputs(cfg, device=DEV, seed=900 + case, with_state=True, with_state_grads=True)
    p = ram.problem(B, H, T, None if U > 1 else S, kw, kr, d, io=io, eps=eps, renorm=rn,
                    cape_heads=cape, t0=t0, U=U, P=P)
    gen = torch.Generator(device="cpu").manual_seed(case)
    mask = (torch.rand((B, T), generator=gen) > 0.2).to(torch.uint8).to(DEV) if masked else None
    s0, m0 = (x["slot0"], x["mass0"]) if state else (None, None)
    ws = ram.workspace(p, True, DEV)
    o = torch.empty_like(x["v"])
    s1 = torch.empty((B, H, S, d), device=DEV)
    m1 = torch.empty((B, H, S), device=DEV)
    ram.ram_forward(p, x["wl"], x["rl"], x["v"], x["gamma"], s0, m0, o, s1, m1, ws, mask=mask)
    g = {"d_wlogits": torch.empty_like(x["wl"]), "d_rlogits": torch.empty_like(x["rl"]),
         "d_v": torch.empty_like(x["v"]), "d_gamma": torch.empty_like(x["gamma"])}
    ds0 = torch.empty((B, H, S, d), device=DEV) if state else None
    dm0 = torch.empty((B, H, S), device=DEV) if state else None
    ram.ram_backward(p, ws, x["wl"], x["rl"], x["v"], x["gamma"], s0, m0, x["d_o"], x["d_slot1"],
                     x["d_mass1"], g["d_wlogits"], g["d_rlogits"], g["d_v"], g["d_gamma"], ds0, dm0,
                     mask=mask)
    torch.cuda.synchronize()
    h = {k: host(v) for k, v in x.items()}
    op = oracle_problem(p)
    hm = mask.cpu().numpy() if masked else None
    hs0, hm0 = (h["slot0"], h["mass0"]) if state else (None, None)
    oo, os_, om = oracle.forward(op, h["wl"], h["rl"], h["v"], h["gamma"], hs0, hm0, mask=hm)
    rg = oracle.backward(op, h["wl"], h["rl"], h["v"], h["gamma"], hs0, hm0, h["d_o"],
                         h["d_slot1"], h["d_mass1"], mask=hm)
    tol = TOL[io]
    for name, got, ref in (("o", o, oo), ("slot1", s1, os_), ("mass1", m1, om),
                           ("d_v", g["d_v"], rg["d_v"]), ("d_gamma", g["d_gamma"], rg["d_gamma"])):
        assert frel(host(got), ref) <= tol, name
    views = ram.ws_views(p, ws)
    for name in ("dw", "dr"):
        assert frel(views[name].cpu().numpy().reshape(rg[name].shape), rg[name]) <= 1e-4, name
    if state:
        assert frel(host(ds0), rg["d_slot0"]) <= tol
        assert frel(host(dm0), rg["d_mass0"]) <= tol
    for name, side in (("d_wlogits", 0), ("d_rlogits", 1)):
        gw_ref = rg["dw" if side == 0 else "dr"]
        if float(np.max(np.abs(gw_ref))) < FLOOR:
            continue
        logits = h["wl" if side == 0 else "rl"]
        idx, w, lse = oracle.decode(op, side, logits)
        sel = parity.selected_entries(idx, U, P, cape, t0)
        scale = parity.dense_scale(logits, lse, parity.gw_products(gw_ref, w, rn[side]), U, P)
        parity.check_logit_grad(host(g[name]), rg[name], sel, tol, name, scale)
