"""GPU parity of the forward and backward over seeded random small shapes:
slot counts from 8 to 1024, 1 to 600 tokens, k up to 16, widths from 1 to
128 (rows of whole 16-byte vectors or not), both io dtypes, renormalised
sides, eps of 0, 1e-3 and 1e-6, with and without the hot-slot bias, the
initial state and the final state's gradients.  The bars are those of the
other parity tests; where an exact gradient is zero (eps = 0 and every
write a slot's first: the fp64 reference then holds rounding noise of
1e-16) the relative error is taken against a floor of 1e-9."""
import random

import numpy as np
import pytest
import torch

import linear_attention_ram_amd as ram
import oracle
from gpu_util import TOL, check_grads, host, oracle_problem, run_backward, run_forward, say
from linear_attention_ram_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FLOOR = 1e-9


def frel(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), FLOOR))


def shapes(seed, n):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        io = rng.choice(["f32", "bf16"])
        S = rng.choice([8, 16, 24, 32, 64, 128, 256, 512, 1024])
        B, H = rng.randint(1, 3), rng.randint(1, 3)
        T = rng.choice([1, 2, 5, 17, 64, 200, 600])
        kw, kr = rng.randint(1, min(S, 16)), rng.randint(1, min(S, 16))
        d = rng.choice([1, 3, 8, 16, 33, 64, 66, 96, 128])
        rn = (rng.random() < 0.3, rng.random() < 0.3)
        eps = rng.choice([1e-6, 1e-3, 0.0])
        zipf = rng.choice([None, None, 1.1])
        out.append((B, H, T, S, kw, kr, d, io, rn, eps, zipf, rng.random() < 0.5, rng.random() < 0.5))
    return out


@pytest.mark.parametrize("case", range(24))
def test_random_shape(case):
    B, H, T, S, kw, kr, d, io, rn, eps, zipf, with_state, with_grads = shapes(2026, 24)[case]
    say("random shape", case, (B, H, T, S, kw, kr, d, io, rn, eps, zipf, with_state, with_grads))
    cfg = synth.Config("random", B, H, T, S, kw, kr, d, io, zipf=zipf)
    x = synth.layer_inputs(cfg, device=DEV, seed=500 + case, with_state=True, with_state_grads=True)
    p = ram.problem(B, H, T, S, kw, kr, d, io=io, eps=eps, renorm=rn)
    s0, m0 = (x["slot0"], x["mass0"]) if with_state else (None, None)
    ds1, dm1 = (x["d_slot1"], x["d_mass1"]) if with_grads else (None, None)
    r = run_forward(p, x, slot0=s0, mass0=m0)
    g = run_backward(p, x, r["ws"], s0, m0, ds1, dm1, want_state=with_state)
    torch.cuda.synchronize()
    h = {k: host(v) for k, v in x.items()}
    op = oracle_problem(p)
    hs0, hm0 = (h["slot0"], h["mass0"]) if with_state else (None, None)
    oo, os_, om = oracle.forward(op, h["wl"], h["rl"], h["v"], h["gamma"], hs0, hm0)
    rg = oracle.backward(op, h["wl"], h["rl"], h["v"], h["gamma"], hs0, hm0, h["d_o"],
                         h["d_slot1"] if with_grads else None, h["d_mass1"] if with_grads else None)
    tol = TOL[io]
    assert frel(host(r["o"]), oo) <= tol
    assert frel(host(r["slot1"]), os_) <= tol
    assert frel(host(r["mass1"]), om) <= tol
    views = ram.ws_views(p, r["ws"])
    for name in ("dw", "dr"):
        assert frel(views[name].cpu().numpy().reshape(rg[name].shape), rg[name]) <= 1e-4, name
    for name in ("d_v", "d_gamma"):
        assert frel(host(g[name]), rg[name]) <= tol, name
    # the logit gradients' bar is relative to the weight gradients' scale,
    # which an all-zero exact dw or dr does not have
    if min(float(np.max(np.abs(rg["dw"]))), float(np.max(np.abs(rg["dr"])))) >= FLOOR:
        check_grads(g, rg, op, h, tol, names=("d_wlogits", "d_rlogits"))
    if with_state:
        assert frel(host(g["d_slot0"]), rg["d_slot0"]) <= tol
        assert frel(host(g["d_mass0"]), rg["d_mass0"]) <= tol
