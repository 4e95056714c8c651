"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
run the CPU oracle on the same inputs (or on one (b, h) slice of them)."""
import sys
import time

import numpy as np
import torch

import linear_attention_ram_amd as ram
import oracle
import parity
from parity import rel  # noqa: F401  (re-exported for the tests)

TOL = {"f32": 1e-5, "bf16": 2e-2}


def say(*a):
    print(time.strftime("%H:%M:%S"), *a, flush=True)
    sys.stdout.flush()


def host(t):
    return t.detach().double().cpu().numpy()


def check_grads(got, ref, op, h, tol, names=("d_wlogits", "d_rlogits", "d_v", "d_gamma")):
    """Gradients against the oracle's: the logit gradients with the split bar
    of parity.check_logit_grad (selected entries normwise, the dense term
    against its scale p_i * sum_j |g_j w_j|), the others normwise.  got: name -> tensor or host array; h:
    the host inputs the oracle ran on (its decode gives the selected slots)."""
    for name in names:
        x = host(got[name]) if isinstance(got[name], torch.Tensor) else got[name]
        if name in ("d_wlogits", "d_rlogits"):
            side = 0 if name == "d_wlogits" else 1
            logits = h["wl" if side == 0 else "rl"]
            idx, w, lse = oracle.decode(op, side, logits)
            U, P = int(op.U), int(op.P)
            sel = parity.selected_entries(idx, U, P, int(op.cape_heads), int(op.t0))
            renorm = bool(op.renorm_w if side == 0 else op.renorm_r)
            gw = parity.gw_products(ref["dw" if side == 0 else "dr"], w, renorm)
            scale = parity.dense_scale(logits, lse, gw, U, P)
            parity.check_logit_grad(x, ref[name], sel, tol, name, scale)
        else:
            err = rel(x, ref[name])
            assert err <= tol, (name, err)


def gpu_problem(cfg, T=None, eps=None, renorm=(False, False), cape_heads=0, t0=0):
    return ram.problem(cfg.B, cfg.H, cfg.T if T is None else T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v,
                       io=cfg.io, eps=cfg.eps if eps is None else eps, renorm=renorm,
                       cape_heads=cape_heads, t0=t0, U=cfg.U, P=cfg.P)


def oracle_problem(gp, B=None, H=None, cape_heads=None):
    """Oracle problem of a GPU problem.  With H given (a slice of heads) the
    CAPE head count must be given too (it depends on which heads)."""
    cape = int(gp.cape_heads) if cape_heads is None else cape_heads
    return oracle.problem(gp.B if B is None else B, gp.H if H is None else H, gp.T, gp.S,
                          gp.k_w, gp.k_r, gp.d_v, U=int(gp.U), P=int(gp.P), eps=float(gp.eps),
                          renorm=(bool(gp.renorm_w), bool(gp.renorm_r)),
                          cape_heads=cape, t0=int(gp.t0))


def run_forward(p, x, ws=None, slot0=None, mass0=None):
    dev = x["v"].device
    if ws is None:
        ws = ram.workspace(p, True, dev)
    o = torch.empty_like(x["v"])
    nseg = p.B * p.H * p.S
    slot1 = torch.empty((p.B, p.H, p.S, p.d_v), dtype=torch.float32, device=dev)
    mass1 = torch.empty((p.B, p.H, p.S), dtype=torch.float32, device=dev)
    assert slot1.numel() == nseg * p.d_v
    ram.ram_forward(p, x["wl"], x["rl"], x["v"], x["gamma"], slot0, mass0, o, slot1, mass1, ws)
    return {"o": o, "slot1": slot1, "mass1": mass1, "ws": ws}


def run_backward(p, x, ws, slot0=None, mass0=None, d_slot1=None, d_mass1=None, want_state=False):
    g = {"d_wlogits": torch.empty_like(x["wl"]), "d_rlogits": torch.empty_like(x["rl"]),
         "d_v": torch.empty_like(x["v"]), "d_gamma": torch.empty_like(x["gamma"]),
         "d_slot0": None, "d_mass0": None}
    if want_state:
        dev = x["v"].device
        g["d_slot0"] = torch.empty((p.B, p.H, p.S, p.d_v), dtype=torch.float32, device=dev)
        g["d_mass0"] = torch.empty((p.B, p.H, p.S), dtype=torch.float32, device=dev)
    ram.ram_backward(p, ws, x["wl"], x["rl"], x["v"], x["gamma"], slot0, mass0, x["d_o"],
                     d_slot1, d_mass1, g["d_wlogits"], g["d_rlogits"], g["d_v"], g["d_gamma"],
                     g["d_slot0"], g["d_mass0"])
    return g


def bh_slice(x, b, h):
    """Host float64 arrays of one (b, h) problem: shapes with B = H = 1."""
    out = {}
    for k in ("wl", "rl", "v", "d_o"):
        if k in x:
            out[k] = host(x[k][b:b + 1, :, h:h + 1])
    out["gamma"] = host(x["gamma"][b:b + 1, :, h:h + 1])
    for k in ("slot0", "d_slot1"):
        if x.get(k) is not None:
            out[k] = host(x[k][b:b + 1, h:h + 1])
    for k in ("mass0", "d_mass1"):
        if x.get(k) is not None:
            out[k] = host(x[k][b:b + 1, h:h + 1])
    return out


def decode_event_codes(codes):
    codes = np.asarray(codes, np.int64)
    return codes >> 7, (codes >> 6) & 1, codes & 63
