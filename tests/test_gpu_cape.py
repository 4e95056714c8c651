"""GPU parity of CAPE (ramnet-ops "Quick start": the first embed_num heads
address the content-selected slot shifted cyclically by the token's absolute
position; paper App. C) against the oracle: addressed slots bit-exact,
outputs, state and gradients within the io dtype's tolerance."""
import numpy as np
import pytest
import torch

import linear_attention_ram_amd as ram
import oracle
from gpu_util import (TOL, check_grads, gpu_problem, host, oracle_problem, rel, run_backward,
                      run_forward, say)
from linear_attention_ram_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("side", [0, 1])
def test_decode_addresses_shifted_slots(side):
    cfg = synth.Config("cape-dec", 2, 3, 37, 64, 4, 3, 16, "f32")
    x = synth.layer_inputs(cfg, device=DEV, seed=21, with_d_o=False)
    p = gpu_problem(cfg, cape_heads=2, t0=1000)
    k = cfg.k_w if side == 0 else cfg.k_r
    N = cfg.B * cfg.T * cfg.H
    idx = torch.empty((N, k), dtype=torch.int32, device=DEV)
    w = torch.empty((N, k), dtype=torch.float32, device=DEV)
    lse = torch.empty((N,), dtype=torch.float32, device=DEV)
    logits = x["wl"] if side == 0 else x["rl"]
    ram.ram_decode(p, side, logits, idx, w, lse)
    torch.cuda.synchronize()
    oi, ow, olse = oracle.decode(oracle_problem(p), side, host(logits))
    np.testing.assert_array_equal(idx.cpu().numpy().reshape(oi.shape), oi)
    assert rel(w.cpu().numpy().reshape(ow.shape), ow) <= 1e-5
    # the non-CAPE head is unshifted, the CAPE heads are not (t0 + t = 1000.. mod 64 != 0)
    plain = oracle.decode(oracle_problem(p, cape_heads=0), side, host(logits))[0]
    assert np.array_equal(oi[:, :, 2], plain[:, :, 2])
    assert not np.array_equal(oi[:, :, :2], plain[:, :, :2])


def full_fwd_bwd(cfg, p, x, tol, with_state):
    slot0 = x["slot0"] if with_state else None
    mass0 = x["mass0"] if with_state else None
    ds1 = x["d_slot1"] if with_state else None
    dm1 = x["d_mass1"] if with_state else None
    r = run_forward(p, x, slot0=slot0, mass0=mass0)
    g = run_backward(p, x, r["ws"], slot0, mass0, ds1, dm1, want_state=with_state)
    torch.cuda.synchronize()
    h = {k: host(v) for k, v in x.items()}
    op = oracle_problem(p)
    say("oracle forward/backward", cfg.name, "cape_heads", p.cape_heads, "t0", p.t0)
    oo, os_, om = oracle.forward(op, h["wl"], h["rl"], h["v"], h["gamma"],
                                 h.get("slot0") if with_state else None,
                                 h.get("mass0") if with_state else None)
    assert rel(host(r["o"]), oo) <= tol
    assert rel(host(r["slot1"]), os_) <= tol
    assert rel(host(r["mass1"]), om) <= tol
    views = ram.ws_views(p, r["ws"])
    iw, _, _ = oracle.decode(op, 0, h["wl"])
    np.testing.assert_array_equal(views["idx_w"].cpu().numpy().reshape(iw.shape), iw)
    rg = oracle.backward(op, h["wl"], h["rl"], h["v"], h["gamma"],
                         h.get("slot0") if with_state else None, h.get("mass0") if with_state else None,
                         h["d_o"], h.get("d_slot1") if with_state else None,
                         h.get("d_mass1") if with_state else None)
    check_grads(g, rg, op, h, tol)
    if with_state:
        assert rel(host(g["d_slot0"]), rg["d_slot0"]) <= tol
        assert rel(host(g["d_mass0"]), rg["d_mass0"]) <= tol


@pytest.mark.parametrize("with_state", [False, True])
def test_small_fp32_fwd_bwd(with_state):
    cfg = synth.Config("cape-small", 2, 4, 200, 64, 4, 3, 16, "f32")
    x = synth.layer_inputs(cfg, device=DEV, seed=22, with_state=True, with_state_grads=True)
    full_fwd_bwd(cfg, gpu_problem(cfg, cape_heads=2, t0=77), x, TOL["f32"], with_state)


def test_340m_bf16_fwd_bwd():
    cfg = synth.CONFIGS["340m"]
    x = synth.layer_inputs(cfg, device=DEV, seed=23)
    full_fwd_bwd(cfg, gpu_problem(cfg, cape_heads=4, t0=5000), x, TOL["bf16"], False)


def test_chunks_carry_the_position():
    # three calls of 32 tokens with t0 advancing give the one-call result
    cfg = synth.Config("cape-chunks", 1, 2, 96, 32, 3, 2, 16, "f32")
    x = synth.layer_inputs(cfg, device=DEV, seed=24, with_d_o=False)
    p_all = gpu_problem(cfg, cape_heads=1, t0=11)
    r_all = run_forward(p_all, x)
    slot = torch.zeros((1, 2, 32, 16), dtype=torch.float32, device=DEV)
    mass = torch.zeros((1, 2, 32), dtype=torch.float32, device=DEV)
    outs = []
    for c in range(3):
        sub = {k: v[:, 32 * c:32 * (c + 1)].contiguous() for k, v in x.items()}
        p = gpu_problem(cfg, T=32, cape_heads=1, t0=11 + 32 * c)
        r = run_forward(p, sub, slot0=slot, mass0=mass)
        slot, mass = r["slot1"], r["mass1"]
        outs.append(r["o"])
    torch.cuda.synchronize()
    assert rel(host(torch.cat(outs, 1)), host(r_all["o"])) <= 1e-6
    assert rel(host(slot), host(r_all["slot1"])) <= 1e-6
    h = {k: host(v) for k, v in x.items()}
    oo, _, _ = oracle.forward(oracle_problem(p_all), h["wl"], h["rl"], h["v"], h["gamma"])
    assert rel(host(r_all["o"]), oo) <= TOL["f32"]


def test_decode_steps_with_positions():
    cfg = synth.Config("cape-step", 3, 2, 1, 64, 4, 3, 16, "f32")
    slot, mass = synth.decode_state(cfg, device=DEV, seed=0)
    o_slot, o_mass = np.ascontiguousarray(host(slot)), np.ascontiguousarray(host(mass))
    o = torch.empty((cfg.B, 1, cfg.H, cfg.d_v), dtype=torch.float32, device=DEV)
    for step in range(24):
        x = synth.decode_step_inputs(cfg, step, device=DEV, seed=0)
        p = ram.problem(cfg.B, cfg.H, 1, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, io="f32",
                        cape_heads=1, t0=300 + step)
        ram.ram_decode_step(p, x["wl"], x["rl"], x["v"], x["gamma"], slot, mass, o)
        torch.cuda.synchronize()
        h = {k: host(v) for k, v in x.items()}
        op = oracle.problem(cfg.B, cfg.H, 1, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, cape_heads=1,
                            t0=300 + step)
        ref = oracle.decode_step(op, h["wl"], h["rl"], h["v"], h["gamma"], o_slot, o_mass)
        assert rel(host(o), ref) <= TOL["f32"], step
    assert rel(host(slot), o_slot) <= TOL["f32"]
    assert rel(host(mass), o_mass) <= TOL["f32"]
