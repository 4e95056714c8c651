"""GPU parity of the token mask (ramnet-ops "Arguments", mask) against the
oracle: a masked token writes and reads nothing, its output row is exactly 0
and every gradient of it is exactly 0; everything else matches the oracle
within the io dtype's tolerance."""
import numpy as np
import pytest
import torch

import linear_attention_ram_amd as ram
import oracle
from gpu_util import TOL, check_grads, gpu_problem, host, oracle_problem, rel, say
from linear_attention_ram_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def random_mask(B, T, seed, frac=0.3):
    g = torch.Generator(device="cpu").manual_seed(seed)
    m = (torch.rand((B, T), generator=g) >= frac).to(torch.uint8)
    m[0, :3] = 0
    return m.to(DEV)


def run(cfg, x, p, mask, with_state):
    slot0 = x["slot0"] if with_state else None
    mass0 = x["mass0"] if with_state else None
    ws = ram.workspace(p, True, DEV)
    o = torch.empty_like(x["v"])
    slot1 = torch.empty((p.B, p.H, p.S, p.d_v), dtype=torch.float32, device=DEV)
    mass1 = torch.empty((p.B, p.H, p.S), dtype=torch.float32, device=DEV)
    ram.ram_forward(p, x["wl"], x["rl"], x["v"], x["gamma"], slot0, mass0, o, slot1, mass1, ws,
                    mask=mask)
    g = {"d_wlogits": torch.empty_like(x["wl"]), "d_rlogits": torch.empty_like(x["rl"]),
         "d_v": torch.empty_like(x["v"]), "d_gamma": torch.empty_like(x["gamma"])}
    ram.ram_backward(p, ws, x["wl"], x["rl"], x["v"], x["gamma"], slot0, mass0, x["d_o"],
                     None, None, g["d_wlogits"], g["d_rlogits"], g["d_v"], g["d_gamma"], mask=mask)
    torch.cuda.synchronize()
    return o, slot1, mass1, g


def check(cfg, x, p, mask, with_state, tol):
    o, slot1, mass1, g = run(cfg, x, p, mask, with_state)
    h = {k: host(v) for k, v in x.items()}
    mk = mask.cpu().numpy()
    op = oracle_problem(p)
    say("oracle masked forward/backward", cfg.name)
    oo, os_, om = oracle.forward(op, h["wl"], h["rl"], h["v"], h["gamma"],
                                 h["slot0"] if with_state else None,
                                 h["mass0"] if with_state else None, mask=mk)
    assert rel(host(o), oo) <= tol
    assert rel(host(slot1), os_) <= tol
    assert rel(host(mass1), om) <= tol
    rg = oracle.backward(op, h["wl"], h["rl"], h["v"], h["gamma"],
                         h["slot0"] if with_state else None, h["mass0"] if with_state else None,
                         h["d_o"], mask=mk)
    check_grads(g, rg, op, h, tol)
    off = mk == 0
    assert not np.any(host(o)[off])
    for name in ("d_wlogits", "d_rlogits", "d_v", "d_gamma"):
        assert not np.any(host(g[name])[off]), name


@pytest.mark.parametrize("with_state", [False, True])
def test_small_fp32(with_state):
    cfg = synth.Config("mask-small", 3, 2, 150, 64, 4, 3, 16, "f32")
    x = synth.layer_inputs(cfg, device=DEV, seed=31, with_state=True)
    check(cfg, x, gpu_problem(cfg), random_mask(3, 150, 1), with_state, TOL["f32"])


def test_340m_bf16():
    cfg = synth.CONFIGS["340m"]
    x = synth.layer_inputs(cfg, device=DEV, seed=32)
    check(cfg, x, gpu_problem(cfg), random_mask(cfg.B, cfg.T, 2), False, TOL["bf16"])


def test_all_masked_keeps_state_bitwise():
    cfg = synth.Config("mask-all", 2, 2, 64, 32, 3, 2, 16, "bf16")
    x = synth.layer_inputs(cfg, device=DEV, seed=33, with_state=True)
    mask = torch.zeros((2, 64), dtype=torch.uint8, device=DEV)
    o, slot1, mass1, g = run(cfg, x, gpu_problem(cfg), mask, True)
    assert torch.equal(slot1, x["slot0"]) and torch.equal(mass1, x["mass0"])
    assert not torch.any(o.float() != 0)
    for t in g.values():
        assert not torch.any(t.float() != 0)


def test_masked_decode_steps():
    cfg = synth.Config("mask-step", 4, 2, 1, 64, 4, 3, 16, "f32")
    slot, mass = synth.decode_state(cfg, device=DEV, seed=0)
    o_slot, o_mass = np.ascontiguousarray(host(slot)), np.ascontiguousarray(host(mass))
    p = ram.problem(cfg.B, cfg.H, 1, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, io="f32")
    op = oracle.problem(cfg.B, cfg.H, 1, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v)
    o = torch.empty((cfg.B, 1, cfg.H, cfg.d_v), dtype=torch.float32, device=DEV)
    for step in range(20):
        x = synth.decode_step_inputs(cfg, step, device=DEV, seed=0)
        mask = torch.tensor([1, step % 2, 1, (step // 3) % 2], dtype=torch.uint8, device=DEV)
        ram.ram_decode_step(p, x["wl"], x["rl"], x["v"], x["gamma"], slot, mass, o, mask=mask)
        torch.cuda.synchronize()
        h = {k: host(v) for k, v in x.items()}
        ref = oracle.decode_step(op, h["wl"], h["rl"], h["v"], h["gamma"], o_slot, o_mass,
                                 mask=mask.cpu().numpy())
        assert rel(host(o), ref) <= TOL["f32"], step
    assert rel(host(slot), o_slot) <= TOL["f32"]
    assert rel(host(mass), o_mass) <= TOL["f32"]


@pytest.mark.parametrize("with_state", [False, True])
def test_nan_inputs_at_masked_tokens(with_state):
    # a masked token is absent, so whatever its rows hold (NaN here: logits
    # of both sides, v, gamma and d_o) reaches nothing; hot slots put its
    # no-op events on the cooperative scan path as well
    cfg = synth.Config("mask-nan", 2, 3, 700, 128, 8, 8, 64, "bf16", zipf=1.1)
    x = synth.layer_inputs(cfg, device=DEV, seed=34, with_state=True)
    mask = random_mask(cfg.B, cfg.T, 3)
    off = mask == 0
    for key in ("wl", "rl", "v", "gamma", "d_o"):
        x[key][off] = float("nan")
    o, slot1, mass1, g = run(cfg, x, gpu_problem(cfg), mask, with_state)
    assert torch.all(torch.isfinite(slot1)) and torch.all(torch.isfinite(mass1))
    assert torch.all(torch.isfinite(o.float()))
    for name, t in g.items():
        assert torch.all(torch.isfinite(t.float())), name
    check(cfg, x, gpu_problem(cfg), mask, with_state, TOL["bf16"])
