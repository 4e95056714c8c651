"""GPU parity of ram_decode_step (one token per (b, h), state updated in
place) against the oracle's autoregressive step."""
import numpy as np
import pytest
import torch

import linear_attention_ram_amd as ram
import oracle
from gpu_util import TOL, host, rel, say
from linear_attention_ram_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_steps(cfg, nsteps, seqs, io_tol, state_tol=None, report_every=0):
    """nsteps autoregressive steps of the whole batch on the GPU; the oracle
    takes the same steps on the sequences `seqs`.  o of those sequences is
    compared at every step (io_tol), their final state at the end
    (state_tol, default io_tol)."""
    state_tol = io_tol if state_tol is None else state_tol
    slot, mass = synth.decode_state(cfg, device=DEV, seed=0)
    p = ram.problem(cfg.B, cfg.H, 1, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, io=cfg.io, eps=cfg.eps)
    op = oracle.problem(len(seqs), cfg.H, 1, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, eps=cfg.eps)
    o_slot = np.ascontiguousarray(host(slot[seqs]))
    o_mass = np.ascontiguousarray(host(mass[seqs]))
    o = torch.empty((cfg.B, 1, cfg.H, cfg.d_v), dtype=cfg.dtype, device=DEV)
    worst = 0.0
    for step in range(nsteps):
        x = synth.decode_step_inputs(cfg, step, device=DEV, seed=0)
        ram.ram_decode_step(p, x["wl"], x["rl"], x["v"], x["gamma"], slot, mass, o)
        torch.cuda.synchronize()
        h = {k: host(v[seqs]) for k, v in x.items()}
        ref = oracle.decode_step(op, h["wl"], h["rl"], h["v"], h["gamma"], o_slot, o_mass)
        err = rel(host(o[seqs]), ref)
        worst = max(worst, err)
        assert err <= io_tol, (step, err)
        if report_every and (step + 1) % report_every == 0:
            say("step", step + 1, "of", nsteps, "worst o error so far", worst)
    assert rel(host(slot[seqs]), o_slot) <= state_tol
    assert rel(host(mass[seqs]), o_mass) <= state_tol


def test_small_fp32():
    cfg = synth.Config("small", 5, 3, 1, 64, 4, 3, 16, "f32")
    run_steps(cfg, 40, list(range(5)), TOL["f32"])


def test_small_bf16_wide():
    cfg = synth.Config("wide", 3, 2, 1, 1024, 8, 8, 128, "bf16")
    run_steps(cfg, 30, list(range(3)), TOL["bf16"])


def test_many_read_slots():
    # more read slots than the step requests before its write phase
    cfg = synth.Config("many-reads", 3, 2, 1, 256, 5, 13, 96, "f32")
    run_steps(cfg, 25, list(range(3)), TOL["f32"])


def test_decode_config_full_horizon():
    # the decode configuration over its whole length: all 1,024 steps of the
    # 256-sequence batch on the GPU, the oracle on sequences 0-15 (every
    # sequence is independent); mass grows and step sizes shrink over the
    # horizon, so drift would show in o at the late steps or in the state
    cfg = synth.CONFIGS["decode"]
    say("decode config: 1024 steps, oracle on sequences 0-15")
    run_steps(cfg, cfg.steps, list(range(16)), TOL["bf16"], state_tol=1e-4, report_every=128)


def test_steps_match_parallel_forward():
    # T decode steps reproduce one parallel forward over the same T tokens
    cfg = synth.Config("chain", 2, 2, 48, 32, 3, 2, 16, "f32")
    x = synth.layer_inputs(cfg, device=DEV, seed=3, with_state=True, with_d_o=False)
    p = ram.problem(cfg.B, cfg.H, cfg.T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, io="f32")
    ws = ram.workspace(p, False, DEV)
    o = torch.empty_like(x["v"])
    slot1 = torch.empty_like(x["slot0"])
    mass1 = torch.empty_like(x["mass0"])
    ram.ram_forward(p, x["wl"], x["rl"], x["v"], x["gamma"], x["slot0"], x["mass0"], o, slot1,
                    mass1, ws)
    ps = ram.problem(cfg.B, cfg.H, 1, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, io="f32")
    slot, mass = x["slot0"].clone(), x["mass0"].clone()
    os_ = torch.empty((cfg.B, 1, cfg.H, cfg.d_v), device=DEV)
    for t in range(cfg.T):
        xs = {k: x[k][:, t:t + 1].contiguous() for k in ("wl", "rl", "v", "gamma")}
        ram.ram_decode_step(ps, xs["wl"], xs["rl"], xs["v"], xs["gamma"], slot, mass, os_)
        assert rel(host(os_[:, 0]), host(o[:, t])) <= 1e-5
    torch.cuda.synchronize()
    assert rel(host(slot), host(slot1)) <= 1e-5
    assert rel(host(mass), host(mass1)) <= 1e-5
