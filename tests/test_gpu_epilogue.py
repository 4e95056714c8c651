"""GPU parity of the gated read-out (ram_forward_gated / ram_backward_gated:
y = sigmoid(gate) * RMSNorm(o), paper §3.4 "Read-out", last step) against the
oracle: its forward followed by its epilogue, and its epilogue backward
followed by its core backward.  Outputs and gradients within the io dtype's
tolerance; the gain gradient within the same bar and bitwise repeatable."""
import numpy as np
import pytest
import torch

import linear_attention_ram_amd as ram
import oracle
from gpu_util import TOL, bh_slice, check_grads, gpu_problem, host, oracle_problem, rel, say
from linear_attention_ram_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_gated(p, x, gx, with_gain=True, eps=1e-6, with_state=False, mask=None):
    ep = ram.epilogue(p, gx["gate"], gx["gain"] if with_gain else None, eps)
    slot0 = x["slot0"] if with_state else None
    mass0 = x["mass0"] if with_state else None
    ws = ram.workspace(p, True, DEV)
    y = torch.empty_like(x["v"])
    slot1 = torch.empty((p.B, p.H, p.S, p.d_v), dtype=torch.float32, device=DEV)
    mass1 = torch.empty((p.B, p.H, p.S), dtype=torch.float32, device=DEV)
    ram.ram_forward_gated(p, ep, x["wl"], x["rl"], x["v"], x["gamma"], slot0, mass0, y, slot1,
                          mass1, ws, mask=mask)
    g = {"d_wlogits": torch.empty_like(x["wl"]), "d_rlogits": torch.empty_like(x["rl"]),
         "d_v": torch.empty_like(x["v"]), "d_gamma": torch.empty_like(x["gamma"]),
         "d_gate": torch.empty_like(gx["gate"]),
         "d_gain": torch.empty((p.d_v,), dtype=torch.float32, device=DEV)}
    ram.ram_backward_gated(p, ep, ws, x["wl"], x["rl"], x["v"], x["gamma"], slot0, mass0,
                           gx["d_y"], None, None, g["d_wlogits"], g["d_rlogits"], g["d_v"],
                           g["d_gamma"], g["d_gate"], g["d_gain"], mask=mask)
    torch.cuda.synchronize()
    return y, slot1, mass1, g


def oracle_gated(op, h, hg, with_gain=True, eps=1e-6, with_state=False, mask=None):
    gain = hg["gain"] if with_gain else None
    o, s1, m1 = oracle.forward(op, h["wl"], h["rl"], h["v"], h["gamma"],
                               h["slot0"] if with_state else None,
                               h["mass0"] if with_state else None, mask=mask)
    y = oracle.epilogue_forward(o, hg["gate"], gain, eps)
    d_o, d_gate, d_gain = oracle.epilogue_backward(o, hg["gate"], hg["d_y"], gain, eps)
    if mask is not None:
        # a masked token is absent: no gradient reaches its gate
        d_gate = d_gate * np.asarray(mask, np.float64)[:, :, None, None]
    rg = oracle.backward(op, h["wl"], h["rl"], h["v"], h["gamma"],
                         h["slot0"] if with_state else None, h["mass0"] if with_state else None,
                         d_o, None, None, mask=mask)
    rg.update({"y": y, "slot1": s1, "mass1": m1, "d_gate": d_gate, "d_gain": d_gain})
    return rg


def compare(p, y, slot1, mass1, g, ref, tol, h):
    assert rel(host(y), ref["y"]) <= tol
    assert rel(host(slot1), ref["slot1"]) <= tol
    assert rel(host(mass1), ref["mass1"]) <= tol
    check_grads(g, ref, oracle_problem(p), h, tol,
                ("d_wlogits", "d_rlogits", "d_v", "d_gamma", "d_gate"))
    err = rel(host(g["d_gain"]), ref["d_gain"])
    assert err <= tol, ("d_gain", err)


@pytest.mark.parametrize("with_gain,eps,with_state", [(True, 1e-6, False), (False, 1e-5, True),
                                                      (True, 0.25, True)])
def test_tiny_full(with_gain, eps, with_state):
    cfg = synth.CONFIGS["tiny"]
    x = synth.layer_inputs(cfg, device=DEV, seed=0, with_state=True)
    gx = synth.gate_inputs(cfg, device=DEV, seed=0)
    p = gpu_problem(cfg)
    y, s1, m1, g = run_gated(p, x, gx, with_gain, eps, with_state)
    h = {k: host(v) for k, v in x.items()}
    hg = {k: host(v) for k, v in gx.items()}
    ref = oracle_gated(oracle_problem(p), h, hg, with_gain, eps, with_state)
    compare(p, y, s1, m1, g, ref, TOL["f32"], h)


GATED_EDGE = [
    # B, H, T, S, k_w, k_r, d_v, io, U
    (2, 3, 57, 64, 3, 5, 24, "f32", 1),
    (1, 2, 129, 128, 4, 4, 128, "bf16", 1),
    (2, 2, 40, 64, 4, 4, 7, "f32", 2),      # odd d_v, product addresses
    (1, 1, 1, 8, 1, 1, 1, "f32", 1),        # one channel: RMSNorm is sign(o) * |o| / sqrt(o^2 + eps)
]


@pytest.mark.parametrize("case", range(len(GATED_EDGE)))
def test_edge_shapes(case):
    B, H, T, S, kw, kr, d, io, U = GATED_EDGE[case]
    cfg = synth.Config("gated-edge", B, H, T, S, kw, kr, d, io, U=U)
    x = synth.layer_inputs(cfg, device=DEV, seed=70 + case, with_state=True)
    gx = synth.gate_inputs(cfg, device=DEV, seed=70 + case)
    p = gpu_problem(cfg)
    y, s1, m1, g = run_gated(p, x, gx, True, 1e-6, case % 2 == 0)
    h = {k: host(v) for k, v in x.items()}
    hg = {k: host(v) for k, v in gx.items()}
    ref = oracle_gated(oracle_problem(p), h, hg, True, 1e-6, case % 2 == 0)
    compare(p, y, s1, m1, g, ref, TOL[io], h)


@pytest.mark.parametrize("d_v", [32, 12])   # vector rows, and rows taken pair by pair
def test_masked_tokens(d_v):
    cfg = synth.Config("gated-mask", 2, 3, 50, 64, 4, 3, d_v, "f32")
    x = synth.layer_inputs(cfg, device=DEV, seed=80)
    gx = synth.gate_inputs(cfg, device=DEV, seed=80)
    mask = np.ones((cfg.B, cfg.T), np.uint8)
    mask[0, 10:20] = 0
    mask[1, :3] = 0
    p = gpu_problem(cfg)
    y, s1, m1, g = run_gated(p, x, gx, mask=torch.as_tensor(mask, device=DEV))
    h = {k: host(v) for k, v in x.items()}
    hg = {k: host(v) for k, v in gx.items()}
    ref = oracle_gated(oracle_problem(p), h, hg, mask=mask)
    compare(p, y, s1, m1, g, ref, TOL["f32"], h)
    assert np.all(host(y)[mask == 0] == 0.0)
    assert np.all(host(g["d_gate"])[mask == 0] == 0.0)


def test_340m_full():
    cfg = synth.CONFIGS["340m"]
    x = synth.layer_inputs(cfg, device=DEV, seed=3)
    gx = synth.gate_inputs(cfg, device=DEV, seed=3)
    p = gpu_problem(cfg)
    y, s1, m1, g = run_gated(p, x, gx)
    h = {k: host(v) for k, v in x.items()}
    hg = {k: host(v) for k, v in gx.items()}
    say("oracle gated 340m")
    ref = oracle_gated(oracle_problem(p), h, hg)
    compare(p, y, s1, m1, g, ref, TOL["bf16"], h)


def test_plain_and_gated_read_out_agree():
    # the gated forward's y equals the epilogue applied to the plain
    # forward's o (float32 io: o is rounded once in the plain path)
    cfg = synth.Config("gated-vs-plain", 2, 2, 64, 64, 4, 4, 32, "f32")
    x = synth.layer_inputs(cfg, device=DEV, seed=90)
    gx = synth.gate_inputs(cfg, device=DEV, seed=90)
    p = gpu_problem(cfg)
    y, _, _, _ = run_gated(p, x, gx)
    ws = ram.workspace(p, False, DEV)
    o = torch.empty_like(x["v"])
    s1 = torch.empty((p.B, p.H, p.S, p.d_v), device=DEV)
    m1 = torch.empty((p.B, p.H, p.S), device=DEV)
    ram.ram_forward(p, x["wl"], x["rl"], x["v"], x["gamma"], None, None, o, s1, m1, ws)
    torch.cuda.synchronize()
    ref = oracle.epilogue_forward(host(o), host(gx["gate"]), host(gx["gain"]), 1e-6)
    assert rel(host(y), ref) <= 1e-5


def test_gated_backward_repeats_on_one_forward():
    # the backward recomputes o from the forward's read contributions, which
    # it never overwrites: further gated backward calls after one forward
    # (as with retain_graph) repeat the first bit for bit
    cfg = synth.Config("gated-retain", 2, 2, 700, 128, 8, 8, 64, "bf16", zipf=1.1)
    x = synth.layer_inputs(cfg, device=DEV, seed=92)
    gx = synth.gate_inputs(cfg, device=DEV, seed=92)
    p = gpu_problem(cfg)
    ep = ram.epilogue(p, gx["gate"], gx["gain"], 1e-6)
    ws = ram.workspace(p, True, DEV)
    y = torch.empty_like(x["v"])
    slot1 = torch.empty((p.B, p.H, p.S, p.d_v), dtype=torch.float32, device=DEV)
    mass1 = torch.empty((p.B, p.H, p.S), dtype=torch.float32, device=DEV)
    ram.ram_forward_gated(p, ep, x["wl"], x["rl"], x["v"], x["gamma"], None, None, y, slot1,
                          mass1, ws)
    outs = []
    for _ in range(2):
        g = {"d_wlogits": torch.empty_like(x["wl"]), "d_rlogits": torch.empty_like(x["rl"]),
             "d_v": torch.empty_like(x["v"]), "d_gamma": torch.empty_like(x["gamma"]),
             "d_gate": torch.empty_like(gx["gate"]),
             "d_gain": torch.empty((p.d_v,), dtype=torch.float32, device=DEV)}
        ram.ram_backward_gated(p, ep, ws, x["wl"], x["rl"], x["v"], x["gamma"], None, None,
                               gx["d_y"], None, None, g["d_wlogits"], g["d_rlogits"], g["d_v"],
                               g["d_gamma"], g["d_gate"], g["d_gain"])
        outs.append(g)
    torch.cuda.synchronize()
    for name in outs[0]:
        assert torch.equal(outs[0][name], outs[1][name]), name
    h = {k: host(v) for k, v in x.items()}
    hg = {k: host(v) for k, v in gx.items()}
    ref = oracle_gated(oracle_problem(p), h, hg)
    compare(p, y, slot1, mass1, outs[1], ref, TOL["bf16"], h)


def test_gain_gradient_is_repeatable():
    cfg = synth.Config("gated-repeat", 2, 4, 300, 256, 8, 8, 64, "bf16")
    x = synth.layer_inputs(cfg, device=DEV, seed=91)
    gx = synth.gate_inputs(cfg, device=DEV, seed=91)
    p = gpu_problem(cfg)
    _, _, _, g1 = run_gated(p, x, gx)
    _, _, _, g2 = run_gated(p, x, gx)
    assert torch.equal(g1["d_gain"], g2["d_gain"])
    assert torch.equal(g1["d_gate"], g2["d_gate"])


def test_1_3b_sampled_slices():
    cfg = synth.CONFIGS["1.3b"]
    x = synth.layer_inputs(cfg, device=DEV, seed=0)
    gx = synth.gate_inputs(cfg, device=DEV, seed=0)
    p = gpu_problem(cfg)
    say("1.3b gated fwd+bwd on GPU")
    y, _, _, g = run_gated(p, x, gx)
    for b, h in [(0, 0), (7, 15)]:
        say("1.3b gated oracle slice", b, h)
        s = bh_slice(x, b, h)
        sg = {k: host(gx[k][b:b + 1, :, h:h + 1]) for k in ("gate", "d_y")}
        sg["gain"] = host(gx["gain"])
        op = oracle.problem(1, 1, cfg.T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, eps=cfg.eps)
        ref = oracle_gated(op, s, sg)
        assert rel(host(y[b:b + 1, :, h:h + 1]), ref["y"]) <= TOL["bf16"]
        names = ("d_wlogits", "d_rlogits", "d_v", "d_gamma", "d_gate")
        got = {name: host(g[name][b:b + 1, :, h:h + 1]) for name in names}
        check_grads(got, ref, op, s, TOL["bf16"], names)
