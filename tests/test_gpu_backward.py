"""GPU parity of ram_backward against the oracle's reverse token loop:
gradients of both logit sides, v, gamma and the initial state within the
tolerance of the io dtype; the decoded-weight gradients (float32 internals)
within 1e-4."""
import numpy as np
import pytest
import torch

import linear_attention_ram_amd as ram
import oracle
from gpu_util import (TOL, bh_slice, check_grads, gpu_problem, host, oracle_problem, rel,
                      run_backward, run_forward, say)
from linear_attention_ram_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def full_check(cfg, x, p, with_state, with_state_grads, tol):
    slot0 = x["slot0"] if with_state else None
    mass0 = x["mass0"] if with_state else None
    ds1 = x["d_slot1"] if with_state_grads else None
    dm1 = x["d_mass1"] if with_state_grads else None
    r = run_forward(p, x, slot0=slot0, mass0=mass0)
    g = run_backward(p, x, r["ws"], slot0, mass0, ds1, dm1, want_state=True)
    torch.cuda.synchronize()
    h = {k: host(v) for k, v in x.items()}
    say("oracle backward", cfg.name)
    rg = oracle.backward(oracle_problem(p), h["wl"], h["rl"], h["v"], h["gamma"],
                         h["slot0"] if with_state else None, h["mass0"] if with_state else None,
                         h["d_o"], h["d_slot1"] if with_state_grads else None,
                         h["d_mass1"] if with_state_grads else None)
    op = oracle_problem(p)
    check_grads(g, rg, op, h, tol)
    views = ram.ws_views(p, r["ws"])
    # float32 internals computed from the same io values: tighter than the io bar
    assert rel(views["dw"].cpu().numpy().reshape(rg["dw"].shape), rg["dw"]) <= 1e-4
    assert rel(views["dr"].cpu().numpy().reshape(rg["dr"].shape), rg["dr"]) <= 1e-4
    if with_state:
        assert rel(host(g["d_slot0"]), rg["d_slot0"]) <= tol
        assert rel(host(g["d_mass0"]), rg["d_mass0"]) <= tol
    return r, g


@pytest.mark.parametrize("with_state,with_state_grads", [(False, False), (True, True),
                                                         (True, False)])
def test_tiny_full(with_state, with_state_grads):
    cfg = synth.CONFIGS["tiny"]
    x = synth.layer_inputs(cfg, device=DEV, seed=0, with_state=True, with_state_grads=True)
    full_check(cfg, x, gpu_problem(cfg), with_state, with_state_grads, TOL["f32"])


def test_tiny_renormalised():
    cfg = synth.CONFIGS["tiny"]
    x = synth.layer_inputs(cfg, device=DEV, seed=4, with_state=True, with_state_grads=True)
    full_check(cfg, x, gpu_problem(cfg, renorm=(True, True)), True, True, TOL["f32"])


@pytest.mark.parametrize("with_state", [False, True])
def test_340m_full(with_state):
    cfg = synth.CONFIGS["340m"]
    x = synth.layer_inputs(cfg, device=DEV, seed=2, with_state=True, with_state_grads=True)
    full_check(cfg, x, gpu_problem(cfg), with_state, with_state, TOL["bf16"])


@pytest.mark.parametrize("S,io,k", [(640, "bf16", 12), (1000, "f32", 9), (2056, "bf16", 16)])
def test_partial_last_kilobyte(S, io, k):
    # the decode backward streams each logits row in 1 KiB pieces, one wave
    # each: rows whose length is not a multiple of 1 KiB (here 1280, 4000 and
    # 4112 bytes) end in a partial piece, and with k up to 16 several selected
    # entries can share a piece
    cfg = synth.Config(f"partial-{S}-{io}", 2, 3, 96, S, k, k, 64 if io == "bf16" else 40, io)
    x = synth.layer_inputs(cfg, device=DEV, seed=11, with_state=True, with_state_grads=True)
    full_check(cfg, x, gpu_problem(cfg), True, True, TOL[io])


def test_1_3b_sampled_slices():
    cfg = synth.CONFIGS["1.3b"]
    x = synth.layer_inputs(cfg, device=DEV, seed=0)
    p = gpu_problem(cfg)
    say("1.3b fwd+bwd on GPU")
    r = run_forward(p, x)
    g = run_backward(p, x, r["ws"])
    torch.cuda.synchronize()
    for b, h in [(0, 0), (6, 9)]:
        say("1.3b oracle backward slice", b, h)
        s = bh_slice(x, b, h)
        op = oracle.problem(1, 1, cfg.T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, eps=cfg.eps)
        rg = oracle.backward(op, s["wl"], s["rl"], s["v"], s["gamma"], None, None, s["d_o"])
        got = {name: host(g[name][b:b + 1, :, h:h + 1])
               for name in ("d_wlogits", "d_rlogits", "d_v", "d_gamma")}
        check_grads(got, rg, op, s, TOL["bf16"])


EDGE = [
    # B, H, T, S, k_w, k_r, d_v, io, renorm, eps
    (1, 1, 1, 8, 1, 1, 1, "f32", (False, False), 1e-6),
    (2, 3, 31, 16, 3, 2, 7, "f32", (False, True), 1e-6),
    (3, 1, 300, 32, 2, 5, 66, "f32", (True, False), 1e-3),
    (1, 2, 257, 128, 4, 4, 128, "bf16", (False, False), 1e-6),
    (2, 2, 600, 8, 8, 8, 16, "f32", (False, False), 1e-6),  # long segments: many chunks
    (1, 2, 2000, 16, 4, 4, 16, "f32", (False, False), 1e-6),  # ~1000-event segments
    (1, 1, 3000, 8, 3, 2, 128, "f32", (True, True), 1e-6),    # long segments, wide slots
    # most slots without events, rows not of whole 16-byte vectors (the
    # second case passes d_slot1 / d_mass1 on through the empty slots)
    (1, 2, 5, 256, 2, 2, 66, "f32", (False, False), 1e-6),
    (1, 2, 5, 256, 2, 2, 7, "bf16", (False, False), 1e-6),
]


@pytest.mark.parametrize("case", range(len(EDGE)))
def test_edge_shapes(case):
    B, H, T, S, kw, kr, d, io, rn, eps = EDGE[case]
    cfg = synth.Config("edge", B, H, T, S, kw, kr, d, io)
    x = synth.layer_inputs(cfg, device=DEV, seed=20 + case, with_state=True, with_state_grads=True)
    p = ram.problem(B, H, T, S, kw, kr, d, io=io, eps=eps, renorm=rn)
    full_check(cfg, x, p, case % 2 == 0, case % 2 == 0, TOL[io])


@pytest.mark.parametrize("hot", [False, True])
def test_backward_repeats_on_the_same_workspace(hot):
    # the workspace's accumulators and work queues are zero again after each
    # call, so further backward calls after one forward repeat the first one
    # bit for bit; the hot-slot case has segments long enough for the
    # cooperative scan (its work queue is cleared by the call itself)
    cfg = (synth.Config("hot-repeat", 2, 2, 1024, 256, 4, 4, 64, "bf16", zipf=1.1) if hot
           else synth.CONFIGS["tiny"])
    x = synth.layer_inputs(cfg, device=DEV, seed=9)
    p = gpu_problem(cfg)
    r = run_forward(p, x)
    if hot:
        offs = ram.ws_views(p, r["ws"])["seg_offset"].cpu().numpy()
        assert (offs[1:] - offs[:-1]).max() > 4 * 128
    g1 = run_backward(p, x, r["ws"])
    g2 = run_backward(p, x, r["ws"])
    g3 = run_backward(p, x, r["ws"])
    r2 = run_forward(p, x)
    torch.cuda.synchronize()
    for name in ("d_wlogits", "d_rlogits", "d_v", "d_gamma"):
        assert torch.equal(g2[name], g1[name]), name
        assert torch.equal(g3[name], g1[name]), name
    assert torch.equal(r2["o"], r["o"])


def test_hot_slots_over_ragged_slot_blocks():
    # as the forward case: a partial last 1024-slot block of the bucketing
    # scan and hot slots on the cooperative reverse path
    cfg = synth.Config("hot-ragged", 2, 2, 1024, 2504, 8, 8, 64, "bf16", zipf=1.1)
    x = synth.layer_inputs(cfg, device=DEV, seed=41, with_state=True, with_state_grads=True)
    full_check(cfg, x, gpu_problem(cfg), True, True, TOL["bf16"])


@pytest.mark.parametrize("nhot,bias,listed", [(512, 2.0, True), (1024, 1.0, False)])
def test_short_segments_listed_or_direct(nhot, bias, listed):
    # as the forward case: both ways of the short-segment reverse scan, and
    # d_slot1 / d_mass1 passed on through the slots without events
    from test_gpu_forward import raised_slots, short_list_mode
    cfg = synth.Config("raised", 1, 2, 512, 2048, 4, 4, 64, "bf16")
    x = raised_slots(cfg, 51, nhot, bias, with_state=True, with_state_grads=True)
    p = gpu_problem(cfg)
    r, g = full_check(cfg, x, p, True, True, TOL["bf16"])
    seg = ram.ws_views(p, r["ws"])["seg_offset"].cpu().numpy()
    assert short_list_mode(seg) == listed
    empty = torch.from_numpy(np.diff(seg.astype(np.int64)) == 0).to(DEV).reshape(cfg.B, cfg.H, cfg.S)
    assert torch.equal(g["d_slot0"][empty], x["d_slot1"][empty])
    assert torch.equal(g["d_mass0"][empty], x["d_mass1"][empty])


def test_widest_address_space():
    cfg = synth.Config("widest", 1, 2, 512, 16384, 8, 8, 64, "bf16", zipf=1.1)
    x = synth.layer_inputs(cfg, device=DEV, seed=45, with_state=True, with_state_grads=True)
    full_check(cfg, x, gpu_problem(cfg), True, True, TOL["bf16"])
