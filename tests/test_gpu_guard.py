"""In-place continuation and the backward (ramnet-ops "Arguments": inplace
runs without gradients).  A forward whose final state overlaps its initial
state overwrites what a backward needs, so ram_backward on that workspace
returns RAM_EINVAL and enqueues nothing; an out-of-place forward on the same
workspace makes the backward valid again.  Calls go through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import linear_attention_ram_amd as ram
import oracle
from gpu_util import TOL, check_grads, gpu_problem, host, oracle_problem, rel
from linear_attention_ram_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def c_forward(p, x, slot0, mass0, o, slot1, mass1, ws):
    return ram.lib().ram_forward(ctypes.byref(p), vp(x["wl"]), vp(x["rl"]), vp(x["v"]),
                                 vp(x["gamma"]), None, vp(slot0), vp(mass0), vp(o), vp(slot1),
                                 vp(mass1), vp(ws), ctypes.c_size_t(ws.numel()), None)


def c_backward(p, x, ws, slot0, mass0, g):
    return ram.lib().ram_backward(
        ctypes.byref(p), vp(ws), ctypes.c_size_t(ws.numel()), vp(x["wl"]), vp(x["rl"]),
        vp(x["v"]), vp(x["gamma"]), None, vp(slot0), vp(mass0), vp(x["d_o"]), None, None,
        vp(g["d_wlogits"]), vp(g["d_rlogits"]), vp(g["d_v"]), vp(g["d_gamma"]), None, None, None)


def grads_like(x):
    return {"d_wlogits": torch.zeros_like(x["wl"]), "d_rlogits": torch.zeros_like(x["rl"]),
            "d_v": torch.zeros_like(x["v"]), "d_gamma": torch.zeros_like(x["gamma"])}


@pytest.mark.parametrize("alias", ["slot and mass", "mass only"])
def test_backward_after_in_place_forward_is_rejected(alias):
    cfg = synth.Config("inplace", 2, 2, 300, 64, 4, 3, 16, "f32")
    x = synth.layer_inputs(cfg, device=DEV, seed=51, with_state=True)
    p = gpu_problem(cfg)
    ws = ram.workspace(p, True, DEV)
    o_ref = torch.empty_like(x["v"])
    s1_ref = torch.empty_like(x["slot0"])
    m1_ref = torch.empty_like(x["mass0"])
    assert c_forward(p, x, x["slot0"], x["mass0"], o_ref, s1_ref, m1_ref, ws) == ram.RAM_OK

    # in place: the continuation overwrites the initial state
    slot = x["slot0"].clone()
    mass = x["mass0"].clone()
    o = torch.empty_like(x["v"])
    s1 = slot if alias == "slot and mass" else torch.empty_like(slot)
    assert c_forward(p, x, slot, mass, o, s1, mass, ws) == ram.RAM_OK
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(s1, s1_ref) and torch.equal(mass, m1_ref)
    g = grads_like(x)
    assert c_backward(p, x, ws, slot, mass, g) == ram.RAM_EINVAL
    torch.cuda.synchronize()
    for t in g.values():      # nothing was enqueued: the outputs are untouched
        assert not torch.any(t != 0)

    # an out-of-place forward on the same workspace: the backward runs again
    assert c_forward(p, x, x["slot0"], x["mass0"], o, s1_ref, m1_ref, ws) == ram.RAM_OK
    assert c_backward(p, x, ws, x["slot0"], x["mass0"], g) == ram.RAM_OK
    torch.cuda.synchronize()
    h = {k: host(v) for k, v in x.items()}
    op = oracle_problem(p)
    rg = oracle.backward(op, h["wl"], h["rl"], h["v"], h["gamma"], h["slot0"], h["mass0"],
                         h["d_o"])
    check_grads(g, rg, op, h, TOL["f32"])


def test_other_workspaces_are_not_affected():
    # the record is per workspace: an in-place forward on one workspace does
    # not block the backward of another
    cfg = synth.Config("inplace-two", 1, 2, 100, 32, 3, 2, 16, "f32")
    x = synth.layer_inputs(cfg, device=DEV, seed=52, with_state=True)
    p = gpu_problem(cfg)
    ws_a, ws_b = ram.workspace(p, True, DEV), ram.workspace(p, True, DEV)
    o = torch.empty_like(x["v"])
    s1, m1 = torch.empty_like(x["slot0"]), torch.empty_like(x["mass0"])
    assert c_forward(p, x, x["slot0"], x["mass0"], o, s1, m1, ws_b) == ram.RAM_OK
    slot, mass = x["slot0"].clone(), x["mass0"].clone()
    assert c_forward(p, x, slot, mass, o, slot, mass, ws_a) == ram.RAM_OK
    g = grads_like(x)
    assert c_backward(p, x, ws_a, slot, mass, g) == ram.RAM_EINVAL
    assert c_backward(p, x, ws_b, x["slot0"], x["mass0"], g) == ram.RAM_OK
    torch.cuda.synchronize()
    assert rel(host(g["d_v"]), host(g["d_v"])) == 0.0
    assert np.all(np.isfinite(host(g["d_wlogits"])))
