"""ram_forward_noalloc (the allocation-free forward) against ram_forward: the
same kernels on a library-held workspace, so o, slot1 and mass1 must agree
bit for bit.  Two calls in a row, the second on a smaller problem (the array
keeps the first call's contents), then a problem too large for the array.

The array belongs to the library's code object: the runtime places it on a
device when that code object is first used there (the first call's address
lookup), and holds it until the process ends.  Calls after that first one
allocate nothing: the device's free memory is the same before and after."""
import ctypes

import pytest
import torch

import linear_attention_ram_amd as ram
from linear_attention_ram_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def outputs(cfg, x, with_state):
    o = torch.full_like(x["v"], float("nan"))
    s1 = torch.full((cfg.B, cfg.H, cfg.S, cfg.d_v), float("nan"), device=DEV)
    m1 = torch.full((cfg.B, cfg.H, cfg.S), float("nan"), device=DEV)
    return o, s1, m1


def run_pair(cfg, seed, with_state, check_free):
    x = synth.layer_inputs(cfg, device=DEV, seed=seed, with_state=with_state, with_d_o=False)
    p = ram.problem(cfg.B, cfg.H, cfg.T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, io=cfg.io)
    assert ram.ram_workspace_size(p, False) <= ram.NOALLOC_SCRATCH_BYTES
    slot0 = x.get("slot0") if with_state else None
    mass0 = x.get("mass0") if with_state else None
    ws = ram.workspace(p, False, DEV)
    o_ref, s_ref, m_ref = outputs(cfg, x, with_state)
    ram.ram_forward(p, x["wl"], x["rl"], x["v"], x["gamma"], slot0, mass0, o_ref, s_ref, m_ref, ws)
    o, s1, m1 = outputs(cfg, x, with_state)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    st = ram.lib().ram_forward_noalloc(ctypes.byref(p), vp(x["wl"]), vp(x["rl"]), vp(x["v"]),
                                       vp(x["gamma"]), None, vp(slot0), vp(mass0), vp(o), vp(s1),
                                       vp(m1), None)
    assert st == ram.RAM_OK, ram.ram_status_string(st)
    torch.cuda.synchronize()
    if check_free:
        assert torch.cuda.mem_get_info()[0] == free0    # nothing allocated on the device
    assert torch.equal(o, o_ref)
    assert torch.equal(s1, s_ref)
    assert torch.equal(m1, m_ref)


def test_noalloc_forward_matches_ram_forward_twice():
    # hot slots (cooperative scan path) at 27 MiB of workspace, then a smaller
    # problem with an initial state on the same array
    run_pair(synth.Config("noalloc-a", 2, 8, 2048, 1024, 4, 4, 64, "bf16", zipf=1.1), 61, False,
             check_free=False)
    run_pair(synth.Config("noalloc-b", 1, 3, 300, 256, 8, 5, 32, "f32", zipf=1.1), 62, True,
             check_free=True)


def test_noalloc_forward_rejects_problems_beyond_the_array():
    p = ram.problem(1, 16, 2048, 4096, 8, 8, 128, io="bf16")
    assert ram.ram_workspace_size(p, False) > ram.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(16 * 1024)     # never dereferenced: the size check fails first
    st = ram.lib().ram_forward_noalloc(ctypes.byref(p), fake, fake, fake, fake, None, None, None,
                                       fake, fake, fake, None)
    assert st == ram.RAM_ECAPACITY
