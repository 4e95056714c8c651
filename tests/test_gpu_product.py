"""GPU parity of product-softmax addresses (U >= 2 digits of P logits; paper
§3.2 "Product Softmax", App. B.1; the pruned prefix search of paper §4
"Efficient Address Decoding") against the oracle's exhaustive decoder:
selected slots bit-exact, weights and per-digit logsumexp within 1e-5,
outputs, state and gradients within the io dtype's tolerance."""
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


def gpu_decode(p, side, logits):
    k = p.k_w if side == 0 else p.k_r
    idx = torch.empty((p.B, p.T, p.H, k), dtype=torch.int32, device=DEV)
    w = torch.empty((p.B, p.T, p.H, k), dtype=torch.float32, device=DEV)
    lse = torch.empty((p.B, p.T, p.H, p.U), dtype=torch.float32, device=DEV)
    ram.ram_decode(p, side, logits, idx, w, lse)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), lse.cpu().numpy()


def check_decode(p, side, logits, w_tol=1e-5):
    gi, gw, gl = gpu_decode(p, side, logits)
    oi, ow, ol = oracle.decode(oracle_problem(p), side, host(logits))
    np.testing.assert_array_equal(gi, oi)
    assert rel(gw, ow) <= w_tol
    assert np.max(np.abs(gl - ol)) <= 1e-5 * max(1.0, float(np.max(np.abs(ol))))


DECODE_CASES = [
    # U, P, k, io, renorm, logits ("int": heavy ties, "normal")
    (2, 8, 8, "f32", False, "normal"),
    (2, 8, 8, "bf16", False, "int"),
    (3, 4, 8, "f32", True, "int"),
    (5, 4, 8, "bf16", False, "normal"),
    (5, 4, 8, "f32", False, "int"),
    (2, 64, 8, "bf16", False, "normal"),
    (2, 64, 8, "f32", True, "int"),          # four rows per wave; ties overflow the row list
    (2, 32, 8, "bf16", False, "int"),        # P = 4K: K lanes of a row hold values
    (2, 48, 12, "bf16", False, "normal"),    # P not a power of two
    (2, 64, 16, "f32", True, "normal"),      # the largest K of the four-row kernel
    (2, 64, 33, "f32", True, "int"),
    (2, 128, 64, "bf16", False, "normal"),   # S = 16384, k = 64
    (2, 5, 25, "f32", False, "int"),         # k = S
    (3, 3, 5, "f32", False, "normal"),
    (4, 3, 6, "bf16", True, "int"),
    (14, 2, 8, "f32", False, "normal"),      # most digits
    (7, 1, 1, "f32", False, "normal"),       # P = 1: one slot
]


@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_decode(case):
    U, P, k, io, rn, kind = DECODE_CASES[case]
    B, T, H = 2, 41, 3                       # 246 rows: several blocks and a ragged tail
    dt = torch.float32 if io == "f32" else torch.bfloat16
    g = torch.Generator(device=DEV).manual_seed(100 + case)
    if kind == "int":
        lg = torch.randint(-2, 3, (B, T, H, U, P), generator=g, device=DEV).to(dt)
    else:
        lg = torch.randn((B, T, H, U, P), generator=g, device=DEV).to(dt)
    p = ram.problem(B, H, T, None, k, k, 16, io=io, renorm=rn, U=U, P=P)
    say("product decode", U, P, k, io, rn, kind)
    for side in (0, 1):
        check_decode(p, side, lg)


def test_rounding_limited_keys():
    # the first digit is large and the others tiny: many float32 key sums
    # round to the same value, so selection hinges on exact rounding and ties
    B, T, H, U, P, k = 1, 64, 2, 3, 16, 8
    g = torch.Generator(device=DEV).manual_seed(7)
    lg = torch.randn((B, T, H, U, P), generator=g, device=DEV) * 1e-5
    lg[..., 0, :] = torch.randn((B, T, H, P), generator=g, device=DEV) * 1000.0
    p = ram.problem(B, H, T, None, k, k, 16, io="f32", U=U, P=P)
    # a weight is exp(sum_u (l_u - lse_u)) in float32: each difference carries
    # up to an ulp of |lse_u| (here ~3000), so the bound scales with sum_u |lse_u|
    ol = oracle.decode(oracle_problem(p), 0, host(lg))[2]
    w_tol = 4 * 2.0 ** -24 * float(np.abs(ol).sum(-1).max())
    check_decode(p, 0, lg.contiguous(), w_tol)


def test_two_digit_rows_by_listed_count():
    # U = 2 rows whose top c digit-0 values and top 8 digit-1 values are all
    # 1 and the rest near -3: exactly 8c slots tie at the best key 2, ranked
    # by index.  Rows of four (one wave) list 32 slots (ranked by count), 40
    # or 64 (ranked by rounds of the row maximum), or mix those; c = 9 lists
    # 72, more than a row holds, and is redone by the whole-wave kernel.
    B, T, H, U, P, k = 1, 48, 2, 2, 64, 8
    pattern = [4, 4, 4, 4, 4, 5, 2, 1, 8, 8, 8, 8, 9, 1, 4, 3]
    g = torch.Generator(device="cpu").manual_seed(11)
    lg = -3.0 + 0.1 * torch.randn((B, T, H, U, P), generator=g)
    for i in range(T * H):
        t, h = divmod(i, H)
        c = pattern[i % len(pattern)]
        d0 = torch.randperm(P, generator=g)[:c]
        d1 = torch.randperm(P, generator=g)[:8]
        lg[0, t, h, 0, d0] = 1.0
        lg[0, t, h, 1, d1] = 1.0
    lg = lg.to(torch.bfloat16).to(DEV)
    p = ram.problem(B, H, T, None, k, k, 16, io="bf16", U=U, P=P)
    for side in (0, 1):
        check_decode(p, side, lg)


@pytest.mark.parametrize("U,P", [(2, 64), (5, 4), (2, 128)])
def test_all_equal_rows_take_the_exhaustive_fallback(U, P):
    # every slot ties: more kept prefixes than the list holds
    B, T, H, k = 1, 3, 2, 8
    lg = torch.zeros((B, T, H, U, P), dtype=torch.bfloat16, device=DEV)
    lg[0, 1, 1, U - 1, P - 1] = 1.0
    p = ram.problem(B, H, T, None, k, k, 16, io="bf16", U=U, P=P)
    check_decode(p, 1, lg)


def full_check(cfg, p, x, tol, with_state=False, mask=None):
    slot0 = x["slot0"] if with_state else None
    mass0 = x["mass0"] if with_state else None
    ds1 = x["d_slot1"] if with_state else None
    dm1 = x["d_mass1"] if with_state else None
    dev_mask = None if mask is None else torch.as_tensor(mask, device=DEV)
    ws = ram.workspace(p, True, DEV)
    o = torch.empty_like(x["v"])
    slot1 = torch.empty((p.B, p.H, p.S, p.d_v), dtype=torch.float32, device=DEV)
    mass1 = torch.empty((p.B, p.H, p.S), dtype=torch.float32, device=DEV)
    ram.ram_forward(p, x["wl"], x["rl"], x["v"], x["gamma"], slot0, mass0, o, slot1, mass1, ws,
                    mask=dev_mask)
    g = {"d_wlogits": torch.empty_like(x["wl"]), "d_rlogits": torch.empty_like(x["rl"]),
         "d_v": torch.empty_like(x["v"]), "d_gamma": torch.empty_like(x["gamma"])}
    d_s0 = torch.empty_like(slot1) if with_state else None
    d_m0 = torch.empty_like(mass1) if with_state else None
    ram.ram_backward(p, ws, x["wl"], x["rl"], x["v"], x["gamma"], slot0, mass0, x["d_o"], ds1,
                     dm1, g["d_wlogits"], g["d_rlogits"], g["d_v"], g["d_gamma"], d_s0, d_m0,
                     mask=dev_mask)
    torch.cuda.synchronize()
    h = {k: host(v) for k, v in x.items()}
    op = oracle_problem(p)
    say("oracle forward/backward", cfg.name, "U", p.U, "P", p.P)
    oo, os_, om = oracle.forward(op, h["wl"], h["rl"], h["v"], h["gamma"],
                                 h["slot0"] if with_state else None,
                                 h["mass0"] if with_state else None, mask=mask)
    assert rel(host(o), oo) <= tol
    assert rel(host(slot1), os_) <= tol
    assert rel(host(mass1), om) <= tol
    views = ram.ws_views(p, ws)
    for side, key, name in ((0, "wl", "idx_w"), (1, "rl", "idx_r")):
        oi, _, ol = oracle.decode(op, side, h[key])
        np.testing.assert_array_equal(views[name].cpu().numpy().reshape(oi.shape), oi)
        lse = views["lse_w" if side == 0 else "lse_r"].cpu().numpy().reshape(ol.shape)
        assert np.max(np.abs(lse - ol)) <= 1e-5 * max(1.0, float(np.max(np.abs(ol))))
    rg = oracle.backward(op, h["wl"], h["rl"], h["v"], h["gamma"],
                         h["slot0"] if with_state else None, h["mass0"] if with_state else None,
                         h["d_o"], h["d_slot1"] if with_state else None,
                         h["d_mass1"] if with_state else None, mask=mask)
    check_grads(g, rg, op, h, tol)
    # decoded-weight gradients (float32 internals) of valid tokens; a masked
    # token's events are weight-0 no-ops whose internal gradient feeds nothing
    valid = np.ones((p.B, p.T), bool) if mask is None else np.asarray(mask, bool)
    for name in ("dw", "dr"):
        got = views[name].cpu().numpy().reshape(rg[name].shape)
        assert rel(got[valid], rg[name][valid]) <= 1e-4, name
    if with_state:
        assert rel(host(d_s0), rg["d_slot0"]) <= tol
        assert rel(host(d_m0), rg["d_mass0"]) <= tol


def test_ops_example_shape():
    # U = 3 digits of 4, B=2, T=32, H=4, C=32, top-8
    cfg = synth.CONFIGS["ops-example"]
    x = synth.layer_inputs(cfg, device=DEV, seed=0, with_state=True, with_state_grads=True)
    full_check(cfg, gpu_problem(cfg), x, TOL["f32"], with_state=True)


def test_default_address_space_u5():
    # 4^5 slots as 5 digits of 4
    cfg = synth.CONFIGS["u5"]
    x = synth.layer_inputs(cfg, device=DEV, seed=1)
    full_check(cfg, gpu_problem(cfg), x, TOL["bf16"])


PRODUCT_EDGE = [
    # B, H, T, U, P, k_w, k_r, d_v, io, renorm
    (1, 1, 1, 2, 4, 1, 1, 1, "f32", (False, False)),
    (2, 3, 57, 2, 16, 3, 5, 24, "f32", (True, False)),
    (1, 2, 300, 3, 2, 4, 2, 16, "f32", (False, True)),     # 8 slots: long segments
    (2, 2, 129, 2, 32, 8, 8, 128, "bf16", (False, False)),
]


@pytest.mark.parametrize("case", range(len(PRODUCT_EDGE)))
def test_edge_shapes(case):
    B, H, T, U, P, kw, kr, d, io, rn = PRODUCT_EDGE[case]
    cfg = synth.Config("prod-edge", B, H, T, P ** U, kw, kr, d, io, U=U)
    x = synth.layer_inputs(cfg, device=DEV, seed=40 + case, with_state=True, with_state_grads=True)
    full_check(cfg, gpu_problem(cfg, renorm=rn), x, TOL[io], with_state=case % 2 == 1)


def test_with_cape_and_mask():
    cfg = synth.Config("prod-cape", 2, 3, 45, 64, 4, 3, 16, "f32", U=2)
    x = synth.layer_inputs(cfg, device=DEV, seed=61)
    mask = np.ones((cfg.B, cfg.T), np.uint8)
    mask[0, 3:9] = 0
    mask[1, -5:] = 0
    full_check(cfg, gpu_problem(cfg, cape_heads=2, t0=77), x, TOL["f32"], mask=mask)


def test_1_3b_factorised_sampled_slices():
    # the 1.3B-layer shape with U = 2 digits of 64: full fwd+bwd on the GPU,
    # oracle on two (b, h) slices
    cfg = synth.CONFIGS["1.3b-u2"]
    x = synth.layer_inputs(cfg, device=DEV, seed=0)
    p = gpu_problem(cfg)
    say("1.3b-u2 fwd+bwd on GPU")
    r = run_forward(p, x)
    g = run_backward(p, x, r["ws"])
    torch.cuda.synchronize()
    for b, h in [(0, 0), (5, 11)]:
        say("1.3b-u2 oracle slice", b, h)
        s = bh_slice(x, b, h)
        op = oracle.problem(1, 1, cfg.T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, U=cfg.U, P=cfg.P,
                            eps=cfg.eps)
        oo, _, _ = oracle.forward(op, s["wl"], s["rl"], s["v"], s["gamma"])
        assert rel(host(r["o"][b:b + 1, :, h:h + 1]), oo) <= TOL["bf16"]
        rg = oracle.backward(op, s["wl"], s["rl"], s["v"], s["gamma"], None, None, s["d_o"])
        got = {name: host(g[name][b:b + 1, :, h:h + 1])
               for name in ("d_wlogits", "d_rlogits", "d_v", "d_gamma")}
        check_grads(got, rg, op, s, TOL["bf16"])


def test_decode_step():
    cfg = synth.Config("prod-step", 3, 2, 1, 256, 4, 3, 32, "f32", U=4)
    slot, mass = synth.decode_state(cfg, device=DEV, seed=0)
    p = gpu_problem(cfg, T=1)
    op = oracle_problem(p)
    o_slot = np.ascontiguousarray(host(slot))
    o_mass = np.ascontiguousarray(host(mass))
    o = torch.empty((cfg.B, 1, cfg.H, cfg.d_v), dtype=torch.float32, device=DEV)
    for step in range(24):
        x = synth.decode_step_inputs(cfg, step, device=DEV, seed=0)
        ram.ram_decode_step(p, x["wl"], x["rl"], x["v"], x["gamma"], slot, mass, o)
        torch.cuda.synchronize()
        h = {k: host(v) for k, v in x.items()}
        ref = oracle.decode_step(op, h["wl"], h["rl"], h["v"], h["gamma"], o_slot, o_mass)
        assert rel(host(o), ref) <= TOL["f32"], step
    assert rel(host(slot), o_slot) <= TOL["f32"]
    assert rel(host(mass), o_mass) <= TOL["f32"]
