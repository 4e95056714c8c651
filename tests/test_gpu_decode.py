"""GPU parity of the address decoder (ram_decode) against the oracle:
indices bit-exact, weights and lse within the fp32 tolerance."""
import numpy as np
import pytest
import torch

import linear_attention_ram_amd as ram
import oracle
from gpu_util import host, rel, say
from linear_attention_ram_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gpu_decode(p, side, logits):
    k = p.k_w if side == 0 else p.k_r
    idx = torch.empty((p.B, p.T, p.H, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((p.B, p.T, p.H, k), dtype=torch.float32, device=logits.device)
    lse = torch.empty((p.B, p.T, p.H), dtype=torch.float32, device=logits.device)
    ram.ram_decode(p, side, logits, idx, w, lse)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), lse.cpu().numpy()


def check_rows(p, side, logits_gpu, rows_host, sel):
    """rows_host: float64 logits (B', T', H', S) of the rows picked by sel."""
    gi, gw, gl = gpu_decode(p, side, logits_gpu)
    k = p.k_w if side == 0 else p.k_r
    B_, T_, H_ = rows_host.shape[:3]
    op = oracle.problem(B_, H_, T_, p.S, k, k, 1, renorm=(bool(p.renorm_w), bool(p.renorm_r)))
    oi, ow, ol = oracle.decode(op, side, rows_host)
    np.testing.assert_array_equal(gi[sel], oi)
    assert rel(gw[sel], ow) <= 1e-5
    assert np.max(np.abs(gl[sel] - ol[..., 0])) <= 1e-5 * max(1.0, np.max(np.abs(ol)))


@pytest.mark.parametrize("side", [0, 1])
def test_tiny_full(side):
    cfg = synth.CONFIGS["tiny"]
    x = synth.layer_inputs(cfg, device=DEV, seed=0)
    p = ram.problem(cfg.B, cfg.H, cfg.T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, io="f32")
    lg = x["wl"] if side == 0 else x["rl"]
    check_rows(p, side, lg, host(lg), np.s_[:])


@pytest.mark.parametrize("S,k,io,renorm", [(1024, 8, "bf16", False), (4096, 8, "bf16", True),
                                           (16384, 8, "bf16", False), (8192, 16, "bf16", True),
                                           (16384, 64, "bf16", False), (8192, 8, "f32", False),
                                           (64, 64, "f32", False),
                                           (8, 1, "bf16", False), (2048, 33, "f32", True),
                                           (512, 5, "bf16", False)])
def test_ties_and_shapes(S, k, io, renorm):
    # integer-valued logits: heavy ties at the k-th boundary; ragged row count
    g = torch.Generator(device=DEV).manual_seed(S + k)
    B, T, H = 1, 37, 3
    dt = torch.float32 if io == "f32" else torch.bfloat16
    lg = torch.randint(-3, 4, (B, T, H, S), generator=g, device=DEV).to(dt)
    p = ram.problem(B, H, T, S, k, k, 16, io=io, renorm=renorm)
    say("ties", S, k, io)
    check_rows(p, 0, lg, host(lg), np.s_[:])


@pytest.mark.parametrize("S", [4096, 8192, 16384])
def test_all_equal_rows_take_the_exact_fallback(S):
    # every logit equal: more candidates than the LDS list holds
    B, T, H, k = 1, 4, 2, 8
    lg = torch.zeros((B, T, H, S), dtype=torch.bfloat16, device=DEV)
    lg[0, 1, 1, S - 96] = 1.0
    p = ram.problem(B, H, T, S, k, k, 16, io="bf16")
    check_rows(p, 1, lg, host(lg), np.s_[:])


def test_340m_full():
    cfg = synth.CONFIGS["340m"]
    x = synth.layer_inputs(cfg, device=DEV, seed=0, with_d_o=False)
    p = ram.problem(cfg.B, cfg.H, cfg.T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, io=cfg.io)
    for side, key in ((0, "wl"), (1, "rl")):
        say("340m side", side)
        check_rows(p, side, x[key], host(x[key]), np.s_[:])


def test_1_3b_sampled_heads():
    cfg = synth.CONFIGS["1.3b"]
    x = synth.layer_inputs(cfg, device=DEV, seed=0, with_d_o=False)
    p = ram.problem(cfg.B, cfg.H, cfg.T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, io=cfg.io)
    for side, key in ((0, "wl"), (1, "rl")):
        for b, h in ((0, 0), (5, 11)):
            say("1.3b side", side, "slice", b, h)
            rows = host(x[key][b:b + 1, :, h:h + 1])
            check_rows(p, side, x[key], rows, np.s_[b:b + 1, :, h:h + 1])


@pytest.mark.parametrize("S,k,io,U", [(4096, 8, "bf16", 1), (16384, 8, "bf16", 1),
                                      (64, 8, "f32", 1), (1024, 8, "bf16", 2),
                                      (64, 5, "f32", 3)])
def test_nan_logits_give_valid_distinct_slots(S, k, io, U):
    # NaN logits rank below every number (the decoder's exact fallback), so a
    # row always yields K distinct slots in range; rows without NaN decode as
    # the oracle does, bit for bit
    P = S if U == 1 else round(S ** (1.0 / U))
    B, T, H = 1, 24, 2
    dt = torch.float32 if io == "f32" else torch.bfloat16
    g = torch.Generator(device=DEV).manual_seed(S + k + U)
    shape = (B, T, H, S) if U == 1 else (B, T, H, U, P)
    lg = torch.randn(shape, generator=g, device=DEV).to(dt)
    flat = lg.view(B, T, H, U * P)
    flat[0, 0, 0] = float("nan")                      # all NaN
    flat[0, 1, 1, 3:] = float("nan")                  # 3 numbers, the rest NaN
    flat[0, 2, 0, ::2] = float("nan")                 # every other entry NaN
    flat[0, 3, 1, : U * P - 1] = float("nan")         # one number
    p = ram.problem(B, H, T, None if U > 1 else S, k, k, 16, io=io, U=U, P=P)
    idx = torch.empty((B, T, H, k), dtype=torch.int32, device=DEV)
    w = torch.empty((B, T, H, k), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, T, H, U), dtype=torch.float32, device=DEV)
    ram.ram_decode(p, 0, lg, idx, w, lse)
    torch.cuda.synchronize()
    gi, gw = idx.cpu().numpy(), w.cpu().numpy()
    assert gi.min() >= 0 and gi.max() < S
    for b in range(B):
        for t in range(T):
            for h in range(H):
                assert len(set(gi[b, t, h].tolist())) == k, (t, h)
    # rows with a single digit and a few numbers: the numbers come first, in
    # (value desc, index asc) order
    if U == 1:
        row = host(flat[0, 1, 1])
        fin = np.flatnonzero(~np.isnan(row))
        order = fin[np.lexsort((fin, -row[fin]))]
        assert gi[0, 1, 1, :len(order)].tolist() == order[:k].tolist()
        assert gi[0, 3, 1, 0] == U * P - 1
    clean = np.ones((B, T, H), bool)
    clean[0, 0, 0] = clean[0, 1, 1] = clean[0, 2, 0] = clean[0, 3, 1] = False
    op = oracle.problem(B, H, T, S, k, k, 1, U=U, P=P)
    oi, ow, _ = oracle.decode(op, 0, host(lg))
    np.testing.assert_array_equal(gi[clean], oi[clean])
    assert rel(gw[clean], ow[clean]) <= 1e-5
