"""The logit-gradient bar of the GPU parity tests can fail (CPU only).

The gradient of a logit row is dl_i = [i selected] g_j w_j - p_i G with
G = sum_j g_j w_j (paper §3.2 "Address Decoder": a softmax over all slots).
parity.check_logit_grad compares the selected entries (normwise) and all
other entries, the dense term -p_i G alone, against the dense scale
p_i * sum_j |g_j w_j| the GPU tests use.  On one
(batch, head) slice of the 340M- and 1.3B-layer shapes, the oracle's own
gradients rounded to bf16 pass that bar, and oracle gradients with a planted
mistake in the dense term fail it: the dense term dropped, the logsumexp
shifted by 0.5 nats, the dense term's sign flipped.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
from linear_attention_ram_amd import synth

TOL_BF16 = 2e-2

SHAPES = {
    "340m": synth.Config("340m-slice", 1, 1, 2048, 1024, 4, 4, 64, "bf16"),
    "1.3b": synth.Config("1.3b-slice", 1, 1, 4096, 4096, 8, 8, 128, "bf16", zipf=1.1),
}


def to_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


@pytest.fixture(scope="module", params=list(SHAPES))
def case(request):
    cfg = SHAPES[request.param]
    x = synth.layer_inputs(cfg, device="cpu", seed=5)
    h = {k: v.double().numpy() for k, v in x.items()}
    op = oracle.problem(1, 1, cfg.T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, eps=cfg.eps)
    rg = oracle.backward(op, h["wl"], h["rl"], h["v"], h["gamma"], None, None, h["d_o"])
    return op, h, rg


def dense_parts(op, h, rg, side):
    """p (softmax of the row), G (sum_j g_j w_j per row, broadcastable), the
    selected-entry mask and the dense scale of one side, from the oracle's
    decode and its decoded-weight gradients (no renormalisation)."""
    logits = h["wl"] if side == 0 else h["rl"]
    idx, w, lse = oracle.decode(op, side, logits)
    gw = parity.gw_products(rg["dw"] if side == 0 else rg["dr"], w)
    G = np.sum(gw, axis=-1)[..., None]
    p = np.exp(logits - lse)
    scale = parity.dense_scale(logits, lse, gw, 1, int(op.P))
    return p, G, parity.selected_entries(idx, 1, int(op.P)), scale


@pytest.mark.parametrize("side", [0, 1])
def test_dense_term_is_what_the_mutants_change(case, side):
    # off the selected entries the oracle's gradient is exactly -p_i G, so the
    # mutants below change the dense term and nothing else
    op, h, rg = case
    ref = rg["d_wlogits" if side == 0 else "d_rlogits"]
    p, G, sel, _ = dense_parts(op, h, rg, side)
    dense = -p * G
    assert parity.rel(ref[~sel], dense[~sel]) <= 1e-12


@pytest.mark.parametrize("side", [0, 1])
def test_bf16_rounded_oracle_passes(case, side):
    op, h, rg = case
    ref = rg["d_wlogits" if side == 0 else "d_rlogits"]
    _, _, sel, scale = dense_parts(op, h, rg, side)
    e_sel, e_dense = parity.check_logit_grad(to_bf16(ref), ref, sel, TOL_BF16, scale=scale)
    assert e_sel <= 4e-3 and e_dense <= 4e-3


@pytest.mark.parametrize("mutant", ["dense dropped", "lse + 0.5", "dense sign"])
@pytest.mark.parametrize("side", [0, 1])
def test_planted_dense_mistakes_fail(case, side, mutant):
    op, h, rg = case
    ref = rg["d_wlogits" if side == 0 else "d_rlogits"]
    p, G, sel, scale = dense_parts(op, h, rg, side)
    if mutant == "dense dropped":
        bad = ref + p * G
    elif mutant == "lse + 0.5":
        bad = ref + (p - p * np.exp(-0.5)) * G
    else:
        bad = ref + 2.0 * p * G
    _, e_dense = parity.logit_grad_errors(to_bf16(bad), ref, sel, scale)
    assert e_dense > 5 * TOL_BF16, (mutant, e_dense)
    with pytest.raises(AssertionError):
        parity.check_logit_grad(to_bf16(bad), ref, sel, TOL_BF16, scale=scale)


@pytest.mark.parametrize("side", [0, 1])
def test_renormalised_dense_term_vanishes(case, side):
    # with renormalised weights sum_j g_j w_j = 0, so the reference dense term
    # is zero up to rounding: the scale keeps the bar finite there, and a
    # dense term that does not vanish still fails it
    op, h, rg = case
    logits = h["wl"] if side == 0 else h["rl"]
    rn = oracle.problem(1, 1, int(op.T), int(op.P), int(op.k_w), int(op.k_r), int(op.d_v),
                        eps=float(op.eps), renorm=True)
    idx, w, lse = oracle.decode(rn, side, logits)
    rgn = oracle.backward(rn, h["wl"], h["rl"], h["v"], h["gamma"], None, None, h["d_o"])
    ref = rgn["d_wlogits" if side == 0 else "d_rlogits"]
    gw = parity.gw_products(rgn["dw"] if side == 0 else rgn["dr"], w, renorm=True)
    sel = parity.selected_entries(idx, 1, int(rn.P))
    scale = parity.dense_scale(logits, lse, gw, 1, int(rn.P))
    off = ~sel.reshape(ref.shape)
    assert np.max(np.abs(ref[off])) <= 1e-12 * np.max(np.abs(ref))
    parity.check_logit_grad(to_bf16(ref), ref, sel, TOL_BF16, scale=scale)
    p = np.exp(logits - lse)
    bad = ref - p * np.sum(np.abs(gw), axis=-1)[..., None] * 0.1
    with pytest.raises(AssertionError):
        parity.check_logit_grad(to_bf16(bad), ref, sel, TOL_BF16, scale=scale)
