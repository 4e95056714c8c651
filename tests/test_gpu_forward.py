"""GPU parity of ram_forward against the oracle: decoded indices, segment
offsets and event lists bit-exact; outputs and final state within the
tolerance of the io dtype (1e-5 fp32, 2e-2 bf16, normwise relative)."""
import numpy as np
import pytest
import torch

import linear_attention_ram_amd as ram
import oracle
from gpu_util import (TOL, bh_slice, decode_event_codes, gpu_problem, host, oracle_problem, rel,
                      run_forward, say)
from linear_attention_ram_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def check_segments(p, views, oracle_idx_w, oracle_idx_r, bh_list=None):
    """Compare the workspace's segment arrays with the oracle's bucketing.
    bh_list: restrict to these flat (b*H + h) pairs (oracle idx given for
    exactly those, as (len, T, 1, k) arrays)."""
    seg = views["seg_offset"].cpu().numpy().astype(np.int64)
    ev = views["events"].cpu().numpy()
    S, K, T = p.S, p.k_w + p.k_r, p.T
    if bh_list is None:
        op = oracle.problem(p.B, p.H, p.T, S, p.k_w, p.k_r, 1)
        o_seg, o_t, o_s, o_j = oracle.bucket(op, oracle_idx_w, oracle_idx_r)
        np.testing.assert_array_equal(seg, o_seg)
        t, s, j = decode_event_codes(ev)
        np.testing.assert_array_equal(t, o_t)
        np.testing.assert_array_equal(s, o_s)
        np.testing.assert_array_equal(j, o_j)
        return
    for n, bh in enumerate(bh_list):
        op = oracle.problem(1, 1, T, S, p.k_w, p.k_r, 1)
        o_seg, o_t, o_s, o_j = oracle.bucket(op, oracle_idx_w[n:n + 1], oracle_idx_r[n:n + 1])
        base = bh * T * K
        np.testing.assert_array_equal(seg[bh * S:(bh + 1) * S + 1] - base, o_seg)
        t, s, j = decode_event_codes(ev[base:base + T * K])
        np.testing.assert_array_equal(t, o_t)
        np.testing.assert_array_equal(s, o_s)
        np.testing.assert_array_equal(j, o_j)


def full_check(cfg, x, p, with_state, tol):
    slot0 = x.get("slot0") if with_state else None
    mass0 = x.get("mass0") if with_state else None
    r = run_forward(p, x, slot0=slot0, mass0=mass0)
    torch.cuda.synchronize()
    h = {k: host(v) for k, v in x.items()}
    op = oracle_problem(p)
    say("oracle forward", cfg.name)
    oo, os_, om = oracle.forward(op, h["wl"], h["rl"], h["v"], h["gamma"],
                                 h.get("slot0") if with_state else None,
                                 h.get("mass0") if with_state else None)
    assert rel(host(r["o"]), oo) <= tol, rel(host(r["o"]), oo)
    assert rel(host(r["slot1"]), os_) <= tol, rel(host(r["slot1"]), os_)
    assert rel(host(r["mass1"]), om) <= tol, rel(host(r["mass1"]), om)
    # decoded indices and weights, then segments
    views = ram.ws_views(p, r["ws"])
    iw, ww, _ = oracle.decode(op, 0, h["wl"])
    ir, wr, _ = oracle.decode(op, 1, h["rl"])
    np.testing.assert_array_equal(views["idx_w"].cpu().numpy().reshape(iw.shape), iw)
    np.testing.assert_array_equal(views["idx_r"].cpu().numpy().reshape(ir.shape), ir)
    assert rel(views["w_w"].cpu().numpy().reshape(ww.shape), ww) <= 1e-5
    assert rel(views["w_r"].cpu().numpy().reshape(wr.shape), wr) <= 1e-5
    check_segments(p, views, iw, ir)
    return r


@pytest.mark.parametrize("with_state", [False, True])
def test_tiny_full(with_state):
    cfg = synth.CONFIGS["tiny"]
    x = synth.layer_inputs(cfg, device=DEV, seed=0, with_state=True)
    full_check(cfg, x, gpu_problem(cfg), with_state, TOL["f32"])


@pytest.mark.parametrize("with_state", [False, True])
def test_340m_full(with_state):
    cfg = synth.CONFIGS["340m"]
    x = synth.layer_inputs(cfg, device=DEV, seed=1, with_state=True, with_d_o=False)
    full_check(cfg, x, gpu_problem(cfg), with_state, TOL["bf16"])


def test_1_3b_sampled_slices():
    cfg = synth.CONFIGS["1.3b"]
    x = synth.layer_inputs(cfg, device=DEV, seed=0, with_d_o=False)
    p = gpu_problem(cfg)
    say("1.3b forward on GPU")
    r = run_forward(p, x)
    torch.cuda.synchronize()
    views = ram.ws_views(p, r["ws"])
    pairs = [(0, 0), (3, 7), (7, 15)]
    iws, irs = [], []
    for b, h in pairs:
        say("1.3b oracle slice", b, h)
        s = bh_slice(x, b, h)
        op = oracle.problem(1, 1, cfg.T, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, eps=cfg.eps)
        oo, os_, om = oracle.forward(op, s["wl"], s["rl"], s["v"], s["gamma"])
        assert rel(host(r["o"][b, :, h]), oo[0, :, 0]) <= TOL["bf16"]
        assert rel(host(r["slot1"][b, h]), os_[0, 0]) <= TOL["bf16"]
        assert rel(host(r["mass1"][b, h]), om[0, 0]) <= TOL["bf16"]
        iw, _, _ = oracle.decode(op, 0, s["wl"])
        ir, _, _ = oracle.decode(op, 1, s["rl"])
        iws.append(iw[:, :, 0])
        irs.append(ir[:, :, 0])
    check_segments(p, views, np.concatenate(iws)[:, :, None], np.concatenate(irs)[:, :, None],
                   bh_list=[b * cfg.H + h for b, h in pairs])


def test_long_context_chunk_carry():
    cfg = synth.CONFIGS["long"]
    heads = (3,)
    p = ram.problem(cfg.B, cfg.H, cfg.chunk, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, io=cfg.io)
    ws = ram.workspace(p, False, DEV)
    slot = mass = None
    o_slot, o_mass = {}, {}
    nchunks = cfg.T // cfg.chunk
    for c in range(nchunks):
        x = synth.chunk_inputs(cfg, c, device=DEV, seed=0)
        r = run_forward(p, x, ws=ws, slot0=slot, mass0=mass)
        torch.cuda.synchronize()
        slot, mass = r["slot1"], r["mass1"]
        say("long chunk", c)
        for h in heads:
            s = bh_slice(x, 0, h)
            op = oracle.problem(1, 1, cfg.chunk, cfg.S, cfg.k_w, cfg.k_r, cfg.d_v, eps=cfg.eps)
            oo, o_slot[h], o_mass[h] = oracle.forward(op, s["wl"], s["rl"], s["v"], s["gamma"],
                                                      o_slot.get(h), o_mass.get(h))
            assert rel(host(r["o"][0, :, h]), oo[0, :, 0]) <= TOL["bf16"], c
    for h in heads:
        assert rel(host(slot[0, h]), o_slot[h][0, 0]) <= TOL["bf16"]
        assert rel(host(mass[0, h]), o_mass[h][0, 0]) <= TOL["bf16"]


EDGE = [
    # B, H, T, S, k_w, k_r, d_v, io, renorm, eps
    (1, 1, 1, 8, 1, 1, 1, "f32", (False, False), 1e-6),
    (2, 3, 31, 16, 3, 2, 7, "f32", (False, False), 1e-6),
    (1, 2, 33, 64, 64, 8, 64, "f32", (True, False), 1e-6),
    (3, 1, 300, 32, 2, 5, 66, "f32", (False, True), 1e-3),
    (1, 2, 257, 128, 4, 4, 128, "bf16", (False, False), 1e-6),
    (2, 2, 600, 8, 8, 8, 16, "bf16", (True, True), 0.0),   # 8 slots, every token writes all
    (1, 2, 2000, 16, 4, 4, 16, "f32", (False, False), 1e-6),  # ~1000-event segments
    (1, 1, 3000, 8, 3, 2, 128, "f32", (False, False), 1e-6),  # long segments, wide slots
    # most slots without events (the short list), rows not of whole 16-byte
    # vectors: the empty slots' state element by element, zero then copied
    (1, 2, 5, 256, 2, 2, 66, "f32", (False, False), 1e-6),
    (1, 2, 5, 256, 2, 2, 7, "bf16", (False, False), 1e-6),
]


@pytest.mark.parametrize("case", range(len(EDGE)))
def test_edge_shapes(case):
    B, H, T, S, kw, kr, d, io, rn, eps = EDGE[case]
    cfg = synth.Config("edge", B, H, T, S, kw, kr, d, io)
    x = synth.layer_inputs(cfg, device=DEV, seed=10 + case, with_state=True, with_d_o=False)
    p = ram.problem(B, H, T, S, kw, kr, d, io=io, eps=eps, renorm=rn)
    full_check(cfg, x, p, case % 2 == 1, TOL[io])


def test_empty_call_copies_state():
    cfg = synth.Config("empty", 2, 3, 0, 64, 2, 2, 16, "bf16")
    p = ram.problem(2, 3, 0, 64, 2, 2, 16, io="bf16")
    g = torch.Generator(device=DEV).manual_seed(3)
    slot0 = torch.randn((2, 3, 64, 16), generator=g, device=DEV)
    mass0 = torch.rand((2, 3, 64), generator=g, device=DEV)
    x = {k: torch.empty((2, 0, 3) + s, dtype=torch.bfloat16, device=DEV)
         for k, s in (("wl", (64,)), ("rl", (64,)), ("v", (16,)), ("gamma", ()))}
    r = run_forward(p, x, slot0=slot0, mass0=mass0)
    torch.cuda.synchronize()
    assert torch.equal(r["slot1"], slot0) and torch.equal(r["mass1"], mass0)
    del cfg


def test_untouched_slots_bitwise_and_overwrite_limit():
    cfg = synth.CONFIGS["340m"].with_(B=2, T=300)
    x = synth.layer_inputs(cfg, device=DEV, seed=5, with_state=True, with_d_o=False)
    # gamma = +1e4, eps = 0: lambda = 0, eta = 1, every write replaces its slot
    x["gamma"] = torch.full_like(x["gamma"], 1e4)
    p = gpu_problem(cfg, eps=0.0)
    r = run_forward(p, x, slot0=x["slot0"], mass0=x["mass0"])
    torch.cuda.synchronize()
    h = {k: host(v) for k, v in x.items()}
    op = oracle_problem(p)
    oo, os_, om = oracle.forward(op, h["wl"], h["rl"], h["v"], h["gamma"], h["slot0"], h["mass0"])
    # final contents are exact copies of values (or untouched initial rows);
    # the final mass is the last write's weight, a float32 probability
    np.testing.assert_array_equal(host(r["slot1"]), os_)
    assert rel(host(r["mass1"]), om) <= 1e-6
    iw, _, _ = oracle.decode(op, 0, h["wl"])
    touched = np.zeros((cfg.B, cfg.H, cfg.S), bool)
    for b in range(cfg.B):
        for hh in range(cfg.H):
            touched[b, hh, np.unique(iw[b, :, hh])] = True
    assert (~touched).sum() > 0
    np.testing.assert_array_equal(host(r["slot1"])[~touched], h["slot0"][~touched])
    assert rel(host(r["o"]), oo) <= TOL["bf16"]


@pytest.mark.parametrize("S", [1504, 2504])   # rows of whole 16-byte vectors
def test_hot_slots_over_ragged_slot_blocks(S):
    # the bucketing scan works in blocks of 1024 slots: S here leaves a
    # partial last block, and the Zipf bias makes hot slots whose segments
    # (thousands of events) take the cooperative scan path
    cfg = synth.Config("hot-ragged", 2, 2, 1024, S, 8, 8, 64, "bf16", zipf=1.1)
    x = synth.layer_inputs(cfg, device=DEV, seed=40 + S, with_state=True, with_d_o=False)
    p = gpu_problem(cfg)
    r = full_check(cfg, x, p, True, TOL["bf16"])
    seg = ram.ws_views(p, r["ws"])["seg_offset"].cpu().numpy()
    assert (seg[1:] - seg[:-1]).max() > 1000


def raised_slots(cfg, seed, nhot, bias, **kw):
    """Inputs whose first nhot slots have their logits raised by bias, so
    that they take most selections."""
    x = synth.layer_inputs(cfg, device=DEV, seed=seed, **kw)
    for side in ("wl", "rl"):
        x[side][..., :nhot] += bias
    return x


def short_list_mode(seg):
    """Whether the short-segment scans take the bucketing's short list (at
    most half of all segments have 1 to 128 events) or map waves to
    segments directly."""
    n = np.diff(seg.astype(np.int64))
    return 2 * int(((n > 0) & (n <= 128)).sum()) <= n.size


# 512 tokens, S = 2048, k = 4: 512 raised slots give about 500 short
# segments per head (the list), 1024 slots raised by 1 about 1100 (direct)
RAISED = [(512, 2.0, True), (1024, 1.0, False)]


@pytest.mark.parametrize("nhot,bias,listed", RAISED)
def test_short_segments_listed_or_direct(nhot, bias, listed):
    # both ways the short-segment scans find their segments, with the state
    # of the slots without events kept bit for bit
    cfg = synth.Config("raised", 1, 2, 512, 2048, 4, 4, 64, "bf16")
    x = raised_slots(cfg, 50, nhot, bias, with_state=True, with_d_o=False)
    p = gpu_problem(cfg)
    r = full_check(cfg, x, p, True, TOL["bf16"])
    seg = ram.ws_views(p, r["ws"])["seg_offset"].cpu().numpy()
    assert short_list_mode(seg) == listed
    empty = torch.from_numpy(np.diff(seg.astype(np.int64)) == 0).to(DEV).reshape(cfg.B, cfg.H, cfg.S)
    assert empty.any()
    assert torch.equal(r["slot1"][empty], x["slot0"][empty])
    assert torch.equal(r["mass1"][empty], x["mass0"][empty])


def test_widest_address_space():
    # S = 16384, the largest flat address space: 16 blocks in the bucketing
    # scan and the largest LDS tables of the bucketing scatter
    cfg = synth.Config("widest", 1, 2, 512, 16384, 8, 8, 64, "bf16", zipf=1.1)
    x = synth.layer_inputs(cfg, device=DEV, seed=44, with_state=True, with_d_o=False)
    full_check(cfg, x, gpu_problem(cfg), True, TOL["bf16"])


def test_bucketing_in_several_rounds():
    # 48 events per token: a bucketing tile of 128 tokens holds 6,144 events,
    # more than one round (4,096) of the scatter's ranking
    cfg = synth.Config("rounds", 1, 2, 300, 64, 24, 24, 16, "f32")
    x = synth.layer_inputs(cfg, device=DEV, seed=46, with_state=True, with_d_o=False)
    p = ram.problem(1, 2, 300, 64, 24, 24, 16, io="f32")
    full_check(cfg, x, p, True, TOL["f32"])


@pytest.mark.parametrize("S", [4096, 16384])
def test_decoder_rows_across_the_side_boundary(S):
    # 111 (token, head) rows per side and k_w != k_r: the decoder workgroup of
    # rows 108..111 holds three write-side rows and the first read-side row.
    # S = 4096 takes the register-resident decoder whose workgroups gather
    # their results in LDS, S = 16384 the one whose waves store their own rows.
    cfg = synth.Config("sides", 1, 3, 37, S, 8, 5, 32, "bf16")
    x = synth.layer_inputs(cfg, device=DEV, seed=48, with_state=False, with_d_o=False)
    full_check(cfg, x, gpu_problem(cfg), False, TOL["bf16"])
