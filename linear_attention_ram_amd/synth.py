"""Seeded synthetic inputs for the RAM-Net attention core.

This module only draws random numbers; it holds none of the method's
arithmetic.  Tests, the benchmark and the smoke check use it to make the
inputs that both the HIP path and the CPU oracle then consume.

Workload shapes follow the configurations the path is measured on (layer
shapes of the paper's 340M and 1.3B models, a long-context chunked forward,
and an autoregressive decode batch); values are N(0, 1) unless stated:

* address logits are drawn directly (the op takes logits, ramnet-ops
  "Arguments"); the tiny case builds them as key/query times a fixed
  N(0, 1/d_k) projection, which yields N(0, 1) logits;
* the forgetting modulator gamma is N(ln 9, 1): ln 9 is the paper's bias
  initialisation of gamma (paper App. A "Bias Initialization");
* the hot-slot case adds a per-head Zipf(1.1) bias -1.1 * ln(1 + pi_h(a)),
  pi_h a seeded permutation of the slots, to both sides' logits before the
  cast to the io dtype (key and query share the address bias in the paper's
  App. A; a few always-on slots appear in the access traces of App. C).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

LN9 = math.log(9.0)


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    T: int
    S: int
    k_w: int
    k_r: int
    d_v: int
    io: str                    # "f32" or "bf16"
    zipf: float | None = None  # Zipf exponent of the per-slot bias, or None
    chunk: int | None = None   # tokens per forward call (long context)
    steps: int | None = None   # autoregressive steps (decode)
    d_k: int | None = None     # key/query width of the projection case
    eps: float = 1e-6
    U: int = 1                 # address digits; S = P**U

    @property
    def P(self) -> int:
        """Digit size."""
        if self.U == 1:
            return self.S
        P = round(self.S ** (1.0 / self.U))
        assert P ** self.U == self.S, (self.S, self.U)
        return P

    @property
    def logit_shape(self) -> tuple:
        """Trailing shape of one (token, head) logit row: (S,) or (U, P)."""
        return (self.S,) if self.U == 1 else (self.U, self.P)

    @property
    def dtype(self) -> torch.dtype:
        return torch.float32 if self.io == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    # B=1,H=1,T=256,S=64,k=2,d=16,fp32; logits = key/query @ N(0,1/d_k) projection
    "tiny": Config("tiny", 1, 1, 256, 64, 2, 2, 16, "f32", d_k=16),
    # 340M-layer shape
    "340m": Config("340m", 4, 8, 2048, 1024, 4, 4, 64, "bf16"),
    # 1.3B-layer shape with hot-slot contention
    "1.3b": Config("1.3b", 8, 16, 4096, 4096, 8, 8, 128, "bf16", zipf=1.1),
    # long context: 16 chunks of 4096 tokens with state carry
    "long": Config("long", 1, 16, 65536, 16384, 8, 8, 128, "bf16", chunk=4096),
    # autoregressive decode: 256 sequences, one token per step
    "decode": Config("decode", 256, 16, 1, 4096, 8, 8, 128, "bf16", steps=1024),
    # product-softmax addresses (U >= 2 digits of P logits each):
    # the 1.3B-layer shape factorised as U = 2 digits of 64 (q/k are the digit logits)
    "1.3b-u2": Config("1.3b-u2", 8, 16, 4096, 4096, 8, 8, 128, "bf16", U=2),
    # the ramnet-ops example shape: U = 3 digits of 4, C = 32, top-8
    "ops-example": Config("ops-example", 2, 4, 32, 64, 8, 8, 32, "f32", U=3),
    # the paper's default address space 4^5: U = 5 digits of 4
    "u5": Config("u5", 2, 4, 512, 1024, 8, 8, 64, "bf16", U=5),
}


def generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, dtype, mean=0.0, std=1.0, bias=None):
    """N(mean, std^2) drawn in float32 one leading slice at a time (bounded
    temporary memory), optionally plus a bias broadcast over the trailing
    dims, then cast to ``dtype``."""
    out = torch.empty(shape, dtype=dtype, device=device)
    for i in range(shape[0]):
        x = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        if mean != 0.0:
            x.add_(mean)
        if bias is not None:
            x.add_(bias)
        out[i].copy_(x)
        del x
    return out


def zipf_bias(cfg: Config, g, device) -> torch.Tensor:
    """(H, S) float32 bias -s * ln(1 + pi_h(a)) with pi_h a seeded permutation."""
    rows = []
    for _ in range(cfg.H):
        perm = torch.randperm(cfg.S, generator=g, device=device)
        rows.append(-cfg.zipf * torch.log1p(perm.to(torch.float32)))
    return torch.stack(rows)


def layer_inputs(cfg: Config, device="cpu", seed: int = 0, T: int | None = None,
                 with_state: bool = False, with_state_grads: bool = False,
                 with_d_o: bool = True):
    """Inputs of one forward(+backward) call.  Draw order: Zipf permutations
    (if any), write logits, read logits, v, gamma, dO, then the optional
    slot0 ~ N(0,1), mass0 ~ U(0,1), d_slot1 ~ N(0,1), d_mass1 ~ N(0,1).

    Returns a dict of tensors on ``device``: wl, rl (B,T,H,S), or (B,T,H,U,P)
    for U >= 2 digits; v (B,T,H,d_v);
    gamma (B,T,H); d_o (B,T,H,d_v); slot0 (B,H,S,d_v) f32; mass0 (B,H,S) f32;
    d_slot1, d_mass1 likewise."""
    T = cfg.T if T is None else T
    g = generator(device, seed)
    dt = cfg.dtype
    out = {}
    if cfg.d_k is not None:
        # key/query times a fixed N(0, 1/d_k) projection to S slots (fp32 host math)
        q = torch.randn((cfg.B, T, cfg.H, cfg.d_k), generator=g, device=device)
        k = torch.randn((cfg.B, T, cfg.H, cfg.d_k), generator=g, device=device)
        v = torch.randn((cfg.B, T, cfg.H, cfg.d_v), generator=g, device=device)
        W = torch.randn((cfg.d_k, cfg.S), generator=g, device=device) / math.sqrt(cfg.d_k)
        out["wl"] = (k @ W).to(dt).contiguous()
        out["rl"] = (q @ W).to(dt).contiguous()
        out["v"] = v.to(dt)
        out["gamma"] = (torch.randn((cfg.B, T, cfg.H), generator=g, device=device) + LN9).to(dt)
    else:
        bias = None
        if cfg.zipf is not None:
            assert cfg.U == 1, "the per-slot bias is defined for flat addresses"
            bias = zipf_bias(cfg, g, device)          # (H, S), broadcast over (T, H, S)
        shape = (cfg.B, T, cfg.H) + cfg.logit_shape
        out["wl"] = _randn(shape, g, device, dt, bias=bias)
        out["rl"] = _randn(shape, g, device, dt, bias=bias)
        out["v"] = _randn((cfg.B, T, cfg.H, cfg.d_v), g, device, dt)
        out["gamma"] = _randn((cfg.B, T, cfg.H), g, device, dt, mean=LN9)
    if with_d_o:
        out["d_o"] = _randn((cfg.B, T, cfg.H, cfg.d_v), g, device, dt)
    if with_state:
        out["slot0"] = _randn((cfg.B, cfg.H, cfg.S, cfg.d_v), g, device, torch.float32)
        out["mass0"] = torch.rand((cfg.B, cfg.H, cfg.S), generator=g, device=device)
    if with_state_grads:
        out["d_slot1"] = _randn((cfg.B, cfg.H, cfg.S, cfg.d_v), g, device, torch.float32)
        out["d_mass1"] = torch.randn((cfg.B, cfg.H, cfg.S), generator=g, device=device)
    return out


def gate_inputs(cfg: Config, device="cpu", seed: int = 0, T: int | None = None):
    """Inputs of the gated read-out, from their own seeded stream (seed * 7 +
    3): gate pre-activations (B,T,H,d_v) ~ N(3, 1) in the io dtype (3 is the
    paper's output-gate bias initialisation, App. A "Bias Initialization"),
    RMSNorm gain (d_v) ~ 1 + 0.1 N(0, 1) float32, and the gradient d_y of the
    gated output (B,T,H,d_v) ~ N(0, 1) io."""
    T = cfg.T if T is None else T
    g = generator(device, seed * 7 + 3)
    shape = (cfg.B, T, cfg.H, cfg.d_v)
    return {"gate": _randn(shape, g, device, cfg.dtype, mean=3.0),
            "gain": 1.0 + 0.1 * torch.randn((cfg.d_v,), generator=g, device=device),
            "d_y": _randn(shape, g, device, cfg.dtype)}


def chunk_inputs(cfg: Config, chunk: int, device="cpu", seed: int = 0):
    """Inputs of chunk ``chunk`` of the long-context forward: its own seeded
    stream (seed * 1_000_003 + chunk) so any chunk can be regenerated alone."""
    sub = cfg.with_(T=cfg.chunk)
    return layer_inputs(sub, device=device, seed=seed * 1_000_003 + chunk, with_d_o=False)


def decode_state(cfg: Config, device="cpu", seed: int = 0, std: float = 0.02):
    """Initial decode state: slot ~ N(0, std^2) float32 (B,H,S,d_v), mass = 0."""
    g = generator(device, seed)
    slot = _randn((cfg.B, cfg.H, cfg.S, cfg.d_v), g, device, torch.float32, std=std)
    mass = torch.zeros((cfg.B, cfg.H, cfg.S), dtype=torch.float32, device=device)
    return slot, mass


def decode_step_inputs(cfg: Config, step: int, device="cpu", seed: int = 0):
    """Inputs of one decode step (T = 1), seeded per step."""
    sub = cfg.with_(T=1, zipf=None)
    return layer_inputs(sub, device=device, seed=(seed + 1) * 7_919 + step, with_d_o=False)
