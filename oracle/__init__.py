"""ctypes wrapper around the plain C oracle (``oracle/ram_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (the HIP library and
its Python binding) never imports this package, and this package imports
nothing from the product.

Every array is a host numpy float64 array (io values of bf16 or fp32 convert
to float64 exactly); indices are int32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ram_oracle.c")
_LIB = os.path.join(_HERE, "libramoracle.so")


def build() -> str:
    """Compile the oracle with gcc (plain C, OpenMP, no fused multiply-add)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
        ("U", ctypes.c_int32), ("P", ctypes.c_int32),
        ("k_w", ctypes.c_int32), ("k_r", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("eps", ctypes.c_double),
        ("renorm_w", ctypes.c_int32), ("renorm_r", ctypes.c_int32),
        ("cape_heads", ctypes.c_int32), ("pad_", ctypes.c_int32),
        ("t0", ctypes.c_int64),
    ]

    @property
    def S(self) -> int:
        return int(self.P) ** int(self.U)


def problem(B, H, T, S=None, k_w=1, k_r=1, d_v=1, *, U=1, P=None, eps=1e-6,
            renorm=(False, False), cape_heads=0, t0=0) -> Problem:
    if P is None:
        if S is None:
            raise ValueError("give S (flat, U=1) or P")
        P = S if U == 1 else round(S ** (1.0 / U))
    if S is not None and P ** U != S:
        raise ValueError("S must equal P**U")
    rw, rr = (renorm, renorm) if isinstance(renorm, bool) else renorm
    return Problem(B, H, T, U, P, k_w, k_r, d_v, float(eps), int(rw), int(rr),
                   int(cape_heads), 0, int(t0))


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.POINTER(Problem)
        vp = ctypes.c_void_p
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_decode.argtypes = [P, ctypes.c_int, vp, vp, vp, vp]
        L.orc_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.orc_decode_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        L.orc_backward.argtypes = [P] + [vp] * 18
        L.orc_bucket.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.orc_epilogue_forward.argtypes = [ctypes.c_int64, ctypes.c_int, vp, vp, vp,
                                           ctypes.c_double, vp]
        L.orc_epilogue_backward.argtypes = [ctypes.c_int64, ctypes.c_int, vp, vp, vp,
                                            ctypes.c_double, vp, vp, vp, vp]
        _lib = L
    return _lib


def set_threads(n: int) -> int:
    """Set the OpenMP thread count (n <= 0 keeps it); returns the count in use."""
    return int(lib().orc_set_threads(int(n)))


def _f64in(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(status, what):
    if status != 0:
        raise RuntimeError(f"oracle {what} failed with status {status}")


def decode(p: Problem, side: int, logits):
    """Decode one side for every row.  logits (B,T,H,U,P) (or (B,T,H,S) when
    U = 1).  Returns idx (B,T,H,k) int32, w (B,T,H,k) float64, lse (B,T,H,U)."""
    lg = _f64in(logits)
    k = p.k_w if side == 0 else p.k_r
    shp = (p.B, p.T, p.H)
    idx = np.empty(shp + (k,), np.int32)
    w = np.empty(shp + (k,), np.float64)
    lse = np.empty(shp + (p.U,), np.float64)
    _check(lib().orc_decode(ctypes.byref(p), side, _ptr(lg), _ptr(idx), _ptr(w), _ptr(lse)),
           "decode")
    return idx, w, lse


def _mask(mask, shape):
    if mask is None:
        return None
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    if m.shape != shape:
        raise ValueError(f"mask must have shape {shape}, got {m.shape}")
    return m


def forward(p: Problem, wlogits, rlogits, v, gamma, slot0=None, mass0=None, mask=None):
    """Token-loop forward.  mask: (B,T), nonzero = valid token, or None.
    Returns o (B,T,H,d_v), slot1 (B,H,S,d_v), mass1 (B,H,S)."""
    wl, rl, vv, gg = _f64in(wlogits), _f64in(rlogits), _f64in(v), _f64in(gamma)
    s0, m0 = _f64(slot0), _f64(mass0)
    mk = _mask(mask, (p.B, p.T))
    o = np.empty((p.B, p.T, p.H, p.d_v), np.float64)
    s1 = np.empty((p.B, p.H, p.S, p.d_v), np.float64)
    m1 = np.empty((p.B, p.H, p.S), np.float64)
    _check(lib().orc_forward(ctypes.byref(p), _ptr(wl), _ptr(rl), _ptr(vv), _ptr(gg), _ptr(mk),
                             _ptr(s0), _ptr(m0), _ptr(o), _ptr(s1), _ptr(m1)), "forward")
    return o, s1, m1


def decode_step(p: Problem, wlogits, rlogits, v, gamma, slot, mass, mask=None):
    """One autoregressive step (p.T == 1); slot and mass (float64, C-contiguous)
    are updated in place.  mask: (B,) or None.  Returns o (B,1,H,d_v)."""
    if slot.dtype != np.float64 or not slot.flags.c_contiguous:
        raise ValueError("slot must be a C-contiguous float64 array")
    if mass.dtype != np.float64 or not mass.flags.c_contiguous:
        raise ValueError("mass must be a C-contiguous float64 array")
    wl, rl, vv, gg = _f64in(wlogits), _f64in(rlogits), _f64in(v), _f64in(gamma)
    o = np.empty((p.B, 1, p.H, p.d_v), np.float64)
    mk = _mask(mask, (p.B,))
    _check(lib().orc_decode_step(ctypes.byref(p), _ptr(wl), _ptr(rl), _ptr(vv), _ptr(gg),
                                 _ptr(mk), _ptr(slot), _ptr(mass), _ptr(o)), "decode_step")
    return o


def backward(p: Problem, wlogits, rlogits, v, gamma, slot0, mass0, d_o,
             d_slot1=None, d_mass1=None, mask=None):
    """Reverse token loop.  Returns a dict with d_wlogits, d_rlogits (shape of
    the logits), d_v, d_gamma, d_slot0, d_mass0 (None without slot0), and the
    decoded-weight gradients dw (B,T,H,k_w), dr (B,T,H,k_r).  mask as in forward."""
    wl, rl, vv, gg, do = _f64in(wlogits), _f64in(rlogits), _f64in(v), _f64in(gamma), _f64in(d_o)
    mk = _mask(mask, (p.B, p.T))
    s0, m0 = _f64(slot0), _f64(mass0)
    ds1, dm1 = _f64(d_slot1), _f64(d_mass1)
    out = {
        "d_wlogits": np.empty(wl.shape, np.float64),
        "d_rlogits": np.empty(rl.shape, np.float64),
        "d_v": np.empty((p.B, p.T, p.H, p.d_v), np.float64),
        "d_gamma": np.empty((p.B, p.T, p.H), np.float64),
        "d_slot0": np.empty((p.B, p.H, p.S, p.d_v), np.float64) if s0 is not None else None,
        "d_mass0": np.empty((p.B, p.H, p.S), np.float64) if s0 is not None else None,
        "dw": np.empty((p.B, p.T, p.H, p.k_w), np.float64),
        "dr": np.empty((p.B, p.T, p.H, p.k_r), np.float64),
    }
    _check(lib().orc_backward(
        ctypes.byref(p), _ptr(wl), _ptr(rl), _ptr(vv), _ptr(gg), _ptr(mk), _ptr(s0), _ptr(m0),
        _ptr(do), _ptr(ds1), _ptr(dm1),
        _ptr(out["d_wlogits"]), _ptr(out["d_rlogits"]), _ptr(out["d_v"]), _ptr(out["d_gamma"]),
        _ptr(out["d_slot0"]), _ptr(out["d_mass0"]), _ptr(out["dw"]), _ptr(out["dr"])),
        "backward")
    return out


def bucket(p: Problem, idx_w, idx_r):
    """Segment view.  Returns seg_offset (B*H*S+1,) int64 and per event position
    its token t, side (0 write / 1 read) and rank j, each (E,) int32."""
    iw = np.ascontiguousarray(idx_w, dtype=np.int32)
    ir = np.ascontiguousarray(idx_r, dtype=np.int32)
    nseg = p.B * p.H * p.S
    E = p.B * p.T * p.H * (p.k_w + p.k_r)
    seg = np.empty(nseg + 1, np.int64)
    ev_t = np.empty(E, np.int32)
    ev_s = np.empty(E, np.int32)
    ev_j = np.empty(E, np.int32)
    _check(lib().orc_bucket(ctypes.byref(p), _ptr(iw), _ptr(ir), _ptr(seg), _ptr(ev_t),
                            _ptr(ev_s), _ptr(ev_j)), "bucket")
    return seg, ev_t, ev_s, ev_j


def epilogue_forward(o, gate, gain=None, eps=1e-6):
    """Read epilogue y = sigmoid(gate) * RMSNorm(o) over the last axis (d_v):
    o / sqrt(mean(o^2) + eps) * gain.  o, gate (..., d_v); gain (d_v) or None."""
    oo, gg = _f64in(o), _f64in(gate)
    if oo.shape != gg.shape:
        raise ValueError("o and gate must have the same shape")
    d_v = oo.shape[-1]
    gn = None if gain is None else _f64in(gain)
    if gn is not None and gn.shape != (d_v,):
        raise ValueError("gain must have d_v entries")
    y = np.empty_like(oo)
    _check(lib().orc_epilogue_forward(ctypes.c_int64(oo.size // d_v), d_v, _ptr(oo), _ptr(gg),
                                      _ptr(gn), ctypes.c_double(eps), _ptr(y)),
           "epilogue_forward")
    return y


def epilogue_backward(o, gate, d_y, gain=None, eps=1e-6):
    """Gradients of epilogue_forward: returns d_o, d_gate (shape of o) and
    d_gain (d_v) summed over all rows (zeros when gain is None)."""
    oo, gg, dy = _f64in(o), _f64in(gate), _f64in(d_y)
    if oo.shape != gg.shape or oo.shape != dy.shape:
        raise ValueError("o, gate and d_y must have the same shape")
    d_v = oo.shape[-1]
    gn = None if gain is None else _f64in(gain)
    d_o, d_g = np.empty_like(oo), np.empty_like(oo)
    d_gain = np.zeros(d_v)
    _check(lib().orc_epilogue_backward(ctypes.c_int64(oo.size // d_v), d_v, _ptr(oo), _ptr(gg),
                                       _ptr(gn), ctypes.c_double(eps), _ptr(dy), _ptr(d_o),
                                       _ptr(d_g), _ptr(d_gain)),
           "epilogue_backward")
    return d_o, d_g, d_gain
