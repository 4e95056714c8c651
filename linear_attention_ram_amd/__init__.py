"""Python binding of the RAM-Net attention core for AMD MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``_lib/libramnet.so`` behind the C ABI declared in
``include/ramnet.h``.  There is no CPU or PyTorch fallback; if the library is
missing the calls raise.  PyTorch supplies device memory and the stream.

Functions keep the C names: ``ram_workspace_size``, ``ram_workspace_layout``,
``ram_decode``, ``ram_forward``, ``ram_forward_noalloc``, ``ram_backward``,
``ram_forward_gated``,
``ram_backward_gated`` (with ``epilogue`` to build their gate argument),
``ram_decode_step``,
``ram_status_string``, plus ``ram_prof_enable`` / ``ram_prof_collect``.
Tensors are passed by device pointer; the stream defaults to PyTorch's current
stream.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libramnet.so")

RAM_OK, RAM_EINVAL, RAM_EDTYPE, RAM_ECAPACITY, RAM_EUNSUPPORTED, RAM_EHIP = 0, -1, -2, -3, -4, -5
RAM_F32, RAM_BF16 = 0, 1
EXPORTED = ("ram_workspace_size", "ram_workspace_layout", "ram_decode", "ram_forward",
            "ram_backward", "ram_forward_gated", "ram_backward_gated", "ram_decode_step",
            "ram_forward_noalloc", "ram_stream_probe", "ram_status_string", "ram_prof_enable",
            "ram_prof_collect")
NOALLOC_SCRATCH_BYTES = 64 << 20   # RAM_NOALLOC_SCRATCH_BYTES


class Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
        ("U", ctypes.c_int32), ("P", ctypes.c_int32),
        ("k_w", ctypes.c_int32), ("k_r", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32), ("eps", ctypes.c_float),
        ("renorm_w", ctypes.c_int32), ("renorm_r", ctypes.c_int32),
        ("cape_heads", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("t0", ctypes.c_int64),
    ]

    @property
    def S(self) -> int:
        return int(self.P) ** int(self.U)

    @property
    def N(self) -> int:
        return int(self.B) * int(self.T) * int(self.H)

    @property
    def row(self) -> int:
        """Logits per (token, head, side): U * P."""
        return int(self.U) * int(self.P)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.io_dtype == RAM_F32 else torch.bfloat16


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "idx_w", "w_w", "lse_w", "idx_r", "w_r", "lse_r", "seg_offset", "events", "ckpt_s",
        "ckpt_m", "stash", "tile_hist", "long_list", "long_count", "short_list", "stash_b", "dw", "dr",
        "dgam", "epi_d_o", "epi_part", "fwd_bytes", "total_bytes")]


class Epilogue(ctypes.Structure):
    """Gated read-out: y = sigmoid(gate) * RMSNorm(o) (gate io (B,T,H,d_v),
    gain float (d_v) or NULL, eps)."""
    _fields_ = [("gate", ctypes.c_void_p), ("gain", ctypes.c_void_p), ("eps", ctypes.c_float)]


class ProfEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


def problem(B, H, T, S=None, k_w=1, k_r=1, d_v=1, io="bf16", eps=1e-6, renorm=(False, False),
            cape_heads=0, t0=0, *, U=1, P=None) -> Problem:
    """Problem description.  One address digit: give S (U = 1, P = S).  U >= 2
    digits of size P: give U and P (S = P**U; if S is given too it must agree)."""
    io_dtype = {"f32": RAM_F32, "bf16": RAM_BF16, torch.float32: RAM_F32,
                torch.bfloat16: RAM_BF16}[io]
    if P is None:
        if S is None or U != 1:
            raise ValueError("give S (one digit) or U and P")
        P = S
    if S is not None and int(P) ** int(U) != S:
        raise ValueError("S must equal P**U")
    rw, rr = (renorm, renorm) if isinstance(renorm, bool) else renorm
    return Problem(B, H, T, int(U), int(P), k_w, k_r, d_v, io_dtype, float(eps), int(rw),
                   int(rr), int(cape_heads), 0, int(t0))


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(hipcc for gfx950); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.ram_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(sz)]
    L.ram_workspace_layout.argtypes = [P, ctypes.POINTER(WsLayout)]
    L.ram_decode.argtypes = [P, ctypes.c_int, vp, vp, vp, vp, vp]
    L.ram_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.ram_backward.argtypes = [P, vp, sz] + [vp] * 17
    L.ram_decode_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.ram_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.ram_stream_probe.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, sz, vp]
    EP = ctypes.POINTER(Epilogue)
    L.ram_forward_gated.argtypes = [P, EP, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.ram_backward_gated.argtypes = [P, EP, vp, sz] + [vp] * 19
    L.ram_status_string.argtypes = [ctypes.c_int]
    L.ram_status_string.restype = ctypes.c_char_p
    L.ram_prof_enable.argtypes = [ctypes.c_int]
    L.ram_prof_collect.argtypes = [ctypes.POINTER(ProfEntry), ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_int)]
    for name in EXPORTED:
        if name not in ("ram_status_string",):
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def ram_status_string(status: int) -> str:
    return lib().ram_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != RAM_OK:
        raise RuntimeError(f"{what}: {ram_status_string(status)} (status {status})")


def _ptr(t, name, dtype=None, numel=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, device=None):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def ram_workspace_size(p: Problem, with_backward: bool = True) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ram_workspace_size(ctypes.byref(p), int(with_backward), ctypes.byref(n)),
           "ram_workspace_size")
    return int(n.value)


def ram_workspace_layout(p: Problem) -> dict:
    L = WsLayout()
    _check(lib().ram_workspace_layout(ctypes.byref(p), ctypes.byref(L)), "ram_workspace_layout")
    return {name: int(getattr(L, name)) for name, _ in WsLayout._fields_}


def workspace(p: Problem, with_backward: bool = True, device="cuda") -> torch.Tensor:
    """A byte tensor of the size the library asks for."""
    return torch.empty(ram_workspace_size(p, with_backward), dtype=torch.uint8, device=device)


def ws_views(p: Problem, ws: torch.Tensor) -> dict:
    """Typed views of the arrays the forward leaves in the workspace."""
    L = ram_workspace_layout(p)
    N, S = p.N, p.S
    E = N * (p.k_w + p.k_r)

    def view(off, n, dt):
        nbytes = n * torch.empty((), dtype=dt).element_size()
        return ws[off:off + nbytes].view(dt)

    return {
        "idx_w": view(L["idx_w"], N * p.k_w, torch.int32),
        "w_w": view(L["w_w"], N * p.k_w, torch.float32),
        "lse_w": view(L["lse_w"], N * p.U, torch.float32),
        "idx_r": view(L["idx_r"], N * p.k_r, torch.int32),
        "w_r": view(L["w_r"], N * p.k_r, torch.float32),
        "lse_r": view(L["lse_r"], N * p.U, torch.float32),
        "seg_offset": view(L["seg_offset"], p.B * p.H * S + 1, torch.int32),
        "events": view(L["events"], 4 * E, torch.int32).view(E, 4)[:, 0],
        "event_w": view(L["events"], 4 * E, torch.float32).view(E, 4)[:, 1],
        "dw": view(L["dw"], N * p.k_w, torch.float32),
        "dr": view(L["dr"], N * p.k_r, torch.float32),
    }


def ram_decode(p: Problem, side: int, logits, idx, weight, lse, stream=None):
    k = p.k_w if side == 0 else p.k_r
    args = (_ptr(logits, "logits", p.torch_dtype, p.N * p.row),
            _ptr(idx, "idx", torch.int32, p.N * k),
            _ptr(weight, "weight", torch.float32, p.N * k),
            _ptr(lse, "lse", torch.float32, p.N * p.U))
    _check(lib().ram_decode(ctypes.byref(p), int(side), *args, _stream(stream, logits.device)),
           "ram_decode")


def ram_forward(p: Problem, wlogits, rlogits, v, gamma, slot0, mass0, o, slot1, mass1, ws,
                stream=None, mask=None):
    """mask: optional (B, T) uint8 tensor, nonzero = valid token."""
    io = p.torch_dtype
    N, S, nseg = p.N, p.S, p.B * p.H * p.S
    args = (_ptr(wlogits, "wlogits", io, N * p.row), _ptr(rlogits, "rlogits", io, N * p.row),
            _ptr(v, "v", io, N * p.d_v), _ptr(gamma, "gamma", io, N),
            _ptr(mask, "mask", torch.uint8, p.B * p.T, optional=True),
            _ptr(slot0, "slot0", torch.float32, nseg * p.d_v, optional=True),
            _ptr(mass0, "mass0", torch.float32, nseg, optional=True),
            _ptr(o, "o", io, N * p.d_v),
            _ptr(slot1, "slot1", torch.float32, nseg * p.d_v),
            _ptr(mass1, "mass1", torch.float32, nseg),
            _ptr(ws, "ws", torch.uint8), ctypes.c_size_t(ws.numel()))
    _check(lib().ram_forward(ctypes.byref(p), *args, _stream(stream, ws.device)), "ram_forward")


def ram_backward(p: Problem, ws, wlogits, rlogits, v, gamma, slot0, mass0, d_o, d_slot1, d_mass1,
                 d_wlogits, d_rlogits, d_v, d_gamma, d_slot0=None, d_mass0=None, stream=None,
                 mask=None):
    """mask: the (B, T) uint8 mask the forward was given, or None."""
    io = p.torch_dtype
    N, S, nseg = p.N, p.S, p.B * p.H * p.S
    args = (_ptr(ws, "ws", torch.uint8), ctypes.c_size_t(ws.numel()),
            _ptr(wlogits, "wlogits", io, N * p.row), _ptr(rlogits, "rlogits", io, N * p.row),
            _ptr(v, "v", io, N * p.d_v), _ptr(gamma, "gamma", io, N),
            _ptr(mask, "mask", torch.uint8, p.B * p.T, optional=True),
            _ptr(slot0, "slot0", torch.float32, nseg * p.d_v, optional=True),
            _ptr(mass0, "mass0", torch.float32, nseg, optional=True),
            _ptr(d_o, "d_o", io, N * p.d_v),
            _ptr(d_slot1, "d_slot1", torch.float32, nseg * p.d_v, optional=True),
            _ptr(d_mass1, "d_mass1", torch.float32, nseg, optional=True),
            _ptr(d_wlogits, "d_wlogits", io, N * p.row),
            _ptr(d_rlogits, "d_rlogits", io, N * p.row),
            _ptr(d_v, "d_v", io, N * p.d_v), _ptr(d_gamma, "d_gamma", io, N),
            _ptr(d_slot0, "d_slot0", torch.float32, nseg * p.d_v, optional=True),
            _ptr(d_mass0, "d_mass0", torch.float32, nseg, optional=True))
    _check(lib().ram_backward(ctypes.byref(p), *args, _stream(stream, ws.device)), "ram_backward")


def ram_forward_noalloc(p: Problem, wlogits, rlogits, v, gamma, slot0, mass0, o, slot1, mass1,
                        stream=None, mask=None):
    """ram_forward without a workspace (the library's per-device array of
    NOALLOC_SCRATCH_BYTES); no backward can follow it."""
    io = p.torch_dtype
    N, nseg = p.N, p.B * p.H * p.S
    args = (_ptr(wlogits, "wlogits", io, N * p.row), _ptr(rlogits, "rlogits", io, N * p.row),
            _ptr(v, "v", io, N * p.d_v), _ptr(gamma, "gamma", io, N),
            _ptr(mask, "mask", torch.uint8, p.B * p.T, optional=True),
            _ptr(slot0, "slot0", torch.float32, nseg * p.d_v, optional=True),
            _ptr(mass0, "mass0", torch.float32, nseg, optional=True),
            _ptr(o, "o", io, N * p.d_v),
            _ptr(slot1, "slot1", torch.float32, nseg * p.d_v),
            _ptr(mass1, "mass1", torch.float32, nseg))
    _check(lib().ram_forward_noalloc(ctypes.byref(p), *args, _stream(stream, o.device)),
           "ram_forward_noalloc")


def epilogue(p: Problem, gate, gain=None, eps=1e-6) -> Epilogue:
    """Gated read-out arguments; gate (B,T,H,d_v) io, gain (d_v) float32 or None.
    The tensors must stay alive while calls that use the result run."""
    return Epilogue(_ptr(gate, "gate", p.torch_dtype, p.N * p.d_v),
                    _ptr(gain, "gain", torch.float32, p.d_v, optional=True), float(eps))


def ram_forward_gated(p: Problem, ep: Epilogue, wlogits, rlogits, v, gamma, slot0, mass0, y,
                      slot1, mass1, ws, stream=None, mask=None):
    """ram_forward with the gated read-out: writes y instead of o."""
    io = p.torch_dtype
    N, nseg = p.N, p.B * p.H * p.S
    args = (_ptr(wlogits, "wlogits", io, N * p.row), _ptr(rlogits, "rlogits", io, N * p.row),
            _ptr(v, "v", io, N * p.d_v), _ptr(gamma, "gamma", io, N),
            _ptr(mask, "mask", torch.uint8, p.B * p.T, optional=True),
            _ptr(slot0, "slot0", torch.float32, nseg * p.d_v, optional=True),
            _ptr(mass0, "mass0", torch.float32, nseg, optional=True),
            _ptr(y, "y", io, N * p.d_v),
            _ptr(slot1, "slot1", torch.float32, nseg * p.d_v),
            _ptr(mass1, "mass1", torch.float32, nseg),
            _ptr(ws, "ws", torch.uint8), ctypes.c_size_t(ws.numel()))
    _check(lib().ram_forward_gated(ctypes.byref(p), ctypes.byref(ep), *args,
                                   _stream(stream, ws.device)), "ram_forward_gated")


def ram_backward_gated(p: Problem, ep: Epilogue, ws, wlogits, rlogits, v, gamma, slot0, mass0,
                       d_y, d_slot1, d_mass1, d_wlogits, d_rlogits, d_v, d_gamma, d_gate,
                       d_gain=None, d_slot0=None, d_mass0=None, stream=None, mask=None):
    """Backward of ram_forward_gated: d_y is the gradient of y."""
    io = p.torch_dtype
    N, nseg = p.N, p.B * p.H * p.S
    args = (_ptr(ws, "ws", torch.uint8), ctypes.c_size_t(ws.numel()),
            _ptr(wlogits, "wlogits", io, N * p.row), _ptr(rlogits, "rlogits", io, N * p.row),
            _ptr(v, "v", io, N * p.d_v), _ptr(gamma, "gamma", io, N),
            _ptr(mask, "mask", torch.uint8, p.B * p.T, optional=True),
            _ptr(slot0, "slot0", torch.float32, nseg * p.d_v, optional=True),
            _ptr(mass0, "mass0", torch.float32, nseg, optional=True),
            _ptr(d_y, "d_y", io, N * p.d_v),
            _ptr(d_slot1, "d_slot1", torch.float32, nseg * p.d_v, optional=True),
            _ptr(d_mass1, "d_mass1", torch.float32, nseg, optional=True),
            _ptr(d_wlogits, "d_wlogits", io, N * p.row),
            _ptr(d_rlogits, "d_rlogits", io, N * p.row),
            _ptr(d_v, "d_v", io, N * p.d_v), _ptr(d_gamma, "d_gamma", io, N),
            _ptr(d_gate, "d_gate", io, N * p.d_v),
            _ptr(d_gain, "d_gain", torch.float32, p.d_v, optional=True),
            _ptr(d_slot0, "d_slot0", torch.float32, nseg * p.d_v, optional=True),
            _ptr(d_mass0, "d_mass0", torch.float32, nseg, optional=True))
    _check(lib().ram_backward_gated(ctypes.byref(p), ctypes.byref(ep), *args,
                                    _stream(stream, ws.device)), "ram_backward_gated")


def ram_decode_step(p: Problem, wlogits, rlogits, v, gamma, slot, mass, o, stream=None,
                    mask=None):
    """mask: optional (B,) uint8 tensor, nonzero = the sequence takes this step."""
    io = p.torch_dtype
    BH, S = p.B * p.H, p.S
    args = (_ptr(wlogits, "wlogits", io, BH * p.row), _ptr(rlogits, "rlogits", io, BH * p.row),
            _ptr(v, "v", io, BH * p.d_v), _ptr(gamma, "gamma", io, BH),
            _ptr(mask, "mask", torch.uint8, p.B, optional=True),
            _ptr(slot, "slot", torch.float32, BH * S * p.d_v),
            _ptr(mass, "mass", torch.float32, BH * S), _ptr(o, "o", io, BH * p.d_v))
    _check(lib().ram_decode_step(ctypes.byref(p), *args, _stream(stream, slot.device)),
           "ram_decode_step")


STREAM_PROBE_VARIANTS = ("8 KiB rows, 4 waves, nontemporal", "8 KiB rows, 4 waves, plain",
                         "16 KiB rows, 4 waves, nontemporal", "4 KiB rows, 4 waves, nontemporal",
                         "8 KiB rows, 8 waves, nontemporal", "1 KiB rows, 1 wave, nontemporal",
                         "2 KiB rows, 1 wave, nontemporal")


def ram_stream_probe(mode: int, variant: int, src, dst, stream=None):
    """HBM streaming roof: mode 0 reads src, mode 1 copies src to dst (uint8
    device tensors of equal size, a multiple of 128 KiB)."""
    n = src.numel()
    _check(lib().ram_stream_probe(int(mode), int(variant), _ptr(src, "src", torch.uint8),
                                  _ptr(dst, "dst", torch.uint8, n), ctypes.c_size_t(n),
                                  _stream(stream, src.device)), "ram_stream_probe")


def ram_prof_enable(on: bool = True):
    _check(lib().ram_prof_enable(int(on)), "ram_prof_enable")


def ram_prof_collect() -> dict:
    """{kernel name: (launches, total ms)} since the last ram_prof_enable."""
    buf = (ProfEntry * 64)()
    n = ctypes.c_int(0)
    _check(lib().ram_prof_collect(buf, 64, ctypes.byref(n)), "ram_prof_collect")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms))
            for i in range(n.value)}
