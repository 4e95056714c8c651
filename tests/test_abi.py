"""C ABI checks that need no GPU: the library loads, exports every function
that include/ramnet.h declares, and rejects bad problems with the documented
status codes (host-side validation; nothing is enqueued)."""
import ctypes
import os
import re

import pytest

import linear_attention_ram_amd as ram

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ramnet.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(ram_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    L = ram.lib()
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(ram.EXPORTED)


def test_problem_struct_matches_header_size():
    assert ctypes.sizeof(ram.Problem) == 64
    assert ctypes.sizeof(ram.WsLayout) == 23 * ctypes.sizeof(ctypes.c_size_t)
    assert ctypes.sizeof(ram.Epilogue) == 24


def status_of(**kw):
    base = dict(B=2, H=3, T=100, S=64, k_w=4, k_r=2, d_v=16, io="bf16")
    base.update(kw)
    p = ram.problem(**base)
    n = ctypes.c_size_t(0)
    return ram.lib().ram_workspace_size(ctypes.byref(p), 1, ctypes.byref(n)), p, n.value


def test_valid_problem_has_positive_workspace():
    st, p, n = status_of()
    assert st == ram.RAM_OK and n > 0
    L = ram.ram_workspace_layout(p)
    assert L["fwd_bytes"] <= L["total_bytes"] == n
    offs = sorted(v for k, v in L.items() if k not in ("fwd_bytes", "total_bytes"))
    assert all(o % 256 == 0 for o in offs)
    assert len(set(offs)) == len(offs)


@pytest.mark.parametrize("kw,code", [
    (dict(k_w=65), ram.RAM_EINVAL),
    (dict(k_r=0), ram.RAM_EINVAL),
    (dict(S=8, k_w=9), ram.RAM_EINVAL),
    (dict(S=4), ram.RAM_EINVAL),              # 4 bf16 logits are not a 16-byte row
    (dict(d_v=129), ram.RAM_EINVAL),
    (dict(d_v=65), ram.RAM_EINVAL),
    (dict(H=0), ram.RAM_EINVAL),
    (dict(eps=-1.0), ram.RAM_EINVAL),
    (dict(S=32768), ram.RAM_EUNSUPPORTED),
    (dict(cape_heads=4), ram.RAM_EINVAL),     # more CAPE heads than heads
    (dict(cape_heads=1, t0=-1), ram.RAM_EINVAL),
    (dict(cape_heads=3, t0=1 << 40), ram.RAM_OK),
    (dict(T=1 << 24), ram.RAM_ECAPACITY),
    (dict(B=4096, T=8192, H=16, S=64, k_w=8, k_r=8), ram.RAM_ECAPACITY),
    # one batch's staging rows (T*H*k*d_v bf16) above the scans' buffer limit
    (dict(B=1, T=70000, H=16, S=64, k_w=8, k_r=8, d_v=128), ram.RAM_ECAPACITY),
    (dict(B=1, T=65000, H=16, S=64, k_w=8, k_r=8, d_v=128), ram.RAM_OK),
])
def test_invalid_problems_are_rejected(kw, code):
    st, _, _ = status_of(**kw)
    assert st == code, ram.ram_status_string(st)


def test_bad_dtype():
    p = ram.problem(1, 1, 4, 64, 2, 2, 16)
    p.io_dtype = 7
    n = ctypes.c_size_t(0)
    assert ram.lib().ram_workspace_size(ctypes.byref(p), 1, ctypes.byref(n)) == ram.RAM_EDTYPE


@pytest.mark.parametrize("U,P,k,code", [
    (2, 8, 8, ram.RAM_OK),
    (3, 4, 8, ram.RAM_OK),            # rows of 12 bf16 logits need no 16-byte multiple
    (2, 128, 64, ram.RAM_OK),         # S = 16384
    (2, 129, 8, ram.RAM_EUNSUPPORTED),
    (14, 2, 8, ram.RAM_OK),
    (15, 1, 1, ram.RAM_EUNSUPPORTED),  # more digits than the decoder keeps
    (14, 1, 1, ram.RAM_OK),
    (14, 1, 2, ram.RAM_EINVAL),        # k > S = 1
    (0, 8, 1, ram.RAM_EINVAL),
    (3, 3, 28, ram.RAM_EINVAL),        # k > S = 27
])
def test_digit_counts(U, P, k, code):
    p = ram.problem(1, 2, 4, None, k, k, 16, U=U, P=P) if U >= 1 else None
    if p is None:
        p = ram.problem(1, 2, 4, 64, 1, 1, 16)
        p.U = U
        p.P = P
    n = ctypes.c_size_t(0)
    st = ram.lib().ram_workspace_size(ctypes.byref(p), 1, ctypes.byref(n))
    assert st == code, ram.ram_status_string(st)
    if code == ram.RAM_OK:
        L = ram.ram_workspace_layout(p)
        # per-digit logsumexp of every row and side
        assert L["idx_r"] - L["lse_w"] >= 4 * p.N * U


def test_problem_helper_checks_digits():
    p = ram.problem(2, 3, 5, 64, 4, 4, 8, U=3, P=4)
    assert (p.U, p.P, p.S, p.row) == (3, 4, 64, 12)
    with pytest.raises(ValueError):
        ram.problem(2, 3, 5, 60, 4, 4, 8, U=3, P=4)
    with pytest.raises(ValueError):
        ram.problem(2, 3, 5, 64, 4, 4, 8, U=3)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert ram.ram_status_string(code)
    assert ram.ram_status_string(-99) == "unknown status"


def test_forward_rejects_small_workspace_before_touching_the_gpu():
    p = ram.problem(1, 1, 8, 64, 2, 2, 16, io="f32")
    L = ram.lib()
    fake = ctypes.c_void_p(16 * 1024)  # never dereferenced: validation fails first
    st = L.ram_forward(ctypes.byref(p), fake, fake, fake, fake, None, None, None, fake, fake,
                       fake, fake, ctypes.c_size_t(16), None)
    assert st == ram.RAM_ECAPACITY
    st = L.ram_forward(ctypes.byref(p), fake, fake, fake, fake, None, fake, None, fake, fake,
                       fake, fake, ctypes.c_size_t(1 << 30), None)
    assert st == ram.RAM_EINVAL             # slot0 without mass0
    st = L.ram_decode_step(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, fake, None)
    assert st == ram.RAM_EINVAL             # T != 1


def test_gated_calls_validate_before_touching_the_gpu():
    p = ram.problem(1, 1, 8, 64, 2, 2, 16, io="f32")
    L = ram.lib()
    fake = ctypes.c_void_p(16 * 1024)  # never dereferenced: validation fails first
    big = ctypes.c_size_t(1 << 40)
    fwd = (fake, fake, fake, fake, None, None, None, fake, fake, fake, fake, big, None)
    assert L.ram_forward_gated(ctypes.byref(p), None, *fwd) == ram.RAM_EINVAL
    no_gate = ram.Epilogue(None, None, 1e-6)
    assert L.ram_forward_gated(ctypes.byref(p), ctypes.byref(no_gate), *fwd) == ram.RAM_EINVAL
    bad_eps = ram.Epilogue(fake, None, -1.0)
    assert L.ram_forward_gated(ctypes.byref(p), ctypes.byref(bad_eps), *fwd) == ram.RAM_EINVAL
    ok = ram.Epilogue(fake, None, 1e-6)
    bwd = [fake, big, fake, fake, fake, fake, None, None, None, fake, None, None, fake, fake,
           fake, fake, None, None, None, None, None]
    # d_gate (position 16 after ep) missing
    assert L.ram_backward_gated(ctypes.byref(p), ctypes.byref(ok), *bwd) == ram.RAM_EINVAL
    assert L.ram_backward_gated(ctypes.byref(p), None, *bwd) == ram.RAM_EINVAL


def test_gated_workspace_areas():
    p = ram.problem(2, 3, 40, 64, 4, 4, 24, io="bf16")
    L = ram.ram_workspace_layout(p)
    assert L["fwd_bytes"] <= L["epi_d_o"] < L["epi_part"] < L["total_bytes"]
    assert L["epi_part"] - L["epi_d_o"] >= 2 * p.N * p.d_v
    assert L["total_bytes"] - L["epi_part"] >= 4 * 8192 * p.d_v


def test_backward_scratch_leaves_the_forward_arrays_alone():
    # the forward's read contributions (stash) stay intact through any number
    # of backward calls: the reverse pass has its own d_v staging (stash_b),
    # past fwd_bytes like the rest of its scratch
    p = ram.problem(2, 3, 40, 64, 4, 5, 24, io="bf16")
    L = ram.ram_workspace_layout(p)
    assert L["stash"] < L["fwd_bytes"]
    assert L["long_count"] - L["stash"] >= 2 * p.N * p.k_r * p.d_v
    for name in ("stash_b", "dw", "dr", "dgam", "epi_d_o", "epi_part"):
        assert L[name] >= L["fwd_bytes"], name
    assert L["dw"] - L["stash_b"] >= 2 * p.N * p.k_w * p.d_v
    assert L["dgam"] - L["dr"] >= 4 * p.N * p.k_r
