"""Comparison bars of the parity tests (numpy only; no GPU needed).

rel(): normwise relative error max|x - ref| / max|ref| over a tensor.

Logit gradients need more than one normwise figure.  The gradient of a
logit row is dl_i = [i selected] g_j w_j - p_i * sum_j g_j w_j (paper §3.2
"Address Decoder": a softmax over all slots, so every logit gets a
gradient).  Over a whole tensor its largest entries are the few selected
ones, and the dense term -p_i * sum_j g_j w_j on every other entry is about
1% of them: a normwise bar of 2e-2 over the whole tensor cannot see that
term at all.  logit_grad_errors() therefore gives two errors, one over the
selected entries and one over all the others (the dense term alone), and
both must meet the bar.

The dense error is measured against the size of what the dense sum adds
up, max over the other entries of p_i * sum_j |g_j w_j|, not against the
sum itself: where the sum cancels, the reference dense term is (close to)
zero and any rounding would look like an unbounded relative error.  It
cancels exactly with renormalised weights (sum_j g_j w_j = 0 because the
weights sum to 1: the unselected logits get no gradient), and nearly under
the gated read-out's RMSNorm (<dL/do, o> = 0 up to its epsilon).  Where it
does not cancel, |sum_j g_j w_j| is a sizeable share of sum_j |g_j w_j|, so
a dropped, shifted or sign-flipped dense term still fails the bar
(tests/test_parity_bars.py).
"""
import numpy as np


def rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


def content_index(idx, S, cape_heads=0, t0=0):
    """Content-selected slot of each decoded index: CAPE heads h < cape_heads
    address (a + t0 + t) mod S for the content index a, so a = (idx - t0 - t)
    mod S there.  idx (B, T, H, k)."""
    idx = np.asarray(idx, np.int64)
    if cape_heads == 0:
        return idx
    a = idx.copy()
    T = idx.shape[1]
    shift = (t0 + np.arange(T, dtype=np.int64)) % S
    a[:, :, :cape_heads] = (idx[:, :, :cape_heads] - shift[None, :, None, None]) % S
    return a


def selected_entries(idx, U, P, cape_heads=0, t0=0):
    """Boolean mask over a logit tensor viewed as (B, T, H, U * P): entry u * P
    + a_u of every selected slot a = sum_u a_u P^(U-1-u) of its row (for
    U = 1 the entry a itself).  idx (B, T, H, k) as decoded (CAPE-shifted)."""
    S = P ** U
    a = content_index(idx, S, cape_heads, t0)
    B, T, H, k = a.shape
    sel = np.zeros((B, T, H, U * P), bool)
    bb, tt, hh = np.meshgrid(np.arange(B), np.arange(T), np.arange(H), indexing="ij")
    for j in range(k):
        rem = a[..., j].copy()
        for u in range(U - 1, -1, -1):
            sel[bb, tt, hh, u * P + rem % P] = True
            rem //= P
    return sel


def gw_products(g, w, renorm=False):
    """g_j w_j of each selected slot from the gradient g of its weight w
    (B, T, H, k); renormalised weights: (g_j - sum_i g_i w_i) w_j."""
    g = np.asarray(g, np.float64)
    w = np.asarray(w, np.float64)
    if renorm:
        return (g - np.sum(g * w, axis=-1, keepdims=True)) * w
    return g * w


def dense_scale(logits, lse, gw, U, P):
    """p_i * sum_j |gw_j| for every entry of a logit tensor viewed as
    (B, T, H, U * P), with p the softmax of the entry's digit: exp(l - lse_u).
    Rows whose logits are not finite (masked tokens may hold anything) get 0."""
    logits = np.asarray(logits, np.float64)
    B, T, H = logits.shape[:3]
    lg = logits.reshape(B, T, H, U, P)
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.exp(lg - np.asarray(lse, np.float64).reshape(B, T, H, U, 1))
        a = np.sum(np.abs(np.asarray(gw, np.float64)), axis=-1)
        sc = p * a[..., None, None]
    return np.nan_to_num(sc, nan=0.0, posinf=0.0, neginf=0.0).reshape(B, T, H, U * P)


def logit_grad_errors(x, ref, sel, scale=None):
    """(error over the selected entries, error over all other entries).  The
    first is normwise relative; the second is max |x - ref| over the other
    entries divided by the largest scale there (dense_scale), or normwise
    relative when no scale is given.  x and ref are logit gradients of any
    shape whose elements line up with sel (B, T, H, U * P)."""
    x = np.asarray(x, np.float64).reshape(sel.shape)
    ref = np.asarray(ref, np.float64).reshape(sel.shape)
    e_sel = rel(x[sel], ref[sel])
    if scale is None:
        return e_sel, rel(x[~sel], ref[~sel])
    off = ~sel
    num = float(np.max(np.abs(x[off] - ref[off]))) if off.any() else 0.0
    den = float(np.max(np.asarray(scale).reshape(sel.shape)[off])) if off.any() else 0.0
    return e_sel, (num / den if den > 0 else num)


def check_logit_grad(x, ref, sel, tol, name="d_logits", scale=None):
    e_sel, e_dense = logit_grad_errors(x, ref, sel, scale)
    assert e_sel <= tol and e_dense <= tol, (name, "selected", e_sel, "others", e_dense)
    return e_sel, e_dense
