"""Pins of the oracle's first-order gradients (ramnet-ops "Autograd and
compile": first-order autograd).

* central finite differences of the oracle's own forward, in float64, on
  every input coordinate whose perturbation leaves the top-K selection
  unchanged (the selection itself is piecewise constant);
* an independent float64 PyTorch-autograd token loop over dense slot arrays
  (softmax over all slots masked to the top-K, dense retention via
  torch.sigmoid(logit(1-w) - gamma), dense content blend, r @ S read-out).
The loss is <d_o, o> + <d_slot1, slot1> + <d_mass1, mass1>.
"""
import numpy as np
import pytest
import torch


def make_case(rng, B, H, T, S, kw, kr, d, U=1, P=None, with_state=True):
    shp = (B, T, H, U, P) if U > 1 else (B, T, H, S)
    x = {
        "wl": rng.standard_normal(shp) * 1.5,
        "rl": rng.standard_normal(shp) * 1.5,
        "v": rng.standard_normal((B, T, H, d)),
        "gamma": rng.normal(np.log(9), 1.0, (B, T, H)),
        "d_o": rng.standard_normal((B, T, H, d)),
        "d_slot1": rng.standard_normal((B, H, S, d)),
        "d_mass1": rng.standard_normal((B, H, S)),
    }
    if with_state:
        x["slot0"] = rng.standard_normal((B, H, S, d))
        x["mass0"] = rng.uniform(0.1, 1.0, (B, H, S))
    else:
        x["slot0"] = None
        x["mass0"] = None
    return x


def loss_of(orc, p, x, **over):
    y = dict(x)
    y.update(over)
    o, s1, m1 = orc.forward(p, y["wl"], y["rl"], y["v"], y["gamma"], y["slot0"], y["mass0"])
    return float(np.sum(o * x["d_o"]) + np.sum(s1 * x["d_slot1"]) + np.sum(m1 * x["d_mass1"]))


def selection(orc, p, wl, rl):
    return orc.decode(p, 0, wl)[0], orc.decode(p, 1, rl)[0]


CASES = [
    dict(B=1, H=2, T=10, S=6, kw=2, kr=3, d=3),
    dict(B=2, H=1, T=8, S=5, kw=1, kr=2, d=2, renorm=(True, True)),
    dict(B=1, H=2, T=9, S=9, kw=3, kr=2, d=2, U=2, P=3),
    dict(B=1, H=3, T=7, S=8, kw=2, kr=2, d=2, cape=2),
    dict(B=1, H=1, T=12, S=4, kw=2, kr=2, d=3, with_state=False),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_finite_differences(orc, case):
    c = dict(CASES[case])
    rng = np.random.default_rng(100 + case)
    U, P = c.get("U", 1), c.get("P")
    x = make_case(rng, c["B"], c["H"], c["T"], c["S"], c["kw"], c["kr"], c["d"], U, P,
                  c.get("with_state", True))
    p = orc.problem(c["B"], c["H"], c["T"], c["S"], c["kw"], c["kr"], c["d"], U=U, P=P,
                    eps=1e-6, renorm=c.get("renorm", (False, False)),
                    cape_heads=c.get("cape", 0), t0=5 if c.get("cape") else 0)
    g = orc.backward(p, x["wl"], x["rl"], x["v"], x["gamma"], x["slot0"], x["mass0"], x["d_o"],
                     x["d_slot1"], x["d_mass1"])
    sel = selection(orc, p, x["wl"], x["rl"])
    h = 1e-6
    names = [("wl", "d_wlogits"), ("rl", "d_rlogits"), ("v", "d_v"), ("gamma", "d_gamma")]
    if x["slot0"] is not None:
        names += [("slot0", "d_slot0"), ("mass0", "d_mass0")]
    for name, gname in names:
        base = x[name]
        num = np.zeros_like(base)
        checked = 0
        for i in np.ndindex(base.shape):
            xp, xm = base.copy(), base.copy()
            xp[i] += h
            xm[i] -= h
            if name in ("wl", "rl"):
                wl_p = xp if name == "wl" else x["wl"]
                rl_p = xp if name == "rl" else x["rl"]
                wl_m = xm if name == "wl" else x["wl"]
                rl_m = xm if name == "rl" else x["rl"]
                sp, sm = selection(orc, p, wl_p, rl_p), selection(orc, p, wl_m, rl_m)
                if not all(np.array_equal(a, b) for a, b in zip(sp + sm, sel + sel)):
                    num[i] = np.nan
                    continue
            num[i] = (loss_of(orc, p, x, **{name: xp}) - loss_of(orc, p, x, **{name: xm})) / (2 * h)
            checked += 1
        ok = ~np.isnan(num)
        assert checked > 0
        err = np.max(np.abs(num[ok] - g[gname][ok]))
        scale = max(1.0, np.max(np.abs(g[gname][ok])))
        assert err <= 2e-6 * scale, (name, err, scale)


def torch_dense_loss(x, S, kw, kr, eps, renorm, cape, t0, U=1, P=None):
    """Dense float64 token loop in PyTorch; returns loss and leaf tensors."""
    leaves = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
              for k, v in x.items() if v is not None and k in
              ("wl", "rl", "v", "gamma", "slot0", "mass0")}
    wl, rl, v, gam = leaves["wl"], leaves["rl"], leaves["v"], leaves["gamma"]
    B, T, H = gam.shape
    d = v.shape[-1]

    def dense(logit_row, k, rn, shift):
        if U == 1:
            prob = torch.softmax(logit_row, dim=-1)
            keys = logit_row.detach().float().numpy()
        else:
            prob = torch.softmax(logit_row[0], -1)
            for u in range(1, U):
                prob = torch.kron(prob, torch.softmax(logit_row[u], -1))
            dig = logit_row.detach().float().numpy()
            keys = np.zeros(P ** U, np.float32)
            for a in range(P ** U):
                acc, rem = np.float32(0), a
                for u in range(U):
                    st = P ** (U - 1 - u)
                    acc = np.float32(acc + dig[u, rem // st])
                    rem %= st
                keys[a] = acc
        order = np.lexsort((np.arange(keys.size), -keys.astype(np.float64)))[:k]
        mask = torch.zeros(keys.size, dtype=torch.float64)
        mask[torch.as_tensor(order)] = 1.0
        wv = prob * mask
        if rn:
            wv = wv / wv.sum()
        return torch.roll(wv, shifts=int(shift))

    loss = torch.zeros((), dtype=torch.float64)
    for b in range(B):
        for h in range(H):
            s = leaves["slot0"][b, h] if "slot0" in leaves else torch.zeros(S, d, dtype=torch.float64)
            m = leaves["mass0"][b, h] if "mass0" in leaves else torch.zeros(S, dtype=torch.float64)
            for t in range(T):
                shift = (t0 + t) % S if h < cape else 0
                w = dense(wl[b, t, h], kw, renorm[0], shift)
                r = dense(rl[b, t, h], kr, renorm[1], shift)
                on = w > 0
                inner = on & (w < 1)          # w = 1 (renormalised top-1): lambda = 0
                wc = torch.where(inner, w, torch.full_like(w, 0.5))
                lam = torch.sigmoid(torch.log1p(-wc) - torch.log(wc) - gam[b, t, h])
                lam = torch.where(inner, lam, torch.where(on, torch.zeros_like(w), torch.ones_like(w)))
                m = lam * m + w
                eta = torch.where(on, w / (m + eps), torch.zeros_like(w))
                s = (1 - eta)[:, None] * s + eta[:, None] * v[b, t, h][None, :]
                o = r @ s
                loss = loss + torch.sum(o * torch.as_tensor(x["d_o"][b, t, h]))
            loss = loss + torch.sum(s * torch.as_tensor(x["d_slot1"][b, h]))
            loss = loss + torch.sum(m * torch.as_tensor(x["d_mass1"][b, h]))
    loss.backward()
    return {k: t.grad.numpy() for k, t in leaves.items()}


@pytest.mark.parametrize("case", range(len(CASES)))
def test_matches_dense_torch_autograd(orc, case):
    c = dict(CASES[case])
    rng = np.random.default_rng(200 + case)
    U, P = c.get("U", 1), c.get("P")
    x = make_case(rng, c["B"], c["H"], c["T"] + 5, c["S"], c["kw"], c["kr"], c["d"], U, P,
                  c.get("with_state", True))
    T = c["T"] + 5
    renorm = c.get("renorm", (False, False))
    cape, t0 = c.get("cape", 0), (5 if c.get("cape") else 0)
    p = orc.problem(c["B"], c["H"], T, c["S"], c["kw"], c["kr"], c["d"], U=U, P=P,
                    eps=1e-6, renorm=renorm, cape_heads=cape, t0=t0)
    g = orc.backward(p, x["wl"], x["rl"], x["v"], x["gamma"], x["slot0"], x["mass0"], x["d_o"],
                     x["d_slot1"], x["d_mass1"])
    ref = torch_dense_loss(x, c["S"], c["kw"], c["kr"], 1e-6, renorm, cape, t0, U, P)
    pairs = [("wl", "d_wlogits"), ("rl", "d_rlogits"), ("v", "d_v"), ("gamma", "d_gamma")]
    if x["slot0"] is not None:
        pairs += [("slot0", "d_slot0"), ("mass0", "d_mass0")]
    for leaf, name in pairs:
        # renormalised top-1 weights are constant: their logit gradient is
        # exactly 0 in the oracle and rounding noise (~1e-17) in the dense loop
        err = np.max(np.abs(g[name] - ref[leaf]))
        assert err <= 1e-10 * max(np.max(np.abs(ref[leaf])), 1.0), (leaf, err)
