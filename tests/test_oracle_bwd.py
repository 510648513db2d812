"""Pins of the oracle's attention backward (CPU, float64).

The pages give no gradient formulas, so each mode is pinned by something other than the
oracle's own algebra:
  * the exact kind, every mode: torch autograd through scaled_dot_product_attention;
  * post-normalisation surrogate (ste_post), every kind: torch autograd through the
    construction z = S + (log w - S).detach(), O = softmax(z) V, whose backward is that of
    a softmax evaluated at the normalised weights;
  * pre-normalisation surrogate and exact modes, attached and detached, every kind: torch
    autograd through the forward rebuilt in torch from its definition (row max and min with
    their gradients, the grid, the rounding passed straight through or held constant, the
    normalisation), with the extrema detached in torch for the detached modes;
  * exact (almost-everywhere) gradients: central finite differences of the oracle forward;
  * exact_detached: central finite differences of the forward with the row extrema held at
    their unperturbed values (the oracle forward's ``extrema`` input).
"""
import math

import numpy as np
import pytest
import torch

import oracle

KINDS = [dict(kind="pot", levels=4), dict(kind="pot", levels=3, flush=True), dict(kind="kint", levels=4),
         dict(kind="kint", levels=3, interp=True), dict(kind="kint", levels=4, window=2.0),
         dict(kind="kint", levels=3, window=1.5, interp=True), dict(kind="kint", levels=3, window=1.5, flush=True),
         dict(kind="kint", levels=3, window=1.2, interp=True, flush=True), dict(kind="trunc", window=1.0),
         dict(kind="uniform", window=1.0)]


def _vid(v):
    return "-".join(f"{k}{v[k]}" for k in v)


def _qkvdo(B=1, H=2, Hkv=1, N=9, d=4, sigma=1.0, seed=0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, H, N, d)) * sigma, r.standard_normal((B, Hkv, N, d)) * sigma,
            r.standard_normal((B, Hkv, N, d)), r.standard_normal((B, H, N, d)))


@pytest.mark.parametrize("grad", ["ste_post", "ste_pre", "ste_pre_detached", "exact", "exact_detached"])
@pytest.mark.parametrize("causal", [False, True])
def test_exact_kind_equals_sdpa_autograd(grad, causal):
    q, k, v, do = _qkvdo(H=4, Hkv=2, N=11, d=8, sigma=1.3, seed=1)
    r = oracle.attn_bwd(q, k, v, do, causal=causal, kind="exact", grad=grad)
    Q, K, V = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal, enable_gqa=True)
    (O * torch.from_numpy(do)).sum().backward()
    for name, t in (("dQ", Q), ("dK", K), ("dV", V)):
        np.testing.assert_allclose(r[name], t.grad.numpy(), atol=1e-13)


@pytest.mark.parametrize("var", KINDS, ids=_vid)
@pytest.mark.parametrize("causal", [False, True])
def test_straight_through_equals_autograd_construction(var, causal):
    q, k, v, do = _qkvdo(N=10, d=4, sigma=1.6, seed=2)
    r = oracle.attn_bwd(q, k, v, do, causal=causal, grad="ste_post", **var)
    Q, K, V = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    dQ, dK, dV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    N, d = q.shape[2], q.shape[3]
    for h in range(q.shape[1]):
        S = (Q[0, h] @ K[0, 0].T) / math.sqrt(d)
        w = oracle.head_rows(q[0, h], k[0, 0], v[0, 0], causal=causal, detail=True, **var)["w"]
        logw = torch.from_numpy(np.where(w > 0, np.log(np.where(w > 0, w, 1.0)), -np.inf))
        z = S + (logw - S).detach()                      # value log w, derivative 1 in S
        O = torch.softmax(z, dim=-1) @ V[0, 0]
        (O * torch.from_numpy(do[0, h])).sum().backward()
    np.testing.assert_allclose(r["dQ"], Q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dK"], K.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dV"], V.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("var", KINDS[:6], ids=_vid)
@pytest.mark.parametrize("causal", [False, True])
def test_detail_weights_and_score_gradients_equal_autograd_at_the_scores(var, causal):
    """``detail``: P and dS are the normalised weights and the gradient of the loss with
    respect to the scaled scores, here with the scores as the autograd leaf (ste_post)."""
    q, k, v, do = _qkvdo(N=10, d=4, sigma=1.6, seed=3)
    d = q.shape[3]
    r = oracle.head_bwd(q[0, 1], k[0, 0], v[0, 0], do[0, 1], causal=causal, grad="ste_post", detail=True, **var)
    S = torch.tensor(q[0, 1] @ k[0, 0].T / math.sqrt(d), requires_grad=True)
    w = oracle.head_rows(q[0, 1], k[0, 0], v[0, 0], causal=causal, detail=True, **var)["w"]
    logw = torch.from_numpy(np.where(w > 0, np.log(np.where(w > 0, w, 1.0)), -np.inf))
    P = torch.softmax(S + (logw - S).detach(), dim=-1)
    ((P @ torch.from_numpy(v[0, 0])) * torch.from_numpy(do[0, 1])).sum().backward()
    np.testing.assert_allclose(r["P"], P.detach().numpy(), atol=1e-14)
    np.testing.assert_allclose(r["dS"], S.grad.numpy(), atol=1e-12)


LOG2E = 1.0 / math.log(2.0)


def _torch_weights(S, vis, var, grad):
    """The forward's weights rebuilt in torch (float64) so that autograd gives the
    pre-normalisation surrogate (grad ste_pre*) or the exact derivative (exact*)."""
    kind = var["kind"]
    ste = grad.startswith("ste_pre")
    neg_inf = torch.full_like(S, -math.inf)
    m = torch.where(vis, S, neg_inf).max(dim=1).values            # gradient to the first arg-max
    mn = torch.where(vis, S, -neg_inf).min(dim=1).values           # ... and the first arg-min
    if grad.endswith("_detached"):
        m, mn = m.detach(), mn.detach()
    zero = torch.zeros_like(S)
    if kind == "exact":
        return torch.where(vis, torch.exp(S - m[:, None]), zero)
    if kind in ("trunc", "uniform"):
        kept = vis & ((m[:, None] - S).detach() <= var["window"])
        val = torch.exp(S - m[:, None]) if kind == "trunc" else torch.ones_like(S)
        return torch.where(kept, val, zero)
    if kind == "pot":
        L = var["levels"]
        y = (m[:, None] - S) * LOG2E
        r = torch.round(y.detach())                                  # half to even
        pas = (r <= L - 1).double() if ste else 0.0
        e = torch.clamp(r, max=L - 1) + (y - y.detach()) * pas
        w = torch.exp2(-e)
        if var.get("flush"):
            w = torch.where(r <= L - 1, w, zero)
        return torch.where(vis, w, zero)
    K = var["levels"]
    lo = (m - var["window"]) if "window" in var else mn
    delta = (m - lo) / K
    deg = (delta.detach() == 0)[:, None]          # a single visible score: every weight 1, no gradient
    y = (m[:, None] - S) / torch.where(deg[:, 0], torch.ones_like(delta), delta)[:, None]
    window = "window" in var
    if var.get("interp"):
        # past the grid's end (fixed windows only) the weight stays at T_K; at y = K the
        # last interval's slope applies, and a min-max grid's arg-min (y = K up to
        # rounding) is inside
        yc = torch.where(y.detach() <= K, y, torch.full_like(y, float(K))) if window else y
        l0 = torch.clamp(torch.floor(yc.detach()), 0, K - 1)
        t = yc - l0
        w = (1 - t) * torch.exp(-l0 * delta[:, None]) + t * torch.exp(-(l0 + 1) * delta[:, None])
    else:
        r = torch.round(y.detach())
        pas = (r <= K).double() if ste else 0.0
        lv = torch.clamp(r, max=K) + (y - y.detach()) * pas
        w = torch.exp(-lv * delta[:, None])
    if var.get("flush") and window:
        w = torch.where(y.detach() <= K, w, zero)
    w = torch.where(deg, torch.ones_like(w), w)
    return torch.where(vis, w, zero)


def _construction_grads(q, k, v, do, var, causal, grad):
    Q, K, V = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    N, d = q.shape[2], q.shape[3]
    vis = torch.ones(N, N, dtype=torch.bool)
    if causal:
        vis = torch.tril(vis)
    group = q.shape[1] // k.shape[1]
    for h in range(q.shape[1]):
        S = (Q[0, h] @ K[0, h // group].T) / math.sqrt(d)
        w = _torch_weights(S, vis, var, grad)
        O = (w / w.sum(dim=1, keepdim=True)) @ V[0, h // group]
        (O * torch.from_numpy(do[0, h])).sum().backward()
    return tuple(np.zeros(t.shape) if t.grad is None else t.grad.numpy() for t in (Q, K, V))


@pytest.mark.parametrize("grad", ["ste_pre", "ste_pre_detached", "exact", "exact_detached"])
@pytest.mark.parametrize("var", KINDS, ids=_vid)
@pytest.mark.parametrize("causal", [False, True])
def test_modes_equal_autograd_through_the_rebuilt_forward(var, causal, grad):
    q, k, v, do = _qkvdo(H=2, Hkv=1, N=10, d=4, sigma=1.6, seed=12)
    r = oracle.attn_bwd(q, k, v, do, causal=causal, grad=grad, **var)
    gq, gk, gv = _construction_grads(q, k, v, do, var, causal, grad)
    np.testing.assert_allclose(r["dQ"], gq, atol=1e-12)
    np.testing.assert_allclose(r["dK"], gk, atol=1e-12)
    np.testing.assert_allclose(r["dV"], gv, atol=1e-12)


def test_pre_surrogate_has_a_calibration_term_the_post_one_lacks():
    # min-max hard rounding: dw/dDelta = w (y - l) moves the gradient of q and k
    q, k, v, do = _qkvdo(N=8, d=4, sigma=1.5, seed=6)
    var = dict(kind="kint", levels=4)
    pre = oracle.attn_bwd(q, k, v, do, grad="ste_pre", **var)
    post = oracle.attn_bwd(q, k, v, do, grad="ste_post", **var)
    det = oracle.attn_bwd(q, k, v, do, grad="ste_pre_detached", **var)
    assert np.abs(pre["dQ"] - post["dQ"]).max() > 1e-3
    # with the extrema detached and nothing clipped (min-max: y <= K) the two placements agree
    np.testing.assert_allclose(det["dQ"], post["dQ"], atol=1e-13)
    np.testing.assert_allclose(det["dK"], post["dK"], atol=1e-13)


def _fd(q, k, v, do, var, causal, extrema=None, h=1e-7):
    """Central finite differences of sum(dO * O) over every entry of q, k, v."""
    N = q.shape[2]

    def loss(qq, kk, vv):
        tot = 0.0
        for hh in range(q.shape[1]):
            ext = None if extrema is None else extrema[hh]
            O = oracle.head_rows(qq[0, hh], kk[0, 0], vv[0, 0], causal=causal, extrema=ext, **var)["O"]
            tot += float((O * do[0, hh]).sum())
        return tot

    out = []
    for which in range(3):
        arrs = [q, k, v]
        g = np.zeros_like(arrs[which])
        for idx in np.ndindex(*g.shape):
            a = [x.copy() for x in arrs]
            a[which][idx] += h
            lp = loss(*a)
            a[which][idx] -= 2 * h
            lm = loss(*a)
            g[idx] = (lp - lm) / (2 * h)
        out.append(g)
    return out


@pytest.mark.parametrize("var", KINDS, ids=_vid)
@pytest.mark.parametrize("causal", [False, True])
def test_exact_mode_equals_finite_differences(var, causal):
    q, k, v, do = _qkvdo(N=7, d=3, sigma=1.5, seed=3)
    r = oracle.attn_bwd(q, k, v, do, causal=causal, grad="exact", **var)
    gq, gk, gv = _fd(q, k, v, do, var, causal)
    np.testing.assert_allclose(r["dQ"], gq, atol=2e-6)
    np.testing.assert_allclose(r["dK"], gk, atol=2e-6)
    np.testing.assert_allclose(r["dV"], gv, atol=2e-6)


@pytest.mark.parametrize("var", [v for v in KINDS if v["kind"] in ("kint", "trunc")], ids=_vid)
@pytest.mark.parametrize("causal", [False, True])
def test_detached_mode_equals_finite_differences_with_fixed_extrema(var, causal):
    # extrema held a little outside the score range, so that no perturbed score crosses them
    q, k, v, do = _qkvdo(N=7, d=3, sigma=1.5, seed=4)
    ext = []
    for h in range(q.shape[1]):
        S = q[0, h] @ k[0, 0].T / math.sqrt(3)
        vis = np.tril(np.ones((7, 7), bool)) if causal else np.ones((7, 7), bool)
        ext.append((np.where(vis, S, -np.inf).max(1) + 0.01, np.where(vis, S, np.inf).min(1) - 0.01))
    dQ, dK, dV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(q.shape[1]):
        r = oracle.head_bwd(q[0, h], k[0, 0], v[0, 0], do[0, h], causal=causal, grad="exact_detached",
                            extrema=ext[h], **var)
        dQ[0, h] = r["dQ"]
        dK[0, 0] += r["dK"]
        dV[0, 0] += r["dV"]
    gq, gk, gv = _fd(q, k, v, do, var, causal, extrema=ext)
    np.testing.assert_allclose(dQ, gq, atol=2e-6)
    np.testing.assert_allclose(dK, gk, atol=2e-6)
    np.testing.assert_allclose(dV, gv, atol=2e-6)


def test_attached_and_detached_differ_for_min_max_grids():
    q, k, v, do = _qkvdo(N=8, d=4, sigma=1.5, seed=5)
    a = oracle.attn_bwd(q, k, v, do, kind="kint", levels=4, interp=True, grad="exact")
    b = oracle.attn_bwd(q, k, v, do, kind="kint", levels=4, interp=True, grad="exact_detached")
    assert np.abs(a["dQ"] - b["dQ"]).max() > 1e-3
    np.testing.assert_allclose(a["dV"], b["dV"], atol=0)


# --------------------------------------------------------------------------- planted mistakes
import os
import types

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "qsa_oracle.py")
MUT_BWD = {
    "ste_clip_ignored": ("dwdy = np.where(r <= K, -delta[:, None] * w, 0.0) if ste else np.zeros((R, N))",
                         "dwdy = -delta[:, None] * w if ste else np.zeros((R, N))"),
    "pot_ste_clip_ignored": ("g = np.where(visible & (e <= levels - 1), dw * w, 0.0)", "g = np.where(visible, dw * w, 0.0)"),
    "ste_drops_D": ("dS = np.where(visible, P * (dP - D[:, None]), 0.0)", "dS = np.where(visible, P * dP, 0.0)"),
    "dlo_sign": ("dlo = -dD / levels", "dlo = dD / levels"),
    "interp_slope_sign": ("dwdy = np.where(inside, T[rows, l0 + 1] - T[rows, l0], 0.0)",
                          "dwdy = np.where(inside, T[rows, l0] - T[rows, l0 + 1], 0.0)"),
    "delta_moves_y_dropped": ("dD = (dw * (dwdD - dwdy * y / safe)).sum(axis=1)", "dD = (dw * dwdD).sum(axis=1)"),
    "dK_without_scale": ("dK = sc * (dS.T @ qh)", "dK = (dS.T @ qh)"),
    "argmax_term_dropped": ("np.add.at(dS, (rows, amax), dm)", "pass"),
}


def _bwd_checks(o):
    try:
        q, k, v, do = _qkvdo(N=6, d=3, sigma=1.5, seed=7)
        for var in (dict(kind="kint", levels=3, interp=True), dict(kind="kint", levels=4),
                    dict(kind="kint", levels=3, window=1.5, interp=True)):
            r = o.attn_bwd(q, k, v, do, grad="exact", **var)
            gq, gk, gv = _fd(q, k, v, do, var, False)
            np.testing.assert_allclose(r["dQ"], gq, atol=2e-6)
            np.testing.assert_allclose(r["dK"], gk, atol=2e-6)
        for var in (dict(kind="kint", levels=4), dict(kind="kint", levels=3, window=1.5),
                    dict(kind="pot", levels=3)):
            r = o.attn_bwd(q, k, v, do, grad="ste_pre", **var)
            gq, gk, gv = _construction_grads(q, k, v, do, var, False, "ste_pre")
            np.testing.assert_allclose(r["dQ"], gq, atol=1e-12)
            np.testing.assert_allclose(r["dK"], gk, atol=1e-12)
        var = dict(kind="pot", levels=4)
        r = o.attn_bwd(q, k, v, do, grad="ste_post", **var)
        Q, K = torch.tensor(q, requires_grad=True), torch.tensor(k, requires_grad=True)
        for h in range(2):
            S = (Q[0, h] @ K[0, 0].T) / math.sqrt(3)
            w = oracle.head_rows(q[0, h], k[0, 0], v[0, 0], detail=True, **var)["w"]
            z = S + (torch.from_numpy(np.log(w)) - S).detach()
            (torch.softmax(z, -1) @ torch.from_numpy(v[0, 0]) * torch.from_numpy(do[0, h])).sum().backward()
        np.testing.assert_allclose(r["dQ"], Q.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(r["dK"], K.grad.numpy(), atol=1e-12)
    except Exception:
        return False
    return True


def test_unmutated_backward_passes_the_checks():
    import oracle.qsa_oracle as real
    assert _bwd_checks(real)


@pytest.mark.parametrize("name", sorted(MUT_BWD))
def test_planted_backward_mistake_is_caught(name):
    old, new = MUT_BWD[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"oracle_bwd_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    assert not _bwd_checks(mod), f"planted mistake {name} went unnoticed"
