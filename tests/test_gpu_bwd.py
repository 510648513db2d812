"""GPU parity of the attention backward (qsa_attn_bwd) against the oracle's float64 backward,
element by element on dQ, dK and dV.

Inputs: seeded Q, K, V (inputs.make_inputs) and dO (inputs.make_dout) in the stored dtype;
the oracle takes the same stored values, decoded exactly.  The quantized weights are piecewise
constant in the scores, so an element whose grid coordinate lies within EDGE_Y of a rounding
edge, or a row whose maximum or minimum is tied within EDGE_S, may take the other side in
float32.  Rows holding one get dO = 0 on both sides: such a row adds exactly zero to every
gradient (its dV terms are P * 0; dP and D vanish, so its dS does in every mode), so the
comparison is exact-decision everywhere else.  Tolerance: max |gpu - oracle| <= TOL times
max(max |oracle|, FLOOR) per tensor (float32 sums of at most N terms; the floor covers
gradients that vanish exactly, as with a single visible key, where float32 leaves rounding
residue of order 1e-8 on inputs of order 1).

bf16 inputs run on the matrix cores, which take the normalised weights P and the score
gradients dS rounded to bfloat16 (nearest even, relative error at most u = 2^-8) as the operands
of dV = P^T dO, dK = scale dS^T Q and dQ = scale dS K.  Rounding the operand of a sum of products
moves it by at most u times the sum of the absolute products, so each element also gets
(u + 2^-12) * (|P|^T |dO|, scale |dS|^T |Q|, scale |dS| |K|) on top of the float32 tolerance (the
2^-12 covers float32 accumulation over the row or column).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import quantized_softmax_approximation_amd as qsa
from quantized_softmax_approximation_amd import inputs as qin
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

EDGE_Y = 2e-4     # grid-coordinate units
EDGE_S = 2e-5     # score units
TOL = 2e-4
FLOOR = 1e-3
BF16_U = 2.0 ** -8 + 2.0 ** -12   # bfloat16 unit roundoff of the P and dS operands, plus fp32 accumulation
MODES = ["ste_post", "ste_pre", "ste_pre_detached", "exact", "exact_detached"]
KINDS = [gc.EXACT, gc.EXACT_ANCH, gc.POT8, gc.POT4F, gc.KH4, gc.KH16, gc.KI4, gc.KI16, gc.KH4W, gc.KI4W, gc.KH4WF,
         gc.KI4WF, gc.TRUNC2, gc.UNIF2]


def _decode(t):
    bits = qin.raw_bits(t)
    f = oracle.decode_bf16(bits) if t.dtype == torch.bfloat16 else oracle.decode_f32(bits)
    return f.reshape(t.shape)


def _near_edge_rows(var, qh, kh, causal, sc):
    """Rows of one head with a decision within EDGE_Y / EDGE_S of flipping."""
    N = qh.shape[0]
    r = oracle.head_rows(qh, kh, kh, causal=causal, detail=True, scale=sc, **var)
    y = r["y"]
    vis = ~np.isnan(y)
    yv = np.where(vis, y, -10.0)
    kind = var["kind"]
    near = np.zeros_like(vis)
    if kind == "kint":
        K = var["levels"]
        win = "window" in var
        if var.get("interp"):
            n = np.rint(yv)
            top = K if win else K - 1              # interior kinks; a window's end is one too
            near = (np.abs(yv - n) < EDGE_Y) & (n >= 1) & (n <= top)
        else:
            h = np.floor(yv) + 0.5
            near = (np.abs(yv - h) < EDGE_Y) & (h <= K + 0.5)
            if var.get("flush") and win:
                near |= np.abs(yv - K) < EDGE_Y
    elif kind == "pot":
        h = np.floor(yv) + 0.5
        near = (np.abs(yv - h) < EDGE_Y) & (h <= var["levels"] - 0.5)
    elif kind in ("trunc", "uniform"):
        near = np.abs(yv - 1.0) * var["window"] < EDGE_S
    bad = (near & vis).any(axis=1)
    S = sc * (qh @ kh.T)
    cols = np.arange(N)
    visible = (cols[None, :] <= cols[:, None]) if causal else np.ones((N, N), bool)
    for sign in (1.0, -1.0) if N > 1 else ():     # near-ties at the maximum and at the minimum
        Z = np.sort(np.where(visible, sign * S, -np.inf), axis=1)
        gap = Z[:, -1] - Z[:, -2]
        bad |= np.isfinite(gap) & (gap < EDGE_S)
    return bad


def _case(wl, var, grad, heads=None):
    x = qin.make_inputs(wl)
    do = qin.make_dout(wl)
    qf, kf, vf = (_decode(t) for t in (x.q, x.k, x.v))
    B, H, N, d = qf.shape
    Hkv = kf.shape[1]
    group = H // Hkv
    sc = 1.0 / np.sqrt(d)
    ovar = gc.oracle_var(var)
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    bs = sorted({b for b, _ in heads})
    # the query heads the compared gradients depend on: the compared heads' KV groups (dK and dV
    # of a KV head sum over its group)
    need = {b: sorted({g for bb, h in heads if bb == b for g in range((h // group) * group, (h // group + 1) * group)})
            for b in bs}
    # zero dO on rows near a decision edge (both sides see the zeroed tensor)
    mask = torch.ones((B, H, N, 1), dtype=torch.bool)
    for b in bs:
        for h in need[b]:
            mask[b, h, _near_edge_rows(ovar, qf[b, h], kf[b, h // group], wl.causal, sc)] = False
    do = torch.where(mask, do, torch.zeros((), dtype=do.dtype))
    dof = _decode(do)
    print(f"[bwd] {wl.name} B{B} H{H}/{Hkv} N{N} d{d} {wl.dtype} causal={wl.causal} {gc.name(var)} grad={grad} "
          f"masked_rows={int((~mask[bs]).sum())}", flush=True, file=sys.stderr)
    q, k, v, g = (t.cuda() for t in (x.q, x.k, x.v, do))
    dq, dk, dv = qsa.attn_bwd(q, k, v, g, causal=wl.causal, grad=grad, **var)
    torch.cuda.synchronize()
    dq, dk, dv = (t.cpu().numpy() for t in (dq, dk, dv))
    worst = {}
    mma = wl.dtype == "bf16"   # the matrix-core path: bf16 P and dS operands
    for b in bs:
        oq = np.zeros((H, N, d))
        ok_ = np.zeros((Hkv, N, d))
        ov = np.zeros((Hkv, N, d))
        bq, bk, bv = np.zeros((H, N, d)), np.zeros((Hkv, N, d)), np.zeros((Hkv, N, d))
        for h in need[b]:
            kv = h // group
            r = oracle.head_bwd(qf[b, h], kf[b, kv], vf[b, kv], dof[b, h], causal=wl.causal, grad=grad, detail=mma,
                                **ovar)
            oq[h], ok_[kv], ov[kv] = r["dQ"], ok_[kv] + r["dK"], ov[kv] + r["dV"]
            if mma:
                aS, aP = np.abs(r["dS"]), np.abs(r["P"])
                bq[h] = BF16_U * sc * (aS @ np.abs(kf[b, kv]))
                bk[kv] += BF16_U * sc * (aS.T @ np.abs(qf[b, h]))
                bv[kv] += BF16_U * (aP.T @ np.abs(dof[b, h]))
        hs = sorted({h for bb, h in heads if bb == b})
        kvs = sorted({h // group for h in hs})
        for name, got, ref, bnd in (("dQ", dq[b][hs], oq[hs], bq[hs]), ("dK", dk[b][kvs], ok_[kvs], bk[kvs]),
                                    ("dV", dv[b][kvs], ov[kvs], bv[kvs])):
            scale = max(np.abs(ref).max(), FLOOR)
            err = np.max(np.maximum(np.abs(got - ref) - bnd, 0.0)) / scale
            worst[name] = max(worst.get(name, 0.0), err)
    print(f"[bwd]   rel err " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in worst.items()), flush=True, file=sys.stderr)
    for name, err in worst.items():
        assert err <= TOL, f"{name}: max error {err:.3e} of max |oracle| > {TOL}"


SMALL = [
    qin.custom("bwd_f32_d64", B=2, H=4, Hkv=2, N=136, d=64, dtype="f32", causal=False, sigma_qk=1.5, seed=2101),
    qin.custom("bwd_f32_d128c", B=1, H=2, Hkv=1, N=200, d=128, dtype="f32", causal=True, sigma_qk=1.3, seed=2102),
    qin.custom("bwd_bf16_d64c", B=1, H=4, Hkv=1, N=150, d=64, dtype="bf16", causal=True, sigma_qk=1.5, seed=2103),
    qin.custom("bwd_bf16_d128", B=1, H=4, Hkv=2, N=200, d=128, dtype="bf16", causal=False, sigma_qk=1.2, seed=2104),
]


@pytest.mark.parametrize("grad", MODES)
@pytest.mark.parametrize("var", KINDS, ids=gc.name)
@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_bwd_small(wl, var, grad):
    _case(wl, var, grad)


def test_bwd_tiny_shapes():
    # one key tile with a ragged tail, a single row, and a single causal row per head
    for wl in (qin.custom("bwd_n1", B=1, H=2, Hkv=2, N=1, d=64, dtype="f32", seed=2111),
               qin.custom("bwd_n65c", B=1, H=2, Hkv=1, N=65, d=64, dtype="bf16", causal=True, seed=2112)):
        for var in (gc.KH4, gc.KI4W, gc.POT8):
            for grad in ("ste_post", "ste_pre", "exact"):
                _case(wl, var, grad)


def test_bwd_causal_tile_order_ragged():
    # B * Hkv a multiple of 8 under a causal mask takes the longest-first block order of all three
    # launches; a ragged N puts a partial tile last in every head
    wl = qin.custom("bwd_order", B=2, H=8, Hkv=4, N=150, d=64, dtype="bf16", causal=True, sigma_qk=1.5, seed=2121)
    for var in (gc.EXACT, gc.KH4, gc.KI4W, gc.POT8):
        for grad in ("ste_post", "ste_pre", "exact"):
            _case(wl, var, grad)


# GPT-2-small shaped pretraining attention (B 8, 12 heads, 1024 keys, d 64, bf16, causal): the
# whole problem on the GPU, two batch entries compared in full.
@pytest.mark.parametrize("var,grad", [(gc.KH4, "ste_pre"), (gc.KH4, "exact"), (gc.KI16W, "ste_post"),
                                      (gc.POT8, "ste_pre_detached"), (gc.EXACT, "ste_post")],
                         ids=lambda p: gc.name(p) if isinstance(p, dict) else p)
def test_bwd_gpt2(var, grad):
    wl = qin.WORKLOADS["gpt2"]
    _case(wl, var, grad, heads=[(b, h) for b in (0, wl.B - 1) for h in range(wl.H)])


# 2K with the attention-sink key (B 4, H 32, N 2048, d 128, bf16, causal): the whole problem on
# the GPU, the first and the last head compared in full; most rows take their maximum at key 0,
# so the attached modes put most rows' gradient of m on one key
@pytest.mark.parametrize("var,grad", [(gc.KH16, "ste_pre"), (gc.POT8, "ste_pre"), (gc.KI16W, "exact")],
                         ids=lambda p: gc.name(p) if isinstance(p, dict) else p)
def test_bwd_pot2k_sampled(var, grad):
    wl = qin.WORKLOADS["pot2k"]
    _case(wl, var, grad, heads=[(0, 0), (wl.B - 1, wl.H - 1)])


def _random_bwd_cases(n, seed):
    r = np.random.default_rng(seed)
    for i in range(n):
        hkv = int(r.choice([1, 2]))
        wl = qin.custom(f"bwd_rnd{i}", B=int(r.choice([1, 2])), H=hkv * int(r.choice([1, 2, 4])), Hkv=hkv,
                        N=int(r.choice([17, 64, 100, 129, 200, 257])), d=int(r.choice([64, 128])),
                        dtype=str(r.choice(["bf16", "bf16", "f32"])), causal=bool(r.random() < 0.6),
                        sigma_qk=float(r.choice([0.7, 1.2, 1.5, 2.5])), seed=int(r.integers(1 << 20)))
        yield wl, KINDS[int(r.integers(len(KINDS)))], MODES[int(r.integers(len(MODES)))]


@pytest.mark.parametrize("block", range(2))
def test_bwd_random_configurations(block):
    # shapes, grouped heads, masks, score scales, weight kinds and gradient modes drawn at random
    # (seeded), away from the fixed cases above
    for wl, var, grad in _random_bwd_cases(30, seed=700 + block):
        _case(wl, var, grad)


def test_bwd_rejects_fp8():
    x = qin.make_inputs(qin.custom("bwd_fp8", N=64, dtype="fp8"))
    q, k, v = (t.cuda() for t in (x.q, x.k, x.v))
    with pytest.raises(ValueError):
        qsa.attn_bwd(q, k, v, q, kind="pot", levels=8)
