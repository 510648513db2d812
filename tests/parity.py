"""GPU-vs-oracle comparison protocol (test helper).

The GPU forms scores in fp32 (MFMA accumulation of exact bf16/fp8 products,
or fp32 FMAs); the oracle in float64.  For a row i the fp32 score error is
bounded by delta*_i = gamma * scale * max_j sum_c |q_ic k_jc| with
gamma = 2 d u, u = 2^-24 (twice the textbook bound for any summation order).
That error moves the grid coordinate y_ij by at most eps_ij (below), so an
element whose y lies within eps of a discontinuity of its weight function is
edge-ambiguous: either neighbouring grid index is a correct result.

Single-pass PoT (``pot_running``) has one more decision per tile: the anchor
ceil(running max of s log2 e).  Where that maximum lies within the band of an
integer, the GPU may take the neighbouring anchor, which moves every exponent
weighed against it by one level (and so the clip); such rows are counted and
left out of the comparison, and must stay rare (``check_anchor_rows``: at most
3 % of the rows compared).

Checks:
  * index agreement >= 99.9 % over visible elements, and every disagreement
    edge-ambiguous; masked codes identical;
  * per row ||O_gpu - O_ref|| <= tol ||O_ref|| + sigma_i, where sigma_i is the
    exact worst-case move of O_i if every ambiguous element took its other
    index.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

import oracle

U = 2.0 ** -24
LOG2E = 1.0 / math.log(2.0)


@dataclass
class Report:
    rows: int = 0
    elems: int = 0
    idx_agree: float = 1.0
    idx_disagree: int = 0
    idx_bad: int = 0              # disagreements outside the ambiguity band
    amb_rows: int = 0
    anchor_amb_rows: int = 0      # pot_running rows whose anchor may round either way
    max_rel_err: float = 0.0      # max over rows of ||dO|| / ||O_ref||
    max_excess: float = 0.0       # max over rows of ||dO|| - tol ||O_ref|| - sigma (<= 0 passes)
    notes: list = field(default_factory=list)

    def merge(self, o: "Report"):
        tot = self.elems + o.elems
        if tot:
            self.idx_agree = (self.idx_agree * self.elems + o.idx_agree * o.elems) / tot
        self.elems = tot
        self.rows += o.rows
        self.idx_disagree += o.idx_disagree
        self.idx_bad += o.idx_bad
        self.amb_rows += o.amb_rows
        self.anchor_amb_rows += o.anchor_amb_rows
        self.max_rel_err = max(self.max_rel_err, o.max_rel_err)
        self.max_excess = max(self.max_excess, o.max_excess)


def _edges(var, y, K):
    """Distance of y to the nearest discontinuity of the weight (and the index)."""
    kind = var["kind"]
    if kind == "exact":
        return np.full_like(y, np.inf), np.full_like(y, np.inf)
    if kind in ("trunc", "uniform"):                             # the support edge y = (m - s)/W = 1
        d = np.abs(y - 1.0)
        return d, d
    frac_half = np.abs(y - np.floor(y) - 0.5)                   # distance to a half-integer
    if kind == "pot" or not var.get("interp", False):
        d_w = frac_half
        if var.get("flush") and kind == "kint":
            d_w = np.minimum(d_w, np.abs(y - K))
        return d_w, d_w
    # interpolation: weight continuous inside the grid; index = floor(y) jumps at integers
    d_w = np.abs(y - K) if var.get("flush") else np.full_like(y, np.inf)
    d_i = np.minimum(np.abs(y - np.rint(y)), d_w)
    return d_w, d_i


def _eps(var, y, m, S, dstar, delta):
    kind = var["kind"]
    if kind == "exact":
        return np.zeros_like(y)
    base = 4 * U * (np.abs(m)[:, None] + np.abs(S))
    if kind in ("pot", "pot_running"):
        return (2 * dstar[:, None] + base) * LOG2E + 4 * U * np.abs(y)
    if kind in ("trunc", "uniform"):
        return (2 * dstar[:, None] + base) / var["window"] + 4 * U * np.abs(y)
    K = var["levels"]
    grow = 0.0 if var.get("window") is not None else (np.abs(y) / K)
    dd = np.where(delta > 0, delta, np.inf)[:, None]
    return (2 * dstar[:, None] * (1 + grow) + base) / dd + 4 * U * np.abs(y)


def _other_weight(var, idx, y, T, shift=None):
    """Weight an ambiguous element gets if it lands across its nearest edge (pot_running:
    ``shift`` = the later rises of the anchor, in levels, that scale the element's weight)."""
    kind = var["kind"]
    if kind == "pot_running":
        fl = np.floor(y)
        other = np.maximum(np.where(y - fl < 0.5, fl + 1, fl), 0)
        L = var["levels"]
        if var.get("flush"):
            return np.where(other >= L, 0.0, np.exp2(-(np.minimum(other, L - 1) + shift)))
        return np.exp2(-(np.minimum(other, L - 1) + shift))
    if kind in ("trunc", "uniform"):   # across the support edge: cut if kept, kept if cut
        inside = np.exp(-y * var["window"]) if kind == "trunc" else np.ones_like(y)
        return np.where(y <= 1.0, 0.0, inside)
    fl = np.floor(y)
    other = np.where(y - fl < 0.5, fl + 1, fl)          # index across the nearest half-integer
    if kind == "pot":
        L = var["levels"]
        other = np.maximum(other, 0)
        if var.get("flush"):
            return np.where(other >= L, 0.0, np.exp2(-np.minimum(other, L - 1)))
        return np.exp2(-np.minimum(other, L - 1))
    K = var["levels"]
    flush = var.get("flush", False)
    if var.get("interp"):
        # inside the grid the weight is continuous; only the flush edge y = K jumps
        return np.where(y <= K, 0.0, T[:, K:K + 1]) if flush else np.zeros_like(y)
    oi = np.clip(other, 0, K).astype(np.int64)
    w_other = np.take_along_axis(T, oi, axis=1)
    if flush:
        near_flush = np.abs(y - K) < np.abs(y - (fl + 0.5))
        w_other = np.where(near_flush, np.where(y <= K, 0.0, T[:, K:K + 1]), w_other)
        w_other = np.where((y > K) & ~near_flush, 0.0, w_other)
    return w_other


def check_anchor_rows(rep: Report, frac: float = 0.03):
    assert rep.anchor_amb_rows <= max(2, frac * rep.rows), \
        f"{rep.anchor_amb_rows} of {rep.rows} rows have an ambiguous anchor"


def compare_head(var, q, k, v, rows, O_gpu, idx_gpu=None, *, causal, scale=None, tol=1e-2, min_agree=0.999,
                 l_gpu=None):
    """Compare one (batch, head): q (Nq,d), k/v (N,d) float64 as stored (decoded,
    descaled); rows: query rows; O_gpu (R,d) float; idx_gpu (R,N) uint8 or None."""
    d = q.shape[1]
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    ref = oracle.head_rows(q, k, v, rows, causal=causal, detail=True, scale=scale,
                           **{kk: var[kk] for kk in var if kk != "kind"}, kind=var["kind"])
    R, N = ref["w"].shape
    rep = Report(rows=R)
    S = sc * (q[rows] @ k.T)
    vis = ref["idx"] != oracle.IDX_MASKED
    dstar = 2 * d * U * sc * np.max(np.abs(q[rows]) @ np.abs(k).T, axis=1)
    K = var.get("levels") or 0
    y = np.where(vis, ref["y"], 0.0)
    d_w, d_i = _edges(var, y, K)
    eps = _eps(var, y, ref["m"], S, dstar, ref["delta"])
    amb_w = vis & (d_w <= eps)
    amb_i = vis & (d_i <= eps)
    shift = None
    skip = np.zeros(R, bool)
    if var["kind"] == "pot_running":
        t = np.where(vis, S * LOG2E, -np.inf)
        tile = oracle.qsa_oracle.ANCHOR_TILE
        nt = (N + tile - 1) // tile
        cm = np.maximum.accumulate(np.stack([t[:, c * tile:(c + 1) * tile].max(1) for c in range(nt)], 1), 1)
        fin = np.isfinite(cm)
        cmv = np.where(fin, cm, 0.0)
        eps_a = (2 * dstar + 8 * U * np.abs(ref["m"]))[:, None] * LOG2E + 4 * U * np.abs(cmv)
        skip = (fin & (np.abs(cmv - np.rint(cmv)) <= eps_a)).any(1)
        rep.anchor_amb_rows = int(skip.sum())
        shift = np.where(vis, np.rint(ref["A"][:, None] - (y + np.where(vis, S * LOG2E, 0.0))), 0.0)
        vis = vis & ~skip[:, None]
        amb_w &= vis
        amb_i &= vis
    if idx_gpu is not None and var["kind"] != "exact":
        assert np.array_equal((idx_gpu == oracle.IDX_MASKED)[~skip], (ref["idx"] == oracle.IDX_MASKED)[~skip]), \
            "masked positions differ"
        dis = vis & (idx_gpu != ref["idx"])
        rep.elems = int(vis.sum())
        rep.idx_disagree = int(dis.sum())
        rep.idx_agree = 1.0 - rep.idx_disagree / max(rep.elems, 1)
        rep.idx_bad = int((dis & ~amb_i).sum())
    # O: per-row relative error with the ambiguity slack
    T = None
    if var["kind"] == "kint":
        T = np.exp(-np.arange(K + 1)[None, :] * ref["delta"][:, None])
    sigma = np.zeros(R)
    dw_sum = np.zeros(R)
    if amb_w.any():
        wo = _other_weight(var, ref["idx"], y, T, shift)
        dw = np.where(amb_w, np.abs(wo - ref["w"]), 0.0)
        spread = np.linalg.norm(v[None, :, :] - ref["O"][:, None, :], axis=2) if R * N * d < 5e7 else None
        if spread is None:
            spread = np.stack([np.linalg.norm(v - ref["O"][i], axis=1) for i in range(R)])
        num = (dw * spread).sum(1)
        den = ref["l"] - dw.sum(1)
        sigma = np.where(den > 0, num / np.maximum(den, 1e-300), np.inf)
        rep.amb_rows = int((dw.sum(1) > 0).sum())
        dw_sum = dw.sum(1)
    err = np.linalg.norm(O_gpu.astype(np.float64) - ref["O"], axis=1)
    nrm = np.linalg.norm(ref["O"], axis=1)
    sigma = np.where(skip, np.inf, sigma)
    rep.max_rel_err = float(np.max(np.where(skip, 0.0, err / np.maximum(nrm, 1e-30))))
    rep.max_excess = float(np.max(err - tol * nrm - sigma))
    if idx_gpu is not None and var["kind"] != "exact":
        if rep.idx_bad:
            bi, bj = np.nonzero(dis & ~amb_i)
            detail = "; ".join(f"row {rows[i]} key {j}: y {y[i, j]:.7f} eps {eps[i, j]:.2e} gpu {idx_gpu[i, j]} "
                               f"oracle {ref['idx'][i, j]}" for i, j in list(zip(bi, bj))[:3])
            raise AssertionError(f"{rep.idx_bad} index disagreements outside the fp32 edge band ({detail})")
        # interpolation's index floor(y) is informative only: its weight is continuous there,
        # and min-max rows put their minimum exactly on the integer y = K
        if not var.get("interp"):
            assert rep.idx_agree >= min_agree, f"index agreement {rep.idx_agree:.5f} < {min_agree}"
    assert rep.max_excess <= 0, f"O error exceeds tol: max rel err {rep.max_rel_err:.3e}"
    if l_gpu is not None:   # row sums: same tolerance plus the weight change of ambiguous elements
        excess = np.abs(np.asarray(l_gpu, np.float64) - ref["l"]) - tol * ref["l"] - dw_sum
        excess = np.where(skip, -1.0, excess)
        assert np.all(excess <= 0), f"row sum off by {np.max(excess):.3e} beyond tolerance"
    return rep, ref
