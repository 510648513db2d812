"""GPU-vs-oracle comparison protocol (test helper).

The GPU forms scores by MFMA accumulation of exact bf16 or fp8 products (or by
fp32 FMAs); the oracle in float64.  For a row i the score error is bounded by
delta*_i = gamma * scale * max_j sum_c |q_ic k_jc|.  With fp32 accumulation
gamma = 2 d u, u = 2^-24 (twice the textbook bound for any summation order).
The 8-bit MFMA of fp8 inputs sums its products more coarsely than fp32: on
MI355X its row maxima, measured against exact float64 (16 seeded cases, d 64
and 128, logit scales 0.25 to 16, 65 536 rows), were off by up to
2^-14.3 scale max_j sum_c |q_ic k_jc|, 3.3 times the fp32 bound at d = 64.  For
fp8 inputs gamma is therefore GAMMA_FP8 = 2^-12, 4.8 times the largest error
measured (the bf16 MFMA stays within 1.4 % of the fp32 bound).
That error moves the grid coordinate y_ij by at most eps_ij (below), so an
element whose y lies within eps of a discontinuity of its weight function is
edge-ambiguous: either neighbouring grid index is a correct result.

Single-pass PoT (``pot_running``) has one more decision per tile: the anchor
ceil(running max of s log2 e), i.e. the running max of ceil(tile max).  Where a
tile's maximum lies within the band of an integer n, the GPU may round it up to
n or to n + 1, which moves every exponent weighed against the anchor by one
level (and so the clip).  Such rows are compared against the oracle once per
possible anchor sequence (the oracle takes the anchors as an input) and pass if
one of them matches; none is left out.

Checks:
  * index agreement >= 99.9 % over visible elements (at least one element may
    differ in any head), and every disagreement edge-ambiguous; masked codes
    identical;
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
GAMMA_FP8 = 2.0 ** -12      # score-error factor of the 8-bit MFMA (module docstring)


def score_gamma(d, fp8=False):
    """gamma of delta* for head dimension d (fp8: the 8-bit MFMA's accumulation)."""
    return max(2 * d * U, GAMMA_FP8) if fp8 else 2 * d * U


@dataclass
class Report:
    rows: int = 0
    elems: int = 0
    idx_agree: float = 1.0
    idx_disagree: int = 0
    idx_bad: int = 0              # disagreements outside the ambiguity band
    amb_rows: int = 0
    anchor_amb_rows: int = 0      # pot_running rows compared under several possible anchor sequences
    max_rel_err: float = 0.0      # max over rows of ||dO|| / ||O_ref||
    max_excess: float = 0.0       # max over rows of ||dO|| - tol ||O_ref|| - sigma (<= 0 passes)
    plain_differs: int = 0        # launches without the index dump whose O differs from the dump's
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
        self.plain_differs += o.plain_differs


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


MAX_AMBIGUOUS_TILES = 8     # per row; 2^8 anchor sequences at most


def anchor_candidates(var, q, k, rows, *, causal, scale=None, fp8=False):
    """pot_running: for each row, the anchor sequences (after each key tile) an fp32
    implementation may produce, the definition's own first.  The score band is the one
    of the weights (delta*, section above); a tile maximum within it of an integer n
    may be rounded up to n or n + 1.  Returns a list (one per row) of (tiles,) arrays."""
    d = q.shape[1]
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    N = k.shape[0]
    S = sc * (q[rows] @ k.T)
    cols = np.arange(N)
    vis = (cols[None, :] <= np.asarray(rows)[:, None]) if causal else np.ones(S.shape, bool)
    t = np.where(vis, S * LOG2E, -np.inf)
    tile = oracle.qsa_oracle.ANCHOR_TILE
    nt = (N + tile - 1) // tile
    tmax = np.stack([t[:, c * tile:(c + 1) * tile].max(1) for c in range(nt)], 1)
    dstar = score_gamma(d, fp8) * sc * np.max(np.abs(q[rows]) @ np.abs(k).T, axis=1)
    m = np.where(vis, S, -np.inf).max(1)
    fin = np.isfinite(tmax)
    tv = np.where(fin, tmax, 0.0)
    eps_a = (2 * dstar + 8 * U * np.abs(m))[:, None] * LOG2E + 4 * U * np.abs(tv)
    amb = fin & (np.abs(tv - np.rint(tv)) <= eps_a)
    base = np.ceil(tmax)
    # A tile's rounding matters only if it can raise the running anchor: where even the smallest
    # running maximum of the tiles before it (every ambiguous tile rounded down) is already at
    # least n + 1, both roundings give the same anchors, so the tile is left out (exactly: no
    # distinct sequence is lost).
    low = np.where(amb, np.rint(tv), base)
    prev = np.concatenate([np.full((len(rows), 1), -np.inf), np.maximum.accumulate(low, axis=1)[:, :-1]], 1)
    amb &= prev < np.rint(tv) + 1
    out = []
    for i in range(len(rows)):
        J = np.nonzero(amb[i])[0]
        assert len(J) <= MAX_AMBIGUOUS_TILES, f"row {rows[i]}: {len(J)} tile anchors within the score band"
        seqs, seen = [], set()
        for bits in range(1 << len(J)):
            a = base[i].copy()
            for b, j in enumerate(J):
                a[j] = np.rint(tv[i, j]) + ((bits >> b) & 1)
            A = np.maximum.accumulate(a)
            key = A.tobytes()
            if key not in seen:
                seen.add(key)
                seqs.append(A)
        default = np.maximum.accumulate(base[i])
        seqs.sort(key=lambda A: not np.array_equal(A, default))
        out.append(seqs)
    return out


def _check_agreement(rep, min_agree):
    """The agreement floor: at most a fraction 1 - min_agree of the visible elements, and never
    less than one element, may take the other index of an edge (each one already checked to lie
    in the band).  A head with fewer than 1 / (1 - min_agree) visible elements may otherwise fail
    on a single element that is correct either way."""
    allowed = max(1, int((1.0 - min_agree) * rep.elems))
    assert rep.idx_disagree <= allowed, \
        f"index agreement {rep.idx_agree:.5f} < {min_agree} ({rep.idx_disagree} of {rep.elems} elements)"


def compare_head(var, q, k, v, rows, O_gpu, idx_gpu=None, *, causal, scale=None, tol=1e-2, min_agree=0.999,
                 l_gpu=None, anchors=None, fp8=False):
    """Compare one (batch, head): q (Nq,d), k/v (N,d) float64 as stored (decoded,
    descaled); rows: query rows; O_gpu (R,d) float; idx_gpu (R,N) uint8 or None.
    ``anchors`` (pot_running): the per-tile anchors of the rows, as the oracle takes them;
    by default every sequence fp32 may produce is tried per row (anchor_candidates).
    ``fp8``: the scores came from the 8-bit MFMA (its wider error band, module docstring)."""
    rows = np.asarray(rows)
    if var["kind"] == "pot_running" and anchors is None:
        cands = anchor_candidates(var, q, k, rows, causal=causal, scale=scale, fp8=fp8)
        single = np.array([len(c) == 1 for c in cands])
        rep, ref = Report(), None
        if single.any():
            sel = np.nonzero(single)[0]
            rep, ref = compare_head(var, q, k, v, rows[sel], O_gpu[sel], None if idx_gpu is None else idx_gpu[sel],
                                    causal=causal, scale=scale, tol=tol, min_agree=min_agree,
                                    l_gpu=None if l_gpu is None else np.asarray(l_gpu)[sel],
                                    anchors=np.stack([cands[i][0] for i in sel]), fp8=fp8)
        for i in np.nonzero(~single)[0]:
            errs = []
            for A in cands[i]:
                try:
                    r1, _ = compare_head(var, q, k, v, rows[i:i + 1], O_gpu[i:i + 1],
                                         None if idx_gpu is None else idx_gpu[i:i + 1], causal=causal, scale=scale,
                                         tol=tol, min_agree=0.0, l_gpu=None if l_gpu is None else
                                         np.asarray(l_gpu)[i:i + 1], anchors=A[None, :], fp8=fp8)
                    break
                except AssertionError as e:
                    errs.append(str(e))
            else:
                raise AssertionError(f"row {rows[i]}: no anchor sequence of {len(cands[i])} matches: {errs}")
            r1.anchor_amb_rows = 1
            rep.merge(r1)
        if rep.elems and idx_gpu is not None and not var.get("interp"):
            _check_agreement(rep, min_agree)
        return rep, ref
    d = q.shape[1]
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    ref = oracle.head_rows(q, k, v, rows, causal=causal, detail=True, scale=scale, anchors=anchors,
                           **{kk: var[kk] for kk in var if kk != "kind"}, kind=var["kind"])
    R, N = ref["w"].shape
    rep = Report(rows=R)
    S = sc * (q[rows] @ k.T)
    vis = ref["idx"] != oracle.IDX_MASKED
    dstar = score_gamma(d, fp8) * sc * np.max(np.abs(q[rows]) @ np.abs(k).T, axis=1)
    K = var.get("levels") or 0
    y = np.where(vis, ref["y"], 0.0)
    d_w, d_i = _edges(var, y, K)
    eps = _eps(var, y, ref["m"], S, dstar, ref["delta"])
    amb_w = vis & (d_w <= eps)
    amb_i = vis & (d_i <= eps)
    shift = None
    if var["kind"] == "pot_running":
        # later rises of the anchor scale an element's weight by 2^-shift
        shift = np.where(vis, np.rint(ref["A"][:, None] - (y + np.where(vis, S * LOG2E, 0.0))), 0.0)
    if idx_gpu is not None and var["kind"] != "exact":
        assert np.array_equal(idx_gpu == oracle.IDX_MASKED, ref["idx"] == oracle.IDX_MASKED), \
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
    rep.max_rel_err = float(np.max(err / np.maximum(nrm, 1e-30)))
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
            _check_agreement(rep, min_agree)
    assert rep.max_excess <= 0, f"O error exceeds tol: max rel err {rep.max_rel_err:.3e}"
    if l_gpu is not None:   # row sums: same tolerance plus the weight change of ambiguous elements
        excess = np.abs(np.asarray(l_gpu, np.float64) - ref["l"]) - tol * ref["l"] - dw_sum
        assert np.all(excess <= 0), f"row sum off by {np.max(excess):.3e} beyond tolerance"
    return rep, ref
