"""Scalar brute-force oracle (pure Python, tiny inputs only).

TEST INFRASTRUCTURE ONLY, like the rest of this package.  A second, deliberately
naive implementation of the same weight functions, written with plain loops
and the ``math`` module, so that the vectorised float64 oracle can be checked
against something that shares none of its code.  Rowmax-PoT weights are exact
dyadic rationals, so the PoT path here works in ``fractions.Fraction`` and
returns the exact rational output.

Definitions followed (readings as in the vectorised oracle):
  K-interval -- "Pretraining Transformers with Quantized Softmax in Attention",
  abstract (K+1 grid values, per-row calibration, hard rounding or
  interpolation) and chapter 1 (exponential read off a grid calibrated per row);
  Rowmax-PoT -- "Approximating Softmax in Pretrained LLMs: Model Sensitivity
  and Kernel Acceleration", abstract (power-of-two weights anchored at each
  row maximum);
  support truncation and uniform weighting -- the same abstract's sensitivity
  study (keep only the scores within W of the row maximum, with their exact
  weights or with equal weights);
  single-pass power-of-two weights (``pot_running``) -- simulated here as a
  pass over the keys that keeps a running integer anchor and rescales the
  weights already formed whenever the anchor rises, instead of the vectorised
  oracle's closed form.
"""
from __future__ import annotations

import math
from fractions import Fraction


def _round_half_even(x: float) -> int:
    f = math.floor(x)
    r = x - f
    if r > 0.5:
        return f + 1
    if r < 0.5:
        return f
    return f if f % 2 == 0 else f + 1


def _running_pot_row(scores, visible, L, flush, tile, exact):
    """Single-pass power-of-two weights: tiles of ``tile`` keys in order; after a
    tile's maximum is seen the anchor A = ceil(max so far of s log2 e) may rise,
    and every weight formed before is multiplied by 2**-(rise)."""
    inv_ln2 = 1.0 / math.log(2.0)
    one = Fraction(1) if exact else 1.0
    w = [0 * one] * len(scores)
    A = None
    for start in range(0, len(scores), tile):
        keys = [j for j in range(start, min(start + tile, len(scores))) if visible[j]]
        if not keys:
            continue
        top = math.ceil(max(scores[j] * inv_ln2 for j in keys))
        if A is not None and top > A:
            for j in range(start):
                w[j] = w[j] / (2 ** (top - A))
        if A is None or top > A:
            A = top
        for j in keys:
            e = _round_half_even(A - scores[j] * inv_ln2)
            if e > L - 1:
                if flush:
                    continue
                e = L - 1
            w[j] = one / (2 ** e)
    return w


def weight_row(scores, visible, kind, levels=None, window=None, interp=False, flush=False, exact_pot=False,
               tile=64):
    """Weights of one row of scaled scores (list of float) -> list of weights.

    Masked keys get weight 0.  With ``exact_pot`` PoT weights are Fractions.
    """
    if kind == "pot_running":
        return _running_pot_row(scores, visible, levels, flush, tile, exact_pot)
    vis = [s for s, ok in zip(scores, visible) if ok]
    m = max(vis)
    mn = min(vis)
    out = []
    if kind == "exact":
        for s, ok in zip(scores, visible):
            out.append(math.exp(s - m) if ok else 0.0)
        return out
    if kind in ("trunc", "uniform"):
        for s, ok in zip(scores, visible):
            if not ok or s < m - window:
                out.append(0.0)
            elif kind == "trunc":
                out.append(math.exp(s - m))
            else:
                out.append(1.0)
        return out
    if kind == "pot":
        L = levels
        for s, ok in zip(scores, visible):
            if not ok:
                out.append(Fraction(0) if exact_pot else 0.0)
                continue
            e = _round_half_even((m - s) / math.log(2.0))
            if e > L - 1:
                if flush:
                    out.append(Fraction(0) if exact_pot else 0.0)
                    continue
                e = L - 1
            out.append(Fraction(1, 2 ** e) if exact_pot else 2.0 ** (-e))
        return out
    # K-interval: grid of K+1 points from the anchor m down to lo
    K = levels
    lo = (m - window) if window is not None else mn
    step = (m - lo) / K
    grid_vals = [math.exp(-l * step) for l in range(K + 1)]
    # A min-max grid ends at the row minimum, so no visible score lies below it: flushing
    # applies to fixed windows only (a y a rounding step above K at the minimum stays in).
    flush = flush and window is not None
    for s, ok in zip(scores, visible):
        if not ok:
            out.append(0.0)
            continue
        if step == 0.0:
            out.append(1.0)
            continue
        y = (m - s) / step
        if y > K and flush:
            out.append(0.0)
            continue
        if not interp:
            l = min(_round_half_even(y), K)
            out.append(grid_vals[l])
        else:
            if y >= K:
                out.append(grid_vals[K])
                continue
            l = int(math.floor(y))
            t = y - l
            out.append(grid_vals[l] + t * (grid_vals[l + 1] - grid_vals[l]))
    return out


def attention(q, k, v, causal=False, kind="exact", levels=None, window=None, interp=False, flush=False,
              scale=None, exact_pot=False, tile=64):
    """One head: q, k, v lists of rows (lists of float).  Returns O rows.

    With ``exact_pot`` (kind "pot"), scores are still floats but the weights
    and the normalised output are exact Fractions of the (exact) V entries.
    """
    n = len(q)
    nk = len(k)
    d = len(q[0])
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    out = []
    for i in range(n):
        scores = []
        for j in range(nk):
            acc = 0.0
            for c in range(d):
                acc += q[i][c] * k[j][c]
            scores.append(sc * acc)
        visible = [(j <= i) if causal else True for j in range(nk)]
        w = weight_row(scores, visible, kind, levels, window, interp, flush,
                       exact_pot and kind in ("pot", "pot_running"), tile)
        total = sum(w)
        row = []
        for c in range(len(v[0])):
            num = sum((w[j] * (Fraction(v[j][c]) if isinstance(w[j], Fraction) else v[j][c]))
                      for j in range(nk))
            row.append(num / total)
        out.append(row)
    return out
