"""Float64 CPU oracle for the quantized-softmax attention forward.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain reference that the
GPU path is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.  It
shares no code, constant or table with the HIP library.

What it computes, per (batch b, query head h), for query rows i and keys j:

    s_ij = scale * q_i . k_j                       (scale = 1/sqrt(d) by default)
    O_i  = sum_j w_ij v_j / sum_j w_ij             (w: the weight function)

with three kinds of weight function w(s) replacing exp(s - m):

* ``exact``  -- w = exp(s - m_i), i.e. ordinary softmax attention, the
  control that the approximate forms replace (both pages note that softmax
  usually stays at higher precision than the attention matmuls).
* ``kint``   -- K-interval attention ("Pretraining Transformers with Quantized
  Softmax in Attention", abstract and chapters 1, 5, 6): the exponential is
  read off K+1 grid values fitted to each row of scores.  The grid spans the
  row's calibration range [lo_i, m_i]: min-max calibration takes lo_i = the
  row minimum, fixed-window calibration takes lo_i = m_i - W.  Grid points are
  g_l = m_i - l*Delta_i with Delta_i = (m_i - lo_i)/K, l = 0..K, and grid
  values T_l = exp(-l*Delta_i).  With y = (m_i - s)/Delta_i, hard rounding
  takes w = T_rint(y); interpolation takes the straight line between the two
  neighbouring grid values.
* ``pot``    -- Rowmax-PoT ("Approximating Softmax in Pretrained LLMs: Model
  Sensitivity and Kernel Acceleration", abstract; the wiki page's flowchart
  "Row max -> Power-of-two weights"): a coarse logarithmic weight anchored at
  the row maximum.  With y = (m_i - s) * log2(e), e = rint(y) clipped to the
  stated level count L, w = 2**-e.
* ``pot_running`` -- a single-pass form of the power-of-two weights with no
  row-maximum pre-pass (the Rowmax-PoT page names a max-anchored variant built
  into FlashAttention-4 without saying how it obtains the maximum).  Keys are
  taken in tiles of ``tile`` consecutive keys (64, the kernels' key tile); after
  each tile the row's anchor becomes A = ceil(running max of s * log2(e)), an
  integer, so that a key's exponent e = rint(A - s log2(e)), clipped to L-1 (or
  flushed beyond it) against the anchor in force when its tile was weighed,
  stays exact when a later rise of the anchor by an integer dA rescales every
  earlier weight by 2**-dA.  Its final weight is 2**-(e + A_final - A_tile).
  Without the clip this is 2**rint(s log2 e) normalised: a power-of-two grid
  fixed at integer log2 values instead of aligned with the row maximum.
* ``trunc`` and ``uniform`` -- the two operators of the sensitivity study on
  the same "Approximating Softmax" page (abstract): the softmax support can be
  cut to the scores close to the row maximum with little loss, while giving
  the kept positions equal weight hurts.  Both keep the support
  {j visible : s_ij >= m_i - W} for a window W; ``trunc`` gives the kept keys
  their exact weights exp(s - m_i), ``uniform`` gives each of them weight 1,
  so O_i is the plain mean of the kept values.  Keys outside the support get
  weight 0 (index code 254, like a flushed element).

Readings taken where the pages are silent (every one is listed in the design
notes of the repository with its reason):
  R1  the grid lives in the score domain and is uniformly spaced;
  R2  K counts intervals, so there are K+1 grid values, both ends included;
  R4  fixed window: scores below m - W saturate to T_K, or give 0 with flush;
  R5  PoT: e saturates at L-1 (L distinct weights), or e >= L gives 0 with
      flush;
  R6  rint is round-half-to-even;
  R7  the index is measured from the anchor m_i (l = rint((m - s)/Delta));
  R8  interpolation is linear in the weight (exp) domain;
  R9  a min-max row whose visible scores are all equal has Delta = 0: every
      visible weight is 1;
  R10 extrema are taken over the keys visible to the row (causal: j <= i,
      top-left aligned);
  R11 normalisation divides by the sum of the approximate weights;
  R15 query head h reads KV head floor(h / (H/Hkv)).

Index code per element (what the GPU may dump for parity): the grid index
l (kint) or exponent e (pot), clipped as the weight was; 254 for a flushed
element, 255 for a masked (invisible) one; exact kinds store 0.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

LOG2E = 1.0 / math.log(2.0)
ANCHOR_TILE = 64          # keys per anchor update of pot_running (the kernels' key tile)
IDX_FLUSHED = 254
IDX_MASKED = 255


# ---------------------------------------------------------------------------
# Decoding of the stored formats (exact; each value maps to one real number)
# ---------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.  A bfloat16 is the upper
    half of an IEEE binary32, so widening the pattern is exact."""
    b32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b32.view(np.float32).astype(np.float64)


def decode_f32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def decode_e4m3fn(bits: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 (``fn``: finite, no infinities) bit patterns -> float64.

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent field 0
    is subnormal: m/8 * 2**-6.  The pattern S.1111.111 is NaN; every other
    pattern is finite, up to 448 = 1.75 * 2**8.
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    ex = (b >> 3) & 0xF
    man = (b & 0x7).astype(np.float64)
    val = np.where(ex == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * np.exp2(ex - 7.0))
    val = np.where((ex == 0xF) & ((b & 0x7) == 0x7), np.nan, val)
    return sign * val


# ---------------------------------------------------------------------------
# The weight functions (one row chunk at a time)
# ---------------------------------------------------------------------------

def _check_kind(kind, levels, window, interp, flush):
    if kind not in ("exact", "kint", "pot", "pot_running", "trunc", "uniform"):
        raise ValueError(f"unknown kind {kind!r}")
    if kind in ("trunc", "uniform"):
        if window is None or not (window > 0 and math.isfinite(window)):
            raise ValueError(f"{kind} needs a finite window W > 0")
        if interp or flush:
            raise ValueError(f"{kind} takes no interpolation or flush option")
        return
    if kind == "kint" and not (isinstance(levels, int) and levels >= 1):
        raise ValueError("kint needs levels = K >= 1 intervals")
    if kind == "pot" and not (isinstance(levels, int) and levels >= 1):
        raise ValueError("pot needs levels = L >= 1")
    if kind == "pot_running" and not (isinstance(levels, int) and levels >= 2):
        # the row maximum sits at e = 0 or 1 below the rounded-up anchor: L >= 2 keeps it
        raise ValueError("pot_running needs levels = L >= 2")
    if window is not None and not (window > 0 and math.isfinite(window)):
        raise ValueError("window must be finite and > 0")
    if interp and kind != "kint":
        raise ValueError("interpolation is a K-interval option")
    if window is not None and kind != "kint":
        raise ValueError("fixed-window calibration is a K-interval option")
    if flush and kind == "exact":
        raise ValueError("flush applies to kint and pot")


def row_weights(S: np.ndarray, visible: np.ndarray, *, kind: str, levels: Optional[int] = None,
                window: Optional[float] = None, interp: bool = False, flush: bool = False,
                extrema: Optional[tuple] = None, tile: int = ANCHOR_TILE, anchors: Optional[np.ndarray] = None):
    """Weights for a block of score rows.

    S: (R, N) float64 scaled scores; visible: (R, N) bool, at least one True
    per row.  Returns dict with w (R,N), idx (R,N) uint8, y (R,N) grid
    coordinate (nan where masked; for exact kinds y = m - s; pot_running: the
    rounded A_tile - s log2 e), m, lo, delta (R,) and the table T (R, K+1) for
    kint; pot_running also gives the final anchor A (R,) in log2 units.  The
    columns of S are the keys in order (pot_running visits them in tiles of
    ``tile``).  ``extrema`` = (m, mn), each (R,),
    replaces the row maximum and minimum (the forward with the calibration held
    fixed, whose derivative is the detached gradient).  ``anchors`` (pot_running
    only), (R, number of tiles), replaces the anchor after each tile, which the
    definition takes as ceil(running max of s log2 e): a tile maximum that lies on
    an integer up to rounding may be rounded up either way by an implementation
    in lower precision, and this lets a comparison weigh the other choice.
    """
    _check_kind(kind, levels, window, interp, flush)
    R, N = S.shape
    neg = np.where(visible, S, -np.inf)
    pos = np.where(visible, S, np.inf)
    m = neg.max(axis=1)                                   # row max over visible keys (anchor)
    mn = pos.min(axis=1)                                  # row min over visible keys
    if extrema is not None:
        m = np.asarray(extrema[0], dtype=np.float64)
        mn = np.asarray(extrema[1], dtype=np.float64)
    out = {"m": m}
    idx = np.full((R, N), IDX_MASKED, dtype=np.uint8)

    if kind == "exact":
        y = np.where(visible, m[:, None] - S, np.nan)
        w = np.where(visible, np.exp(np.where(visible, S - m[:, None], 0.0)), 0.0)
        idx[visible] = 0
        out.update(w=w, idx=idx, y=y, lo=mn, delta=np.zeros(R))
        return out

    if kind in ("trunc", "uniform"):
        # support: the visible keys whose score is at least m - W (the row max is always kept)
        kept = visible & (m[:, None] - S <= window)
        if kind == "trunc":
            w = np.where(kept, np.exp(np.where(kept, S - m[:, None], 0.0)), 0.0)
        else:
            w = kept.astype(np.float64)
        idx[kept] = 0
        idx[visible & ~kept] = IDX_FLUSHED
        y = np.where(visible, (m[:, None] - S) / window, np.nan)   # the support edge is y = 1
        out.update(w=w, idx=idx, y=y, lo=m - window, delta=np.full(R, float(window)))
        return out

    if kind == "pot_running":
        L = levels
        t = np.where(visible, S * LOG2E, -np.inf)             # scores in log2 units
        nt = (N + tile - 1) // tile
        tmax = np.stack([t[:, c * tile:(c + 1) * tile].max(axis=1) for c in range(nt)], axis=1)
        A = np.ceil(np.maximum.accumulate(tmax, axis=1))      # anchor after each tile (-inf before any key)
        if anchors is not None:
            A = np.asarray(anchors, dtype=np.float64).reshape(R, nt)
        Aj = np.repeat(A, tile, axis=1)[:, :N]                # the anchor a key's tile was weighed with
        Afin = A[:, -1]
        y = np.where(visible, Aj - np.where(visible, t, 0.0), np.nan)
        ex = np.rint(np.where(visible, y, 0.0))               # exponent against the tile's anchor
        if flush:
            keep = visible & (ex <= L - 1)
        else:
            ex = np.minimum(ex, L - 1)
            keep = visible
        shift = np.where(visible, Afin[:, None] - Aj, 0.0)    # later rises of the anchor
        w = np.where(keep, np.exp2(-(np.where(keep, ex, 0.0) + shift)), 0.0)
        idx[keep] = ex[keep].astype(np.uint8)
        idx[visible & ~keep] = IDX_FLUSHED
        out.update(w=w, idx=idx, y=y, lo=mn, delta=np.full(R, 1.0 / LOG2E), A=Afin)
        return out

    if kind == "pot":
        L = levels
        y = np.where(visible, (m[:, None] - S) * LOG2E, np.nan)
        e = np.rint(np.where(visible, y, 0.0))            # round half to even
        if flush:
            kept = visible & (e <= L - 1)
            flushed = visible & ~kept
        else:
            e = np.minimum(e, L - 1)
            kept = visible
            flushed = np.zeros_like(visible)
        w = np.where(kept, np.exp2(-np.where(kept, e, 0.0)), 0.0)
        idx[kept] = e[kept].astype(np.uint8)
        idx[flushed] = IDX_FLUSHED
        out.update(w=w, idx=idx, y=y, lo=mn, delta=np.full(R, 1.0 / LOG2E))
        return out

    # K-interval
    K = levels
    lo = (m - window) if window is not None else mn
    delta = (m - lo) / K
    ell = np.arange(K + 1, dtype=np.float64)
    T = np.exp(-ell[None, :] * delta[:, None])            # K+1 grid values per row, T_0 = 1
    degenerate = delta == 0.0                             # min-max row with all scores equal
    safe = np.where(degenerate, 1.0, delta)
    y = np.where(visible, (m[:, None] - S) / safe[:, None], np.nan)
    y = np.where(degenerate[:, None] & visible, 0.0, y)
    yv = np.where(visible, y, 0.0)
    rows = np.arange(R)[:, None]
    # A min-max grid spans every visible score (y <= K), so flushing removes nothing
    # there; it applies to fixed-window grids, whose window can end above the row minimum.
    flush = flush and window is not None
    if not interp:
        l = np.rint(yv)                                   # nearest grid point, half to even
        if flush:
            kept = visible & (yv <= K)                    # below the window -> flushed
        else:
            kept = visible
        l = np.minimum(l, K)
        li = l.astype(np.int64)
        w = np.where(kept, T[rows, li], 0.0)
    else:
        if flush:
            kept = visible & (yv <= K)
        else:
            kept = visible
        yc = np.minimum(yv, float(K))
        l0 = np.minimum(np.floor(yc), K - 1).astype(np.int64)   # left grid point
        t = yc - l0
        w_lin = (1.0 - t) * T[rows, l0] + t * T[rows, l0 + 1]
        w = np.where(kept, w_lin, 0.0)
        li = np.minimum(np.floor(yc), K).astype(np.int64)
    flushed = visible & ~kept
    idx[kept] = li[kept].astype(np.uint8)
    idx[flushed] = IDX_FLUSHED
    out.update(w=w, idx=idx, y=y, lo=lo, delta=delta, T=T)
    return out


# ---------------------------------------------------------------------------
# Attention forward
# ---------------------------------------------------------------------------

def head_rows(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, rows: Optional[Sequence[int]] = None, *,
              causal: bool = False, kind: str = "exact", levels: Optional[int] = None,
              window: Optional[float] = None, interp: bool = False, flush: bool = False,
              scale: Optional[float] = None, detail: bool = False, chunk: int = 512,
              extrema: Optional[tuple] = None, tile: int = ANCHOR_TILE, anchors: Optional[np.ndarray] = None):
    """One (batch, head) pair: qh (N, d), kh/vh (N, d) float64.

    ``rows`` selects query rows (default: all).  Returns dict with O (R, d),
    m, lo, l (R,) and, if ``detail``, w, idx, y (R, N) and delta (R,).
    ``anchors`` (pot_running): per-tile anchors of the selected rows, (R, tiles).
    """
    Nq, d = qh.shape
    N = kh.shape[0]                                        # keys (equal to Nq in attention proper)
    sc = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    parts = {}
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        S = sc * (qh[r] @ kh.T)                            # scaled scores, float64
        cols = np.arange(N)
        visible = (cols[None, :] <= r[:, None]) if causal else np.ones((len(r), N), dtype=bool)
        ext = None if extrema is None else (np.asarray(extrema[0])[r], np.asarray(extrema[1])[r])
        anc = None if anchors is None else np.asarray(anchors)[c0:c0 + chunk]
        rw = row_weights(S, visible, kind=kind, levels=levels, window=window, interp=interp, flush=flush,
                         extrema=ext, tile=tile, anchors=anc)
        w = rw["w"]
        l = w.sum(axis=1)                                  # row sum of the approximate weights
        O = (w @ vh) / l[:, None]                          # normalise, then P.V
        piece = {"O": O, "m": rw["m"], "lo": rw["lo"], "l": l}
        if detail:
            piece.update(w=w, idx=rw["idx"], y=rw["y"], delta=rw["delta"])
            if "A" in rw:
                piece["A"] = rw["A"]
        for key, val in piece.items():
            parts.setdefault(key, []).append(val)
    return {key: np.concatenate(val, axis=0) for key, val in parts.items()}


def attn_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool = False, kind: str = "exact",
             levels: Optional[int] = None, window: Optional[float] = None, interp: bool = False,
             flush: bool = False, scale: Optional[float] = None, rows: Optional[Sequence[int]] = None,
             detail: bool = False):
    """Attention forward over all heads.

    q: (B, H, N, d); k, v: (B, Hkv, N, d), float64 (already decoded from the
    stored format and multiplied by any per-tensor descale).  Returns dict of
    arrays with leading (B, H) axes.
    """
    B, H, Nq, d = q.shape
    Hkv = k.shape[1]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    group = H // Hkv
    res = {}
    for b in range(B):
        for h in range(H):
            kv = h // group                                # query head h reads KV head floor(h/group)
            r = head_rows(q[b, h], k[b, kv], v[b, kv], rows, causal=causal, kind=kind, levels=levels,
                          window=window, interp=interp, flush=flush, scale=scale, detail=detail)
            for key, val in r.items():
                res.setdefault(key, []).append(val)
    return {key: np.stack(val).reshape((B, H) + val[0].shape) for key, val in res.items()}


# ---------------------------------------------------------------------------
# Attention backward (gradients of sum(dO * O) with respect to q, k, v)
# ---------------------------------------------------------------------------
#
# The pages train K-interval attention with a straight-through surrogate whose
# placement relative to the normalisation they vary, with backward rules that
# include the derivatives through the calibration and with the row extrema
# either attached or detached ("Pretraining Transformers with Quantized Softmax
# in Attention", abstract; chapter 5 "Build the method").  They print no
# formulas, so the gradient modes here are readings (listed in the design notes):
#
# * ``ste_post`` -- surrogate after the normalisation: the normalised weights
#   P = w / l are passed back as if they were a softmax of the scores, so
#   dS_ij = P_ij (dP_ij - D_i) with dP = dO V^T and D_i = dO_i . O_i.  The
#   extrema do not enter, so there is no attached/detached distinction.
# * ``ste_pre`` -- surrogate before the normalisation, where the forward needs
#   one: the rounding of the grid coordinate (K-interval hard rounding:
#   l = rint(y); PoT: e = rint(y)) is passed straight through (dl/dy := 1 where
#   the clip to the last level is not active, 0 where it is).  Everything else
#   takes its exact derivative: the normalisation, the interpolation, and the
#   calibration (the row maximum m through y and, for min-max grids, through
#   Delta = (m - lo) / K, which also moves the grid values T_l = exp(-l Delta);
#   the row minimum lo through Delta).  For hard rounding this gives
#   dw/ds = w inside the clip and dw/dDelta = w (y - l), a calibration term
#   that the post-normalisation placement does not have.  The gradients of m
#   and lo land on the arg-max and arg-min keys of the row (first in key order).
# * ``exact`` -- the derivative of the forward function wherever it exists
#   (almost everywhere): as ``ste_pre`` but with no surrogate, so hard rounding,
#   PoT and uniform weights are constant in each score.
# * ``ste_pre_detached``, ``exact_detached`` -- the same with m and lo held
#   constant.
#
# Rows whose min-max grid has zero width (every visible score equal) get no
# gradient through their weights in the modes that differentiate the grid.

GRADS = ("ste_post", "ste_pre", "ste_pre_detached", "exact", "exact_detached")


def _weight_partials(rw, kind, levels, interp, flush, visible, window, ste=False):
    """dw/dy and dw/dDelta (at fixed y) of each K-interval element; y as in
    row_weights.  ``ste``: hard rounding passed straight through (dl/dy := 1).
    At y = K the last interval's slope applies (the side of the visible scores);
    on a min-max grid every visible key counts as inside (y <= K by construction:
    the arg-min key sits on y = K whichever way the division rounds)."""
    R, N = visible.shape
    z = np.zeros((R, N))
    if kind != "kint":
        return z, z
    K = levels
    flush = flush and window is not None
    delta = rw["delta"]
    T = rw["T"]
    y = np.where(visible, rw["y"], 0.0)
    rows = np.arange(R)[:, None]
    if interp:
        yc = np.minimum(y, float(K))
        l0 = np.minimum(np.floor(yc), K - 1).astype(np.int64)
        t = yc - l0
        inside = visible if window is None else (y <= K)
        dwdy = np.where(inside, T[rows, l0 + 1] - T[rows, l0], 0.0)
        dT0 = -l0 * T[rows, l0]                        # dT_l/dDelta = -l T_l
        dT1 = -(l0 + 1) * T[rows, l0 + 1]
        dwdD = (1.0 - t) * dT0 + t * dT1
        beyond = -K * T[:, K:K + 1] * np.ones((1, N))
        dwdD = np.where(inside, dwdD, 0.0 if flush else beyond)
    else:
        r = np.rint(y)
        l = np.minimum(r, K).astype(np.int64)
        w = rw["w"]
        # T_l = exp(-l Delta): with l := y the weight moves as -Delta w in y (zero once clipped)
        dwdy = np.where(r <= K, -delta[:, None] * w, 0.0) if ste else np.zeros((R, N))
        dwdD = -l * T[rows, l]
        if flush:
            dwdD = np.where(y <= K, dwdD, 0.0)
    keep = visible & (delta > 0)[:, None]
    return np.where(keep, dwdy, 0.0), np.where(keep, dwdD, 0.0)


def head_bwd(qh, kh, vh, doh, *, causal=False, kind="exact", levels=None, window=None, interp=False,
             flush=False, scale=None, grad="ste_post", extrema=None, detail=False):
    """Gradients for one (batch, head): qh (N, d), kh/vh (N, d), doh (N, d) float64.
    Returns dict dQ (N, d), dK (N, d), dV (N, d) (this head's share of dK, dV); with
    ``detail`` also the normalised weights P and the score gradients dS (N, N) they come from.
    ``extrema`` (detached modes only) = (m, mn) per row, as in row_weights."""
    if grad not in GRADS:
        raise ValueError(f"unknown gradient mode {grad!r}")
    if kind == "pot_running":
        raise ValueError("the backward covers the max-anchored kinds, not pot_running")
    detached = grad.endswith("_detached")
    if extrema is not None and not detached:
        raise ValueError("fixed extrema go with a detached gradient")
    ste = grad.startswith("ste_pre")
    N, d = qh.shape
    sc = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    S = sc * (qh @ kh.T)
    cols = np.arange(N)
    visible = (cols[None, :] <= cols[:, None]) if causal else np.ones((N, N), dtype=bool)
    rw = row_weights(S, visible, kind=kind, levels=levels, window=window, interp=interp, flush=flush,
                     extrema=extrema)
    w = rw["w"]
    l = w.sum(axis=1)
    P = w / l[:, None]
    O = P @ vh
    D = (doh * O).sum(axis=1)                               # D_i = dO_i . O_i
    dP = doh @ vh.T
    dV = P.T @ doh
    if grad == "ste_post":
        dS = np.where(visible, P * (dP - D[:, None]), 0.0)
    else:
        dw = np.where(visible, (dP - D[:, None]) / l[:, None], 0.0)
        m = rw["m"]
        if kind == "exact" or kind == "trunc":              # w = exp(s - m) where kept
            dS = dw * w
            dm = -(dw * w).sum(axis=1)
            dlo = np.zeros(N)
        elif kind == "kint":
            dwdy, dwdD = _weight_partials(rw, kind, levels, interp, flush, visible, window, ste=ste)
            delta = rw["delta"]
            safe = np.where(delta > 0, delta, 1.0)[:, None]
            y = np.where(visible, rw["y"], 0.0)
            dS = dw * dwdy * (-1.0 / safe)                   # y = (m - s) / Delta
            dm = (dw * dwdy / safe).sum(axis=1)
            dD = (dw * (dwdD - dwdy * y / safe)).sum(axis=1)  # total dDelta, y moving with Delta
            if window is None:                                # min-max: Delta = (m - lo) / K
                dm = dm + dD / levels
                dlo = -dD / levels
            else:                                            # window: Delta = W / K is constant
                dlo = np.zeros(N)
        elif kind == "pot" and ste:                          # 2^-e with e := y = (m - s) log2(e)
            e = np.rint(np.where(visible, rw["y"], 0.0))
            g = np.where(visible & (e <= levels - 1), dw * w, 0.0)   # dw/ds = w inside the clip
            dS = g
            dm = -g.sum(axis=1)
            dlo = np.zeros(N)
        else:                                                # pot, uniform: piecewise constant
            dS = np.zeros((N, N))
            dm = np.zeros(N)
            dlo = np.zeros(N)
        if not detached:
            rows = np.arange(N)
            amax = np.argmax(np.where(visible, S, -np.inf), axis=1)
            amin = np.argmin(np.where(visible, S, np.inf), axis=1)
            dS = dS.copy()
            np.add.at(dS, (rows, amax), dm)
            if kind == "kint" and window is None:
                np.add.at(dS, (rows, amin), dlo)
    dQ = sc * (dS @ kh)
    dK = sc * (dS.T @ qh)
    out = {"dQ": dQ, "dK": dK, "dV": dV}
    if detail:
        out.update(P=P, dS=dS)
    return out


def attn_bwd(q, k, v, do, *, causal=False, kind="exact", levels=None, window=None, interp=False, flush=False,
             scale=None, grad="ste_post"):
    """Attention backward over all heads: q, do (B, H, N, d); k, v (B, Hkv, N, d) float64.
    dK and dV of a KV head sum the shares of the query heads that read it."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    group = H // Hkv
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            kv = h // group
            r = head_bwd(q[b, h], k[b, kv], v[b, kv], do[b, h], causal=causal, kind=kind, levels=levels,
                         window=window, interp=interp, flush=flush, scale=scale, grad=grad)
            dQ[b, h] = r["dQ"]
            dK[b, kv] += r["dK"]
            dV[b, kv] += r["dV"]
    return {"dQ": dQ, "dK": dK, "dV": dV}
