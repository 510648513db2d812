"""The GPU comparison protocol accepts a correct fp32 computation and rejects a wrong one.

A float32 emulation of the kernels' arithmetic (fp32 scores accumulated in a
different order, fp32 row constants, the same rounding steps) stands in for
the GPU here.  It must pass `parity.compare_head` with every index
disagreement inside the fp32 edge band, while a result with one wrong grid
index outside the band, or a perturbed O, must fail.
"""
import math

import numpy as np
import pytest

from tests import parity

F = np.float32


def emulate(var, q, k, v, causal, anchor_override=()):
    """fp32 emulation of one head: scores in float32 (BLAS order), weights via fp32 ops.
    anchor_override (pot_running): (row, tile, value) entries that replace the rounded-up
    maximum of that tile before the running maximum is taken."""
    q32, k32, v32 = q.astype(F), k.astype(F), v.astype(F)
    N, d = q.shape
    sc = F(1.0 / math.sqrt(d))
    acc = (q32 @ k32.T).astype(F)                               # raw dot products
    vis = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
    M = np.where(vis, acc, -np.inf).max(1).astype(F)
    MN = np.where(vis, acc, np.inf).min(1).astype(F)
    kind = var["kind"]
    idx = np.full((N, N), 255, np.uint8)
    if kind == "exact":
        c = F(sc * F(1.4426950408889634))
        w = np.exp2((acc * c - M[:, None] * c).astype(F))
        idx[vis] = 0
    elif kind == "pot_running":
        # anchor after each 64-key tile: ceil of the fp32 product (running raw max) * c; the
        # exponent rounds A - acc c exactly once (one FMA), as the kernels do
        L = var["levels"]
        c = F(sc * F(1.4426950408889634))
        raw = np.where(vis, acc, -np.inf).astype(F)
        nt = (N + 63) // 64
        tm = np.stack([raw[:, j * 64:(j + 1) * 64].max(1) for j in range(nt)], 1)
        a = np.ceil((tm * c).astype(F)).astype(np.float64)
        for (i, j, val) in anchor_override:
            a[i, j] = val
        A = np.maximum.accumulate(a, 1)
        Aj = np.repeat(A, 64, axis=1)[:, :N]
        e = np.rint(Aj - acc.astype(np.float64) * np.float64(c))
        shift = A[:, -1:] - Aj
        if var.get("flush"):
            kept = e <= L - 1
            w = np.where(kept, np.exp2(-np.minimum(e + shift, 126)), 0).astype(F)
            idx = np.where(kept, e, 254).astype(np.uint8)
        else:
            e = np.clip(e, 0, L - 1)
            w = np.exp2(-(e + shift)).astype(F)
            idx = e.astype(np.uint8)
        w = np.where(vis, w, 0).astype(F)
    elif kind == "pot":
        L = var["levels"]
        c = F(sc * F(1.4426950408889634))
        y = (M[:, None] * c - acc * c).astype(F)
        e = np.rint(y)
        if var.get("flush"):
            kept = e <= L - 1
            w = np.where(kept, np.exp2(-np.minimum(e, 126)), 0).astype(F)
            idx = np.where(kept, e, 254).astype(np.uint8)
        else:
            e = np.clip(e, 0, L - 1)
            w = np.exp2(-e).astype(F)
            idx = e.astype(np.uint8)
    else:
        K = var["levels"]
        if var.get("window") is not None:
            W = F(var["window"])
            c = np.full(N, F(sc * F(K) / W), F)
            delta = np.full(N, F(W / F(K)), F)
        else:
            rng = (M - MN).astype(F)
            c = np.where(rng > 0, F(K) / np.where(rng > 0, rng, 1), 0).astype(F)
            delta = (rng * sc / F(K)).astype(F)
        T = np.exp2(-np.arange(K + 1)[None, :] * (delta[:, None] * F(1.4426950408889634))).astype(F)
        y = (M[:, None] * c[:, None] - acc * c[:, None]).astype(F)
        rows = np.arange(N)[:, None]
        if not var.get("interp"):
            l = np.clip(np.rint(y), 0, K).astype(np.int64)
            w = T[rows, l]
            idx = l.astype(np.uint8)
        else:
            yc = np.clip(y, 0, K)
            l = np.floor(yc).astype(np.int64)
            t = (yc - l).astype(F)
            Tn = np.concatenate([T, T[:, -1:]], axis=1)
            w = (T[rows, l] + t * (Tn[rows, l + 1] - T[rows, l])).astype(F)
            idx = l.astype(np.uint8)
        if var.get("flush"):
            w = np.where(y > K, 0, w).astype(F)
            idx = np.where(y > K, 254, idx).astype(np.uint8)
    w = np.where(vis, w, 0).astype(F)
    idx = np.where(vis, idx, 255).astype(np.uint8)
    O = (w @ v32) / w.sum(1, keepdims=True)
    return O.astype(F), idx


VARS = [dict(kind="exact"), dict(kind="pot", levels=8), dict(kind="pot", levels=4, flush=True),
        dict(kind="pot_running", levels=8), dict(kind="pot_running", levels=4, flush=True),
        dict(kind="pot_running", levels=16),
        dict(kind="kint", levels=4), dict(kind="kint", levels=16, interp=True),
        dict(kind="kint", levels=4, window=8.0), dict(kind="kint", levels=16, window=8.0, flush=True),
        dict(kind="kint", levels=4, window=3.0, interp=True, flush=True)]


@pytest.mark.parametrize("var", VARS, ids=lambda v: "-".join(f"{k}{v[k]}" for k in v))
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_emulation_passes(var, causal):
    r = np.random.default_rng(5)
    N, d = 300, 64
    q = r.standard_normal((N, d)) * 1.5
    k = r.standard_normal((N, d)) * 1.5
    v = r.standard_normal((N, d))
    O, idx = emulate(var, q, k, v, causal)
    rep, _ = parity.compare_head(var, q, k, v, np.arange(N), O, idx, causal=causal, tol=1e-4)
    assert rep.idx_bad == 0
    if not var.get("interp"):
        assert rep.idx_agree >= 0.999


def test_wrong_index_outside_band_fails():
    r = np.random.default_rng(6)
    N, d = 128, 64
    q, k, v = r.standard_normal((N, d)) * 1.5, r.standard_normal((N, d)) * 1.5, r.standard_normal((N, d))
    var = dict(kind="pot", levels=8)
    O, idx = emulate(var, q, k, v, False)
    ref_rep, ref = parity.compare_head(var, q, k, v, np.arange(N), O, idx, causal=False, tol=1e-4)
    y = ref["y"]
    i, j = np.unravel_index(np.argmin(np.abs(y - np.floor(y) - 0.5) * -1 + (idx == 7) * 9), y.shape)
    bad = idx.copy()
    bad[i, j] = (bad[i, j] + 1) % 7                               # a flip far from any edge
    with pytest.raises(AssertionError):
        parity.compare_head(var, q, k, v, np.arange(N), O, bad, causal=False, tol=1e-4)
    O2 = O.copy()
    O2[3] *= 1.05
    with pytest.raises(AssertionError):
        parity.compare_head(var, q, k, v, np.arange(N), O2, idx, causal=False, tol=1e-2)


def test_fp8_band_still_catches_a_wrong_index():
    # the 8-bit MFMA's band (gamma 2^-12) is still far narrower than the distance of a
    # planted flip from its edge
    r = np.random.default_rng(9)
    N, d = 128, 64
    q, k, v = r.standard_normal((N, d)) * 1.5, r.standard_normal((N, d)) * 1.5, r.standard_normal((N, d))
    var = dict(kind="pot", levels=8)
    O, idx = emulate(var, q, k, v, False)
    rep, ref = parity.compare_head(var, q, k, v, np.arange(N), O, idx, causal=False, tol=1e-4, fp8=True)
    assert rep.idx_bad == 0 and rep.idx_agree >= 0.999
    y = ref["y"]
    far = (np.abs(y - np.floor(y) - 0.5) > 0.25) & (idx < 7)
    i, j = np.argwhere(far)[0]
    bad = idx.copy()
    bad[i, j] += 1
    with pytest.raises(AssertionError):
        parity.compare_head(var, q, k, v, np.arange(N), O, bad, causal=False, tol=1e-4, fp8=True)
    assert parity.score_gamma(64, fp8=True) == 2.0 ** -12 and parity.score_gamma(64) == 128 * 2.0 ** -24


def _on_integer_anchor(N=150, d=64, row=100, key=10, n=3, seed=8):
    """Inputs whose row `row` has its largest score of key tile 0 at key `key`, equal to
    n ln 2 up to float64 rounding: that tile's anchor is n or n + 1 in fp32."""
    r = np.random.default_rng(seed)
    q, k, v = r.standard_normal((N, d)) * 0.5, r.standard_normal((N, d)) * 0.5, r.standard_normal((N, d))
    sc = 1.0 / math.sqrt(d)
    k[key] = q[row] * (n * math.log(2.0) / (sc * (q[row] @ q[row])))
    return q, k, v


def test_single_pass_ambiguous_anchor_either_way_passes():
    q, k, v = _on_integer_anchor()
    var = dict(kind="pot_running", levels=8)
    cands = parity.anchor_candidates(var, q, k, np.arange(150), causal=False)
    assert len(cands[100]) == 2 and {c[0] for c in cands[100]} == {3.0, 4.0}
    for val in (3.0, 4.0):   # the emulation takes either rounding of the tile maximum
        O, idx = emulate(var, q, k, v, False, anchor_override=[(100, 0, val)])
        rep, _ = parity.compare_head(var, q, k, v, np.arange(150), O, idx, causal=False, tol=1e-4)
        assert rep.idx_bad == 0 and rep.anchor_amb_rows >= 1


def test_single_pass_wrong_anchor_fails():
    q, k, v = _on_integer_anchor()
    var = dict(kind="pot_running", levels=8)
    O, idx = emulate(var, q, k, v, False)
    A0 = np.ceil(np.max(q[7] @ k[:64].T) / 8.0 / math.log(2.0))
    cands = parity.anchor_candidates(var, q, k, np.arange(150), causal=False)
    assert len(cands[7]) == 1                    # row 7's anchors are decided
    O2, idx2 = emulate(var, q, k, v, False, anchor_override=[(7, 0, A0 + 1)])
    with pytest.raises(AssertionError):
        parity.compare_head(var, q, k, v, np.arange(150), O2, idx2, causal=False, tol=1e-4)


def test_agreement_floor_allows_one_element_in_a_small_head():
    # 20 x 20 visible elements (below the 1000 at which 0.1 % is one element): rows 0 and 1 each
    # get a key on the PoT edge y = 1/2 (inside the band), where both indices are correct.  One
    # flipped there passes; two fail the floor, although each lies in the band.
    r = np.random.default_rng(11)
    N, d = 20, 64
    q, k, v = r.standard_normal((N, d)), r.standard_normal((N, d)), r.standard_normal((N, d))
    sc = 1.0 / math.sqrt(d)
    for i, j in ((0, 5), (1, 6)):
        s = sc * (q[i] @ k.T)
        m = np.max(np.delete(s, j))
        t = m - 0.5 * math.log(2.0)                    # the score that puts key j on y = 1/2
        k[j] += (t - s[j]) / (sc * (q[i] @ q[i])) * q[i]
    var = dict(kind="pot", levels=8)
    O, _ = emulate(var, q, k, v, False)
    _, ref = parity.compare_head(var, q, k, v, np.arange(N), O, None, causal=False, tol=1e-4)
    assert abs(ref["y"][0, 5] - 0.5) < 1e-12 and abs(ref["y"][1, 6] - 0.5) < 1e-12
    one = ref["idx"].astype(np.uint8)                  # the oracle's choices at both ties ...
    one[0, 5] ^= 1                                      # ... and the other one at (0, 5)
    rep, _ = parity.compare_head(var, q, k, v, np.arange(N), O, one, causal=False, tol=1e-4)
    assert rep.idx_disagree == 1 and rep.idx_bad == 0
    two = one.copy()
    two[1, 6] ^= 1
    with pytest.raises(AssertionError, match="index agreement"):
        parity.compare_head(var, q, k, v, np.arange(N), O, two, causal=False, tol=1e-4)
