"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a private copy of the oracle's source (a
dropped term, a wrong sign, an off-by-one index, a swapped operand, a wrong
head mapping) and checks that at least one independent pin fails on it.  The
real oracle is never modified.
"""
import importlib.util
import json
import math
import os
import sys
import types

import numpy as np
import pytest
import torch

from oracle import scalar

HERE = os.path.dirname(__file__)
SRC = os.path.join(os.path.dirname(HERE), "oracle", "qsa_oracle.py")
GOLDEN = os.path.join(HERE, "golden", "hand_examples.json")

MUTATIONS = {
    "pot_floor_not_rint": ("e = np.rint(np.where(visible, y, 0.0))", "e = np.floor(np.where(visible, y, 0.0))"),
    "pot_anchor_sign": ("y = np.where(visible, (m[:, None] - S) * LOG2E, np.nan)",
                        "y = np.where(visible, (S - m[:, None]) * LOG2E, np.nan)"),
    "pot_no_clip": ("e = np.minimum(e, L - 1)", "e = e"),
    "kint_grid_off_by_one": ("delta = (m - lo) / K", "delta = (m - lo) / (K + 1)"),
    "kint_index_from_lo": ("y = np.where(visible, (m[:, None] - S) / safe[:, None], np.nan)",
                           "y = np.where(visible, (S - lo[:, None]) / safe[:, None], np.nan)"),
    "kint_window_sign": ("lo = (m - window) if window is not None else mn",
                         "lo = (m + window) if window is not None else mn"),
    "interp_swapped": ("w_lin = (1.0 - t) * T[rows, l0] + t * T[rows, l0 + 1]",
                       "w_lin = t * T[rows, l0] + (1.0 - t) * T[rows, l0 + 1]"),
    "exact_sign": ("np.exp(np.where(visible, S - m[:, None], 0.0))", "np.exp(np.where(visible, m[:, None] - S, 0.0))"),
    "causal_off_by_one": ("(cols[None, :] <= r[:, None])", "(cols[None, :] <= r[:, None] + 1)"),
    "no_normalisation": ("O = (w @ vh) / l[:, None]", "O = (w @ vh)"),
    "missing_scale": ("S = sc * (qh[r] @ kh.T)", "S = (qh[r] @ kh.T)"),
    "gqa_wrong_head": ("kv = h // group                                # query head h reads",
                       "kv = h % Hkv                                # query head h reads"),
    "flush_threshold": ("kept = visible & (e <= L - 1)", "kept = visible & (e <= L)"),
    "support_edge_exclusive": ("kept = visible & (m[:, None] - S <= window)", "kept = visible & (m[:, None] - S < window)"),
    "support_sign": ("kept = visible & (m[:, None] - S <= window)", "kept = visible & (S - m[:, None] <= window)"),
    "uniform_takes_exact_weights": ("w = kept.astype(np.float64)",
                                    "w = np.where(kept, np.exp(np.where(kept, S - m[:, None], 0.0)), 0.0)"),
    "running_anchor_not_running": ("A = np.ceil(np.maximum.accumulate(tmax, axis=1))", "A = np.ceil(tmax)"),
    "running_anchor_floor": ("A = np.ceil(np.maximum.accumulate(tmax, axis=1))",
                             "A = np.floor(np.maximum.accumulate(tmax, axis=1))"),
    "running_rescale_sign": ("shift = np.where(visible, Afin[:, None] - Aj, 0.0)",
                             "shift = np.where(visible, Aj - Afin[:, None], 0.0)"),
    "running_no_clip": ("ex = np.minimum(ex, L - 1)", "ex = ex"),
    "running_flush_threshold": ("keep = visible & (ex <= L - 1)", "keep = visible & (ex <= L)"),
    "minmax_flush_applied": ("whose window can end above the row minimum.\n    flush = flush and window is not None",
                             "whose window can end above the row minimum.\n    flush = flush"),
    "trunc_takes_unit_weights": ("w = np.where(kept, np.exp(np.where(kept, S - m[:, None], 0.0)), 0.0)\n        else:",
                                 "w = kept.astype(np.float64)\n        else:"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation target not unique: {name}"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _checks(o):
    """Independent pins; returns True when all pass."""
    rng = np.random.default_rng(3)
    try:
        g = json.load(open(GOLDEN))
        for ex in g["rows"]:
            env = {"exp": math.exp, "log": math.log}
            S = np.array([[float(eval(s, {"__builtins__": {}}, env)) for s in ex["scores"]]])
            rw = o.row_weights(S, np.ones_like(S, bool), kind=ex["kind"], levels=ex["levels"],
                               window=ex.get("window"), interp=ex.get("interp", False), flush=ex.get("flush", False))
            want = [float(eval(w, {"__builtins__": {}}, env)) for w in ex["weights"]]
            np.testing.assert_allclose(rw["w"][0], want, rtol=1e-13)
        for causal in (False, True):
            q = rng.standard_normal((1, 4, 12, 8)) * 1.5
            k = rng.standard_normal((1, 2, 12, 8)) * 1.5
            v = rng.standard_normal((1, 2, 12, 8))
            r = o.attn_fwd(q, k, v, causal=causal, kind="exact")
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal,
                enable_gqa=True).numpy()
            np.testing.assert_allclose(r["O"], ref, atol=1e-12)
            for var in (dict(kind="pot", levels=4), dict(kind="pot", levels=3, flush=True),
                        dict(kind="kint", levels=4), dict(kind="kint", levels=3, window=2.0),
                        dict(kind="kint", levels=3, interp=True)):
                for s in range(3):
                    qq = rng.standard_normal((1, 1, 6, 4)) * 1.7
                    kk = rng.standard_normal((1, 1, 6, 4)) * 1.7
                    vv = rng.standard_normal((1, 1, 6, 4))
                    r = o.attn_fwd(qq, kk, vv, causal=causal, **var)
                    rs = scalar.attention(qq[0, 0].tolist(), kk[0, 0].tolist(), vv[0, 0].tolist(), causal=causal, **var)
                    np.testing.assert_allclose(r["O"][0, 0], np.array(rs), atol=1e-12)
        # single-pass power-of-two weights: the stateful scalar simulation, several tiles per row
        for var in (dict(levels=2), dict(levels=3), dict(levels=3, flush=True), dict(levels=2, flush=True)):
            for causal in (False, True):
                for tile in (2, 3):
                    qq = rng.standard_normal((1, 1, 9, 4)) * 2.5
                    kk = rng.standard_normal((1, 1, 9, 4)) * 2.5
                    vv = rng.standard_normal((1, 1, 9, 4))
                    r = o.head_rows(qq[0, 0], kk[0, 0], vv[0, 0], causal=causal, kind="pot_running", tile=tile,
                                    **var)
                    rs = scalar.attention(qq[0, 0].tolist(), kk[0, 0].tolist(), vv[0, 0].tolist(), causal=causal,
                                          kind="pot_running", tile=tile, **var)
                    np.testing.assert_allclose(r["O"], np.array(rs), atol=1e-12)
        # sensitivity operators: the inclusive support edge on integer scores, then the closed forms
        qe = np.array([[[[1.0, 0.0]]]])
        ke = np.array([[[[5.0, 0.0], [3.0, 0.0], [2.0, 0.0], [4.0, 0.0]]]])
        ve = np.array([[[[1.0, 0.0], [0.0, 1.0], [7.0, 7.0], [0.0, 0.0]]]])
        for kind, w in (("trunc", [1.0, math.exp(-2.0), 0.0, math.exp(-1.0)]), ("uniform", [1.0, 1.0, 0.0, 1.0])):
            r = o.attn_fwd(qe, ke, ve, kind=kind, window=2.0, scale=1.0)
            w = np.array(w)
            np.testing.assert_allclose(r["O"][0, 0, 0], (w @ ve[0, 0]) / w.sum(), atol=1e-15)
        q = rng.standard_normal((1, 1, 10, 8)) * 1.3
        k = rng.standard_normal((1, 1, 10, 8)) * 1.3
        v = rng.standard_normal((1, 1, 10, 8))
        S = (q[0, 0] @ k[0, 0].T) / math.sqrt(8)
        P = torch.softmax(torch.from_numpy(S), dim=-1).numpy()
        for W in (0.3, 1.2):
            keep = S >= S.max(axis=1, keepdims=True) - W
            ru = o.attn_fwd(q, k, v, kind="uniform", window=W)
            np.testing.assert_allclose(ru["O"][0, 0], (keep @ v[0, 0]) / keep.sum(1, keepdims=True), atol=1e-13)
            rt = o.attn_fwd(q, k, v, kind="trunc", window=W)
            p = np.where(keep, P, 0.0)
            np.testing.assert_allclose(rt["O"][0, 0], (p @ v[0, 0]) / p.sum(1, keepdims=True), atol=1e-13)
    except Exception:      # a failed assertion or a crash: either way the pins notice
        return False
    return True


def test_unmutated_oracle_passes_the_checks():
    import oracle.qsa_oracle as real
    assert _checks(real)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    assert not _checks(_mutant(name)), f"planted mistake {name} went unnoticed"
