"""Pins of the oracle's single-pass power-of-two weights (kind ``pot_running``).

The pages do not define the single-pass form (the Rowmax-PoT page names a
max-anchored variant inside FlashAttention-4 without saying how its maximum is
found), so the function is this library's reading and its parity against the
pages is unpinned.  The oracle's closed form is pinned to:
  * a stateful scalar simulation (running integer anchor, rescaling of the weights
    already formed) in exact rationals, over many tile sizes;
  * 2**rint(s log2 e), normalised, when no level is clipped (any number of tiles);
  * Rowmax-PoT anchored at ceil(max s log2 e) when all keys fit one tile;
  * invariance under adding an integer multiple of ln 2 to a row's scores;
  * weights that are exact powers of two, and the final anchor ceil(max s log2 e).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import scalar
from oracle.qsa_oracle import row_weights


def _qkv(N, d=4, sigma=2.0, seed=0):
    r = np.random.default_rng(seed)
    return r.standard_normal((N, d)) * sigma, r.standard_normal((N, d)) * sigma, r.standard_normal((N, d))


@pytest.mark.parametrize("seed", range(12))
def test_closed_form_equals_the_stateful_scalar_simulation(seed):
    r = np.random.default_rng(100 + seed)
    for _ in range(8):
        N = int(r.integers(1, 14))
        tile = int(r.choice([1, 2, 3, 5, 64]))
        L = int(r.integers(2, 6))
        flush = bool(r.integers(0, 2))
        causal = bool(r.integers(0, 2))
        q, k, v = _qkv(N, d=3, sigma=2.0, seed=int(r.integers(1 << 30)))
        ref = scalar.attention(q.tolist(), k.tolist(), v.tolist(), causal=causal, kind="pot_running", levels=L,
                               flush=flush, exact_pot=True, tile=tile)
        got = oracle.head_rows(q, k, v, causal=causal, kind="pot_running", levels=L, flush=flush, tile=tile)["O"]
        np.testing.assert_allclose(got, np.array([[float(x) for x in row] for row in ref]), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_without_clipping_the_weights_are_a_fixed_power_of_two_grid(causal):
    N = 300
    q, k, v = _qkv(N, d=16, sigma=1.6, seed=3)
    S = q @ k.T / 4.0
    vis = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
    g = np.where(vis, np.exp2(np.rint(S / math.log(2.0))), 0.0)
    O = oracle.head_rows(q, k, v, causal=causal, kind="pot_running", levels=400)["O"]
    np.testing.assert_allclose(O, (g @ v) / g.sum(1, keepdims=True), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("flush", [False, True])
def test_one_tile_is_rowmax_pot_at_the_rounded_up_anchor(flush):
    q, k, v = _qkv(60, d=8, sigma=2.0, seed=4)
    S = q @ k.T / math.sqrt(8)
    vis = np.ones_like(S, bool)
    run = row_weights(S, vis, kind="pot_running", levels=4, flush=flush)
    A = np.ceil(S.max(1) / math.log(2.0))
    ref = row_weights(S, vis, kind="pot", levels=4, flush=flush, extrema=(A * math.log(2.0), S.min(1)))
    np.testing.assert_allclose(run["w"], ref["w"], rtol=1e-14)
    np.testing.assert_array_equal(run["A"], A)


def test_integer_multiples_of_ln2_added_to_a_row_change_nothing():
    q, k, _ = _qkv(150, d=8, sigma=2.0, seed=5)
    S = q @ k.T / math.sqrt(8)
    vis = np.tril(np.ones_like(S, bool))
    base = row_weights(S, vis, kind="pot_running", levels=6, flush=True)["w"]
    for n in (-3, 5):
        shifted = row_weights(S + n * math.log(2.0), vis, kind="pot_running", levels=6, flush=True)["w"]
        np.testing.assert_array_equal(shifted, base)


def test_weights_are_powers_of_two_and_the_anchor_is_the_rounded_up_maximum():
    q, k, _ = _qkv(200, d=8, sigma=2.0, seed=6)
    S = q @ k.T / math.sqrt(8)
    vis = np.tril(np.ones_like(S, bool))
    rw = row_weights(S, vis, kind="pot_running", levels=8)
    w = rw["w"][vis]
    lg = np.log2(w)
    np.testing.assert_array_equal(lg, np.rint(lg))
    assert w.max() == 1.0
    np.testing.assert_array_equal(rw["A"], np.ceil(np.where(vis, S, -np.inf).max(1) / math.log(2.0)))


def test_level_count_and_kind_checks():
    S = np.zeros((1, 3))
    with pytest.raises(ValueError):
        row_weights(S, np.ones_like(S, bool), kind="pot_running", levels=1)
    with pytest.raises(ValueError):
        oracle.head_bwd(np.ones((2, 2)), np.ones((2, 2)), np.ones((2, 2)), np.ones((2, 2)), kind="pot_running",
                        levels=4)
    assert oracle.qsa_oracle.ANCHOR_TILE == 64


def test_anchor_override():
    # the anchors an implementation in lower precision may produce enter as an input: the
    # definition's own sequence reproduces the default, and raising every anchor by one moves
    # every exponent up one level (weights halved where the clip does not bind)
    q, k, v = _qkv(150, d=8, sigma=1.0, seed=31)
    base = oracle.head_rows(q, k, v, kind="pot_running", levels=64, detail=True)
    S = (q @ k.T) / math.sqrt(8)
    nt = 3
    tmax = np.stack([(S[:, c * 64:(c + 1) * 64] / math.log(2.0)).max(1) for c in range(nt)], 1)
    A = np.ceil(np.maximum.accumulate(tmax, 1))
    same = oracle.head_rows(q, k, v, kind="pot_running", levels=64, detail=True, anchors=A)
    np.testing.assert_array_equal(same["w"], base["w"])
    up = oracle.head_rows(q, k, v, kind="pot_running", levels=64, detail=True, anchors=A + 1)
    np.testing.assert_array_equal(up["idx"].astype(int), base["idx"].astype(int) + 1)
    np.testing.assert_array_equal(up["w"], base["w"] / 2)
    np.testing.assert_array_equal(up["O"], base["O"])
