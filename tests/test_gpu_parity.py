"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Inputs are the seeded synthetic workloads (quantized_softmax_approximation_amd
.inputs); sizes run from the tiny fp32 case to the full long-context GQA
workload (sampled row windows there), plus ragged tails, degenerate rows and
the maximum sequence length.
"""
import numpy as np
import pytest
import torch

import quantized_softmax_approximation_amd as qsa
from quantized_softmax_approximation_amd import inputs as qin
from tests import gpu_cases as gc
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qsa.lib()
    yield


# ---------------------------------------------------------------- tiny (fp32)

TINY_VARS = [gc.EXACT, gc.EXACT_ANCH, gc.KH4, gc.POT8, gc.POT4F, gc.KI4, gc.KH4W, gc.KI4W, gc.KH4WF, gc.KI4WF,
             gc.TRUNC2, gc.UNIF2]


@pytest.mark.parametrize("var", TINY_VARS, ids=gc.name)
def test_tiny_fp32(var):
    gc.run_parity(qin.WORKLOADS["tiny"], var)


# ---------------------------------------------------------------- GPT-2 shaped (bf16, causal)

GPT2_VARS = [gc.EXACT, gc.POT8, gc.KH4, gc.KH16, gc.KI4, gc.KI16, gc.KH4W, gc.KH16W, gc.KI4W, gc.KI16W, gc.TRUNC2,
             gc.UNIF2, gc.KH4F, gc.KI4F]


@pytest.fixture(scope="module")
def gpt2():
    wl = qin.WORKLOADS["gpt2"]
    x = qin.make_inputs(wl)
    return wl, x, gc.to_gpu(x), gc.decoded(x)


@pytest.mark.parametrize("var", GPT2_VARS, ids=gc.name)
def test_gpt2(gpt2, var):
    wl, x, dev_t, f64 = gpt2
    heads = [(0, 0), (3, 5), (7, 11)]
    gc.run_parity(wl, var, heads=heads, x=x, dev_t=dev_t, f64=f64)


@pytest.fixture(scope="module")
def gpt2_wide():
    # d = 64 on a grid large enough for the pre-pass with two 32-row blocks per wave
    # (B H N/256 >= 512; the GPT-2 shape runs one block per wave)
    wl = qin.custom("gpt2_wide", B=2, H=64, Hkv=64, N=1024, d=64, dtype="bf16", causal=True, sigma_qk=1.5, seed=1012)
    x = qin.make_inputs(wl)
    return wl, x, gc.to_gpu(x), gc.decoded(x)


@pytest.mark.parametrize("var", [gc.EXACT_ANCH, gc.POT8, gc.KH4, gc.KI4, gc.KI16W, gc.KH4F, gc.TRUNC2], ids=gc.name)
def test_gpt2_wide_prepass(gpt2_wide, var):
    wl, x, dev_t, f64 = gpt2_wide
    gc.run_parity(wl, var, heads=[(0, 0), (1, 63)], windows=gc.sample_windows(wl.N, n=3, seed=21), x=x,
                  dev_t=dev_t, f64=f64)


# ---------------------------------------------------------------- 2K with attention sink (bf16, d=128)

@pytest.fixture(scope="module")
def pot2k():
    wl = qin.WORKLOADS["pot2k"]
    x = qin.make_inputs(wl)
    return wl, x, gc.to_gpu(x), gc.decoded(x)


@pytest.mark.parametrize("var", [gc.EXACT, gc.EXACT_ANCH, gc.POT8, gc.POT16, gc.KH16W], ids=gc.name)
def test_pot2k(pot2k, var):
    wl, x, dev_t, f64 = pot2k
    gc.run_parity(wl, var, heads=[(0, 0), (2, 17), (3, 31)], x=x, dev_t=dev_t, f64=f64)


# ---------------------------------------------------------------- long-context GQA (bf16, 16K, sampled rows)

@pytest.fixture(scope="module")
def gqa16k():
    wl = qin.WORKLOADS["gqa16k"]
    x = qin.make_inputs(wl)
    return wl, x, gc.to_gpu(x), gc.decoded(x)


@pytest.mark.parametrize("var", [gc.EXACT, gc.EXACT_ANCH, gc.POT8, gc.POT16, gc.KH4, gc.KH16, gc.KI4, gc.KI16, gc.KH4W,
                                 gc.KH16W, gc.KI4W, gc.KI16W, gc.TRUNC2, gc.UNIF2], ids=gc.name)
def test_gqa16k_sampled(gqa16k, var):
    wl, x, dev_t, f64 = gqa16k
    heads = [(0, 0), (0, 9), (0, 63)]
    gc.run_parity(wl, var, heads=heads, windows=gc.sample_windows(wl.N, n=4, seed=5), x=x, dev_t=dev_t, f64=f64)


# ---------------------------------------------------------------- ragged tails, tiny N, GQA, d

EDGE_N = [1, 2, 17, 63, 64, 65, 127, 129, 200, 255, 257, 333]


@pytest.mark.parametrize("N", EDGE_N)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged(N, d, causal):
    wl = qin.custom(f"ragged{N}", B=2, H=4, Hkv=2, N=N, d=d, dtype="bf16", causal=causal, sigma_qk=1.5, seed=N + d)
    x = qin.make_inputs(wl)
    dev_t, f64 = gc.to_gpu(x), gc.decoded(x)
    for var in (gc.EXACT, gc.EXACT_ANCH, gc.POT8, gc.POT4F, gc.KH4, gc.KI16, gc.KH4WF, gc.KI4WF, gc.TRUNC2, gc.UNIF2,
                gc.KH4F):
        gc.run_parity(wl, var, x=x, dev_t=dev_t, f64=f64, verbose=False)


# ---------------------------------------------------------------- the 8K shape in bf16 (the stricter 60 % reading)

@pytest.fixture(scope="module")
def bf16_8k():
    wl = qin.WORKLOADS["fp8_8k"].replace(dtype="bf16")
    x = qin.make_inputs(wl)
    return wl, x, gc.to_gpu(x), gc.decoded(x)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("var", [gc.EXACT, gc.EXACT_ANCH, gc.POT16, gc.POT8, gc.POTR16, gc.KH16W, gc.KI16W, gc.KH16,
                                 gc.TRUNC2], ids=gc.name)
def test_bf16_8k_sampled(bf16_8k, var, causal):
    # the launch bench.py times at B 1, H 32, N 8192, d 128 with bf16 inputs; seeded 64-row windows
    # (always the first and the last 64 rows) of three heads
    wl, x, dev_t, f64 = bf16_8k
    gc.run_parity(wl.replace(causal=causal), var, heads=[(0, 0), (0, 13), (0, 31)],
                  windows=gc.sample_windows(wl.N, n=3, seed=12), x=x, dev_t=dev_t, f64=f64)


@pytest.mark.parametrize("N", [1, 5, 64, 100, 129, 200, 257])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_fp32(N, causal):
    # fp32 kernel: 128-row workgroups, 64-key tiles; N = 129 and 257 start a new workgroup
    wl = qin.custom(f"f32_{N}", B=1, H=2, Hkv=1, N=N, d=128, dtype="f32", causal=causal, sigma_qk=1.2, seed=N)
    x = qin.make_inputs(wl)
    for var in (gc.EXACT, gc.EXACT_ANCH, gc.POT8, gc.KH4, gc.KI4W, gc.TRUNC2, gc.UNIF2, gc.KH4F):
        gc.run_parity(wl, var, x=x, verbose=False)


def test_large_levels_and_windows():
    wl = qin.custom("levels", B=1, H=2, N=300, d=64, dtype="bf16", causal=False, sigma_qk=2.0, seed=3)
    x = qin.make_inputs(wl)
    dev_t, f64 = gc.to_gpu(x), gc.decoded(x)
    for var in (dict(kind="pot", levels=64), dict(kind="pot", levels=1), dict(kind="pot", levels=2, flush=True),
                dict(kind="kint", levels=64), dict(kind="kint", levels=64, interp=True),
                dict(kind="kint", levels=1), dict(kind="kint", levels=64, window=0.5, flush=True),
                dict(kind="kint", levels=2, window=40.0, interp=True)):
        gc.run_parity(wl, var, x=x, dev_t=dev_t, f64=f64)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_very_wide_score_range(dtype):
    # logit std ~6400: score gaps far beyond 2^15 log2 units, where a 16-bit exponent field
    # would wrap; every weight past the clip must still be the last level (or 0 with flush)
    wl = qin.custom(f"wide_{dtype}", B=1, H=2, N=200, d=128, dtype=dtype, causal=True, sigma_qk=80.0, seed=11)
    x = qin.make_inputs(wl)
    dev_t, f64 = gc.to_gpu(x), gc.decoded(x)
    for var in (gc.POT8, gc.POT16, gc.POT4F, gc.EXACT_ANCH, gc.KH4):
        gc.run_parity(wl, var, x=x, dev_t=dev_t, f64=f64)


def test_degenerate_rows_all_scores_equal():
    # q = 0: every score is 0; min-max grids have zero width, all weights 1
    wl = qin.custom("flat", B=1, H=2, N=130, d=64, dtype="bf16", causal=True, seed=4)
    x = qin.make_inputs(wl)
    x.q.zero_()
    for var in (gc.EXACT, gc.POT8, gc.KH4, gc.KI4, gc.KH4W):
        rep = gc.run_parity(wl, var, x=x, verbose=False)
        assert rep.max_rel_err < 1e-2


# ---------------------------------------------------------------- maximum sequence length

@pytest.mark.parametrize("var", [gc.POT8, gc.EXACT], ids=gc.name)
def test_max_sequence_length(var):
    N = 1 << 20
    wl = qin.custom("maxN", B=1, H=1, N=N, d=64, dtype="bf16", causal=True, sigma_qk=1.5, seed=11)
    x = qin.make_inputs(wl)
    gc.run_parity(wl, var, x=x, windows=[(0, 16), (N // 2 - 7, 16), (N - 16, 16)])


# ---------------------------------------------------------------- properties

def test_row_stats_match_oracle():
    import oracle
    wl = qin.custom("stats", B=1, H=2, N=257, d=128, dtype="bf16", causal=True, sigma_qk=1.5, seed=8)
    x = qin.make_inputs(wl)
    dev_t = gc.to_gpu(x)
    qf, kf, vf = gc.decoded(x)
    for var in (gc.EXACT, gc.POT8, gc.KH4, gc.KH4W, gc.EXACT_ANCH, gc.TRUNC2, gc.UNIF2):
        o, _, st = gc.gpu_call(x, dev_t, var, causal=True, stats=True)
        for h in range(2):
            ref = oracle.head_rows(qf[0, h], kf[0, h], vf[0, h], causal=True, **gc.oracle_var(var))
            m = st["row_max"][0, h].cpu().numpy()
            dstar = 2 * 128 * 2.0 ** -24 / np.sqrt(128) * np.max(np.abs(qf[0, h]) @ np.abs(kf[0, h]).T, axis=1)
            assert np.all(np.abs(m - ref["m"]) <= dstar + 1e-6 * np.abs(ref["m"]))
            l = st["row_sum"][0, h].cpu().numpy()    # online exact: relative to the final running max = m
            parity.compare_head(gc.oracle_var(var), qf[0, h], kf[0, h], vf[0, h], np.arange(257),
                                o[0, h].float().cpu().numpy(), causal=True, l_gpu=l)
            if var["kind"] != "exact":
                lo = st["row_lo"][0, h].cpu().numpy()
                assert np.all(np.abs(lo - ref["lo"]) <= dstar + 1e-5 * (1 + np.abs(ref["lo"])))


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
def test_support_window_extremes(dtype):
    # a window far below the top score gap keeps only the row maximum; one wider than every
    # score range keeps every visible key (truncation = exact softmax, uniform = mean of V)
    d = 128 if dtype != "f32" else 64
    wl = qin.custom(f"support_{dtype}", B=1, H=2, N=150, d=d, dtype=dtype, causal=True, sigma_qk=1.5, seed=21)
    x = qin.make_inputs(wl)
    dev_t, f64 = gc.to_gpu(x), gc.decoded(x)
    for var in (dict(kind="trunc", window=1e-3), dict(kind="uniform", window=1e-3), dict(kind="trunc", window=1e4),
                dict(kind="uniform", window=1e4)):
        gc.run_parity(wl, var, x=x, dev_t=dev_t, f64=f64, verbose=False)


def test_deterministic_and_gqa_equals_repeated_kv():
    wl = qin.custom("det", B=2, H=8, Hkv=2, N=300, d=128, dtype="bf16", causal=True, sigma_qk=1.5, seed=9)
    x = qin.make_inputs(wl)
    q, k, v = gc.to_gpu(x)
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    for var in (gc.EXACT, gc.POT8, gc.KH16W, gc.KI4):
        a = qsa.attn_fwd(q, k, v, causal=True, **var)
        b = qsa.attn_fwd(q, k, v, causal=True, **var)
        c = qsa.attn_fwd(q, kr, vr, causal=True, **var)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        assert torch.equal(a, c)


def test_side_stream_and_out_argument():
    wl = qin.custom("stream", B=1, H=2, N=200, d=64, dtype="bf16", causal=False, seed=10)
    x = qin.make_inputs(wl)
    q, k, v = gc.to_gpu(x)
    ref = qsa.attn_fwd(q, k, v, kind="pot", levels=8)
    s = torch.cuda.Stream()
    out = torch.empty_like(ref)
    with torch.cuda.stream(s):
        qsa.attn_fwd(q, k, v, kind="pot", levels=8, out=out, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(ref, out)


def test_errors_raise_without_launch():
    q = torch.zeros(1, 3, 64, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qsa.QSAError) as e:
        qsa.attn_fwd(q, k, k, kind="pot", levels=8)
    assert e.value.status == qsa.ERR_SHAPE
    q96 = torch.zeros(1, 2, 64, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qsa.QSAError) as e:
        qsa.attn_fwd(q96, q96, q96)
    assert e.value.status == qsa.ERR_UNSUPPORTED
    with pytest.raises(qsa.QSAError) as e:
        qsa.attn_fwd(k, k, k, kind="kint", levels=0)
    assert e.value.status == qsa.ERR_PARAM


# ---------------------------------------------------------------- fp8 e4m3 at 8K (per-tensor descales)

@pytest.fixture(scope="module")
def fp8_8k():
    wl = qin.WORKLOADS["fp8_8k"]
    x = qin.make_inputs(wl)
    return wl, x, gc.to_gpu(x), gc.decoded(x)


FP8_VARS = [gc.EXACT, gc.EXACT_ANCH, gc.POT16, gc.POT8, gc.POT4F, gc.KH16W, gc.KH16, gc.KI16W, gc.KH4WF, gc.TRUNC2,
            gc.UNIF2]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("var", FP8_VARS, ids=gc.name)
def test_fp8_8k_sampled(fp8_8k, var, causal):
    wl, x, dev_t, f64 = fp8_8k
    gc.run_parity(wl.replace(causal=causal), var, heads=[(0, 0), (0, 17), (0, 31)],
                  windows=gc.sample_windows(wl.N, n=3, seed=8), x=x, dev_t=dev_t, f64=f64)


@pytest.mark.parametrize("N", [1, 17, 64, 65, 200, 255, 257, 333])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_ragged(N, d, causal):
    wl = qin.custom(f"fp8_{N}", B=2, H=4, Hkv=2, N=N, d=d, dtype="fp8", causal=causal, sigma_qk=1.5, seed=3 * N + d)
    x = qin.make_inputs(wl)
    dev_t, f64 = gc.to_gpu(x), gc.decoded(x)
    for var in (gc.EXACT, gc.EXACT_ANCH, gc.POT16, gc.POT4F, gc.KH4, gc.KI16, gc.KH4WF, gc.KI4WF, gc.TRUNC2,
                gc.UNIF2, gc.KH4F):
        gc.run_parity(wl, var, x=x, dev_t=dev_t, f64=f64, verbose=False)


# ---------------------------------------------------------------- the score-error model of the protocol

@pytest.mark.parametrize("dtype,d,sigma", [("fp8", 64, 1.0), ("fp8", 128, 1.5), ("fp8", 128, 4.0), ("bf16", 64, 1.5),
                                           ("bf16", 128, 1.5)])
def test_score_error_within_band(dtype, d, sigma):
    # the band of the parity protocol rests on a bound of the score error: fp32 accumulation for
    # bf16 inputs, GAMMA_FP8 for the 8-bit MFMA.  The row maxima (the largest score of each row,
    # as the kernel's MMAs computed it) against exact float64 check that bound on every row.
    import oracle
    wl = qin.custom(f"err_{dtype}{d}", B=1, H=4, N=1024, d=d, dtype=dtype, causal=False, sigma_qk=sigma,
                    seed=40 + d + int(4 * sigma))
    x = qin.make_inputs(wl)
    dev_t = gc.to_gpu(x)
    qf, kf, vf = gc.decoded(x)
    _, _, st = gc.gpu_call(x, dev_t, gc.EXACT_ANCH, causal=False, stats=True)
    sc = 1.0 / np.sqrt(d)
    for h in range(4):
        m_gpu = st["row_max"][0, h].cpu().numpy().astype(np.float64)
        m = (sc * (qf[0, h] @ kf[0, h].T)).max(1)
        A = sc * np.max(np.abs(qf[0, h]) @ np.abs(kf[0, h]).T, axis=1)
        gamma = parity.score_gamma(d, fp8=dtype == "fp8")
        # (+ the rounding of the exported m = M * scale, one fp32 product)
        assert np.all(np.abs(m_gpu - m) <= gamma * A + 2 * parity.U * np.abs(m))


# ---------------------------------------------------------------- seeded random configurations

def _random_cases(n, seed):
    r = np.random.default_rng(seed)
    for i in range(n):
        dtype = r.choice(["bf16", "bf16", "fp8"])
        kind = r.choice(["ki", "ki", "kh", "pot", "potr"])
        if kind == "pot":
            var = dict(kind="pot", levels=int(r.choice([2, 8, 16])), flush=bool(r.random() < 0.3))
        elif kind == "potr":
            var = dict(kind="pot_running", levels=int(r.choice([2, 8, 16])), flush=bool(r.random() < 0.3))
        else:
            var = dict(kind="kint", levels=int(r.choice([1, 2, 4, 7, 16])), interp=bool(kind == "ki"))
            win = r.choice([0.0, 0.0, 2.0, 8.0])
            if win:
                var["window"] = float(win)
                if r.random() < 0.4:
                    var["flush"] = True
        wl = qin.custom(f"rnd{i}", B=1, H=int(r.choice([1, 2, 4])), N=int(r.choice([33, 127, 200, 257, 511, 640])),
                        d=int(r.choice([64, 128])), dtype=str(dtype), causal=bool(r.random() < 0.6),
                        sigma_qk=float(r.choice([0.5, 1.0, 1.5, 2.5, 4.0])), seed=int(r.integers(1 << 20)))
        yield wl, var


@pytest.mark.parametrize("block", range(4))
def test_random_configurations(block):
    # sizes, scales, dtypes, head dimensions and K-interval / PoT parameters drawn at random
    # (seeded), away from the fixed workloads: the interpolation lines, the clamps of the grid
    # coordinate and the single-pass anchors on inputs no other case uses
    for wl, var in _random_cases(25, seed=500 + block):
        gc.run_parity(wl, var, verbose=False)


def _random_wide_cases(n, seed):
    r = np.random.default_rng(seed)
    for i in range(n):
        dtype = str(r.choice(["bf16", "bf16", "fp8", "fp8", "f32"]))
        kind = str(r.choice(["ki", "kh", "pot", "potr", "exact", "exact_anchored", "trunc", "uniform"]))
        top = 16 if dtype == "fp8" else 64
        if kind == "pot":
            var = dict(kind="pot", levels=min(top, int(r.choice([1, 2, 3, 8, 16, 32]))), flush=bool(r.random() < 0.3))
        elif kind == "potr":
            var = dict(kind="pot_running", levels=int(r.choice([2, 5, 8, 16])), flush=bool(r.random() < 0.3))
        elif kind in ("exact", "exact_anchored"):
            var = dict(kind=kind)
        elif kind in ("trunc", "uniform"):
            var = dict(kind=kind, window=float(r.choice([0.5, 2.0, 8.0])))
        else:
            var = dict(kind="kint", levels=min(top, int(r.choice([1, 2, 3, 4, 8, 16, 31]))), interp=kind == "ki")
            win = float(r.choice([0.0, 0.0, 1.0, 4.0, 8.0]))
            if win:
                var["window"] = win
            if r.random() < 0.3:
                var["flush"] = True
        hkv = int(r.choice([1, 2]))
        wl = qin.custom(f"wide{i}", B=int(r.choice([1, 2, 3])), H=hkv * int(r.choice([1, 2, 4, 8])), Hkv=hkv,
                        N=int(r.choice([1, 2, 31, 64, 65, 129, 200, 383, 520])), d=int(r.choice([64, 128])),
                        dtype=dtype, causal=bool(r.random() < 0.5), sigma_qk=float(r.choice([0.5, 1.0, 1.5, 2.5, 4.0])),
                        seed=int(r.integers(1 << 20)), sink=bool(r.random() < 0.2))
        yield wl, var


@pytest.mark.parametrize("block", range(2))
def test_random_configurations_wide(block):
    # every kind and dtype, batch > 1, grouped key/value heads, the attention-sink key, and sizes
    # down to a single key, drawn at random (seeded)
    for wl, var in _random_wide_cases(50, seed=900 + block):
        gc.run_parity(wl, var, verbose=False)
