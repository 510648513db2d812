"""Shared helpers of the GPU parity tests: run the library through its C ABI on
seeded inputs and compare with the oracle (tests.parity)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import quantized_softmax_approximation_amd as qsa
from quantized_softmax_approximation_amd import inputs as qin
from tests import parity

# Variant specs: keyword arguments of qsa.attn_fwd_ex; the oracle reads
# exact_anchored as exact (the same function, computed another way).
EXACT = dict(kind="exact")
EXACT_ANCH = dict(kind="exact_anchored")
POT8 = dict(kind="pot", levels=8)
POT16 = dict(kind="pot", levels=16)
POT4F = dict(kind="pot", levels=4, flush=True)
KH4 = dict(kind="kint", levels=4)
KH16 = dict(kind="kint", levels=16)
KI4 = dict(kind="kint", levels=4, interp=True)
KI16 = dict(kind="kint", levels=16, interp=True)
KH4W = dict(kind="kint", levels=4, window=8.0)
KH16W = dict(kind="kint", levels=16, window=8.0)
KI4W = dict(kind="kint", levels=4, window=8.0, interp=True)
KI16W = dict(kind="kint", levels=16, window=8.0, interp=True)
KH4WF = dict(kind="kint", levels=4, window=3.0, flush=True)
KI4WF = dict(kind="kint", levels=4, window=3.0, interp=True, flush=True)
KH4F = dict(kind="kint", levels=4, flush=True)          # min-max + flush: the flag removes nothing
KI4F = dict(kind="kint", levels=4, interp=True, flush=True)
POTR8 = dict(kind="pot_running", levels=8)
POTR16 = dict(kind="pot_running", levels=16)
POTR4F = dict(kind="pot_running", levels=4, flush=True)
TRUNC2 = dict(kind="trunc", window=2.0)
UNIF2 = dict(kind="uniform", window=2.0)

ALL = [EXACT, EXACT_ANCH, POT8, POT16, POT4F, KH4, KH16, KI4, KI16, KH4W, KH16W, KI4W, KI16W, KH4WF, KI4WF,
       TRUNC2, UNIF2]


def name(var):
    return "-".join(f"{k}{v}" for k, v in var.items())


def oracle_var(var):
    o = dict(var)
    if o["kind"] == "exact_anchored":
        o["kind"] = "exact"
    return o


def decoded(x: qin.Inputs):
    """Stored tensors -> float64 numpy (descales applied)."""
    out = []
    for t, s in ((x.q, x.q_descale), (x.k, x.k_descale), (x.v, x.v_descale)):
        bits = qin.raw_bits(t)
        if t.dtype == torch.bfloat16:
            f = oracle.decode_bf16(bits)
        elif t.dtype == torch.float8_e4m3fn:
            f = oracle.decode_e4m3fn(bits) * s
        else:
            f = oracle.decode_f32(bits)
        out.append(f.reshape(t.shape))
    return out


def to_gpu(x: qin.Inputs):
    return x.q.cuda(), x.k.cuda(), x.v.cuda()


def gpu_call(x, dev_t, var, *, causal, idx_window=None, stats=False):
    q, k, v = dev_t
    B, H, N, d = q.shape
    grid = None
    r0 = 0
    if idx_window is not None and var["kind"] not in ("exact", "exact_anchored"):
        r0, nr = idx_window
        grid = torch.full((B, H, nr, N), 77, dtype=torch.uint8, device=q.device)
    st = {}
    if stats:
        for key in ("row_max", "row_sum") + (("row_lo",) if var["kind"] not in ("exact", "pot_running") else ()):
            st[key] = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    o = qsa.attn_fwd_ex(q, k, v, causal=causal, q_descale=x.q_descale if q.dtype == torch.float8_e4m3fn else 0.0,
                        k_descale=x.k_descale if q.dtype == torch.float8_e4m3fn else 0.0,
                        v_descale=x.v_descale if q.dtype == torch.float8_e4m3fn else 0.0,
                        grid_idx=grid, idx_row0=r0, **var, **st)
    torch.cuda.synchronize()
    return o, grid, st


def run_parity(wl, var, *, windows=None, heads=None, tol=None, x=None, dev_t=None, f64=None, verbose=True):
    """Launch the full problem once per row window; compare the chosen (b, h).

    Kinds with a grid index run twice per window: once with the index dump (compared
    element by element) and once without it, which is the kernel build a plain call (and
    the benchmark) uses; its O must equal the dump launch's bit for bit, or else match the
    oracle on its own."""
    x = x if x is not None else qin.make_inputs(wl)
    dev_t = dev_t if dev_t is not None else to_gpu(x)
    qf, kf, vf = f64 if f64 is not None else decoded(x)
    B, H, N, d = x.q.shape
    group = H // x.k.shape[1]
    fp8 = x.q.dtype == torch.float8_e4m3fn
    if tol is None:
        tol = 3e-2 if fp8 else 1e-2
    windows = windows or [(0, N)]
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    ovar = oracle_var(var)
    rep = parity.Report()
    for (r0, nr) in windows:
        print(f"[parity] {wl.name} B{B} H{H} N{N} d{d} causal={wl.causal} {name(var)} rows {r0}+{nr}",
              flush=True, file=sys.stderr)
        o, grid, _ = gpu_call(x, dev_t, var, causal=wl.causal, idx_window=(r0, nr))
        o_np = o.float().cpu().numpy()
        g_np = grid.cpu().numpy() if grid is not None else None
        o_plain = None
        if grid is not None:   # the launch without the dump: the build plain calls run
            o2, _, _ = gpu_call(x, dev_t, var, causal=wl.causal)
            if not torch.equal(o2, o):
                o_plain = o2.float().cpu().numpy()
        rows = np.arange(r0, r0 + nr)
        for (b, h) in heads:
            kvh = h // group
            r, _ = parity.compare_head(ovar, qf[b, h], kf[b, kvh], vf[b, kvh], rows, o_np[b, h, r0:r0 + nr],
                                       None if g_np is None else g_np[b, h], causal=wl.causal, tol=tol, fp8=fp8)
            rep.merge(r)
            if o_plain is not None:
                parity.compare_head(ovar, qf[b, h], kf[b, kvh], vf[b, kvh], rows, o_plain[b, h, r0:r0 + nr], None,
                                    causal=wl.causal, tol=tol, fp8=fp8)
        rep.plain_differs += int(o_plain is not None)
    if verbose:
        print(f"[parity] {name(var)}: rows={rep.rows} agree={rep.idx_agree:.6f} disagree={rep.idx_disagree} "
              f"amb_rows={rep.amb_rows} anchor_amb_rows={rep.anchor_amb_rows} max_rel_err={rep.max_rel_err:.3e} "
              f"plain_launch_differs={rep.plain_differs}", flush=True, file=sys.stderr)
    return rep


def sample_windows(N, n=8, width=64, seed=0):
    """Seeded row windows: always rows 0..width-1 and the last width rows."""
    width = min(width, N)
    r = np.random.default_rng(seed)
    starts = {0, N - width}
    while len(starts) < min(n, max(1, N // width)):
        starts.add(int(r.integers(0, N - width + 1)))
    return sorted((s, width) for s in starts)
