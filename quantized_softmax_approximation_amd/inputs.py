"""Seeded synthetic inputs for the quantized-softmax attention forward.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests.  It draws random numbers, scales them and casts them to the
storage dtype; it holds none of the attention arithmetic (no scores, no
weights, no normalisation).

Workloads (shapes and value distributions) follow the settings the pages
describe for the method: a GPT-2-small-shaped pretraining attention (124M
parameters, K-interval paper, abstract), a 2K BF16 path, FP8 forward at 8K
(causal and non-causal) and causal 16K (Rowmax-PoT paper, abstract).  The
models and datasets behind those runs are not available, so seeded Gaussian
tensors of the same shapes stand in for them.

Recipe (identical bytes go to the GPU and to the oracle):
  * generator ``numpy.random.Generator(PCG64(seed))``, draw order Q, K, V,
    each ``standard_normal`` in float32 of shape ``[B,H,N,d]`` (K, V:
    ``[B,Hkv,N,d]``), multiplied by the config's sigma in float32;
  * the attention-sink workload sets feature ``d-1`` of every query to sigma
    and adds ``6*sqrt(d)/sigma`` to feature ``d-1`` of key 0, which adds 6 to
    the scaled score of key 0 in every row (before rounding to bf16);
  * cast on the CPU: bf16 by round-to-nearest-even (torch), fp8 e4m3fn by a
    per-tensor scale ``amax/448`` (values divided by it, clamped to +-448,
    rounded by torch), the scale returned as the tensor's descale.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

FP8_E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    dtype: str          # "f32" | "bf16" | "fp8"
    causal: bool
    sigma_qk: float     # per-coordinate std of Q and K
    seed: int
    sink: bool = False  # attention-sink key 0 (+6 on every row's score)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the method is evaluated on (shapes, distributions).
WORKLOADS = {
    # tiny fp32 case the oracle finishes in well under a second
    "tiny": Workload("tiny", 1, 2, 2, 256, 64, "f32", False, 1.0, 1001),
    # GPT-2-small shaped pretraining attention, logit std 2.25
    "gpt2": Workload("gpt2", 8, 12, 12, 1024, 64, "bf16", True, 1.5, 1002),
    # 2K bf16, logit std 3 plus an attention-sink key
    "pot2k": Workload("pot2k", 4, 32, 32, 2048, 128, "bf16", True, math.sqrt(3.0), 1003, sink=True),
    # fp8 e4m3 at 8K, non-causal (the causal run uses the same tensors)
    "fp8_8k": Workload("fp8_8k", 1, 32, 32, 8192, 128, "fp8", False, 1.5, 1004),
    # long-context GQA 64/8 at 16K, logit std 4
    "gqa16k": Workload("gqa16k", 1, 64, 8, 16384, 128, "bf16", True, 2.0, 1005),
}


@dataclasses.dataclass
class Inputs:
    """Stored tensors (CPU) plus per-tensor descales (1.0 unless fp8)."""
    wl: Workload
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    q_descale: float = 1.0
    k_descale: float = 1.0
    v_descale: float = 1.0


def _draw(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def _to_fp8(x: np.ndarray):
    amax = float(np.max(np.abs(x)))
    scale = amax / FP8_E4M3_MAX if amax > 0 else 1.0
    y = torch.from_numpy(x / np.float32(scale)).clamp_(-FP8_E4M3_MAX, FP8_E4M3_MAX)
    return y.to(torch.float8_e4m3fn), float(np.float32(scale))


def make_inputs(wl: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw Q, K, V for workload ``wl`` (CPU tensors in the stored dtype)."""
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    B, H, Hkv, N, d = wl.B, wl.H, wl.Hkv, wl.N, wl.d
    q = _draw(rng, (B, H, N, d), wl.sigma_qk)
    k = _draw(rng, (B, Hkv, N, d), wl.sigma_qk)
    v = _draw(rng, (B, Hkv, N, d), 1.0)
    if wl.sink:
        s = np.float32(wl.sigma_qk)
        q[..., d - 1] = s
        k[:, :, 0, d - 1] += np.float32(6.0 * math.sqrt(d)) / s
    if wl.dtype == "f32":
        return Inputs(wl, torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v))
    if wl.dtype == "bf16":
        return Inputs(wl, *(torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v)))
    if wl.dtype == "fp8":
        (q8, qs), (k8, ks), (v8, vs) = (_to_fp8(x) for x in (q, k, v))
        return Inputs(wl, q8, k8, v8, qs, ks, vs)
    raise ValueError(f"unknown dtype {wl.dtype!r}")


def make_dout(wl: Workload, seed: Optional[int] = None) -> torch.Tensor:
    """Output gradient dO for workload ``wl``: ``standard_normal`` float32 of shape
    [B,H,N,d] from ``PCG64(seed)`` (default: the workload's seed + 1), cast to the
    stored dtype (float32 or bf16)."""
    rng = np.random.Generator(np.random.PCG64(wl.seed + 1 if seed is None else seed))
    g = torch.from_numpy(_draw(rng, (wl.B, wl.H, wl.N, wl.d), 1.0))
    if wl.dtype == "f32":
        return g
    if wl.dtype == "bf16":
        return g.to(torch.bfloat16)
    raise ValueError(f"the backward takes f32 or bf16, not {wl.dtype!r}")


def custom(name="custom", *, B=1, H=1, Hkv=None, N=64, d=64, dtype="bf16", causal=False,
           sigma_qk=1.0, seed=7, sink=False) -> Workload:
    """A workload with explicit sizes (tests: ragged tails, edge cases)."""
    return Workload(name, B, H, H if Hkv is None else Hkv, N, d, dtype, causal, sigma_qk, seed, sink)


def raw_bits(t: torch.Tensor) -> np.ndarray:
    """The stored bytes of a CPU tensor as an unsigned-integer numpy array."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.contiguous().view(torch.uint8).numpy()
    if t.dtype == torch.float32:
        return t.contiguous().numpy().view(np.uint32)
    raise TypeError(t.dtype)
