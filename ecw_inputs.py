"""Seeded synthetic workloads for the fused entropy-decode + batch-1 GEMV path.

This module only draws random tensors in the shapes and value statistics of the
workloads that the method's pages measure on (Llama-3.1-8B-shaped linear layers;
BF16 weights; FP8 E4M3 weights quantised per row).  It holds none of the method's
arithmetic: no entropy coding, no table building, no reconstruction and no GEMV.
Both the CPU oracle and the GPU path take their inputs from here.

Recipes (numpy PCG64 ``default_rng``):

* 16-level Gaussian codes: q = clip(rint(N(0, 2^2)), -8, 7); fp16 row scales
  0.01 * U[0.5, 1.5); x ~ N(0, 1) in fp16.  Draw order: codes, scales, x.
* 16-level Laplacian codes: q = clip(rint(Laplace(0, b)), -8, 7) with b chosen so
  the analytic entropy of the clamped discretised Laplacian is 2.2 bits; fp16 row
  scales (0.02 / sd(q)) * U[0.5, 1.5); x ~ N(0, 1) in fp16.
* BF16 weights: N(0, 0.02^2) drawn in fp64, rounded to fp32 then to bf16 (RNE);
  x ~ N(0, 1) in bf16.
* FP8 E4M3 weights: N(0, 0.02^2); row scale fp16(max|w_r| / 448); codes are the
  e4m3fn bytes of clamp(w / scale, +-448) (torch's RNE cast); x ~ N(0,1) in bf16.

``rint`` is numpy's round-half-to-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

LLAMA8B_SHAPES = {  # name: (out rows N, in cols K), tensor id
    "q": ((4096, 4096), 0),
    "k": ((1024, 4096), 1),
    "v": ((1024, 4096), 2),
    "o": ((4096, 4096), 3),
    "gate": ((14336, 4096), 4),
    "up": ((14336, 4096), 5),
    "down": ((4096, 14336), 6),
}
LM_HEAD_SHAPE = ((128256, 4096), 7)


def rng_for(cfg: int, layer: int, tid: int) -> np.random.Generator:
    return np.random.default_rng([0, cfg, layer, tid])


# ---------------------------------------------------------------- code statistics
def _laplace_code_pmf(b: float, lo: int = -8, hi: int = 7) -> np.ndarray:
    """pmf of clip(rint(Laplace(0, b)), lo, hi) (continuous ties have measure 0)."""
    def cdf(t):
        return 0.5 * math.exp(t / b) if t < 0 else 1.0 - 0.5 * math.exp(-t / b)
    p = []
    for n in range(lo, hi + 1):
        a = -math.inf if n == lo else n - 0.5
        c = math.inf if n == hi else n + 0.5
        pa = 0.0 if a == -math.inf else cdf(a)
        pc = 1.0 if c == math.inf else cdf(c)
        p.append(pc - pa)
    return np.array(p)


def _gauss_code_pmf(sigma: float, lo: int = -8, hi: int = 7) -> np.ndarray:
    def cdf(t):
        return 0.5 * (1.0 + math.erf(t / (sigma * math.sqrt(2.0))))
    p = []
    for n in range(lo, hi + 1):
        pa = 0.0 if n == lo else cdf(n - 0.5)
        pc = 1.0 if n == hi else cdf(n + 0.5)
        p.append(pc - pa)
    return np.array(p)


def _h_bits(p: np.ndarray) -> float:
    p = p[p > 0]
    return float(-(p * np.log2(p)).sum())


def laplace_b_for_entropy(target_bits: float = 2.2) -> float:
    """Bisection (60 steps) on b so that H(clip(rint(Laplace(0,b)))) = target."""
    lo, hi = 1e-3, 50.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if _h_bits(_laplace_code_pmf(mid)) < target_bits:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


LAPLACE_B = laplace_b_for_entropy(2.2)
LAPLACE_PMF = _laplace_code_pmf(LAPLACE_B)
GAUSS_PMF = _gauss_code_pmf(2.0)
_LEVELS = np.arange(-8, 8)
LAPLACE_SD = float(math.sqrt((LAPLACE_PMF * _LEVELS**2).sum() - (LAPLACE_PMF * _LEVELS).sum() ** 2))


# ---------------------------------------------------------------- tensors
@dataclass
class IntCodeTensor:
    codes: np.ndarray      # int8 [N][K], values in [-8, 7]
    scales: np.ndarray     # float16 [N]
    x: np.ndarray          # float16 [batch][K]


@dataclass
class Bf16Tensor:
    bits: np.ndarray       # uint16 [N][K] (bf16 bit patterns)
    x_bits: np.ndarray     # uint16 [batch][K] (bf16 bit patterns)


@dataclass
class Fp8Tensor:
    codes: np.ndarray      # uint8 [N][K] (e4m3fn bytes)
    scales: np.ndarray     # float16 [N]
    x_bits: np.ndarray     # uint16 [batch][K] (bf16 bit patterns)


def _fp16(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def gaussian_codes(shape, rng: np.random.Generator, batch: int = 1) -> IntCodeTensor:
    n, k = shape
    q = np.clip(np.rint(rng.normal(0.0, 2.0, (n, k))), -8, 7).astype(np.int8)
    s = _fp16(0.01 * rng.uniform(0.5, 1.5, n))
    x = _fp16(rng.standard_normal((batch, k)))
    return IntCodeTensor(q, s, x)


def laplace_codes(shape, rng: np.random.Generator, batch: int = 1) -> IntCodeTensor:
    n, k = shape
    q = np.clip(np.rint(rng.laplace(0.0, LAPLACE_B, (n, k))), -8, 7).astype(np.int8)
    s = _fp16((0.02 / LAPLACE_SD) * rng.uniform(0.5, 1.5, n))
    x = _fp16(rng.standard_normal((batch, k)))
    return IntCodeTensor(q, s, x)


def bf16_weights(shape, rng: np.random.Generator, batch: int = 1) -> Bf16Tensor:
    n, k = shape
    w = _bf16_bits(rng.normal(0.0, 0.02, (n, k)))
    x = _bf16_bits(rng.standard_normal((batch, k)))
    return Bf16Tensor(w, x)


def fp8_weights(shape, rng: np.random.Generator, batch: int = 1) -> Fp8Tensor:
    import torch
    n, k = shape
    w = rng.normal(0.0, 0.02, (n, k))
    s = _fp16(np.abs(w).max(axis=1) / 448.0)
    s = np.where(s == 0, np.float16(1.0), s)
    v = np.clip(w / s.astype(np.float64)[:, None], -448.0, 448.0).astype(np.float32)
    q = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    x = _bf16_bits(rng.standard_normal((batch, k)))
    return Fp8Tensor(q, s, x)


# ---------------------------------------------------------------- named workloads
def config1(batch: int = 1) -> IntCodeTensor:
    """One 1024x1024 matrix of 16-level Gaussian codes (sigma = 2 levels), seed 0."""
    return gaussian_codes((1024, 1024), np.random.default_rng(0), batch)


def config2_tensor(name: str, layer: int = 0, batch: int = 1) -> IntCodeTensor:
    """One Llama-3.1-8B-shaped linear layer of 2.2-bit Laplacian codes."""
    shape, tid = LLAMA8B_SHAPES[name]
    return laplace_codes(shape, rng_for(2, layer, tid), batch)


def config3_tensor(name: str, batch: int = 1) -> Bf16Tensor:
    """BF16 N(0, 0.02^2) weights at the gate (14336x4096) or down (4096x14336) shape."""
    shape, tid = LLAMA8B_SHAPES[name]
    return bf16_weights(shape, rng_for(3, 0, tid), batch)


def config4_tensor(name: str, layer: int = 0, batch: int = 1) -> Fp8Tensor:
    if name == "lm_head":
        shape, tid = LM_HEAD_SHAPE
    else:
        shape, tid = LLAMA8B_SHAPES[name]
    return fp8_weights(shape, rng_for(4, layer, tid), batch)


def small_int_codes(n: int, k: int, seed: int, dist: str = "laplace", batch: int = 1) -> IntCodeTensor:
    rng = np.random.default_rng([0, 100, seed])
    if dist == "laplace":
        return laplace_codes((n, k), rng, batch)
    return gaussian_codes((n, k), rng, batch)


def normal_matrix(shape, rng: np.random.Generator, sd: float = 0.02) -> np.ndarray:
    """Plain fp64 N(0, sd^2) matrix (input of the lattice conversion)."""
    return rng.normal(0.0, sd, shape)
