"""Seeded synthetic workloads for batched token sampling over a logits matrix [B, V].

This module only draws inputs. It holds none of the sampling method's arithmetic and is the
one module that both the CPU oracle's tests and the HIP library's tests and benchmark read.

Shapes, value distributions and masking follow the sampling-step workloads of the mlxcel
issue "Softmax-free GPU sampling: Gumbel-max categorical sampling kernel" (section
"Performance validation": vocabularies of 32K/64K/152K, batches of 1/4/8; section
"Regression guard": peaked, flat, bimodal and -inf-masked synthetic logits) and the 262K
vocabulary mentioned in the mlx-bun HLG design document ("Open questions / risks").

Recipe (every config draws from its own numpy Generator, in this order):
  1. logits, row block by row block, from ``default_rng(data_seed)``;
  2. the masked set of each row: exactly round(p * V) distinct indices set to -inf;
  3. per-row temperatures (where they vary), then any spike positions;
  4. per-row Philox seeds from ``default_rng(1000 + cfg)``, offsets (where they vary) next.
bf16 / f16 inputs are the float64 draws rounded to nearest-even by torch.
The curve pivot mu, where the curve is on, is the mean of the row's finite log-probs
(log-probs from the bf16/f16/f32 values actually stored), computed in float64 and handed to
both sides as float32: it is an input of the method, not part of it.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch
from scipy.special import logsumexp as _scipy_logsumexp

HLG_A = {"m": 1.5, "w": 2.0, "beta_t": 1.0, "beta_h": 2.0}      # bimodal and 262K configs
HLG_B = {"m": 1.25, "w": 1.5, "beta_t": 0.5, "beta_h": 1.0}     # 256 x 151936 headline


@dataclasses.dataclass
class Workload:
    name: str
    logits: torch.Tensor            # CPU tensor [B, V], dtype float32 / bfloat16 / float16
    T: np.ndarray                   # float32 [B]
    seed: np.ndarray                # uint64 [B]
    offset: np.ndarray              # uint64 [B]
    K: int = 1
    hlg: Optional[dict] = None      # None = curve off
    mu: Optional[np.ndarray] = None  # float32 [B] when the curve is on

    @property
    def B(self) -> int:
        return int(self.logits.shape[0])

    @property
    def V(self) -> int:
        return int(self.logits.shape[1])

    @property
    def dtype(self) -> torch.dtype:
        return self.logits.dtype

    def nbytes(self) -> int:
        return self.logits.numel() * self.logits.element_size()


def _mask_rows(x: np.ndarray, frac: float, rng: np.random.Generator) -> None:
    B, V = x.shape
    n = int(round(frac * V))
    if n == 0:
        return
    for b in range(B):
        idx = rng.choice(V, size=n, replace=False)
        x[b, idx] = -np.inf


def mean_finite_logprob(x: torch.Tensor) -> np.ndarray:
    """Per-row mean of the finite log-probs of the stored logits, float64 -> float32."""
    xd = x.double().numpy()
    out = np.empty(xd.shape[0], dtype=np.float64)
    for b in range(xd.shape[0]):
        row = xd[b]
        fin = row[np.isfinite(row)]
        if fin.size == 0:
            out[b] = 0.0
            continue
        out[b] = fin.mean() - _scipy_logsumexp(fin)
    return out.astype(np.float32)


def _philox_seeds(cfg: int, B: int) -> np.random.Generator:
    return np.random.default_rng(1000 + cfg)


def _normal_blocks(rng, B, V, loc, scale, block=64) -> np.ndarray:
    x = np.empty((B, V), dtype=np.float64)
    for b0 in range(0, B, block):
        b1 = min(B, b0 + block)
        x[b0:b1] = rng.normal(loc, scale, size=(b1 - b0, V))
    return x


def config1(B: int = 1, V: int = 32768, K: int = 1000) -> Workload:
    """B=1 x V=32768 fp32 ~ N(0, 3^2), 5% of entries -inf, T=1, curve off, K draws at
    offsets 0..K-1."""
    rng = np.random.default_rng(0)
    x = _normal_blocks(rng, B, V, 0.0, 3.0)
    _mask_rows(x, 0.05, rng)
    srng = _philox_seeds(1, B)
    seed = srng.integers(0, 2**64, size=B, dtype=np.uint64)
    return Workload("fp32 B=%d V=%d N(0,3^2) 5%% masked, T=1, K=%d" % (B, V, K),
                    torch.from_numpy(x.astype(np.float32)), np.ones(B, np.float32), seed,
                    np.zeros(B, np.uint64), K=K)


def chi_square_rows(V: int = 16) -> np.ndarray:
    """The V=16 logits linspace(-4, 4) of the chi-square side test."""
    return np.linspace(-4.0, 4.0, V)


def config2(B: int = 8, T: float = 0.5, V: int = 65536) -> Workload:
    """B x V=65536 bf16 peaked rows: N(0, 1) plus +15 at one random index per row."""
    rng = np.random.default_rng(2)
    x = _normal_blocks(rng, B, V, 0.0, 1.0)
    spikes = rng.integers(0, V, size=B)
    x[np.arange(B), spikes] += 15.0
    srng = _philox_seeds(2, B)
    seed = srng.integers(0, 2**64, size=B, dtype=np.uint64)
    return Workload("bf16 B=%d V=%d peaked, T=%g" % (B, V, T),
                    torch.from_numpy(x).to(torch.bfloat16), np.full(B, T, np.float32), seed,
                    np.zeros(B, np.uint64))


def config3(B: int = 8, V: int = 151936) -> Workload:
    """B=8 x V=151936 fp32 bimodal (50/50 N(-2,1), N(4,0.5^2)), 10% -inf, curve on
    (m=1.5, w=2, beta_t=1, beta_h=2), T=1."""
    rng = np.random.default_rng(3)
    lo = _normal_blocks(rng, B, V, -2.0, 1.0)
    hi = _normal_blocks(rng, B, V, 4.0, 0.5)
    pick = rng.random(size=(B, V)) < 0.5
    x = np.where(pick, lo, hi)
    _mask_rows(x, 0.10, rng)
    srng = _philox_seeds(3, B)
    seed = srng.integers(0, 2**64, size=B, dtype=np.uint64)
    t = torch.from_numpy(x.astype(np.float32))
    return Workload("fp32 B=%d V=%d bimodal 10%% masked, HLG m=1.5 w=2 bt=1 bh=2, T=1" % (B, V),
                    t, np.ones(B, np.float32), seed, np.zeros(B, np.uint64),
                    hlg=dict(HLG_A), mu=mean_finite_logprob(t))


def config4(B: int = 256, V: int = 151936) -> Workload:
    """B=256 x V=151936 bf16 flat ~ N(0, 0.5^2), per-row T ~ U[0.3, 1.5], per-row seeds and
    offsets, curve on (m=1.25, w=1.5, beta_t=0.5, beta_h=1.0), one draw."""
    rng = np.random.default_rng(4)
    x = _normal_blocks(rng, B, V, 0.0, 0.5)
    T = rng.uniform(0.3, 1.5, size=B).astype(np.float32)
    srng = _philox_seeds(4, B)
    seed = srng.integers(0, 2**64, size=B, dtype=np.uint64)
    offset = srng.integers(0, 2**32, size=B, dtype=np.uint64)
    t = torch.from_numpy(x).to(torch.bfloat16)
    return Workload("bf16 B=%d V=%d N(0,0.5^2), T~U[0.3,1.5], HLG m=1.25 w=1.5 bt=0.5 bh=1" % (B, V),
                    t, T, seed, offset, hlg=dict(HLG_B), mu=mean_finite_logprob(t))


def config5(B: int = 1024, V: int = 262144, K: int = 16) -> Workload:
    """B=1024 x V=262144 fp32 ~ N(0, 2^2), 30% -inf, curve on (m=1.5, w=2, beta_t=1,
    beta_h=2), T=1, K=16 draws at offsets 0..15 from one read."""
    rng = np.random.default_rng(5)
    x = _normal_blocks(rng, B, V, 0.0, 2.0)
    _mask_rows(x, 0.30, rng)
    srng = _philox_seeds(5, B)
    seed = srng.integers(0, 2**64, size=B, dtype=np.uint64)
    t = torch.from_numpy(x.astype(np.float32))
    del x
    return Workload("fp32 B=%d V=%d N(0,2^2) 30%% masked, HLG m=1.5 w=2 bt=1 bh=2, T=1, K=%d" % (B, V, K),
                    t, np.ones(B, np.float32), seed, np.zeros(B, np.uint64), K=K,
                    hlg=dict(HLG_A), mu=mean_finite_logprob(t))


def generic(B: int, V: int, dtype=torch.float32, *, seed: int = 7, scale: float = 2.0,
            mask_frac: float = 0.0, hlg: Optional[dict] = None, K: int = 1,
            T: Optional[np.ndarray] = None, offset_max: int = 0) -> Workload:
    """Free-form shapes for edge-case tests (ragged V, tiny rows, many draws)."""
    rng = np.random.default_rng(seed)
    x = _normal_blocks(rng, B, V, 0.0, scale)
    if mask_frac > 0:
        _mask_rows(x, mask_frac, rng)
    if T is None:
        T = rng.uniform(0.3, 1.5, size=B).astype(np.float32)
    seeds = rng.integers(0, 2**64, size=B, dtype=np.uint64)
    offs = rng.integers(0, offset_max + 1, size=B, dtype=np.uint64) if offset_max else \
        np.zeros(B, np.uint64)
    t = torch.from_numpy(x).to(dtype)
    mu = mean_finite_logprob(t) if hlg is not None else None
    return Workload("generic B=%d V=%d %s" % (B, V, dtype), t, np.asarray(T, np.float32),
                    seeds, offs, K=K, hlg=hlg, mu=mu)


WORKLOADS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}
