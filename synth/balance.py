"""Seeded synthetic inputs for the routing bias update.

Shapes and distributions only (no arithmetic of the update).  Recipe:

* top-k choice arrays [T, k] int32: k distinct experts per token, drawn with
  per-expert popularity p_e ~ rank(e)^-skew (rank a seeded permutation of
  1..E; skew 0 is uniform), as a router with uneven expert affinity would
  pick them (Gumbel top-k of log p_e);
* loads [E] int32 around an exact integer mean m: experts in pairs with
  deviations +d and -d (d uniform in 1..spread), a quarter of them exactly at
  m, shuffled, so that the three directions of the update all occur;
* bias [E] ~ N(0, 0.01) fp32, the spread of the router's correction bias.
"""
from __future__ import annotations

import numpy as np
import torch

from .gen import _gen, _seed

ROLE_CHOICE, ROLE_LOAD, ROLE_BIASV = 31, 32, 33


def topk_choices(T: int, k: int, E: int, seed: int = 0, skew: float = 1.0,
                 device="cpu") -> torch.Tensor:
    rng = np.random.default_rng(_seed(seed, ROLE_CHOICE, T, k, E))
    rank = rng.permutation(E) + 1
    logp = -skew * np.log(rank.astype(np.float64))
    gumbel = -np.log(-np.log(rng.random((T, E)).clip(1e-300, 1.0)))
    ids = np.argsort(-(logp[None, :] + gumbel), axis=1, kind="stable")[:, :k]
    return torch.from_numpy(ids.astype(np.int32)).to(device)


def expert_loads(E: int, mean: int, spread: int, seed: int = 0, device="cpu") -> torch.Tensor:
    assert E % 4 == 0 and spread < mean
    rng = np.random.default_rng(_seed(seed, ROLE_LOAD, E, mean))
    n_pairs = (3 * E // 4) // 2
    d = rng.integers(1, spread + 1, n_pairs)
    dev = np.concatenate([d, -d, np.zeros(E - 2 * n_pairs, dtype=np.int64)])
    c = (mean + rng.permutation(dev)).astype(np.int32)
    return torch.from_numpy(c).to(device)


def bias_values(E: int, seed: int = 0, device="cpu") -> torch.Tensor:
    g = _gen(device, seed, ROLE_BIASV, E)
    return torch.randn(E, generator=g, device=device, dtype=torch.float32) * 0.01
