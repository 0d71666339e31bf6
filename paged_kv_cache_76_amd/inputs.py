"""Seeded synthetic inputs shared by the tests, the bench and the oracle leg.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no attention, no block-table logic), so both the HIP path
and the CPU oracle may consume what it produces.

The pages measure on OPT models with ShareGPT/Alpaca length distributions;
none of those are available, and these generators stand in for them with the
shapes the pages fix (OPT-13B: 40 heads of 128, i.e. 5120 hidden, 2-byte KV)
and length mixes of the stated medians and caps.

Conventions:

* Workload ``k`` uses ``numpy.random.SeedSequence(76_000 + k)``; its children
  (``spawn``) feed independent streams (lengths, q, k, v, pool order, beams).
* "~N(0,1)" values are drawn as float32 by ``Generator.standard_normal`` and
  rounded to the storage type round-to-nearest-even by ``torch.Tensor.to``;
  consumers read the rounded values back (exact widening) as their input.
"""

from __future__ import annotations

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def seed_sequence(config_index: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(76_000 + int(config_index))


def streams(config_index: int, n: int) -> list[np.random.Generator]:
    """``n`` independent generators for workload ``config_index``."""
    return [np.random.default_rng(s) for s in seed_sequence(config_index).spawn(n)]


def normal(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    """A CPU tensor of the storage dtype holding N(0,1) draws."""
    x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    return torch.from_numpy(x).to(DTYPES[dtype])


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a stored fp32/fp16/bf16 CPU tensor to float64."""
    return t.detach().cpu().to(torch.float64).numpy()


def pool_order(rng: np.random.Generator, num_blocks: int) -> np.ndarray:
    """A seeded permutation of the physical block ids (free-list order)."""
    return rng.permutation(num_blocks).astype(np.int64)


def uniform_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """``n`` integers uniform on ``[lo, hi]`` inclusive."""
    return rng.integers(lo, hi + 1, size=n).astype(np.int64)


def lognormal_lengths(rng: np.random.Generator, n: int, median: float, sigma: float,
                      lo: int, hi: int | None) -> np.ndarray:
    """``n`` rounded lognormal lengths with the given median and log-sd,
    clipped to ``[lo, hi]`` (``hi=None``: no upper clip)."""
    x = np.rint(rng.lognormal(mean=np.log(median), sigma=sigma, size=n))
    x = np.maximum(x, lo)
    if hi is not None:
        x = np.minimum(x, hi)
    return x.astype(np.int64)


def uniform_fraction(rng: np.random.Generator, n: int) -> np.ndarray:
    """``n`` floats uniform on [0, 1)."""
    return rng.random(n)


def choice_with_replacement(rng: np.random.Generator, n_groups: int, width: int) -> np.ndarray:
    """``[n_groups][width]`` indices in ``[0, width)`` drawn with replacement,
    sorted within each group (beam parents in the shared-block workload)."""
    return np.sort(rng.integers(0, width, size=(n_groups, width)), axis=1).astype(np.int64)
