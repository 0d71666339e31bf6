"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""

import contextlib

import numpy as np
import torch

BITS = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}
NP_BITS = {torch.float32: np.uint32, torch.float16: np.uint16, torch.bfloat16: np.uint16}

# tolerances of attention outputs vs the float64 oracle (max-abs, fp32 accumulation)
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits of a tensor as an unsigned numpy array (NaN-safe
    bit-exact comparisons)."""
    return t.detach().contiguous().view(BITS[t.dtype]).cpu().numpy().view(NP_BITS[t.dtype])


def from_bits(a: np.ndarray, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    signed = {np.uint32: np.int32, np.uint16: np.int16}[a.dtype.type]
    return torch.from_numpy(np.ascontiguousarray(a).view(signed)).to(device).view(dtype)


def random_bits(rng, shape, dtype: torch.dtype) -> np.ndarray:
    nb = NP_BITS[dtype]
    hi = 2**32 if nb is np.uint32 else 2**16
    return rng.integers(0, hi, size=shape, dtype=np.uint64).astype(nb)


def half_ulp(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Half a unit in the last place of |x| in ``dtype`` (rounding of the output)."""
    mant = {torch.float32: 23, torch.float16: 10, torch.bfloat16: 7}[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    e = np.maximum(e, {torch.float32: -126, torch.float16: -14, torch.bfloat16: -126}[dtype])
    return 0.5 * 2.0 ** (e - mant)


def check_close(got: torch.Tensor, ref: np.ndarray, tol: float, what: str = "") -> float:
    g = got.detach().cpu().to(torch.float64).numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    allowed = tol if got.dtype == torch.float32 else tol + half_ulp(ref, got.dtype)
    err = np.abs(g - ref)
    bad = err > allowed
    assert not bad.any(), f"{what}: max err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"
    return float(err.max())


@contextlib.contextmanager
def debug_checks(on: bool):
    """The library's index-precondition checks on or off for the block
    (restored afterwards, whatever PA_DEBUG set for the process)."""
    from paged_kv_cache_76_amd import _lib as L
    before = L.get_debug()
    L.set_debug(on)
    try:
        yield
    finally:
        L.set_debug(before)
