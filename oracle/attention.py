"""Exact attention over a logically contiguous history, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the reference for the HIP
decode and prefill kernels, never called by the product.

Definition followed ("vLLM / PagedAttention", awesome.papernotes.org,
"方法详解" → key design 1, eq. 1): for query i,

    a_ij = exp(q_i . k_j / sqrt(d)) / sum_{t <= i} exp(q_i . k_t / sqrt(d)),
    o_i  = sum_{j <= i} a_ij v_j .

Readings taken where the pages are silent:

* ``d`` is the head dimension, so the default scale is ``1/sqrt(head_dim)``;
  a caller may pass another scale (the score is ``scale * q . k``).
* The sum runs to ``t = i`` inclusive: the token being decoded attends to its
  own key, so the history handed to :func:`decode` already contains it.
* Eq. 2 of the same section (the block-wise form) is the same quantity with
  the history cut into blocks of B tokens; the oracle evaluates eq. 1 on the
  logically contiguous history and never sees a block table.

Subtracting the row maximum before ``exp`` multiplies numerator and
denominator of eq. 1 by the same factor, so it changes nothing but the range.
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def default_scale(head_dim: int) -> float:
    """1/sqrt(d) with d the head dimension (key design 1, eq. 1)."""
    return 1.0 / np.sqrt(float(head_dim))


def attention_weights(q, K, scale: float) -> np.ndarray:
    """Softmax weights ``a_j`` of one query ``q [d]`` over keys ``K [L][d]``.

    Key design 1, eq. 1: ``a_j = exp(s_j) / sum_t exp(s_t)`` with
    ``s_j = scale * q . k_j``.  Returns a float64 vector of length L.
    """
    q = _f64(q)
    K = _f64(K)
    if K.ndim != 2 or q.ndim != 1 or K.shape[1] != q.shape[0]:
        raise ValueError(f"shape mismatch q{q.shape} K{K.shape}")
    if K.shape[0] == 0:
        raise ValueError("attention over an empty history is undefined")
    s = (K @ q) * float(scale)
    e = np.exp(s - s.max())
    return e / e.sum()


def attend(q, K, V, scale: float) -> np.ndarray:
    """``o = sum_j a_j v_j`` for one query and one head (key design 1, eq. 1).

    ``q [d]``, ``K [L][d]``, ``V [L][dv]`` → ``o [dv]`` in float64.
    """
    a = attention_weights(q, K, scale)
    V = _f64(V)
    if V.shape[0] != a.shape[0]:
        raise ValueError("K and V histories differ in length")
    return a @ V


def decode(q, K, V, scale: float | None = None) -> np.ndarray:
    """One decode step of one sequence, every head.

    ``q [H][d]`` is the new token's query; ``K, V [L][H][d]`` are the
    sequence's whole key/value history in logical order, the new token's own
    key/value included (``L >= 1``).  Returns ``o [H][d]`` in float64.
    """
    q = _f64(q)
    K = _f64(K)
    V = _f64(V)
    H, d = q.shape
    if K.ndim != 3 or K.shape[1:] != (H, d) or V.shape != K.shape:
        raise ValueError(f"shape mismatch q{q.shape} K{K.shape} V{V.shape}")
    if scale is None:
        scale = default_scale(d)
    out = np.empty((H, d), dtype=np.float64)
    for h in range(H):
        out[h] = attend(q[h], K[:, h, :], V[:, h, :], scale)
    return out


def prefill(Q, K, V, scale: float | None = None) -> np.ndarray:
    """Causal attention for the last ``n`` positions of one sequence.

    ``K, V [L][H][d]`` hold the whole history; ``Q [n][H][d]`` (``n <= L``)
    are the queries of logical positions ``L-n .. L-1``.  Query row ``i``
    attends to positions ``t <= L-n+i`` (key design 1, eq. 1: the sum runs to
    the query's own position).  Returns ``[n][H][d]`` in float64.
    """
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    n, H, d = Q.shape
    L = K.shape[0]
    if K.shape != (L, H, d) or V.shape != K.shape or not (1 <= n <= L):
        raise ValueError(f"shape mismatch Q{Q.shape} K{K.shape} V{V.shape}")
    if scale is None:
        scale = default_scale(d)
    # eq. 1 for every query row at once: a score matrix over all key
    # positions, the keys after the row's own position removed (weight 0);
    # row i is sum_t exp(s_it) v_t divided by sum_t exp(s_it)
    first = L - n
    pos = first + np.arange(n)
    allowed = np.arange(L)[None, :] <= pos[:, None]          # [n][L]: t <= position of the row
    out = np.empty((n, H, d), dtype=np.float64)
    for h in range(H):
        Qh = np.ascontiguousarray(Q[:, h, :])
        Kh = np.ascontiguousarray(K[:, h, :])
        Vh = np.ascontiguousarray(V[:, h, :])
        s = (Qh @ Kh.T) * float(scale)                         # [n][L]
        s = np.where(allowed, s, -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (e @ Vh) / e.sum(axis=1, keepdims=True)
    return out
