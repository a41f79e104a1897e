"""fp64 CPU oracle: gradients of exact dot-product attention.

TEST INFRASTRUCTURE ONLY (see the package docstring). Only ``tests/``, the
smoke check and the benchmark's CPU-baseline leg may use it.

For one (batch, head), with ``S = scale * Q K^T`` (causal: ``S[i, j] = -inf``
for key j > query i), ``P = softmax(S)`` row-wise and ``O = P V``, and an
upstream gradient ``dO = dL/dO``, the gradients are
("FlashAttention · InkStack", section 1.2.1, the backward pass of plain
attention):

1. ``dV = P^T dO`` and ``dP = dO V^T``;
2. ``D_i = sum_k P[i, k] dP[i, k]``, which equals ``rowsum(dO * O)``
   (the same section rewrites the first as the second);
3. ``dS = P * (dP - D)`` (the softmax Jacobian applied row by row);
4. ``dQ = scale * dS K`` and ``dK = scale * dS^T Q``.

P is rebuilt from the scores and the saved statistic, ``P = exp(S - LSE)``
with ``LSE = m + ln l`` (section 1.2.2, recomputation from the saved m and l).
Nothing is rounded here; the inputs are the exact values the GPU receives.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_rows


def _as64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def attention_bwd_head(q, k, v, do, scale: float, causal: bool = False):
    """Gradients for one head. q, k, v, do: [N, d] (q and do may have Nq rows,
    k and v Nk rows). Returns (dq, dk, dv, delta) as float64, where ``delta``
    is D = rowsum(dO * O)."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    rows = np.arange(q.shape[0])
    o, lse = attention_rows(q, k, v, rows, scale, causal)
    # rebuild P from the scores and the saved LSE (section 1.2.2)
    s = np.float64(scale) * (q @ k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > rows[:, None], -np.inf, s)
    p = np.exp(s - lse[:, None])
    dv = p.T @ do                       # step 1
    dp = do @ v.T
    delta = np.sum(do * o, axis=1)      # step 2, the rowsum(dO * O) form
    ds = p * (dp - delta[:, None])      # step 3
    dq = np.float64(scale) * (ds @ k)   # step 4
    dk = np.float64(scale) * (ds.T @ q)
    return dq, dk, dv, delta


def attention_bwd_bhnd(q, k, v, do, scale: float, causal: bool = False):
    """``attention_bwd_head`` over every (batch, head) of [B, H, N, d] arrays."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H = q.shape[:2]
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    delta = np.empty(q.shape[:3])
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h], delta[b, h] = attention_bwd_head(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
    return dq, dk, dv, delta


def attention_bwd_sampled(q, k, v, do, rows, keys, scale: float, causal: bool = False):
    """The same gradients, for a subset of one head's outputs: dQ at the query
    rows ``rows`` and dK, dV at the key rows ``keys`` (each still sums over
    every key, respectively every query, exactly as ``attention_bwd_head``).
    Returns (dq[rows], dk[keys], dv[keys])."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    all_rows = np.arange(q.shape[0])
    o, lse = attention_rows(q, k, v, all_rows, scale, causal)   # every query's O, LSE
    delta = np.sum(do * o, axis=1)
    # dQ rows: P and dP of those queries against every key
    s = np.float64(scale) * (q[rows] @ k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > rows[:, None], -np.inf, s)
    p = np.exp(s - lse[rows, None])
    ds = p * ((do[rows] @ v.T) - delta[rows, None])
    dq = np.float64(scale) * (ds @ k)
    # dK, dV rows: P and dP of every query against those keys
    s = np.float64(scale) * (q @ k[keys].T)
    if causal:
        s = np.where(keys[None, :] > all_rows[:, None], -np.inf, s)
    p = np.exp(s - lse[:, None])
    ds = p * ((do @ v[keys].T) - delta[:, None])
    dv = p.T @ do
    dk = np.float64(scale) * (ds.T @ q)
    return dq, dk, dv
