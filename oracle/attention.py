"""fp64 CPU oracle: exact dot-product attention, written from its definition.

TEST INFRASTRUCTURE ONLY (see the package docstring). Only ``tests/``, the
smoke check and the benchmark's CPU-baseline leg may use it.

What is computed, for one (batch, head) with Q, K, V in R^{N x d}:

1. ``S = scale * Q K^T``; with ``causal``, ``S[i, j] = -inf`` for key j > query i.
2. a two-pass safe softmax over each row: ``m_i = max_j S[i, j]``, then
   ``l_i = sum_j exp(S[i, j] - m_i)`` and ``P = exp(S - m) / l``.
3. ``O = P V`` and ``LSE_i = m_i + ln l_i`` (natural logarithm).

Sources: the three-step definition S -> P -> O in the introduction of
"FlashAttention · InkStack" and in the "standard three-step computation" of
the MUSA guide "FlashAttention 优化"; the safe (max-subtracted) softmax of the
MUSA guide's "standard softmax" passage; the statistic ``L = m + log l`` of
"FlashAttention · InkStack", section 2.1. The page states the log without a
base; the exponentials there are base e, so this is the natural log.

The values passed in are the exact real values the GPU receives (its fp16 /
bf16 / dequantised e4m3 inputs, upcast to float64); nothing is rounded here.

The online recurrences below (``online_attention_head*``) are the block-wise
update rules of "FlashAttention · InkStack" sections 1.1.2 (normalise at every
step) and 2.1 (deferred normalisation), kept here only so the tests can show
that they reach the same numbers as the two-pass definition.
"""
from __future__ import annotations

import numpy as np


def _as64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _scores(q: np.ndarray, k: np.ndarray, scale: float, rows: np.ndarray,
            causal: bool) -> np.ndarray:
    """Step 1: S = scale * Q K^T for the query rows ``rows``; causal masking sets
    the entries with key index greater than the query index to -inf."""
    s = np.float64(scale) * (q[rows] @ k.T)
    if causal:
        keys = np.arange(k.shape[0])[None, :]
        s = np.where(keys > rows[:, None], -np.inf, s)
    return s


def _softmax_two_pass(s: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Step 2: safe softmax, two passes over each row (max, then sum of exps).
    Returns P, m and l."""
    m = np.max(s, axis=1)
    e = np.exp(s - m[:, None])
    ell = np.sum(e, axis=1)
    return e / ell[:, None], m, ell


def attention_rows(q, k, v, rows, scale: float, causal: bool = False):
    """Oracle for the query rows ``rows`` of one head.

    q: [Nq, d], k and v: [Nk, d] (any real dtype, upcast to float64).
    Returns (O[rows] as [len(rows), d], LSE[rows] as [len(rows)]), float64.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    rows = np.asarray(rows, dtype=np.int64)
    s = _scores(q, k, scale, rows, causal)
    p, m, ell = _softmax_two_pass(s)
    o = p @ v                                   # step 3
    lse = m + np.log(ell)
    return o, lse


def attention_head(q, k, v, scale: float, causal: bool = False):
    """Oracle for every query row of one head: (O [N, d], LSE [N])."""
    return attention_rows(q, k, v, np.arange(np.shape(q)[0]), scale, causal)


def attention_bhnd(q, k, v, scale: float, causal: bool = False):
    """Oracle over [B, H, N, d] tensors, one (b, h) head at a time.
    Returns O [B, H, N, d] and LSE [B, H, N] in float64."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse


# ------------------------------------------------------ online recurrences --

def online_attention_head(q, k, v, scale: float, causal: bool = False,
                          splits=None):
    """Deferred-normalisation online softmax ("FlashAttention · InkStack" 2.1).

    Keys are consumed in consecutive blocks whose sizes are ``splits`` (default:
    one block per key). Per block: m' = max(m, rowmax S_blk), alpha = e^{m-m'},
    l' = alpha*l + rowsum e^{S_blk-m'}, O~' = alpha*O~ + e^{S_blk-m'} V_blk; at the
    end O = O~ / l and LSE = m + ln l.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    N = q.shape[0]
    rows = np.arange(N)
    nk = k.shape[0]
    splits = [1] * nk if splits is None else list(splits)
    assert sum(splits) == nk
    m = np.full(N, -np.inf)
    ell = np.zeros(N)
    acc = np.zeros((N, v.shape[1]))
    start = 0
    for size in splits:
        blk = slice(start, start + size)
        s = np.float64(scale) * (q @ k[blk].T)
        if causal:
            keys = np.arange(start, start + size)[None, :]
            s = np.where(keys > rows[:, None], -np.inf, s)
        m_new = np.maximum(m, np.max(s, axis=1))
        # rows whose keys so far are all masked keep m = -inf; use 0 there so
        # that exp(-inf - (-inf)) never appears (those rows have l = 0, O~ = 0)
        ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(m - ref)
        p = np.exp(s - ref[:, None])
        ell = alpha * ell + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[blk]
        m = m_new
        start += size
    return acc / ell[:, None], m + np.log(ell)


def online_attention_head_fa1(q, k, v, scale: float, causal: bool = False,
                              splits=None):
    """Online softmax with normalisation at every block ("FlashAttention ·
    InkStack" 1.1.2): O' = (alpha*l*O + P_new V_new) / l'."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    N = q.shape[0]
    rows = np.arange(N)
    nk = k.shape[0]
    splits = [1] * nk if splits is None else list(splits)
    assert sum(splits) == nk
    m = np.full(N, -np.inf)
    ell = np.zeros(N)
    o = np.zeros((N, v.shape[1]))
    start = 0
    for size in splits:
        blk = slice(start, start + size)
        s = np.float64(scale) * (q @ k[blk].T)
        if causal:
            keys = np.arange(start, start + size)[None, :]
            s = np.where(keys > rows[:, None], -np.inf, s)
        m_new = np.maximum(m, np.max(s, axis=1))
        ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(m - ref)
        p = np.exp(s - ref[:, None])
        ell_new = alpha * ell + p.sum(axis=1)
        safe = np.where(ell_new > 0, ell_new, 1.0)
        o = ((alpha * ell)[:, None] * o + p @ v[blk]) / safe[:, None]
        m, ell = m_new, ell_new
        start += size
    return o, m + np.log(ell)


# ------------------------------------------- grouped heads, Nq != Nk, decode --

def attention_gqa(q, k, v, scale: float, causal: bool = False):
    """Oracle for grouped-query attention with a key/value history.

    q: [B, H, Nq, d]; k, v: [B, Hkv, Nk, d] with H a multiple of Hkv. Query
    head h reads key/value head h // (H // Hkv) (grouped-query and multi-query
    attention, the "qhead_per_kvhead" sharing of the FA4 walkthrough, section
    3.3, and the GQA/MQA broadcast of the vLLM deep dive). The Nq queries are
    the last Nq positions of the Nk-long sequence (a decode or chunked-prefill
    step over a key/value cache): with ``causal``, query i sees key j only if
    j <= i + (Nk - Nq). For Nq = Nk this is the causal mask of ``attention_rows``.
    Returns O [B, H, Nq, d] and LSE [B, H, Nq] in float64.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    assert H % Hkv == 0 and Nq <= Nk
    group = H // Hkv
    off = Nk - Nq
    o = np.empty((B, H, Nq, v.shape[-1]))
    lse = np.empty((B, H, Nq))
    rows = np.arange(Nq)
    for b in range(B):
        for h in range(H):
            kh, vh = k[b, h // group], v[b, h // group]
            s = np.float64(scale) * (q[b, h] @ kh.T)
            if causal:
                s = np.where(np.arange(Nk)[None, :] > rows[:, None] + off, -np.inf, s)
            p, m, ell = _softmax_two_pass(s)
            o[b, h] = p @ vh
            lse[b, h] = m + np.log(ell)
    return o, lse


def attention_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool = False):
    """Oracle for a batch of sequences of different lengths, packed token-major.

    q: [Tq, H, d]; k, v: [Tk, Hkv, d]; cu_q, cu_k: B+1 nondecreasing token
    offsets. Sequence b is query tokens cu_q[b]..cu_q[b+1]-1 against key tokens
    cu_k[b]..cu_k[b+1]-1 and nothing else (the variable-length batching of the
    vLLM deep dive: sequences are concatenated, not padded, and never attend to
    each other). Within a sequence it is ``attention_gqa``: query head h reads
    K/V head h // (H // Hkv), and with ``causal`` query i sees key j only if
    j <= i + (Nk_b - Nq_b).

    A query that sees no key (an empty key sequence, or causal rows of a
    sequence with more queries than keys) has an empty softmax sum; its O is
    taken as 0 and its LSE as ln 0 = -inf.
    Returns O [Tq, H, d] and LSE [Tq, H] in float64.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    Tq, H, _ = q.shape
    Hkv = k.shape[1]
    assert H % Hkv == 0
    group = H // Hkv
    o = np.zeros((Tq, H, v.shape[-1]))
    lse = np.full((Tq, H), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        nq, nk = q1 - q0, k1 - k0
        if nq == 0 or nk == 0:
            continue
        # visible[i, j]: query i of this sequence may see key j
        visible = np.ones((nq, nk), dtype=bool)
        if causal:
            visible = np.arange(nk)[None, :] <= np.arange(nq)[:, None] + (nk - nq)
        seen = visible.any(axis=1)
        for h in range(H):
            s = np.float64(scale) * (q[q0:q1, h] @ k[k0:k1, h // group].T)   # step 1
            s = np.where(visible, s, -np.inf)[seen]
            p, m, ell = _softmax_two_pass(s)                                   # step 2
            o[q0:q1, h][seen] = p @ v[k0:k1, h // group]                       # step 3
            lse[q0:q1, h][seen] = m + np.log(ell)
    return o, lse
