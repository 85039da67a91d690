"""Plain fp64 CPU attention forward: the oracle that parity tests trust.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module. The product path never
calls it, and it imports nothing from the HIP package.

What it computes, per batch b, head h and query row i (sources are the pages
this project is built from):

* "[GPU] Deep Learning for HPC", section "Flash Attention": attention multiplies
  Q by K transposed to form the score matrix, applies softmax to it, then
  multiplies the result by V.
* null-ptr.tistory.com, category "development", teaser of the softmax post:
  softmax_i(z) = e^{z_i} / sum_j e^{z_j}; the exponential overflows for large
  inputs, so the maximum is subtracted first (the text is cut off; this is the
  standard reading and it leaves the value unchanged).
* Same page, teaser of the Triton FlashAttention post: the forward kernel takes
  a ``softmax_scale``, an ``IS_CAUSAL`` flag and writes ``Out`` and ``Lse``.

Readings taken where the pages are silent (each is listed in the design notes):

* ``scale`` multiplies Q K^T before masking and softmax.
* causal: key j is visible to query i iff j <= i (queries and keys share one
  position axis); masked keys get weight exactly 0. With M queries and N keys
  (M != N) the two axes are aligned at their ends: query i sits at position
  i + (N - M) on the key axis. A query that then sees no key at all gets
  o = 0 and lse = -inf (the empty sum).
* lse is the natural log of sum_j exp(s_ij) over the visible keys, using the
  scaled scores.

The score row is materialised in full (no online recurrence, no tiling), rows
are processed in chunks only to bound memory.

The backward (``attend_head_grad``) is the derivative of that same definition,
written out with the chain rule; the pages call the FlashAttention backward
much harder than the forward (Hacker News comments on the "GPUの爆発的な性能向上"
page) and print nothing of it. For L = sum(dO * O), with P the softmax
weights (masked entries 0):
  dV = P^T dO;  dP = dO V^T;  dS = P * (dP - rowsum(P * dP));
  dQ = scale * dS K;  dK = scale * dS^T Q.
The last factor of dS is the Jacobian-vector product of a softmax row. A row
that sees no key has P = 0 and contributes nothing. Because O = P V, that row
term also equals rowsum(dO * O): a backward handed the stored output O (as
the FlashAttention backward is) may form it from O, and ``attend_head_grad``
does so when given an ``o``.
"""

from __future__ import annotations

import numpy as np

__all__ = ["attend_head", "attention_ref", "attend_head_grad", "attention_grad_ref"]


def attend_head(q, k, v, scale, causal, q_pos=None, return_weights=False,
                chunk=1024):
    """Attention of one head: returns (o [M,d], lse [M]) in float64.

    q: [M, d] query rows; k, v: [N, d] keys and values of the head.
    scale: the softmax scale (used as given, widened to float64).
    causal: if true, query row r sees keys 0..q_pos[r] only (none if q_pos[r]
      is negative: that row gets o = 0, lse = -inf).
    q_pos: position of each query row on the key axis (default r + N - M, the
      M queries aligned with the end of the N keys; r for M == N). Lets a
      test check a sample of rows.
    return_weights: also return the normalised weights [M, N] (debug aid).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    scale = float(scale)
    m_rows, d = q.shape
    n_keys = k.shape[0]
    if k.shape != (n_keys, d) or v.shape[0] != n_keys:
        raise ValueError("q, k, v shapes do not agree")
    if q_pos is None:
        q_pos = np.arange(m_rows) + (n_keys - m_rows)
    q_pos = np.asarray(q_pos, dtype=np.int64)

    o = np.empty((m_rows, v.shape[1]), dtype=np.float64)
    lse = np.empty(m_rows, dtype=np.float64)
    weights = np.empty((m_rows, n_keys), dtype=np.float64) if return_weights else None
    key_idx = np.arange(n_keys)
    for r0 in range(0, m_rows, chunk):
        r1 = min(r0 + chunk, m_rows)
        # scores s_ij = scale * <q_i, k_j> over the full key axis
        s = scale * (q[r0:r1] @ k.T)
        if causal:
            hidden = key_idx[None, :] > q_pos[r0:r1, None]
            s[hidden] = -np.inf
        # safe softmax: subtract the row maximum, exponentiate, normalise
        m = s.max(axis=1, keepdims=True) if n_keys else np.full((r1 - r0, 1), -np.inf)
        empty = ~np.isfinite(m[:, 0]) & (m[:, 0] < 0)  # no visible key
        m[empty] = 0.0
        w = np.exp(s - m)  # masked entries: exp(-inf) == 0 exactly
        l = w.sum(axis=1, keepdims=True)
        l[empty] = 1.0  # empty sum: o = 0 below, lse = -inf
        o[r0:r1] = (w @ v) / l
        lse[r0:r1] = m[:, 0] + np.log(l[:, 0])
        lse[r0:r1][empty] = -np.inf
        if return_weights:
            weights[r0:r1] = w / l
    if return_weights:
        return o, lse, weights
    return o, lse


def attention_ref(q, k, v, scale, causal):
    """Attention over a batch: q [B, H, M, d], k and v [B, H, N, d]; returns
    (o [B,H,M,d], lse [B,H,M]). M == N is the usual self-attention shape.

    Every (b, h) pair is an independent head; each is handed to attend_head.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    if (q.ndim != 4 or k.ndim != 4 or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]
            or v.shape[:3] != k.shape[:3]):
        raise ValueError("expected q [B, H, M, d] and k, v [B, H, N, d]")
    b_n, h_n, n, _ = q.shape
    o = np.empty((b_n, h_n, n, v.shape[3]), dtype=np.float64)
    lse = np.empty((b_n, h_n, n), dtype=np.float64)
    for b in range(b_n):
        for h in range(h_n):
            o[b, h], lse[b, h] = attend_head(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse


def attend_head_grad(q, k, v, do, scale, causal, q_pos=None, chunk=1024, o=None):
    """Gradients of one head: returns (dq [M,d], dk [N,d], dv [N,d]) in float64,
    of L = sum(do * o) with o the output of attend_head(q, k, v, scale, causal).

    The weights are recomputed from the definition exactly as attend_head
    forms them (full score rows, masked entries -inf, max subtracted); then
    the chain rule of the module docstring. q_pos as for attend_head.

    o: optional [M, d] stored forward output. When given, each row's softmax
    term is rowsum(do * o) instead of rowsum(P * dP): the same value for the
    exact output, and for a rounded one the result of the backward formula
    applied to the output it is handed.

    L is a sum over query rows, and a row's weights depend on that row alone,
    so the rows are taken ``chunk`` at a time only to bound memory: each chunk
    gives its rows' dq outright and adds its rows' share of dk and dv (the
    sums over i in dV = P^T dO and dK = scale dS^T Q, split by rows).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    scale = float(scale)
    m_rows, d = q.shape
    n_keys = k.shape[0]
    if k.shape != (n_keys, d) or v.shape[0] != n_keys or do.shape != (m_rows, v.shape[1]):
        raise ValueError("q, k, v, do shapes do not agree")
    if q_pos is None:
        q_pos = np.arange(m_rows) + (n_keys - m_rows)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    if o is not None:
        o = np.asarray(o, dtype=np.float64)
        if o.shape != do.shape:
            raise ValueError("o must be shaped like do")

    dq = np.empty((m_rows, d), dtype=np.float64)
    dk = np.zeros((n_keys, d), dtype=np.float64)
    dv = np.zeros((n_keys, v.shape[1]), dtype=np.float64)
    key_idx = np.arange(n_keys)
    for r0 in range(0, m_rows, chunk):
        r1 = min(r0 + chunk, m_rows)
        # softmax weights P of these rows over the full key axis
        s = scale * (q[r0:r1] @ k.T)
        if causal:
            s[key_idx[None, :] > q_pos[r0:r1, None]] = -np.inf
        if n_keys:
            m = s.max(axis=1, keepdims=True)
        else:
            m = np.full((r1 - r0, 1), -np.inf)
        empty = np.isneginf(m[:, 0])
        m[empty] = 0.0
        w = np.exp(s - m)
        l = w.sum(axis=1, keepdims=True)
        l[empty] = 1.0
        p = w / l  # rows that see no key: all zero

        dv += p.T @ do[r0:r1]
        dp = do[r0:r1] @ v.T
        if o is None:
            row = (p * dp).sum(axis=1, keepdims=True)
        else:
            row = (do[r0:r1] * o[r0:r1]).sum(axis=1, keepdims=True)
        ds = p * (dp - row)
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv


def attention_grad_ref(q, k, v, do, scale, causal):
    """Gradients over a batch: q, do [B, H, M, d], k and v [B, H, N, d]; returns
    (dq, dk, dv) in float64, each head handed to attend_head_grad."""
    q, k, v, do = (np.asarray(t) for t in (q, k, v, do))
    if (q.ndim != 4 or k.ndim != 4 or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]
            or v.shape[:3] != k.shape[:3] or do.shape != q.shape[:3] + (v.shape[3],)):
        raise ValueError("expected q, do [B, H, M, d] and k, v [B, H, N, d]")
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(k.shape, dtype=np.float64)
    dv = np.empty(v.shape, dtype=np.float64)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            dq[b, h], dk[b, h], dv[b, h] = attend_head_grad(q[b, h], k[b, h], v[b, h], do[b, h],
                                                            scale, causal)
    return dq, dk, dv
