"""fp64 reference of the hybrids' attention layer -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the bench's CPU-baseline leg may use
this module; the GPU library never loads it and shares no code with it.

What it computes.  The hybrid backbones put multi-head softmax attention
between the bidirectional Mamba-2 blocks: full bidirectional attention in
the hybrid checkpoints ("DiffMamba Checkpoints" model card, section "Hybrid
Mamba+attention checkpoints"; "DiffuMamba: High-Throughput Diffusion LMs with
Mamba Backbone", Technical Summary, Core Architecture: one multi-head
attention block every five Mamba blocks), and block-wise attention in the
block-diffusion hybrids ("Training Hybrid Block Diffusion Language Models
with Partial Bidirectionality", Methodology: the BDLM attention baseline,
whose active block sees the cached prefix and itself).  Per batch row b and
head h, with queries Q, keys K and values V (L x D each):

    O = softmax(scale * Q K^T + M) V          (softmax over the keys)

M[t, s] = 0 where query t may see key s, -inf elsewhere: everywhere for full
bidirectional attention; for block-wise attention with blocks of `block`
tokens, where floor(s / block) <= floor(t / block) (the query's own block and
every block before it).  scale defaults to 1 / sqrt(D).  Layout as the GPU
library's: q, k, v, o [Z, L, H, D].

Written as the definition: the scores, an explicit row maximum subtracted
before exp (the textbook stable form of the same softmax), normalisation,
and the product with V, in numpy float64.

Backward: the reverse-mode derivative of that definition for a loss with
gradient dO (plain matrix calculus of softmax, no source on the pages):
    P = softmax(S), S = scale Q K^T + M
    dV = P^T dO,   dP = dO V^T,   dS = P * (dP - rowsum(dP * P))
    dQ = scale dS K,   dK = scale dS^T Q
and rowsum(dP * P) = rowsum(dO * O) for each query.
"""
from __future__ import annotations

import numpy as np


def visible(L: int, block: int = 0) -> np.ndarray:
    """[L, L] bool: query t (row) may see key s (column)."""
    if block <= 0:
        return np.ones((L, L), dtype=bool)
    blk = np.arange(L) // block
    return blk[None, :] <= blk[:, None]


def forward(q, k, v, block: int = 0, scale: float | None = None) -> np.ndarray:
    """O = softmax(scale Q K^T + M) V per (batch row, head), float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Z, L, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    vis = visible(L, block)
    out = np.empty((Z, L, H, D))
    for b in range(Z):
        for h in range(H):
            s = scale * (q[b, :, h] @ k[b, :, h].T)
            s = np.where(vis, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[b, :, h] = p @ v[b, :, h]
    return out


def _probs(q, k, vis, scale):
    s = scale * (q @ k.T)
    s = np.where(vis, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


def backward(q, k, v, do, block: int = 0, scale: float | None = None) -> dict:
    """Gradients dq, dk, dv of sum(dO * O) for O = forward(q, k, v), float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    Z, L, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    vis = visible(L, block)
    g = {n: np.empty((Z, L, H, D)) for n in ("dq", "dk", "dv")}
    for b in range(Z):
        for h in range(H):
            p = _probs(q[b, :, h], k[b, :, h], vis, scale)
            g["dv"][b, :, h] = p.T @ do[b, :, h]
            dp = do[b, :, h] @ v[b, :, h].T
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
            g["dq"][b, :, h] = scale * (ds @ k[b, :, h])
            g["dk"][b, :, h] = scale * (ds.T @ q[b, :, h])
    return g

