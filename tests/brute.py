"""Brute-force dense attention in float64 numpy, for pinning the oracle.

Independent of ``oracle/``: builds the full N x N logit matrix with an explicit
additive bias and a boolean mask, and applies a max-subtracted softmax.
"""
import numpy as np


def dense_attention(q, k, v, bias=None, mask=None):
    """q [Nq, d], k/v [Nk, d]; bias/mask [Nq, Nk]; returns [Nq, d] float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    logits = q @ k.T / np.sqrt(q.shape[-1])
    if bias is not None:
        logits = logits + bias
    if mask is not None:
        logits = np.where(mask, logits, -np.inf)
    m = logits.max(axis=-1, keepdims=True)
    w = np.exp(logits - m)
    return (w / w.sum(axis=-1, keepdims=True)) @ v


def softmax(z):
    z = np.asarray(z, np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()
