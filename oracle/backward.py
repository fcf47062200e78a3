"""Backward pass of the DashAttention causal prefill -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` (and the benchmark's CPU-baseline leg) may use this module.
It shares no code with the GPU library.

The pages (DashAttention explainer, gist.science, arXiv 2605.18753, Technical
summary and Contributions) stress that the whole hierarchy is differentiable:
alpha-entmax lets gradients flow from the fine attention back through the
routing to the chunk summaries.  This module writes that chain rule out for
the forward pass of ``oracle.prefill`` (mean pooling, one W_s, prior strength
sigma, near-diagonal window), in IEEE double, one query row at a time:

  Stage 2  o = sum_t P_t v_t,  P = softmax(q.k_t / sqrt(d) + bias_t)
           dv_t += P_t dO;  dl_t = P_t (dO.v_t - dO.o)
           dq += sum_t dl_t k_t / sqrt(d);  dk_t += dl_t q / sqrt(d)
           routed block j carries bias sigma log pbar_j, so
           d pbar_j += sigma * (sum_{t in j} dl_t) / pbar_j
  GQA      pbar = mean of the group's p_h:  dp_h = d pbar / G
  Stage 1  p = alpha-entmax(x), x = (alpha-1) gamma zbar.  On the support,
           dp/dx = (diag(u) - u u^T / sum u) / (alpha - 1) with u = p^(2-alpha)
           (zero off the support), so dzbar = gamma (u dp - u (u.dp) / sum u)
           zbar_j = q.s_j / sqrt(d):  dq += sum_j dzbar_j s_j / sqrt(d);
           ds_j += dzbar_j q / sqrt(d)
  Stage 0  s_j = m_j W_s, m_j = mean of block j's keys:
           dW_s += m_j^T ds_j;  dk_t += (ds_j W_s^T) / bs for t in block j

Blocks with pbar = 0 are masked and take no gradient (the entmax Jacobian
vanishes off the support).  The forward quantities (p, pbar) come from the
pinned forward oracle; the backward arithmetic is plain numpy.

Parity pins (tests/test_oracle_backward.py): central finite differences of
the forward oracle for every input, and the W_s = 0 reduction to the
autograd of dense biased attention.

``prefill_backward_native`` is the same chain rule written out in C
(``oracle_prefill_backward`` in dash_oracle.c, one thread per (sequence, KV
head) pair), for inputs too large for the numpy loops; it carries the same
finite-difference pins and agrees with ``prefill_backward`` to rounding.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _load, _ptr, prefill


def prefill_backward(q, k, v, w_s, d_o, *, bs: int, alpha: float, gamma: float,
                     sigma: float = 1.0, window: int = 1):
    """Gradients of the causal prefill output with respect to q, k, v and W_s.

    q, d_o [B, H, N, d]; k, v [B, Hkv, N, d]; w_s [d, d].  Returns a dict
    with "dq", "dk", "dv" (float64, shapes of q, k, v), "dw_s" [d, d] and the
    forward output "o" [B, H, N, d].
    """
    q = np.asarray(q, np.float32)
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    w_s = np.asarray(w_s, np.float32)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    nb = N // bs
    nbo = max(nb, 1)
    fwd = prefill(q, k, v, w_s, bs=bs, alpha=alpha, gamma=gamma, nb_out=nbo,
                  want=("o", "p", "pbar"), sigma=sigma, window=window)
    p_all = fwd["p"].reshape(B, N, H, nbo)
    pbar_all = fwd["pbar"].reshape(B, N, Hkv, nbo)

    q64, k64, v64 = (a.astype(np.float64) for a in (q, k, v))
    dO = np.asarray(d_o, np.float64)
    ws64 = w_s.astype(np.float64)
    m = k64[:, :, :nb * bs].reshape(B, Hkv, nb, bs, d).mean(axis=3)      # block means
    summ = m @ ws64                                                      # [B, Hkv, nb, d]
    rs = 1.0 / np.sqrt(d)

    dq = np.zeros_like(q64)
    dk = np.zeros_like(k64)
    dv = np.zeros_like(v64)
    ds = np.zeros_like(summ)
    o = np.zeros_like(q64)
    for b in range(B):
        for i in range(N):
            own = i // bs
            win0 = max(own - (window - 1), 0)
            ncand = win0
            for g in range(Hkv):
                pbar = pbar_all[b, i, g, :ncand]
                routed = np.flatnonzero(pbar > 0)
                keys = np.concatenate([np.arange(j * bs, (j + 1) * bs) for j in routed]
                                      + [np.arange(win0 * bs, i + 1)])
                nrt = len(routed) * bs
                bias = np.zeros(len(keys))
                if nrt:
                    bias[:nrt] = sigma * np.repeat(np.log(pbar[routed]), bs)
                dlogpbar = np.zeros(ncand)
                for h in range(g * G, (g + 1) * G):
                    qv = q64[b, h, i]
                    logit = k64[b, g, keys] @ qv * rs + bias
                    P = np.exp(logit - logit.max())
                    P /= P.sum()
                    orow = P @ v64[b, g, keys]
                    o[b, h, i] = orow
                    do = dO[b, h, i]
                    dl = P * (v64[b, g, keys] @ do - do @ orow)
                    dv[b, g, keys] += P[:, None] * do
                    dq[b, h, i] += dl @ k64[b, g, keys] * rs
                    dk[b, g, keys] += dl[:, None] * qv * rs
                    if nrt:
                        dlogpbar[routed] += sigma * dl[:nrt].reshape(-1, bs).sum(axis=1)
                if ncand == 0:
                    continue
                dpbar = np.zeros(ncand)
                dpbar[routed] = dlogpbar[routed] / pbar[routed]
                for h in range(g * G, (g + 1) * G):
                    ph = p_all[b, i, h, :ncand]
                    u = np.where(ph > 0, ph ** (2.0 - alpha), 0.0)
                    dp = dpbar / G
                    dz = gamma * (u * dp - u * (u @ dp) / u.sum())
                    dq[b, h, i] += dz @ summ[b, g, :ncand] * rs
                    ds[b, g, :ncand] += dz[:, None] * q64[b, h, i] * rs
    dws = np.einsum("bgjc,bgje->ce", m, ds)
    dm = ds @ ws64.T
    dk[:, :, :nb * bs] += np.repeat(dm / bs, bs, axis=2)
    return {"dq": dq, "dk": dk, "dv": dv, "dw_s": dws, "o": o, "o_forward": fwd["o"]}


def prefill_backward_native(q, k, v, w_s, d_o, *, bs: int, alpha: float, gamma: float,
                            sigma: float = 1.0, window: int = 1, threads: int = 0):
    """prefill_backward computed by the C oracle: returns "dq", "dk", "dv"
    (float64, shapes of q, k, v) and "dw_s" [d, d]."""
    q = np.ascontiguousarray(q, np.float32)
    k = np.ascontiguousarray(k, np.float32)
    v = np.ascontiguousarray(v, np.float32)
    w_s = np.ascontiguousarray(w_s, np.float32)
    d_o = np.ascontiguousarray(d_o, np.float32)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape or d_o.shape != q.shape:
        raise ValueError("shape mismatch")
    out = {"dq": np.empty(q.shape), "dk": np.empty(k.shape), "dv": np.empty(v.shape),
           "dw_s": np.empty((d, d))}
    fp, dp = ctypes.c_float, ctypes.c_double
    rc = _load().oracle_prefill_backward(
        _ptr(q, fp), _ptr(k, fp), _ptr(v, fp), _ptr(w_s, fp), _ptr(d_o, fp), B, H, Hkv, N, d,
        bs, float(alpha), float(gamma), float(sigma), int(window), _ptr(out["dq"], dp),
        _ptr(out["dk"], dp), _ptr(out["dv"], dp), _ptr(out["dw_s"], dp), int(threads))
    if rc != 0:
        raise ValueError("oracle_prefill_backward rejected its arguments")
    return out
