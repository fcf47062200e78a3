"""Pins of the oracle's backward pass (oracle/backward.py).

Pages: DashAttention explainer (gist.science, arXiv 2605.18753), Technical
summary (alpha-entmax is differentiable, so gradients reach the chunk
summaries through the routing) and Contributions (end-to-end differentiable
sparse attention).

  * central finite differences of the pinned forward oracle, for q, k, v and
    W_s, with a loss sum(o * R), on inputs whose routing is sparse (masked
    blocks present), for several alpha, sigma, window and GQA settings;
  * W_s = 0: every summary is 0, the routing is uniform and the prior is a
    constant per query, so dq, dk, dv equal PyTorch autograd (float64, CPU)
    of dense attention with that fixed bias, and dW_s is the only gradient
    left in the routing path.

Both writings of the backward carry these pins: the numpy loops
(prefill_backward) and the C one (prefill_backward_native, which the GPU
parity tests use at sizes the numpy loops cannot finish).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.backward import prefill_backward, prefill_backward_native

H_FD = 2.0 ** -10      # exact offset on float32 inputs of magnitude < 2^13


def inputs(B, H, Hkv, N, d, seed, qscale=1.0):
    rng = np.random.default_rng(seed)
    q = (qscale * rng.standard_normal((B, H, N, d))).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    ws = (np.eye(d) + 0.3 * rng.standard_normal((d, d))).astype(np.float32)
    # float32 values, exact in both writings of the backward
    R = rng.standard_normal((B, H, N, d)).astype(np.float32).astype(np.float64)
    return q, k, v, ws, R


IMPLS = {"numpy": prefill_backward, "native": prefill_backward_native}


def loss(q, k, v, ws, R, kw):
    r = oracle.prefill(q, k, v, ws, **kw)
    B, H, N, d = q.shape
    o = r["o"].reshape(B, N, H, d).transpose(0, 2, 1, 3)
    return float((o * R).sum())


CASES = [
    dict(alpha=1.5, gamma=6.0, sigma=1.0, window=1, H=2, Hkv=1, seed=11),
    dict(alpha=2.0, gamma=5.0, sigma=1.0, window=1, H=2, Hkv=2, seed=12),
    dict(alpha=1.5, gamma=6.0, sigma=0.5, window=2, H=4, Hkv=2, seed=13),
    dict(alpha=1.25, gamma=8.0, sigma=2.0, window=1, H=2, Hkv=1, seed=14),
]


@pytest.mark.parametrize("impl", list(IMPLS))
@pytest.mark.parametrize("case", range(len(CASES)))
def test_gradients_match_finite_differences(case, impl):
    c = CASES[case]
    N, d, bs = 80, 8, 16
    q, k, v, ws, R = inputs(1, c["H"], c["Hkv"], N, d, c["seed"], qscale=2.0)
    kw = dict(bs=bs, alpha=c["alpha"], gamma=c["gamma"], sigma=c["sigma"], window=c["window"])
    g = IMPLS[impl](q, k, v, ws, R, **kw)
    if impl == "numpy":
        # the backward's own forward agrees with the oracle's
        np.testing.assert_allclose(g["o"].transpose(0, 2, 1, 3).reshape(-1, c["H"], d),
                                   g["o_forward"], rtol=0, atol=1e-12)
    pb = oracle.prefill(q, k, v, ws, nb_out=N // bs, want=("o", "pbar"), **kw)["pbar"]
    assert (pb[bs * c["window"]:] == 0).any(), "expected masked blocks"
    rng = np.random.default_rng(100 + case)
    arrays = {"dq": q, "dk": k, "dv": v, "dw_s": ws}
    for name, arr in arrays.items():
        for _ in range(12):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += H_FD
            minus[idx] -= H_FD
            args = {"dq": (q, k, v, ws), "dk": (q, k, v, ws), "dv": (q, k, v, ws),
                    "dw_s": (q, k, v, ws)}[name]
            pos = list(args)
            which = ["dq", "dk", "dv", "dw_s"].index(name)
            pos[which] = plus
            lp = loss(*pos, R, kw)
            pos[which] = minus
            lm = loss(*pos, R, kw)
            fd = (lp - lm) / (2 * H_FD)
            an = g[name][idx]
            assert abs(fd - an) <= 2e-4 * max(1.0, abs(an)), f"{name}{idx}: fd {fd} vs {an}"


@pytest.mark.parametrize("impl", list(IMPLS))
@pytest.mark.parametrize("sigma,window", [(1.0, 1), (0.5, 2)])
def test_zero_projection_matches_autograd_of_dense_attention(sigma, window, impl):
    N, d, bs = 96, 16, 16
    q, k, v, _, R = inputs(1, 2, 1, N, d, 21)
    ws = np.zeros((d, d), np.float32)
    g = IMPLS[impl](q, k, v, ws, R, bs=bs, alpha=1.5, gamma=3.0, sigma=sigma, window=window)
    i = np.arange(N)[:, None]
    t = np.arange(N)[None, :]
    ncand = np.maximum(i // bs - (window - 1), 0)
    routed = t < ncand * bs
    branch = (t >= ncand * bs) & (t <= i)
    bias = torch.from_numpy(np.where(routed, -sigma * np.log(np.maximum(ncand, 1)), 0.0))
    mask = torch.from_numpy(routed | branch)
    qt = torch.tensor(q[0], dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k[0, 0], dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v[0, 0], dtype=torch.float64, requires_grad=True)
    logits = qt @ kt.T / np.sqrt(d) + bias                       # [2, N, N]
    logits = logits.masked_fill(~mask, float("-inf"))
    o = torch.softmax(logits, dim=-1) @ vt
    (o * torch.from_numpy(R[0])).sum().backward()
    np.testing.assert_allclose(g["dq"][0], qt.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(g["dk"][0, 0], kt.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(g["dv"][0, 0], vt.grad.numpy(), rtol=0, atol=1e-10)
    assert np.abs(g["dw_s"]).max() > 0          # the routing still has a gradient


@pytest.mark.parametrize("case", [dict(B=2, H=4, Hkv=2, N=100, d=8, bs=16, alpha=2.0, gamma=5.0,
                                       sigma=0.5, window=2),
                                  dict(B=1, H=8, Hkv=2, N=130, d=16, bs=32, alpha=1.25,
                                       gamma=8.0, sigma=1.0, window=1)])
def test_native_agrees_with_numpy(case):
    c = dict(case)
    B, H, Hkv, N, d = (c.pop(x) for x in ("B", "H", "Hkv", "N", "d"))
    q, k, v, ws, R = inputs(B, H, Hkv, N, d, 31, qscale=2.0)
    a = prefill_backward(q, k, v, ws, R, **c)
    b = prefill_backward_native(q, k, v, ws, R, **c)
    for name in ("dq", "dk", "dv", "dw_s"):
        np.testing.assert_allclose(b[name], a[name], rtol=0, atol=1e-12 * np.abs(a[name]).max())
