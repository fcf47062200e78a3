"""Pins of the oracle's prior strength sigma and near-diagonal window W.

Pages: DashAttention explainer (gist.science, arXiv 2605.18753), Technical
summary, Stage 2 (prior-induced sparse softmax): a hyperparameter sigma sets
how strongly the routing prior weighs against a uniform baseline, and chunks
near the diagonal, which may lack summaries, go through a separate branch.

Readings: the routed-block bias is sigma * log pbar (reference distribution
proportional to pbar^sigma on the support; sigma = 0 keeps only the mask);
the branch holds the own block and the W - 1 blocks before it (bias 0,
token-causal), and routing candidates are the blocks before the branch.

Pins (each against brute force or an independent solve, not a retyped formula):
  * W_s = 0 makes the routing uniform over the C = max(0, own - W + 1)
    candidates: a dense causal softmax with bias -sigma log C on the
    candidates' keys and 0 on the branch, for several (sigma, W);
  * W at least the number of blocks gives plain causal attention;
  * the general case equals a dense masked softmax whose bias is
    sigma * log pbar of each key's block (pbar read from the oracle's routing,
    which W and sigma must leave consistent: the candidates end before the
    branch and sigma does not touch Stage 1);
  * the Stage 2 weights maximise z.p - KL(p || g) with g proportional to
    pbar^sigma (SLSQP), for sigma in {0, 0.5, 2};
  * sigma = 1, W = 1 reproduces the default call bit for bit.
"""
import numpy as np
import pytest
from scipy.optimize import minimize

import oracle
import workloads as W
from brute import dense_attention


def rand_inputs(B, H, Hkv, N, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    ws = (np.eye(d) + 0.05 * rng.standard_normal((d, d))).astype(np.float32)
    return q, k, v, ws


@pytest.mark.parametrize("sigma,window", [(1.0, 2), (0.5, 1), (2.0, 3), (0.0, 2), (1.0, 4)])
def test_uniform_routing_with_window_and_strength(sigma, window):
    N, d, bs = 256, 16, 16
    q, k, v, _ = rand_inputs(1, 2, 1, N, d, 101)
    r = oracle.prefill(q, k, v, np.zeros((d, d), np.float32), bs=bs, alpha=1.5, gamma=1.0,
                       sigma=sigma, window=window)
    o = r["o"].reshape(N, 2, d)
    i = np.arange(N)[:, None]
    t = np.arange(N)[None, :]
    ncand = np.maximum(i // bs - (window - 1), 0)
    routed = t < ncand * bs
    branch = (t >= ncand * bs) & (t <= i)
    bias = np.where(routed, -sigma * np.log(np.maximum(ncand, 1)), 0.0)
    for h in range(2):
        ref = dense_attention(q[0, h], k[0, 0], v[0, 0], bias=bias, mask=routed | branch)
        np.testing.assert_allclose(o[:, h], ref, atol=1e-12)
    # rows whose branch covers every earlier block have nothing to route
    no_route = (np.arange(N) // bs) < window
    assert np.all(np.isnan(r["tau"][no_route]))
    assert np.all(np.isfinite(r["tau"][~no_route]))


def test_window_covering_everything_is_causal_attention():
    N, d, bs = 192, 16, 32
    q, k, v, ws = rand_inputs(1, 2, 2, N, d, 102)
    r = oracle.prefill(q, k, v, ws, bs=bs, alpha=1.5, gamma=5.0, window=N // bs)
    o = r["o"].reshape(N, 2, d)
    mask = np.tril(np.ones((N, N), bool))
    for h in range(2):
        np.testing.assert_allclose(o[:, h], dense_attention(q[0, h], k[0, h], v[0, h], mask=mask),
                                   atol=1e-12)


@pytest.mark.parametrize("sigma,window", [(0.5, 2), (2.0, 1), (0.0, 3), (1.0, 2)])
def test_general_case_is_dense_masked_softmax(sigma, window):
    w = W.get("tiny").replace(seq_len=512, head_dim=32, n_heads=4, n_kv_heads=2,
                              planted=True, block_size=32)
    inp = W.make_prefill(w)
    N, bs, nb = 512, 32, 16
    r = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["w_s"], bs=bs, alpha=1.5, gamma=6.0,
                       nb_out=nb, want=("o", "tau", "pbar"), sigma=sigma, window=window)
    pbar = r["pbar"]                                   # [N, Hkv, nb]
    o = r["o"].reshape(N, 4, 32)
    t = np.arange(N)
    kb, qb = t[None, :] // bs, t[:, None] // bs
    branch = (kb > qb - window) & (t[None, :] <= t[:, None])
    cand = kb <= qb - window
    # routing never reaches into the branch
    for g in range(2):
        pk = pbar[:, g, t // bs]                       # [N, N]
        assert not np.any((pk > 0) & ~cand)
    for h in range(4):
        g = h // 2
        pk = pbar[:, g, t // bs]
        routed = cand & (pk > 0)
        with np.errstate(divide="ignore"):
            bias = np.where(branch, 0.0, sigma * np.log(np.where(routed, pk, 1.0)))
        ref = dense_attention(inp["q"][0, h], inp["k"][0, g], inp["v"][0, g], bias=bias,
                              mask=branch | routed)
        np.testing.assert_allclose(o[:, h], ref, atol=1e-12)
    # Stage 1 does not depend on sigma: same thresholds as sigma = 1
    r1 = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["w_s"], bs=bs, alpha=1.5, gamma=6.0,
                        window=window)
    np.testing.assert_array_equal(np.isnan(r["tau"]), np.isnan(r1["tau"]))
    np.testing.assert_allclose(r["tau"], r1["tau"], atol=0, equal_nan=True)


@pytest.mark.parametrize("sigma", [0.0, 0.5, 2.0])
def test_prior_strength_is_the_gibbs_maximiser(sigma):
    """Stage 2 weights (one-hot values) maximise z.p - KL(p || g) with
    g proportional to pbar^sigma on the routed keys (independent SLSQP solve)."""
    d, bs, N = 64, 4, 32
    rng = np.random.default_rng(103)
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    v = np.eye(N, d, dtype=np.float32)[None, None]
    ws = (np.eye(d) + 0.3 * rng.standard_normal((d, d))).astype(np.float32)
    i = N - 1
    r = oracle.prefill(q, k, v, ws, bs=bs, alpha=1.5, gamma=1.0, causal=False, positions=[i],
                       nb_out=N // bs, want=("o", "pbar"), sigma=sigma)
    wts = r["o"][0, 0, :N]
    pbar = r["pbar"][0, 0]
    routed = np.repeat(pbar > 0, bs)
    assert 1 < (pbar > 0).sum() < N // bs
    z = (k[0, 0].astype(np.float64) @ q[0, 0, i].astype(np.float64)) / np.sqrt(d)
    gk = np.repeat(np.where(pbar > 0, pbar, 1.0) ** sigma, bs)
    zr, gr = z[routed], gk[routed] / gk[routed].sum()
    obj = lambda p: -(p @ zr - np.sum(np.where(p > 0, p * np.log(np.maximum(p, 1e-300) / gr), 0)))
    res = minimize(obj, gr, method="SLSQP", bounds=[(0, 1)] * len(zr),
                   constraints=[{"type": "eq", "fun": lambda p: p.sum() - 1}],
                   options={"ftol": 1e-15, "maxiter": 1000})
    np.testing.assert_allclose(wts[routed], res.x, atol=2e-5)
    assert np.all(wts[~routed] == 0)


def test_defaults_are_sigma_one_window_one():
    q, k, v, ws = rand_inputs(1, 4, 2, 320, 16, 104)
    a = oracle.prefill(q, k, v, ws, bs=64, alpha=1.5, gamma=6.0)
    b = oracle.prefill(q, k, v, ws, bs=64, alpha=1.5, gamma=6.0, sigma=1.0, window=1)
    np.testing.assert_array_equal(a["o"], b["o"])
    # and sigma changes the output once something is routed
    c = oracle.prefill(q, k, v, ws, bs=64, alpha=1.5, gamma=6.0, sigma=0.5)
    assert np.abs(c["o"][64:] - a["o"][64:]).max() > 1e-6


def test_decode_with_window_and_strength_is_last_prefill_row():
    w = W.get("tiny").replace(seq_len=384, head_dim=32, n_heads=4, n_kv_heads=2)
    inp = W.make_prefill(w)
    for L in (1, 64, 65, 130, 300, 384):
        kw = dict(bs=64, alpha=1.5, gamma=8.0, sigma=0.7, window=2)
        dec = oracle.decode(inp["q"][:, :, L - 1], inp["k"], inp["v"], [L], inp["w_s"], **kw)
        pre = oracle.prefill(inp["q"][:, :, :L], inp["k"][:, :, :L], inp["v"][:, :, :L],
                             inp["w_s"], positions=[L - 1], **kw)
        np.testing.assert_array_equal(dec["o"], pre["o"])


def test_invalid_strength_and_window_rejected():
    q, k, v, ws = rand_inputs(1, 2, 2, 64, 16, 105)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, ws, bs=32, alpha=1.5, gamma=1.0, sigma=-0.5)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, ws, bs=32, alpha=1.5, gamma=1.0, window=0)
