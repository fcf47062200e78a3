"""Pins of the oracle's Stage 0 (block summaries) and Stage 2 (prior-induced
sparse softmax) against brute force and closed forms.

Pages: DashAttention explainer (gist.science, arXiv 2605.18753), Technical
summary -- Stage 0 (local chunk summarization: a zero-initialised learned
query pools a chunk uniformly), Stage 1 (GQA heads average their routing
probabilities), Stage 2 (softmax as argmax z.p - KL(p||u) with u replaced by a
routing-derived g; g = 0 where w = 0 masks the chunk; near-diagonal chunks get
their own branch).
"""
import numpy as np
import pytest
from scipy.optimize import minimize

import oracle
import workloads as W
from brute import dense_attention, softmax


def rand_inputs(B, H, Hkv, N, d, seed, scale_q=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, H, N, d)) * scale_q).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    ws = (np.eye(d) + 0.05 * rng.standard_normal((d, d))).astype(np.float32)
    return q, k, v, ws


# --------------------------------------------------------------------------
# Stage 0
# --------------------------------------------------------------------------

def test_summary_identity_projection_is_block_mean():
    _, k, _, _ = rand_inputs(2, 2, 2, 256, 16, 1)
    s = oracle.summaries(k, np.eye(16, dtype=np.float32), 64, 4)
    ref = k.astype(np.float64).reshape(2, 2, 4, 64, 16).mean(axis=3)
    np.testing.assert_allclose(s, ref, rtol=0, atol=1e-14)


def test_summary_of_constant_block_is_row_times_ws():
    rng = np.random.default_rng(2)
    d, bs = 8, 32
    rows = rng.standard_normal((3, d)).astype(np.float32)
    k = np.repeat(rows, bs, axis=0)[None, None]           # blocks of identical rows
    ws = rng.standard_normal((d, d)).astype(np.float32)
    s = oracle.summaries(k, ws, bs, 3)[0, 0]
    np.testing.assert_allclose(s, rows.astype(np.float64) @ ws.astype(np.float64), atol=1e-12)


def test_summary_only_complete_blocks():
    _, k, _, ws = rand_inputs(1, 1, 1, 100, 8, 3)
    with pytest.raises(ValueError):
        oracle.summaries(k, ws, 64, 2)


# --------------------------------------------------------------------------
# dense equivalences
# --------------------------------------------------------------------------

@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_noncausal_uniform_routing_is_dense_attention(alpha):
    """W_s = 0 makes every coarse score equal, entmax uniform over all blocks,
    every key gets the same bias -log nb: exactly dense attention."""
    q, k, v, _ = rand_inputs(1, 4, 2, 256, 32, 4)
    ws = np.zeros((32, 32), np.float32)
    r = oracle.prefill(q, k, v, ws, bs=64, alpha=alpha, gamma=3.0, causal=False)
    o = r["o"].reshape(1, 256, 4, 32).transpose(0, 2, 1, 3)
    for h in range(4):
        ref = dense_attention(q[0, h], k[0, h // 2], v[0, h // 2])
        np.testing.assert_allclose(o[0, h], ref, atol=1e-12)


@pytest.mark.parametrize("bs", [16, 64])
def test_causal_uniform_routing_is_biased_dense_causal(bs):
    """Causal, W_s = 0: p = 1/|C(i)| on every earlier block, so routed keys get
    bias -log|C(i)|, own-block keys (t <= i) bias 0, later keys are masked."""
    N, d = 256, 16
    q, k, v, _ = rand_inputs(1, 2, 1, N, d, 5)
    r = oracle.prefill(q, k, v, np.zeros((d, d), np.float32), bs=bs, alpha=1.5, gamma=1.0)
    o = r["o"].reshape(N, 2, d)
    i = np.arange(N)[:, None]
    t = np.arange(N)[None, :]
    ncand = i // bs
    routed = t < ncand * bs
    own = (t >= ncand * bs) & (t <= i)
    bias = np.where(routed, -np.log(np.maximum(ncand, 1)), 0.0)
    for h in range(2):
        ref = dense_attention(q[0, h], k[0, 0], v[0, 0], bias=bias, mask=routed | own)
        np.testing.assert_allclose(o[:, h], ref, atol=1e-12)
    assert np.all(np.isnan(r["tau"][:bs]))          # first block: nothing to route
    assert np.all(np.isfinite(r["tau"][bs:]))


@pytest.mark.parametrize("alpha,gamma", [(1.5, 6.0), (2.0, 4.0), (1.25, 10.0)])
def test_block_sparse_equals_dense_masked_softmax(alpha, gamma):
    """General case: the sparse Stage 2 equals a dense N x N softmax whose bias
    matrix holds log pbar of each key's block, -inf where pbar = 0, and 0 on
    the causal part of the own block."""
    w = W.get("tiny").replace(seq_len=512, head_dim=32, n_heads=4, n_kv_heads=2,
                              planted=True, block_size=32)
    inp = W.make_prefill(w)
    N, bs, nb = 512, 32, 16
    r = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["w_s"], bs=bs, alpha=alpha,
                       gamma=gamma, nb_out=nb, want=("o", "tau", "pbar"))
    pbar = r["pbar"]                                   # [N, Hkv, nb]
    o = r["o"].reshape(N, 4, 32)
    t = np.arange(N)
    for h in range(4):
        g = h // 2
        pk = pbar[:, g, t // bs]                       # [N, N] pbar of each key's block
        own = (t[None, :] // bs == t[:, None] // bs) & (t[None, :] <= t[:, None])
        routed = (t[None, :] // bs < t[:, None] // bs) & (pk > 0)
        with np.errstate(divide="ignore"):
            bias = np.where(own, 0.0, np.log(pk))
        ref = dense_attention(inp["q"][0, h], inp["k"][0, g], inp["v"][0, g], bias=bias,
                              mask=own | routed)
        np.testing.assert_allclose(o[:, h], ref, atol=1e-12)
    sel = (pbar > 0).sum(-1)
    assert sel[bs:].min() < sel[bs:].max()            # adaptive support: sizes vary


def test_first_block_rows_are_plain_causal_attention():
    q, k, v, ws = rand_inputs(1, 2, 2, 128, 16, 6)
    r = oracle.prefill(q, k, v, ws, bs=64, alpha=1.5, gamma=2.0, positions=np.arange(64))
    o = r["o"].reshape(64, 2, 16)
    mask = np.tril(np.ones((64, 64), bool))
    for h in range(2):
        ref = dense_attention(q[0, h, :64], k[0, h, :64], v[0, h, :64], mask=mask)
        np.testing.assert_allclose(o[:, h], ref, atol=1e-12)


# --------------------------------------------------------------------------
# coarse scores, GQA, prior
# --------------------------------------------------------------------------

def test_coarse_score_of_constant_block_is_its_fine_logit():
    """With W_s = I and blocks of identical keys, a block's summary is its key,
    so zbar_j = q . k_j / sqrt(d), the dense attention logit; routing then is
    the entmax of gamma times those logits (SLSQP-free: alpha = 2 closed form
    checked against a direct sparsemax by sorting in numpy)."""
    rng = np.random.default_rng(7)
    d, bs, nb = 16, 8, 6
    keys = rng.standard_normal((nb, d)).astype(np.float32)
    k = np.repeat(keys, bs, axis=0)[None, None]
    v = rng.standard_normal(k.shape).astype(np.float32)
    q = rng.standard_normal((1, 1, nb * bs, d)).astype(np.float32)
    i = nb * bs - 1
    gamma = 2.5
    r = oracle.prefill(q, k, v, np.eye(d, dtype=np.float32), bs=bs, alpha=2.0, gamma=gamma,
                       positions=[i], nb_out=nb, want=("o", "x", "p"))
    logits = keys[: nb - 1].astype(np.float64) @ q[0, 0, i].astype(np.float64) / np.sqrt(d)
    np.testing.assert_allclose(r["x"][0, 0, : nb - 1], gamma * logits, atol=1e-12)
    y = np.sort(gamma * logits)[::-1]
    ks = np.arange(1, len(y) + 1)
    kstar = ks[1 + ks * y > np.cumsum(y)].max()
    tau = (y[:kstar].sum() - 1) / kstar
    np.testing.assert_allclose(r["p"][0, 0, : nb - 1], np.maximum(gamma * logits - tau, 0),
                               atol=1e-12)


def test_gqa_heads_share_the_averaged_support():
    q, k, v, ws = rand_inputs(1, 4, 2, 256, 16, 8, scale_q=3.0)
    r = oracle.prefill(q, k, v, ws, bs=32, alpha=1.5, gamma=4.0, nb_out=8,
                       want=("o", "p", "pbar"))
    p, pbar = r["p"], r["pbar"]
    for g in range(2):
        union = (p[:, 2 * g] > 0) | (p[:, 2 * g + 1] > 0)
        assert np.array_equal(pbar[:, g] > 0, union)
        np.testing.assert_allclose(pbar[:, g].sum(-1)[32:], 1.0, atol=1e-12)
    # with one query head per KV head the average is the identity
    r1 = oracle.prefill(q[:, :2], k, v, ws, bs=32, alpha=1.5, gamma=4.0, nb_out=8,
                        want=("o", "p", "pbar"))
    np.testing.assert_array_equal(r1["p"], r1["pbar"])


def test_prior_softmax_is_the_gibbs_maximiser():
    """The Stage 2 weights w (read out with one-hot values) maximise
    z.p - KL(p || g) with z = q.k/sqrt(d) and g_t = pbar(block of t)/bs on the
    routed keys: compare with an independent SLSQP solve."""
    d, bs, N = 64, 4, 32
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    v = np.eye(N, d, dtype=np.float32)[None, None]      # v_t = e_t: o = attention weights
    ws = (np.eye(d) + 0.3 * rng.standard_normal((d, d))).astype(np.float32)
    i = N - 1
    r = oracle.prefill(q, k, v, ws, bs=bs, alpha=1.5, gamma=3.0, causal=False, positions=[i],
                       nb_out=N // bs, want=("o", "pbar"), )
    wts = r["o"][0, 0, :N]
    pbar = r["pbar"][0, 0]
    routed = np.repeat(pbar > 0, bs)
    z = (k[0, 0].astype(np.float64) @ q[0, 0, i].astype(np.float64)) / np.sqrt(d)
    gk = np.repeat(pbar, bs) / bs
    zr, gr = z[routed], gk[routed]
    obj = lambda p: -(p @ zr - np.sum(np.where(p > 0, p * np.log(np.maximum(p, 1e-300) / gr), 0)))
    res = minimize(obj, gr / gr.sum(), method="SLSQP", bounds=[(0, 1)] * len(zr),
                   constraints=[{"type": "eq", "fun": lambda p: p.sum() - 1}],
                   options={"ftol": 1e-15, "maxiter": 1000})
    np.testing.assert_allclose(wts[routed], res.x, atol=2e-5)
    assert np.all(wts[~routed] == 0)
    assert -obj(wts[routed]) >= -obj(res.x) - 1e-12


def test_unselected_blocks_do_not_touch_the_output():
    """g = 0 where the routing weight is 0 masks the chunk: perturbing the
    values of unrouted blocks leaves every output bit-identical."""
    w = W.get("tiny").replace(seq_len=512, head_dim=32, planted=False)
    inp = W.make_prefill(w)
    N, bs, nb = 512, 64, 8
    kw = dict(bs=bs, alpha=1.5, gamma=30.0, nb_out=nb, want=("o", "pbar"))
    r = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["w_s"], **kw)
    pbar = r["pbar"]
    i = N - 1                                           # last row
    unsel = [(g, j) for g in range(2) for j in range(nb - 1) if pbar[i, g, j] == 0]
    assert unsel, "expected some unrouted block"
    v2 = inp["v"].copy()
    for g, j in unsel:
        v2[:, g, j * bs:(j + 1) * bs] += 100.0
    r2 = oracle.prefill(inp["q"], inp["k"], v2, inp["w_s"], positions=[i], **kw)
    np.testing.assert_array_equal(r2["o"][0], r["o"][i])


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------

def test_decode_equals_last_prefill_row_and_writes_summary():
    w = W.get("tiny").replace(seq_len=384, head_dim=32, n_heads=4, n_kv_heads=2)
    inp = W.make_prefill(w)
    ws = inp["w_s"]
    for L in (1, 63, 64, 65, 128, 300, 384):
        q = inp["q"][:, :, L - 1]                      # [B, H, d]
        dec = oracle.decode(q, inp["k"], inp["v"], [L], ws, bs=64, alpha=1.5, gamma=8.0)
        pre = oracle.prefill(inp["q"][:, :, :L], inp["k"][:, :, :L], inp["v"][:, :, :L], ws,
                             bs=64, alpha=1.5, gamma=8.0, positions=[L - 1])
        np.testing.assert_array_equal(dec["o"], pre["o"])
        np.testing.assert_array_equal(np.isnan(dec["tau"]), np.isnan(pre["tau"]))
        if L % 64 == 0:
            ref = oracle.summaries(inp["k"][:, :, L - 64:L], ws, 64, 1)[0, :, 0]
            np.testing.assert_allclose(dec["new_summary"][0], ref, atol=1e-14)
        else:
            assert dec["new_summary"][0] is None
