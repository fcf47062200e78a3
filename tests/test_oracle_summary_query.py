"""Pins of the oracle's Stage 0 with a summary query q_bar.

Pages: DashAttention explainer (gist.science, arXiv 2605.18753), Technical
summary, Stage 0 (local chunk summarization): a learned query vector attends
to the keys of each chunk through local scaled dot-product attention; it
starts at zero, where the pooling is the uniform mean.  Reading: one query per
KV head, the keys serve as the values, and the pooled vector is projected by
W_s as in the uniform case.

Each pin holds for the mathematics, not for a retyped formula:
  * q_bar = 0 reduces to the uniform block mean (numpy's mean);
  * the pooled key is the gradient of sqrt(d) * logsumexp(q_bar . k_t / sqrt(d))
    with respect to q_bar (scipy's logsumexp, central differences);
  * a block holding two distinct keys with counts n1, n2 weighs them with the
    logistic sigma(q_bar . (a - b) / sqrt(d) + ln(n1 / n2));
  * a constant block summarises to its key for any q_bar;
  * the summary does not depend on the order of the keys inside a block;
  * as q_bar grows along a direction the summary tends to the key with the
    largest projection (the hardmax limit);
  * head h uses row h of q_bar.
"""
import numpy as np
import pytest
from scipy.special import expit, logsumexp

import oracle


def _keys(B, Hkv, L, d, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, Hkv, L, d)).astype(np.float32)


def test_zero_query_is_uniform_mean():
    k = _keys(2, 3, 192, 16, 11)
    rng = np.random.default_rng(12)
    ws = rng.standard_normal((16, 16)).astype(np.float32)
    s0 = oracle.summaries(k, ws, 64, 3, q_bar=np.zeros((3, 16), np.float32))
    mean = k.astype(np.float64).reshape(2, 3, 3, 64, 16).mean(axis=3)
    np.testing.assert_allclose(s0, mean @ ws.astype(np.float64), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(s0, oracle.summaries(k, ws, 64, 3))


@pytest.mark.parametrize("d", [8, 64])
def test_pooled_key_is_gradient_of_log_partition(d):
    bs = 32
    k = _keys(1, 1, bs, d, 21)
    q = np.random.default_rng(22).standard_normal(d).astype(np.float32)
    pooled = oracle.summaries(k, np.eye(d, dtype=np.float32), bs, 1, q_bar=q[None])[0, 0, 0]
    kd = k[0, 0].astype(np.float64)

    def lse(qv):
        return np.sqrt(d) * logsumexp(kd @ qv / np.sqrt(d))

    h = 1e-5
    grad = np.empty(d)
    for c in range(d):
        e = np.zeros(d)
        e[c] = h
        grad[c] = (lse(q + e) - lse(q - e)) / (2 * h)
    np.testing.assert_allclose(pooled, grad, rtol=0, atol=1e-8)


@pytest.mark.parametrize("n1", [1, 17, 40])
def test_two_distinct_keys_logistic(n1):
    d, bs = 16, 64
    rng = np.random.default_rng(31 + n1)
    a, b = rng.standard_normal((2, d)).astype(np.float32)
    q = (2.0 * rng.standard_normal(d)).astype(np.float32)
    order = rng.permutation(bs)
    rows = np.where((order < n1)[:, None], a, b)
    k = rows[None, None].astype(np.float32)
    pooled = oracle.summaries(k, np.eye(d, dtype=np.float32), bs, 1, q_bar=q[None])[0, 0, 0]
    ad, bd, qd = (x.astype(np.float64) for x in (a, b, q))
    w = expit(qd @ (ad - bd) / np.sqrt(d) + np.log(n1 / (bs - n1)))
    np.testing.assert_allclose(pooled, w * ad + (1 - w) * bd, rtol=0, atol=1e-12)


def test_constant_block_is_key_times_ws_for_any_query():
    d, bs = 16, 64
    rng = np.random.default_rng(41)
    rows = rng.standard_normal((3, d)).astype(np.float32)
    k = np.repeat(rows, bs, axis=0)[None, None]
    ws = rng.standard_normal((d, d)).astype(np.float32)
    q = (10.0 * rng.standard_normal((1, d))).astype(np.float32)
    s = oracle.summaries(k, ws, bs, 3, q_bar=q)[0, 0]
    np.testing.assert_allclose(s, rows.astype(np.float64) @ ws.astype(np.float64), atol=1e-11)


def test_order_inside_block_does_not_matter():
    d, bs = 32, 128
    k = _keys(1, 2, 2 * bs, d, 51)
    rng = np.random.default_rng(52)
    ws = rng.standard_normal((d, d)).astype(np.float32)
    q = rng.standard_normal((2, d)).astype(np.float32)
    perm = np.concatenate([rng.permutation(bs), bs + rng.permutation(bs)])
    s = oracle.summaries(k, ws, bs, 2, q_bar=q)
    sp = oracle.summaries(np.ascontiguousarray(k[:, :, perm]), ws, bs, 2, q_bar=q)
    np.testing.assert_allclose(sp, s, rtol=0, atol=1e-12)
    # keys moved across blocks do change the summaries
    swap = np.concatenate([np.arange(bs // 2), bs + np.arange(bs // 2),
                           np.arange(bs // 2, bs), bs + np.arange(bs // 2, bs)])
    sx = oracle.summaries(np.ascontiguousarray(k[:, :, swap]), ws, bs, 2, q_bar=q)
    assert np.abs(sx - s).max() > 1e-3


def test_large_query_selects_the_top_key():
    d, bs = 16, 64
    k = _keys(1, 1, bs, d, 61)
    u = np.random.default_rng(62).standard_normal(d)
    u /= np.linalg.norm(u)
    proj = k[0, 0].astype(np.float64) @ u
    top = int(np.argmax(proj))
    gap = np.sort(proj)[-1] - np.sort(proj)[-2]
    scale = 60.0 * np.sqrt(d) / gap        # every other weight below e^-60 of the top
    pooled = oracle.summaries(k, np.eye(d, dtype=np.float32), bs, 1,
                              q_bar=(scale * u)[None].astype(np.float32))[0, 0, 0]
    np.testing.assert_allclose(pooled, k[0, 0, top].astype(np.float64), rtol=0, atol=1e-20)


def test_each_head_uses_its_own_query():
    d, bs = 16, 64
    k = _keys(2, 2, 2 * bs, d, 71)
    rng = np.random.default_rng(72)
    ws = rng.standard_normal((d, d)).astype(np.float32)
    q = np.stack([np.zeros(d), 3.0 * rng.standard_normal(d)]).astype(np.float32)
    s = oracle.summaries(k, ws, bs, 2, q_bar=q)
    mean = oracle.summaries(k, ws, bs, 2)
    np.testing.assert_array_equal(s[:, 0], mean[:, 0])
    assert np.abs(s[:, 1] - mean[:, 1]).max() > 1e-2
    # swapping both the heads of k and the rows of q_bar swaps the outputs
    s_sw = oracle.summaries(np.ascontiguousarray(k[:, ::-1]), ws, bs, 2,
                            q_bar=np.ascontiguousarray(q[::-1]))
    np.testing.assert_array_equal(s_sw[:, ::-1], s)


def test_query_shape_checked():
    k = _keys(1, 2, 64, 8, 81)
    with pytest.raises(ValueError):
        oracle.summaries(k, np.eye(8, dtype=np.float32), 64, 1,
                         q_bar=np.zeros((1, 8), np.float32))


def test_prefill_and_decode_use_the_query_summaries():
    B, H, Hkv, N, d, bs = 1, 4, 2, 256, 16, 64
    rng = np.random.default_rng(91)
    q = rng.standard_normal((B, H, N, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    ws = np.eye(d, dtype=np.float32)
    qb = (2.0 * rng.standard_normal((Hkv, d))).astype(np.float32)
    res = oracle.prefill(q, k, v, ws, bs=bs, alpha=1.5, gamma=1.0, positions=[N - 1],
                         q_bar=qb)
    np.testing.assert_array_equal(res["summ"], oracle.summaries(k, ws, bs, N // bs, qb))
    dec = oracle.decode(q[:, :, N - 1], k, v, [N], ws, bs=bs, alpha=1.5, gamma=1.0, q_bar=qb)
    np.testing.assert_allclose(dec["o"], res["o"], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(dec["new_summary"][0], res["summ"][0, :, -1])
    # and the routing result differs from uniform pooling
    res0 = oracle.prefill(q, k, v, ws, bs=bs, alpha=1.5, gamma=1.0, positions=[N - 1])
    assert np.abs(res0["o"] - res["o"]).max() > 1e-6
