"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Small cases run every row through the oracle (several query tiles, ragged
tails, batch > 1, GQA groups 1/2/4/8, head dims 64/128, blocks 64/128,
alpha 1.25/1.5/2, fp32 and bf16).  Full-size workloads are in
test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_hierarchical_attention_block_amd as dash
from brute import dense_attention
import workloads as W
from gpu_helpers import (TOL, check_bias, check_list, check_supports, check_tau,
                         check_tile_mask, dev, params, run_decode,
                         run_prefill, run_prefill_fused, tile_union_ref, to_dev)

pytestmark = pytest.mark.gpu

QT = 64


def tiny(**kw):
    return W.get("tiny").replace(**kw)


PREFILL_CASES = {
    "tiny_f32_sparse": tiny(gamma=8.0),
    "tiny_f32_dense": tiny(gamma=1.0),
    "tiny_bf16": tiny(dtype="bf16", gamma=8.0),
    "gqa4_d128_bs64": W.get("prefill_8k").replace(seq_len=2048),
    "gqa4_d128_bs128": W.get("prefill_64k").replace(seq_len=2048, gamma=2.0),
    "gqa8_d64_alpha2": tiny(n_heads=16, n_kv_heads=2, seq_len=1536, dtype="bf16", alpha=2.0,
                            gamma=6.0, planted=True),
    "gqa2_alpha125_ragged": W.get("prefill_8k").replace(n_heads=4, n_kv_heads=2, seq_len=1000,
                                                        alpha=1.25, gamma=4.0),
    "batch3_ragged_f32": tiny(batch=3, seq_len=700, n_heads=4, n_kv_heads=1, gamma=5.0),
    "alpha175_general": tiny(seq_len=640, dtype="bf16", alpha=1.75, gamma=6.0),
    # Stage 0 pooled by per-KV-head summary queries
    "qbar_tiny_f32": tiny(gamma=8.0, summary_query=1.0),
    "qbar_gqa4_d128_bf16": W.get("prefill_8k").replace(seq_len=2048, summary_query=1.0),
    "qbar_sharp_bs128_d64": tiny(batch=2, n_heads=8, n_kv_heads=4, seq_len=1100,
                                 block_size=128, dtype="bf16", gamma=6.0, summary_query=4.0),
    # prior strength and near-diagonal window
    "sigma05_window2_gqa4": W.get("prefill_8k").replace(seq_len=2048, sigma=0.5, window=2),
    "sigma0_window3_f32": tiny(batch=2, seq_len=900, gamma=8.0, sigma=0.0, window=3),
    "sigma2_window4_bs128": W.get("prefill_64k").replace(seq_len=2048, gamma=2.0, sigma=2.0,
                                                         window=4),
    "window_covers_all_bf16": tiny(seq_len=700, dtype="bf16", gamma=8.0, window=11),
    # 64 < candidates <= 128 in the last tiles, full oracle parity
    "cand74_gqa4": W.get("prefill_8k").replace(seq_len=4800, n_heads=8, n_kv_heads=2),
    # one query head per KV head at d = 128 (the two-wave attend workgroup and its
    # four-buffer LDS ring), ragged, at both block sizes
    "mha_d128_bs64_ragged": W.get("prefill_8k").replace(seq_len=1500, n_heads=2, n_kv_heads=2),
    "mha_d128_bs128_ragged": W.get("prefill_64k").replace(seq_len=1700, n_heads=2, n_kv_heads=2,
                                                          gamma=2.0),
    # more than 128 candidates in the last tiles (bf16, G >= 2: the long-row
    # routing kernel; G / 2 workgroups per tile whose unions are merged),
    # ragged tails
    "long_rows_gqa2_d64": W.get("prefill_8k").replace(seq_len=9000, n_heads=4, n_kv_heads=2,
                                                      head_dim=64),
    "long_rows_gqa4_bs128": W.get("prefill_64k").replace(seq_len=18000, n_heads=4,
                                                         n_kv_heads=1),
    "long_rows_gqa8_window2": W.get("prefill_8k").replace(seq_len=8800, n_heads=8,
                                                          n_kv_heads=1, head_dim=64, window=2,
                                                          sigma=0.5),
    "long_rows_alpha125_gqa4": W.get("prefill_8k").replace(seq_len=8500, n_heads=8,
                                                           n_kv_heads=2, alpha=1.25),
    "long_rows_alpha2_gqa4": W.get("prefill_8k").replace(seq_len=8500, n_heads=4, n_kv_heads=1,
                                                         alpha=2.0),
    # general alpha (Newton steps with log / exp) on the long-row kernel with one part per tile
    "long_rows_alpha175_gqa2": W.get("prefill_8k").replace(seq_len=9000, n_heads=4, n_kv_heads=2,
                                                           alpha=1.75),
}


def oracle_prefill(w, inp, nb):
    r = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["w_s"], bs=w.block_size, alpha=w.alpha,
                       gamma=w.gamma, nb_out=nb, want=("o", "tau", "x", "pbar"),
                       q_bar=inp.get("q_bar"), sigma=w.sigma, window=w.window)
    B, N, H, Hkv = w.batch, w.seq_len, w.n_heads, w.n_kv_heads
    return {"o": r["o"].reshape(B, N, H, -1).transpose(0, 2, 1, 3),
            "tau": r["tau"].reshape(B, N, H), "x": r["x"].reshape(B, N, H, nb),
            "pbar": r["pbar"].reshape(B, N, Hkv, nb), "summ": r["summ"]}


def compare_prefill(w, g, ref):
    B, H, Hkv, N, bs, G = w.batch, w.n_heads, w.n_kv_heads, w.seq_len, w.block_size, w.group
    nb = -(-N // bs)
    tol = TOL[w.dtype]
    # Stage 0
    np.testing.assert_allclose(g["summ"], ref["summ"], rtol=1e-5, atol=2e-5)
    # Stage 1: thresholds and per-head supports
    check_tau(g["tau"].transpose(0, 2, 1), ref["tau"])
    pos = np.arange(N)
    ncand = np.tile(np.maximum(pos // bs - (w.window - 1), 0), B)
    bits = g["bits"].transpose(0, 2, 1, 3).reshape(B * N, H, nb)
    check_supports(bits, ref["x"].reshape(B * N, H, nb), ref["tau"].reshape(B * N, H), ncand)
    # tile lists and log priors
    n_qt = -(-N // QT)
    for b in range(B):
        for gg in range(Hkv):
            for qt in range(n_qt):
                p0, p1 = qt * QT, min(N, qt * QT + QT)
                t = max(p0 // bs - (w.window - 1), 0)
                hs = slice(gg * G, gg * G + G)
                union, solid, near = tile_union_ref(ref["pbar"][b, p0:p1, gg, :t],
                                                    ref["x"][b, p0:p1, hs, :t],
                                                    ref["tau"][b, p0:p1, hs], G)
                cnt = g["count"][b, gg, qt]
                check_list(cnt, g["idx"][b, gg, qt], union, solid, near)
                lst = g["idx"][b, gg, qt, :cnt]
                check_bias(g["logp"][b, gg, qt, lst, : p1 - p0].T,           # [P, listed]
                           ref["pbar"][b, p0:p1, gg][:, lst], w.sigma)
    # the bit-packed mask of each tile holds exactly its list
    check_tile_mask(g["tile_words"], g["tile_bits"], g["count"], g["idx"])
    # Stage 2 output
    err = np.abs(g["o"] - ref["o"]).max()
    assert err <= tol, f"output max-abs error {err:.3e} > {tol}"
    return err


@pytest.mark.parametrize("case", list(PREFILL_CASES))
def test_prefill_parity(case):
    w = PREFILL_CASES[case]
    print(f"[prefill parity] {case}: {w}", flush=True)
    inp = W.make_prefill(w)
    nb = -(-w.seq_len // w.block_size)
    g = run_prefill(w, inp)
    ref = oracle_prefill(w, inp, nb)
    err = compare_prefill(w, g, ref)
    # the fused entry point runs the same kernels
    fused = run_prefill_fused(w, inp)
    np.testing.assert_array_equal(fused, g["o"])
    print(f"  max-abs err {err:.3e}", flush=True)


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 128, 129, 200])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_short_and_ragged(n, dtype):
    w = tiny(seq_len=n, dtype=dtype, n_heads=4, n_kv_heads=2, gamma=3.0)
    print(f"[prefill ragged] n={n} {dtype}", flush=True)
    inp = W.make_prefill(w)
    ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["w_s"], bs=w.block_size,
                         alpha=w.alpha, gamma=w.gamma)
    got = run_prefill_fused(w, inp)
    err = np.abs(got.transpose(0, 2, 1, 3).reshape(n, 4, -1) - ref["o"]).max()
    assert err <= TOL[dtype], err


def test_attend_given_oracle_route():
    """Stage 2 alone: feed the oracle's routing (lists and log pbar) to
    dash_attend, so routing flips cannot mask an attend error."""
    import sparse_hierarchical_attention_block_amd as dash
    w = W.get("prefill_8k").replace(seq_len=1536)
    inp = W.make_prefill(w)
    B, H, Hkv, N, d, bs = w.batch, w.n_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block_size
    nb = N // bs
    ref = oracle_prefill(w, inp, nb)
    p = params(w)
    sizes = dash.dash_route_sizes_prefill(p, N)
    n_qt = sizes["n_qt"]
    count = np.zeros((B, Hkv, n_qt), np.int32)
    idx = np.zeros((B, Hkv, n_qt, nb), np.int32)
    logp = np.full((B, Hkv, n_qt, nb, QT), -np.inf, np.float32)
    for b in range(B):
        for g in range(Hkv):
            for qt in range(n_qt):
                pb = ref["pbar"][b, qt * QT:(qt + 1) * QT, g]              # [QT, nb]
                lst = np.flatnonzero((pb > 0).any(0))
                count[b, g, qt] = len(lst)
                idx[b, g, qt, :len(lst)] = lst
                with np.errstate(divide="ignore"):
                    logp[b, g, qt] = np.log(pb).T
    rb = dash.RouteBuffers(sizes, dev())
    rb.sel_count.copy_(torch.from_numpy(count.ravel()))
    rb.sel_idx.copy_(torch.from_numpy(idx.ravel()))
    rb.sel_logp.copy_(torch.from_numpy(logp.ravel()))
    q, k, v = (to_dev(inp[x], "bf16") for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    dash.dash_attend(p, q, k, v, N, rb, o)
    torch.cuda.synchronize()
    err = np.abs(o.float().cpu().numpy() - ref["o"]).max()
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("dtype,window", [("f32", 1), ("bf16", 1), ("bf16", 3), ("f32", 2)])
def test_external_mask_drives_stage2(dtype, window):
    """Stage 2 from a bit-packed mask made outside the library: seeded random
    tile masks (with bits set on blocks outside the candidates, which must be
    ignored) and random biases; dash_mask_to_list builds the lists, dash_attend
    runs on them; checked against brute-force dense attention with that mask
    and bias.  Also: the lists round-trip through the mask dash_route writes."""
    w = tiny(batch=2, n_heads=4, n_kv_heads=2, seq_len=700, dtype=dtype, gamma=8.0,
             window=window)
    print(f"[external mask] {dtype} window={window}", flush=True)
    inp = W.make_prefill(w)
    B, H, Hkv, N, d, bs, G = w.batch, w.n_heads, w.n_kv_heads, w.seq_len, w.head_dim, \
        w.block_size, w.group
    p = params(w)
    sizes = dash.dash_route_sizes_prefill(p, N)
    n_qt, nb = sizes["n_qt"], sizes["nb"]
    nwords = (nb + 31) // 32
    rng = np.random.default_rng(1234 + window)
    bits = rng.random((B, Hkv, n_qt, nwords * 32)) < 0.4
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)          # bit j % 32 of word j // 32
    words = (bits.reshape(B, Hkv, n_qt, nwords, 32) * weights).sum(-1).astype(np.uint32)
    logp = np.log(rng.uniform(0.05, 1.0, (B, Hkv, n_qt, nb, QT))).astype(np.float32)
    logp[rng.random(logp.shape) < 0.1] = -np.inf
    rb = dash.RouteBuffers(sizes, dev(), tile_bits=True)
    rb.tile_bits.copy_(torch.from_numpy(words.view(np.int32).ravel()))
    rb.sel_logp.copy_(torch.from_numpy(logp.ravel()))
    dash.dash_mask_to_list(p, N, rb)
    q, k, v = (to_dev(inp[x], dtype) for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    dash.dash_attend(p, q, k, v, N, rb, o)
    torch.cuda.synchronize()
    count = rb.sel_count.cpu().numpy().reshape(B, Hkv, n_qt)
    idx = rb.sel_idx.cpu().numpy().reshape(B, Hkv, n_qt, nb)
    got = o.float().cpu().numpy()
    t = np.arange(N)
    for b in range(B):
        for g in range(Hkv):
            bias = np.full((N, N), -np.inf)
            for qt in range(n_qt):
                p0, p1 = qt * QT, min(N, qt * QT + QT)
                ncand = max(p0 // bs - (window - 1), 0)
                want = np.flatnonzero(bits[b, g, qt, :ncand])
                np.testing.assert_array_equal(idx[b, g, qt, :count[b, g, qt]], want)
                for j in want:
                    bias[p0:p1, j * bs:(j + 1) * bs] = logp[b, g, qt, j, :p1 - p0, None]
                for i in range(p0, p1):
                    bias[i, ncand * bs:i + 1] = 0.0
            mask = np.isfinite(bias)
            for hh in range(G):
                h = g * G + hh
                ref = dense_attention(inp["q"][b, h], inp["k"][b, g], inp["v"][b, g],
                                      bias=np.where(mask, bias, 0.0), mask=mask)
                err = np.abs(got[b, h] - ref).max()
                assert err <= TOL[dtype], f"b={b} h={h}: {err:.3e}"
    # round trip: the mask dash_route writes rebuilds its own lists
    g1 = run_prefill(w, inp, bits=False)
    rb2 = dash.RouteBuffers(sizes, dev(), tile_bits=True)
    rb2.tile_bits.copy_(torch.from_numpy(g1["tile_words"].ravel()))
    dash.dash_mask_to_list(p, N, rb2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(rb2.sel_count.cpu().numpy().reshape(B, Hkv, n_qt), g1["count"])
    idx2 = rb2.sel_idx.cpu().numpy().reshape(B, Hkv, n_qt, nb)
    for (b, g, qt), c in np.ndenumerate(g1["count"]):
        np.testing.assert_array_equal(idx2[b, g, qt, :c], g1["idx"][b, g, qt, :c])


def test_unselected_values_do_not_matter():
    """Zero-probability blocks are masked: changing V of every block that a
    tile neither selected nor owns leaves that tile's outputs bit-identical."""
    w = W.get("prefill_8k").replace(seq_len=2048)
    inp = W.make_prefill(w)
    g1 = run_prefill(w, inp, bits=False)
    N, bs, G = w.seq_len, w.block_size, w.group
    qt, gg = N // QT - 1, 3
    used = np.zeros(N // bs, bool)
    used[g1["idx"][0, gg, qt, :g1["count"][0, gg, qt]]] = True
    used[(qt * QT) // bs] = True
    assert (~used).any()
    v2 = inp["v"].copy()
    for j in np.flatnonzero(~used):
        v2[0, gg, j * bs:(j + 1) * bs] = 7.0
    g2 = run_prefill(w, dict(inp, v=v2), bits=False)
    rows = slice(qt * QT, qt * QT + QT)
    heads = slice(gg * G, gg * G + G)
    np.testing.assert_array_equal(g1["o"][0, heads, rows], g2["o"][0, heads, rows])
    assert not np.array_equal(g1["o"], g2["o"])      # other tiles did read those blocks


def test_deterministic():
    w = W.get("prefill_8k").replace(seq_len=2048)
    inp = W.make_prefill(w)
    a = run_prefill_fused(w, inp)
    b = run_prefill_fused(w, inp)
    np.testing.assert_array_equal(a, b)


# ----------------------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,bs", [(64, 64), (128, 64), (64, 128), (128, 128)])
@pytest.mark.parametrize("scale", [0.0, 1.0, 6.0])
def test_summarize_with_query(dtype, d, bs, scale):
    """dash_summarize with summary queries against the oracle; blocks [2, 7) of
    a 3-sequence, 3-KV-head cache (7 workgroups per head, odd split)."""
    print(f"[summarize q_bar] {dtype} d={d} bs={bs} scale={scale}", flush=True)
    w = tiny(batch=3, n_heads=3, n_kv_heads=3, head_dim=d, block_size=bs, seq_len=7 * bs + 5,
             dtype=dtype, summary_query=max(scale, 1.0))
    inp = W.make_prefill(w)
    qb = inp["q_bar"] * (scale / max(scale, 1.0))
    p = params(w)
    N, B, Hkv = w.seq_len, w.batch, w.n_kv_heads
    k = to_dev(inp["k"], dtype)
    ws = torch.from_numpy(inp["w_s"]).to(dev())
    summ = torch.full((B * Hkv * 8 * d,), 7.0, dtype=torch.float32, device=dev())
    qbt = torch.from_numpy(np.ascontiguousarray(qb)).to(dev())
    dash.dash_summarize(p, k, N, 2, 7, ws, summ, 8, q_bar=qbt)
    g = summ.cpu().numpy().reshape(B, Hkv, 8, d)
    ref = oracle.summaries(inp["k"], inp["w_s"], bs, 7, qb)
    np.testing.assert_allclose(g[:, :, 2:7], ref[:, :, 2:7], rtol=1e-5, atol=2e-5)
    assert (g[:, :, :2] == 7.0).all() and (g[:, :, 7] == 7.0).all()
    if scale == 0.0:
        # a zero query pools like the mean-pooling path
        summ0 = torch.zeros_like(summ)
        dash.dash_summarize(p, k, N, 2, 7, ws, summ0, 8)
        g0 = summ0.cpu().numpy().reshape(B, Hkv, 8, d)
        np.testing.assert_allclose(g[:, :, 2:7], g0[:, :, 2:7], rtol=1e-6, atol=1e-6)


DECODE_CASES = {
    "tiny_f32_ragged": (tiny(batch=7, gamma=8.0, kind="decode"),
                        [1, 63, 64, 65, 300, 1000, 1024]),
    "tiny_bf16_ragged": (tiny(batch=4, gamma=8.0, kind="decode", dtype="bf16"),
                         [1024, 640, 129, 2]),
    "gqa4_d128": (W.get("decode_32k").replace(batch=4, seq_len=4096, count_lo=4, count_hi=40),
                  [4096, 4000, 2049, 64]),
    "gqa8_loguniform": (W.get("decode_128k").replace(batch=2, seq_len=8192, count_hi=64),
                        [8192, 5555]),
    "bs128_alpha2": (W.get("decode_32k").replace(batch=3, seq_len=3072, block_size=128,
                                                 alpha=2.0, gamma=3.0, count_lo=2, count_hi=12),
                     [3072, 3000, 130]),
    # 512 < candidates <= 1024 (16 register slots per lane), two heads per group
    "gqa2_slots16": (W.get("decode_32k").replace(batch=2, n_heads=4, n_kv_heads=2, seq_len=49152),
                     [49152, 33001]),
    # at least 128 (sequence, KV head) pairs: scores and routing fused per pair,
    # lengths with no candidate, block completions and ragged tails
    "fused_gqa4_d128": (W.get("decode_32k").replace(batch=16, seq_len=3000, count_lo=4,
                                                    count_hi=30),
                        [1, 2, 63, 64, 65, 127, 128, 129, 500, 1000, 1024, 2047, 2048, 2049,
                         2999, 3000]),
    "fused_gqa2_d64": (W.get("decode_32k").replace(batch=32, n_heads=8, n_kv_heads=4,
                                                   head_dim=64, seq_len=1500, count_lo=2,
                                                   count_hi=16),
                       [1500 - 37 * i for i in range(32)]),
    "fused_gqa8": (W.get("decode_128k").replace(batch=16, seq_len=2000, count_hi=24),
                   [2000 - 61 * i for i in range(16)]),
    # Stage 0 pooled by summary queries: routed summaries and the completed block's
    "qbar_f32_ragged": (tiny(batch=5, gamma=8.0, kind="decode", summary_query=1.0),
                        [64, 65, 640, 1000, 1024]),
    "qbar_fused_bf16": (W.get("decode_32k").replace(batch=16, seq_len=2048, count_lo=2,
                                                    count_hi=20, summary_query=2.0),
                        [2048 - 64 * i for i in range(16)]),
    # prior strength and near-diagonal window: two-kernel f32, fused bf16 (lists
    # that start past the first split), and windows longer than short sequences
    "sigma05_window2_f32": (tiny(batch=6, gamma=8.0, kind="decode", sigma=0.5, window=2),
                            [1, 64, 65, 129, 700, 1024]),
    "sigma0_window3_fused": (W.get("decode_32k").replace(batch=16, seq_len=3000, count_lo=4,
                                                         count_hi=30, sigma=0.0, window=3),
                             [1, 63, 64, 128, 129, 192, 193, 500, 1000, 1024, 2047, 2048,
                              2049, 2500, 2999, 3000]),
    "sigma2_window40_gqa8": (W.get("decode_128k").replace(batch=2, seq_len=8192, count_hi=64,
                                                          sigma=2.0, window=40),
                             [8192, 2600]),
    # more than 2048 candidates: scores and routing as two kernels, the row in memory
    "long_row_in_memory": (W.get("decode_32k").replace(batch=1, n_heads=4, n_kv_heads=1,
                                                       seq_len=139264),
                           [139264]),
}


@pytest.mark.parametrize("case", list(DECODE_CASES))
def test_decode_parity(case):
    w, lens = DECODE_CASES[case]
    print(f"[decode parity] {case}: {w} lens={lens}", flush=True)
    inp = W.make_decode(w, cache_len=lens)
    B, H, Hkv, d, bs, G = w.batch, w.n_heads, w.n_kv_heads, w.head_dim, w.block_size, w.group
    Lmax = inp["k_cache"].shape[2]
    nb = -(-Lmax // bs)
    lens = np.asarray(lens)
    # summary cache holds exactly the blocks complete before each new token
    summ = oracle.summaries(inp["k_cache"], inp["w_s"], bs, Lmax // bs, inp.get("q_bar"))
    for b in range(B):
        summ[b, :, max((lens[b] - 1) // bs - (w.window - 1), 0):] = 0.0
    g = run_decode(w, inp, summ_np=summ)
    ref = oracle.decode(inp["q"], inp["k_cache"], inp["v_cache"], lens, inp["w_s"], bs=bs,
                        alpha=w.alpha, gamma=w.gamma, nb_out=nb, want=("o", "tau", "x", "pbar"),
                        q_bar=inp.get("q_bar"), sigma=w.sigma, window=w.window)
    check_tau(g["tau"], ref["tau"])
    ncand = np.maximum((lens - 1) // bs - (w.window - 1), 0)
    check_supports(g["bits"], ref["x"], ref["tau"], ncand)
    for b in range(B):
        for gg in range(Hkv):
            hs = slice(gg * G, gg * G + G)
            t = ncand[b]
            union, solid, near = tile_union_ref(ref["pbar"][b:b + 1, gg, :t],
                                                ref["x"][b:b + 1, hs, :t], ref["tau"][b:b + 1, hs], G)
            cnt = g["count"][b, gg]
            check_list(cnt, g["idx"][b, gg], union, solid, near)
            lst = g["idx"][b, gg, :cnt]
            check_bias(g["logp"][b, gg, lst], ref["pbar"][b, gg, lst], w.sigma)
    check_tile_mask(g["tile_words"], g["tile_bits"], g["count"], g["idx"])
    err = np.abs(g["o"] - ref["o"]).max()
    assert err <= TOL[w.dtype], f"decode max-abs err {err:.3e}"
    # summary written exactly when the step completes a block
    for b in range(B):
        blk = lens[b] // bs - 1
        after, before = g["summ"][b], g["summ_before"][b]
        changed = np.flatnonzero(np.abs(after - before).max(axis=(0, 2)) > 0)
        if lens[b] % bs == 0:
            np.testing.assert_allclose(after[:, blk], ref["new_summary"][b], rtol=1e-5, atol=2e-5)
            assert set(changed.tolist()) <= {blk}
        else:
            assert changed.size == 0
    print(f"  max-abs err {err:.3e}", flush=True)


def test_decode_matches_prefill_last_row():
    """decode(L) is row L-1 of a causal prefill over the first L tokens."""
    w = W.get("prefill_8k").replace(seq_len=1024)
    inp = W.make_prefill(w)
    pre = run_prefill_fused(w, inp)
    L = 1024
    wd = w.replace(kind="decode")
    dinp = {"q": inp["q"][:, :, L - 1], "k_cache": inp["k"], "v_cache": inp["v"],
            "cache_len": np.array([L], np.int32), "w_s": inp["w_s"]}
    g = run_decode(wd, dinp, route=False)
    err = np.abs(g["o"][0] - pre[0, :, L - 1]).max()
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("fill", [1e30, float("nan"), -1e30])
def test_attend_ignores_unwritten_bias_rows(fill):
    """Stage 1 writes the bias of valid rows only; whatever the rest of the
    buffer holds (rows past the end of a ragged last tile) must not change any
    valid output bit (it could otherwise trigger the wave's lazy rescale)."""
    w = W.get("prefill_8k").replace(seq_len=8500, n_heads=8, n_kv_heads=2, alpha=1.25)
    inp = W.make_prefill(w)
    p = params(w)
    B, Hkv, N, d, bs = w.batch, w.n_kv_heads, w.seq_len, w.head_dim, w.block_size
    q, k, v = (to_dev(inp[x], w.dtype) for x in ("q", "k", "v"))
    ws = torch.from_numpy(inp["w_s"]).to(dev())
    nb = N // bs
    summ = torch.zeros(B * Hkv * nb * d, dtype=torch.float32, device=dev())
    dash.dash_summarize(p, k, N, 0, nb, ws, summ, nb)
    outs = []
    for value in (0.0, fill):
        rb = dash.RouteBuffers(dash.dash_route_sizes_prefill(p, N), dev())
        rb.sel_logp.fill_(value)
        dash.dash_route(p, q, N, summ, nb, rb)
        o = torch.empty_like(q)
        dash.dash_attend(p, q, k, v, N, rb, o)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
