"""GPU: decoding over a paged KV cache (one block of keys per page, a block
table per sequence) against the contiguous-cache decode and the oracle.

The pages are the contiguous caches cut into blocks and scattered over a
larger pool in a seeded random order; unused table entries hold garbage
(negative or past the pool), which the kernels must never use.  The paged
step does the same arithmetic as the contiguous one, so outputs, routing and
the summary written for a completed block must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_hierarchical_attention_block_amd as dash
import workloads as W
from gpu_helpers import TOL, dev, params, qbar_dev, to_dev

pytestmark = pytest.mark.gpu


def tiny(**kw):
    return W.get("tiny").replace(**kw)


CASES = {
    "f32_ragged": (tiny(batch=5, gamma=8.0, kind="decode"), [1, 64, 65, 700, 1024]),
    "bf16_gqa4_d128": (W.get("decode_32k").replace(batch=4, seq_len=4096, count_lo=4,
                                                   count_hi=40), [4096, 4000, 2049, 64]),
    "bf16_bs128_window2_sigma": (W.get("decode_32k").replace(batch=3, seq_len=3072,
                                                             block_size=128, alpha=2.0,
                                                             gamma=3.0, count_lo=2, count_hi=12,
                                                             window=2, sigma=0.5),
                                 [3072, 3000, 130]),
    "bf16_fused_qbar": (W.get("decode_32k").replace(batch=16, seq_len=2048, count_lo=2,
                                                    count_hi=20, summary_query=1.0),
                        [2048 - 63 * i for i in range(16)]),
}


def make_pages(kc, vc, bs, seed, spare=7):
    """Scatter [B, Hkv, L, d] caches into [num_pages, Hkv, bs, d] pages."""
    B, Hkv, L, d = kc.shape
    nblk = (L + bs - 1) // bs
    rng = np.random.default_rng(seed)
    num_pages = B * nblk + spare
    order = rng.permutation(num_pages)[:B * nblk].reshape(B, nblk)
    kp = np.zeros((num_pages, Hkv, bs, d), np.float32)
    vp = np.zeros_like(kp)
    for b in range(B):
        for j in range(nblk):
            n = min(bs, L - j * bs)
            kp[order[b, j], :, :n] = kc[b, :, j * bs:j * bs + n]
            vp[order[b, j], :, :n] = vc[b, :, j * bs:j * bs + n]
    max_blocks = nblk + 3
    table = rng.integers(-5, 2 * num_pages, (B, max_blocks)).astype(np.int32)
    table[:, :nblk] = order
    return kp, vp, table


@pytest.mark.parametrize("case", list(CASES))
def test_paged_decode_matches_contiguous(case):
    w, lens = CASES[case]
    print(f"[paged decode] {case}: {w} lens={lens}", flush=True)
    inp = W.make_decode(w, cache_len=lens)
    p = params(w)
    B, H, Hkv, d, bs = w.batch, w.n_heads, w.n_kv_heads, w.head_dim, w.block_size
    Lmax = inp["k_cache"].shape[2]
    nb = (Lmax + bs - 1) // bs
    kp, vp, table = make_pages(inp["k_cache"], inp["v_cache"], bs, seed=77)
    kc, vc = to_dev(inp["k_cache"], w.dtype), to_dev(inp["v_cache"], w.dtype)
    kpd, vpd = to_dev(kp, w.dtype), to_dev(vp, w.dtype)
    tab = torch.from_numpy(table).to(dev())
    q = to_dev(inp["q"], w.dtype)
    lens_d = torch.from_numpy(np.asarray(lens, np.int32)).to(dev())
    ws_mat = torch.from_numpy(inp["w_s"]).to(dev())
    qb = qbar_dev(inp)
    # the summary cache of the blocks complete before each new token
    summ0 = oracle.summaries(inp["k_cache"], inp["w_s"], bs, Lmax // bs, inp.get("q_bar"))
    for b in range(B):
        summ0[b, :, max((lens[b] - 1) // bs - (w.window - 1), 0):] = 0.0
    summ_init = torch.zeros(B * Hkv * nb * d, dtype=torch.float32, device=dev())
    summ_init.view(B, Hkv, nb, d)[:, :, :summ0.shape[2]] = torch.from_numpy(
        summ0.astype(np.float32)).to(dev())
    outs = {}
    for paged in (False, True):
        summ = summ_init.clone()
        o = torch.empty_like(q)
        ws = dash.workspace(dash.dash_decode_workspace_bytes(p, Lmax), dev())
        rb = dash.RouteBuffers(dash.dash_route_sizes_decode(p, Lmax), dev(), tile_bits=True)
        if paged:
            dash.dash_decode_paged(p, q, kpd, vpd, tab, lens_d, Lmax, ws_mat, summ, nb, o, ws,
                                   route=rb, q_bar=qb)
        else:
            dash.dash_decode(p, q, kc, vc, lens_d, Lmax, ws_mat, summ, nb, o, ws, route=rb,
                             q_bar=qb)
        torch.cuda.synchronize()
        outs[paged] = {"o": o.float().cpu().numpy(), "summ": summ.cpu().numpy(),
                       "count": rb.sel_count.cpu().numpy(), "idx": rb.sel_idx.cpu().numpy(),
                       "tau": rb.tau.cpu().numpy(), "bits": rb.tile_bits.cpu().numpy()}
    for key in ("o", "summ", "count", "tau", "bits"):
        np.testing.assert_array_equal(outs[True][key], outs[False][key], err_msg=key)
    cnt = outs[True]["count"].reshape(B * Hkv)
    idx_p, idx_c = (outs[x]["idx"].reshape(B * Hkv, nb) for x in (True, False))
    for r in range(B * Hkv):
        np.testing.assert_array_equal(idx_p[r, :cnt[r]], idx_c[r, :cnt[r]])
    # and against the oracle
    ref = oracle.decode(inp["q"], inp["k_cache"], inp["v_cache"], lens, inp["w_s"], bs=bs,
                        alpha=w.alpha, gamma=w.gamma, q_bar=inp.get("q_bar"), sigma=w.sigma,
                        window=w.window)
    err = np.abs(outs[True]["o"] - ref["o"]).max()
    assert err <= TOL[w.dtype], f"paged decode max-abs err {err:.3e}"
    summ_p = outs[True]["summ"].reshape(B, Hkv, nb, d)
    for b in range(B):
        if lens[b] % bs == 0:
            np.testing.assert_allclose(summ_p[b, :, lens[b] // bs - 1], ref["new_summary"][b],
                                       rtol=1e-5, atol=2e-5)
    print(f"  max-abs err {err:.3e}", flush=True)


def test_paged_binding_checks_shapes():
    w = tiny(batch=2, kind="decode")
    p = params(w)
    q = torch.zeros((2, 2, 64), device=dev())
    pages = torch.zeros((4, 2, 64, 64), device=dev())
    table = torch.zeros((2, 16), dtype=torch.int32, device=dev())
    lens = torch.full((2,), 100, dtype=torch.int32, device=dev())
    ws_mat = torch.zeros((64, 64), device=dev())
    summ = torch.zeros(2 * 2 * 16 * 64, device=dev())
    ws = dash.workspace(dash.dash_decode_workspace_bytes(p, 1024), dev())
    with pytest.raises(ValueError):
        dash.dash_decode_paged(p, q, pages[:, :1], pages[:, :1], table, lens, 1024, ws_mat, summ,
                               16, torch.empty_like(q), ws)
    with pytest.raises(dash.DashError):     # max_blocks below ceil(max_len / bs)
        dash.dash_decode_paged(p, q, pages, pages, table[:, :15].contiguous(), lens, 1024, ws_mat,
                               summ, 16,
                               torch.empty_like(q), ws)
