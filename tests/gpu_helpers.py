"""Helpers for the GPU parity tests: run the HIP path through the C-ABI
binding on seeded inputs and bring results back as numpy; compare with the
oracle by the parity rules.

Parity rules (tolerances as the target states them):
  * per-head supports bit-exact, except blocks whose oracle entmax input lies
    within BAND of the oracle threshold (x-space);
  * outputs max-abs <= 1e-4 (float32 path) or 2e-2 (bf16 path).
"""
from __future__ import annotations

import numpy as np
import torch

import sparse_hierarchical_attention_block_amd as dash

BAND = 1e-5
TOL = {"f32": 1e-4, "bf16": 2e-2}


def dev():
    return torch.device("cuda:0")


def to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(dev(), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def qbar_dev(inp):
    """The summary queries of ``inp`` on the GPU, or None."""
    qb = inp.get("q_bar")
    return None if qb is None else torch.from_numpy(np.ascontiguousarray(qb, np.float32)).to(dev())


def params(w, **over):
    kw = dict(batch=w.batch, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
              block_size=w.block_size, alpha=w.alpha, gamma=w.gamma, dtype=w.dtype,
              sigma=w.sigma, window=w.window)
    kw.update(over)
    return dash.make_params(**kw)


def unpack_bits(words, nb):
    """[..., nwords] int32 -> [..., nb] bool"""
    w = words.astype(np.uint32)
    bits = ((w[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(bool)
    return bits.reshape(*w.shape[:-1], -1)[..., :nb]


def run_prefill(w, inp, bits=True):
    """dash_summarize + dash_route + dash_attend, stage by stage.  Returns a
    dict of numpy arrays in the route-buffer layouts of include/dash.h."""
    p = params(w)
    B, H, Hkv, N, d, bs = w.batch, w.n_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block_size
    q, k, v = (to_dev(inp[x], w.dtype) for x in ("q", "k", "v"))
    ws = torch.from_numpy(inp["w_s"]).to(dev())
    nbf = N // bs
    summ_blocks = max(nbf, 1)
    summ = torch.zeros(B * Hkv * summ_blocks * d, dtype=torch.float32, device=dev())
    dash.dash_summarize(p, k, N, 0, nbf, ws, summ, summ_blocks, q_bar=qbar_dev(inp))
    sizes = dash.dash_route_sizes_prefill(p, N)
    rb = dash.RouteBuffers(sizes, dev(), bits=bits, tile_bits=True)
    # NaN in every bias entry Stage 1 does not write: a listed row it left
    # out, or an entry Stage 2 reads without its being written, shows
    rb.sel_logp.fill_(float("nan"))
    dash.dash_route(p, q, N, summ, summ_blocks, rb)
    o = torch.empty_like(q)
    dash.dash_attend(p, q, k, v, N, rb, o)
    torch.cuda.synchronize()
    n_qt, nb = sizes["n_qt"], sizes["nb"]
    out = {
        "o": o.float().cpu().numpy(),                                  # [B, H, N, d]
        "summ": summ.cpu().numpy().reshape(B, Hkv, summ_blocks, d)[:, :, :nbf],
        "tau": rb.tau.cpu().numpy().reshape(B, H, N),
        "count": rb.sel_count.cpu().numpy().reshape(B, Hkv, n_qt),
        "idx": rb.sel_idx.cpu().numpy().reshape(B, Hkv, n_qt, nb),
        "logp": rb.sel_logp.cpu().numpy().reshape(B, Hkv, n_qt, nb, dash.QUERY_TILE),
        "tile_bits": unpack_bits(rb.tile_bits.cpu().numpy().reshape(B, Hkv, n_qt, -1), nb),
        "tile_words": rb.tile_bits.cpu().numpy().reshape(B, Hkv, n_qt, -1),
    }
    if bits:
        out["bits"] = unpack_bits(rb.support_bits.cpu().numpy().reshape(B, H, N, -1), nb)
    return out


def run_prefill_fused(w, inp):
    p = params(w)
    B, H, Hkv, N, d, bs = w.batch, w.n_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block_size
    q, k, v = (to_dev(inp[x], w.dtype) for x in ("q", "k", "v"))
    ws_mat = torch.from_numpy(inp["w_s"]).to(dev())
    summ_blocks = max(N // bs, 1)
    summ = torch.zeros(B * Hkv * summ_blocks * d, dtype=torch.float32, device=dev())
    o = torch.empty_like(q)
    ws = dash.workspace(dash.dash_prefill_workspace_bytes(p, N), dev())
    dash.dash_prefill(p, q, k, v, N, ws_mat, summ, summ_blocks, o, ws, q_bar=qbar_dev(inp))
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


def run_decode(w, inp, summ_np=None, route=True):
    """dash_decode on the caches of ``inp``.  The summary cache is filled
    with the GPU's own Stage 0 (dash_summarize) of every complete block unless
    ``summ_np`` is given."""
    p = params(w)
    B, H, Hkv, d, bs = w.batch, w.n_heads, w.n_kv_heads, w.head_dim, w.block_size
    Lmax = inp["k_cache"].shape[2]
    kc, vc = to_dev(inp["k_cache"], w.dtype), to_dev(inp["v_cache"], w.dtype)
    q = to_dev(inp["q"], w.dtype)
    lens = torch.from_numpy(np.asarray(inp["cache_len"], np.int32)).to(dev())
    ws_mat = torch.from_numpy(inp["w_s"]).to(dev())
    summ_blocks = (Lmax + bs - 1) // bs
    summ = torch.zeros(B * Hkv * summ_blocks * d, dtype=torch.float32, device=dev())
    if summ_np is not None:
        summ.view(B, Hkv, summ_blocks, d)[:, :, :summ_np.shape[2]] = torch.from_numpy(
            np.ascontiguousarray(summ_np, np.float32)).to(dev())
    elif Lmax // bs > 0:
        # blocks complete before each sequence's new token
        dash.dash_summarize(p, kc, Lmax, 0, Lmax // bs, ws_mat, summ, summ_blocks,
                            q_bar=qbar_dev(inp))
    summ_before = summ.clone()
    o = torch.empty_like(q)
    ws = dash.workspace(dash.dash_decode_workspace_bytes(p, Lmax), dev())
    rb = dash.RouteBuffers(dash.dash_route_sizes_decode(p, Lmax), dev(), bits=True,
                           tile_bits=True) if route else None
    dash.dash_decode(p, q, kc, vc, lens, Lmax, ws_mat, summ, summ_blocks, o, ws, route=rb,
                     q_bar=qbar_dev(inp))
    torch.cuda.synchronize()
    nb = summ_blocks
    out = {"o": o.float().cpu().numpy(),
           "summ": summ.cpu().numpy().reshape(B, Hkv, summ_blocks, d),
           "summ_before": summ_before.cpu().numpy().reshape(B, Hkv, summ_blocks, d)}
    if route:
        out.update({
            "tau": rb.tau.cpu().numpy().reshape(B, H),
            "count": rb.sel_count.cpu().numpy().reshape(B, Hkv),
            "idx": rb.sel_idx.cpu().numpy().reshape(B, Hkv, nb),
            "logp": rb.sel_logp.cpu().numpy().reshape(B, Hkv, nb),
            "bits": unpack_bits(rb.support_bits.cpu().numpy().reshape(B, H, -1), nb),
            "tile_bits": unpack_bits(rb.tile_bits.cpu().numpy().reshape(B, Hkv, -1), nb),
            "tile_words": rb.tile_bits.cpu().numpy().reshape(B, Hkv, -1)})
    return out


def check_bias(logp, pbar, sigma):
    """Stage 2 bias sigma * log pbar written by Stage 1, against the oracle's
    pbar: in probability units for sigma > 0; for sigma = 0 the bias is 0 on
    the support and -inf off it (entries within 2e-5 of 0 may go either way)."""
    if sigma > 0:
        with np.errstate(over="ignore"):
            np.testing.assert_allclose(np.exp(logp / sigma), pbar, atol=2e-5)
        return
    off = np.isneginf(logp)
    assert np.all(logp[~off] == 0.0)
    bad = (off != (pbar == 0)) & (pbar > 2e-5)
    assert not bad.any(), f"{int(bad.sum())} support entries differ"


def check_tile_mask(words, bits, count, idx):
    """The bit-packed mask holds exactly the listed blocks: bits [..., nb] and
    words [..., nwords] against sel_count / sel_idx (bit-exact), padding bits 0."""
    nb = bits.shape[-1]
    flat_bits = bits.reshape(-1, nb)
    flat_words = words.reshape(flat_bits.shape[0], -1)
    cnt, lst = count.reshape(-1), idx.reshape(flat_bits.shape[0], -1)
    for r in range(flat_bits.shape[0]):
        np.testing.assert_array_equal(np.flatnonzero(flat_bits[r]), lst[r, :cnt[r]])
    pad = flat_words.shape[1] * 32 - nb
    if pad:
        assert not np.any(flat_words[:, -1].astype(np.uint32) >> np.uint32(32 - pad))


def check_supports(gpu_bits, x, tau, ncand):
    """gpu_bits, x [rows, H, nb]; tau [rows, H]; ncand [rows].  Bit-exact
    outside the band.  Returns the number of band-exempt entries."""
    rows, H, nb = gpu_bits.shape
    j = np.arange(nb)[None, None, :]
    valid = j < ncand[:, None, None]
    with np.errstate(invalid="ignore"):
        ref = (x > tau[:, :, None]) & valid
        band = valid & (np.abs(x - tau[:, :, None]) <= BAND)
    bad = (gpu_bits != ref) & ~band
    assert not bad.any(), f"{int(bad.sum())} support bits differ outside the band; first at " \
                          f"{np.argwhere(bad)[:5].tolist()}"
    assert not (gpu_bits & ~valid).any(), "support bit set on a non-candidate block"
    return int(band.sum())


def check_tau(gpu_tau, tau, tol=1e-5):
    """tau is a convex combination's fixed point: d tau / d x_j = u_j / sum u
    (u = p^(2-alpha)), so it inherits at most the largest float32 error of the
    scores x (a few float32 ulp of the largest |x|) plus the Newton loop's
    stopping step (1e-7 relative); 1e-5 of max(1, |tau|) bounds both."""
    nan = np.isnan(tau)
    assert np.array_equal(np.isnan(gpu_tau), nan), "NaN pattern of tau differs"
    err = np.abs(gpu_tau[~nan] - tau[~nan]) / np.maximum(1.0, np.abs(tau[~nan]))
    if err.size:
        print(f"  tau max rel err {err.max():.2e}", flush=True)
    assert err.size == 0 or err.max() <= tol, f"tau max rel err {err.max():.3e}"


def tile_union_ref(pbar_tile, x_tile, tau_tile, G):
    """Oracle tile union (pbar > 0 for any position of the tile) and the set of
    blocks whose membership may flip because every supporting entry lies in
    the band.  pbar_tile [P, nb]; x_tile/tau_tile [P, G, nb] / [P, G]."""
    union = (pbar_tile > 0).any(0)
    with np.errstate(invalid="ignore"):
        solid = ((x_tile - tau_tile[:, :, None]) > BAND).any((0, 1))
        near = (np.abs(x_tile - tau_tile[:, :, None]) <= BAND).any((0, 1))
    return union, solid, near


def check_list(gpu_count, gpu_idx, union, solid, near):
    """The GPU list must be ascending, contain every solidly selected block and
    no block outside the (union + band) set."""
    lst = gpu_idx[:gpu_count]
    assert np.all(np.diff(lst) > 0), "list not strictly ascending"
    got = np.zeros_like(union)
    got[lst] = True
    assert not (solid & ~got).any(), f"missing blocks {np.flatnonzero(solid & ~got)[:8]}"
    assert not (got & ~(union | near)).any(), f"extra blocks {np.flatnonzero(got & ~(union|near))[:8]}"
