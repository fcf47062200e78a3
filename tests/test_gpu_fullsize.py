"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the fused dash_prefill / dash_decode entry points), checked
on sampled outputs the oracle computes row by row.

Workloads: causal prefill 8K (32/8 heads, d 128, block 64, bf16), batched
decode 32 x 32K, long prefill 64K (block 128, alpha 1.25 / 1.5 / 2) and long
decode 8 x 128K (64/8 heads, log-uniform planted counts).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_hierarchical_attention_block_amd as dash
import workloads as W
from gpu_helpers import TOL, check_supports, check_tau, dev, params, to_dev, unpack_bits

pytestmark = pytest.mark.gpu
QT = 64


def _prefill_full(w):
    inp = W.make_prefill(w)
    p = params(w)
    B, H, Hkv, N, d, bs = w.batch, w.n_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block_size
    q, k, v = (to_dev(inp[x], w.dtype) for x in ("q", "k", "v"))
    ws_mat = torch.from_numpy(inp["w_s"]).to(dev())
    nb = N // bs
    summ = torch.zeros(B * Hkv * nb * d, dtype=torch.float32, device=dev())
    o = torch.empty_like(q)
    ws = dash.workspace(dash.dash_prefill_workspace_bytes(p, N), dev())
    # all bits set: the bias rows Stage 1 does not write read as NaN, so an
    # output that used one would show it
    ws.fill_(255)
    dash.dash_prefill(p, q, k, v, N, ws_mat, summ, nb, o, ws)
    # stage-wise run with per-head supports (same kernels, same launch shapes)
    sizes = dash.dash_route_sizes_prefill(p, N)
    rb = dash.RouteBuffers(sizes, dev(), bits=True)
    dash.dash_route(p, q, N, summ, nb, rb)
    torch.cuda.synchronize()
    return inp, o, rb, sizes


def _sample_positions(N, rng, tiles=(1, 2), extra=24):
    n_qt = N // QT
    full = [t % n_qt for t in tiles] + [n_qt - 1]
    pos = np.concatenate([np.arange(t * QT, t * QT + QT) for t in sorted(set(full))] +
                         [rng.choice(N, size=extra, replace=False)])
    return np.unique(pos)


@pytest.mark.parametrize("name,alpha", [("prefill_8k", 1.5), ("prefill_64k", 1.5),
                                        ("prefill_64k", 1.25), ("prefill_64k", 2.0)])
def test_prefill_full_size_sampled(name, alpha):
    w = W.get(name).replace(alpha=alpha)
    print(f"[full prefill] {w}", flush=True)
    inp, o, rb, sizes = _prefill_full(w)
    N, H, Hkv, bs, G = w.seq_len, w.n_heads, w.n_kv_heads, w.block_size, w.group
    nb = N // bs
    rng = np.random.default_rng(123)
    pos = _sample_positions(N, rng, tiles=(1, 2, N // QT // 2))
    ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["w_s"], bs=bs, alpha=alpha,
                         gamma=w.gamma, positions=pos, nb_out=nb, want=("o", "tau", "x", "pbar"))
    got = o[0][:, torch.from_numpy(pos).to(dev())].float().cpu().numpy().transpose(1, 0, 2)
    err = np.abs(got - ref["o"]).max()
    assert err <= TOL["bf16"], f"output max-abs err {err:.3e}"
    tau = rb.tau.view(1, H, N)[0][:, torch.from_numpy(pos).to(dev())].cpu().numpy().T
    check_tau(tau, ref["tau"])
    bits = unpack_bits(rb.support_bits.view(1, H, N, -1)[0].cpu().numpy()[:, pos], nb)
    nband = check_supports(bits.transpose(1, 0, 2), ref["x"], ref["tau"], pos // bs)
    # complete tiles in the sample: lists must match the oracle unions
    count = rb.sel_count.view(Hkv, -1).cpu().numpy()
    idx = rb.sel_idx.view(Hkv, -1, nb).cpu().numpy()
    for qt in np.unique(pos // QT):
        rows = np.flatnonzero(pos // QT == qt)
        if len(rows) < QT:
            continue
        t = (qt * QT) // bs
        for g in range(Hkv):
            hs = slice(g * G, g * G + G)
            sel = np.zeros(nb, bool)
            sel[idx[g, qt, :count[g, qt]]] = True
            union = (ref["pbar"][rows, g, :t] > 0).any(0)
            with np.errstate(invalid="ignore"):
                near = (np.abs(ref["x"][rows][:, hs, :t] - ref["tau"][rows][:, hs, None])
                        <= 1e-5).any((0, 1))
            assert not ((sel[:t] != union) & ~near).any(), f"tile {qt} head {g}"
    print(f"  max-abs err {err:.3e}, band-exempt bits {nband}", flush=True)


@pytest.mark.parametrize("name,seqs", [("decode_32k", [0, 13, 31]), ("decode_128k", [0, 5])])
def test_decode_full_size_sampled(name, seqs):
    w = W.get(name)
    print(f"[full decode] {w}", flush=True)
    p = params(w)
    B, H, Hkv, d, bs, L = w.batch, w.n_heads, w.n_kv_heads, w.head_dim, w.block_size, w.seq_len
    nb = L // bs
    kc = torch.empty((B, Hkv, L, d), dtype=torch.bfloat16, device=dev())
    vc = torch.empty_like(kc)
    q = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev())
    keep = {}
    for b in range(B):            # upload one sequence at a time
        one = W.make_decode(w, batches=[b])
        kc[b] = to_dev(one["k_cache"][0], "bf16")
        vc[b] = to_dev(one["v_cache"][0], "bf16")
        q[b] = to_dev(one["q"][0], "bf16")
        if b in seqs:
            keep[b] = one
        w_s = one["w_s"]
    ws_mat = torch.from_numpy(w_s).to(dev())
    summ = torch.zeros(B * Hkv * nb * d, dtype=torch.float32, device=dev())
    dash.dash_summarize(p, kc, L, 0, nb - 1, ws_mat, summ, nb)
    lens = torch.full((B,), L, dtype=torch.int32, device=dev())
    o = torch.empty_like(q)
    ws = dash.workspace(dash.dash_decode_workspace_bytes(p, L), dev())
    rb = dash.RouteBuffers(dash.dash_route_sizes_decode(p, L), dev(), bits=True)
    dash.dash_decode(p, q, kc, vc, lens, L, ws_mat, summ, nb, o, ws, route=rb)
    torch.cuda.synchronize()
    og = o.float().cpu().numpy()
    bits = unpack_bits(rb.support_bits.view(B, H, -1).cpu().numpy(), nb)
    tau = rb.tau.view(B, H).cpu().numpy()
    for b in seqs:
        one = keep[b]
        ref = oracle.decode(one["q"], one["k_cache"], one["v_cache"], [L], one["w_s"], bs=bs,
                            alpha=w.alpha, gamma=w.gamma, nb_out=nb, want=("o", "tau", "x", "pbar"))
        err = np.abs(og[b] - ref["o"][0]).max()
        assert err <= TOL["bf16"], f"seq {b}: max-abs err {err:.3e}"
        check_tau(tau[b:b + 1], ref["tau"])
        check_supports(bits[b:b + 1], ref["x"], ref["tau"], np.array([(L - 1) // bs]))
        summ_ref = ref["new_summary"][0]
        got = summ.view(B, Hkv, nb, d)[b, :, nb - 1].cpu().numpy()
        np.testing.assert_allclose(got, summ_ref, rtol=1e-5, atol=2e-5)
        print(f"  seq {b}: max-abs err {err:.3e}", flush=True)
