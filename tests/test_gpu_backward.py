"""GPU backward of the causal prefill (dash_prefill_backward) against the
fp64 oracle backward (oracle/backward.py, pinned by finite differences; the
C writing prefill_backward_native carries the same pins).

The forward runs stage by stage on the GPU (its summaries, routing and
output feed the backward, as in training); the oracle recomputes everything
in float64 from the same inputs.  Both must route identically outside the
1e-5 band of tau (checked per head).  For alpha <= 1.5 an entry inside the
band that one side keeps and the other drops has
u = (x - tau)^((2-alpha)/(alpha-1)) at most 1e-5, and its bias gradient is
O(pbar), so dp = dlogp / pbar stays O(1): its share of any gradient is below
1e-5 of the gradient's scale, far inside the tolerance.  Above 1.5 the
exponent falls below 1 (sparsemax: u = 1 on the support), so there both
sides must route identically.

Coverage of the kernels' paths:
  * routing-gradient lists longer than one 32-entry LDS chunk, for 64- and
    128-key blocks (alpha 1.25 routes nearly every candidate);
  * 257 query tiles: the keys kernel finds its tiles in two batches of 256
    and the per-tile arrays take two slabs;
  * the full 8K workload (32/8 heads, d 128, up to 127 candidates per tile),
    every gradient compared in full;
  * bitwise-equal results of two runs (no floating-point atomics).

Tolerance: the GPU backward is float32 arithmetic, so on float32 inputs the
gradients agree to ~1e-5 of their scale; near a support boundary the
gradient of log pbar grows like 1/(x - tau) and inherits the forward's
float32 error in x, hence a bound relative to each tensor's largest entry:
1e-4 for float32 inputs.  bf16 inputs round the forward output o (in
delta = dO.o) and the MFMA operands P and dS to bf16 (relative error 2^-9
each, summed over a row's keys): dq, whose fine and coarse parts both carry
dS, within 1e-2 of its scale (observed up to 6.4e-3), dk within 8e-3
(observed 4.2e-3), dv, a sum of P dO, within 4e-3 (observed 1.7e-3), and
dW_s, summed over every block, within 1e-3 (observed 3.0e-4).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_hierarchical_attention_block_amd as dash
import workloads as W
from gpu_helpers import dev, params, to_dev, unpack_bits
from oracle.backward import prefill_backward, prefill_backward_native

pytestmark = pytest.mark.gpu

P8K = W.get("prefill_8k")
BF16_TOL = {"dq": 1e-2, "dk": 8e-3, "dv": 4e-3, "dw_s": 1e-3}
CASES = {
    "f32_gqa2_d64": (W.get("tiny").replace(n_heads=4, n_kv_heads=2, seq_len=640, gamma=8.0),
                     1e-4),
    "f32_alpha2_sigma_window": (W.get("tiny").replace(n_heads=2, n_kv_heads=1, seq_len=520,
                                                      alpha=2.0, gamma=6.0, sigma=0.5,
                                                      window=2), 1e-4),
    "bf16_gqa4_d128": (P8K.replace(seq_len=768, n_heads=8, n_kv_heads=2), BF16_TOL),
    "bf16_bs128_batch2": (W.get("tiny").replace(batch=2, n_heads=4, n_kv_heads=2, seq_len=700,
                                                block_size=128, dtype="bf16", gamma=6.0),
                          BF16_TOL),
    # 128-key blocks with a two-block branch (the summary-gradient sum starts at tile 2 j + 4)
    "bf16_bs128_window2": (W.get("tiny").replace(n_heads=4, n_kv_heads=2, seq_len=900,
                                                 block_size=128, dtype="bf16", gamma=6.0,
                                                 window=2), BF16_TOL),
    # one head per KV head (two-wave rows workgroups), ragged tail
    "bf16_mha_d128": (P8K.replace(seq_len=600, n_heads=2, n_kv_heads=2), BF16_TOL),
    # eight heads per KV head (two workgroups per tile), window and prior strength
    "bf16_gqa8_window2_sigma": (P8K.replace(seq_len=640, n_heads=16, n_kv_heads=2, window=2,
                                            sigma=0.5), BF16_TOL),
    # lists of up to 39 (64-key blocks) and 35 (128-key blocks) entries: more
    # than one 32-entry chunk of the routing gradient
    "bf16_bs64_lists_over_32": (P8K.replace(seq_len=2560, n_heads=8, n_kv_heads=2, alpha=1.25),
                                BF16_TOL),
    "bf16_bs128_lists_over_32": (W.get("prefill_64k").replace(seq_len=4608, n_heads=8,
                                                              n_kv_heads=4, alpha=1.25),
                                 BF16_TOL),
    # 257 query tiles: two batches of the keys kernel's tile flags, two slabs
    "bf16_257_tiles_d64": (P8K.replace(seq_len=16448, n_heads=8, n_kv_heads=8, head_dim=64),
                           BF16_TOL),
}


def _run(w, seed=4321):
    """GPU forward stage by stage, then the backward; returns inputs, dO,
    the GPU routing buffers and the gradients."""
    inp = W.make_prefill(w)
    B, H, Hkv, N, d, bs = w.batch, w.n_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block_size
    rng = np.random.default_rng(seed)
    d_o = W.round_bf16(rng.standard_normal((B, H, N, d)).astype(np.float32)) \
        if w.dtype == "bf16" else rng.standard_normal((B, H, N, d)).astype(np.float32)
    p = params(w)
    q, k, v, dO = (to_dev(x, w.dtype) for x in (inp["q"], inp["k"], inp["v"], d_o))
    ws_mat = torch.from_numpy(inp["w_s"]).to(dev())
    nb = max(N // bs, 1)
    summ = torch.zeros(B * Hkv * nb * d, dtype=torch.float32, device=dev())
    dash.dash_summarize(p, k, N, 0, N // bs, ws_mat, summ, nb)
    rb = dash.RouteBuffers(dash.dash_route_sizes_prefill(p, N), dev(), bits=True)
    dash.dash_route(p, q, N, summ, nb, rb)
    o = torch.empty_like(q)
    dash.dash_attend(p, q, k, v, N, rb, o)
    ws = dash.workspace(dash.dash_prefill_backward_workspace_bytes(p, N), dev())

    def backward():
        grads = {name: torch.empty(shape, dtype=torch.float32, device=dev())
                 for name, shape in (("dq", q.shape), ("dk", k.shape), ("dv", v.shape),
                                     ("dw_s", (d, d)))}
        dash.dash_prefill_backward(p, q, k, v, o, dO, N, ws_mat, summ, nb, rb, grads["dq"],
                                   grads["dk"], grads["dv"], grads["dw_s"], ws)
        return grads
    grads = backward()
    torch.cuda.synchronize()
    return inp, d_o, rb, grads, backward


def _check_routing(w, inp, rb):
    """GPU per-head supports against the oracle's x > tau; returns the number
    of differing entries (all inside the 1e-5 band)."""
    B, H, N, bs = w.batch, w.n_heads, w.seq_len, w.block_size
    nbo = -(-N // bs)
    ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["w_s"], bs=bs, alpha=w.alpha,
                         gamma=w.gamma, nb_out=nbo, want=("tau", "x"), sigma=w.sigma,
                         window=w.window)
    gb = unpack_bits(rb.support_bits.cpu().numpy().reshape(B, H, N, -1), nbo)
    gb = gb.transpose(0, 2, 1, 3).reshape(B * N, H, nbo)
    with np.errstate(invalid="ignore"):
        ob = ref["x"] > ref["tau"][:, :, None]
        near = np.abs(ref["x"] - ref["tau"][:, :, None]) <= 1e-5
    diff = gb != ob
    assert not (diff & ~near).any(), "routing differs from the oracle outside the tau band"
    nd = int(diff.sum())
    assert w.alpha <= 1.5 or nd == 0, f"{nd} support entries inside the tau band differ"
    return nd


def _compare(grads, ref, tols):
    for name in ("dq", "dk", "dv", "dw_s"):
        tol = tols[name] if isinstance(tols, dict) else tols
        g = grads[name].cpu().numpy().astype(np.float64)
        r = ref[name]
        scale = np.abs(r).max()
        err = np.abs(g - r).max()
        print(f"  {name}: max |ref| {scale:.3e}, max err {err:.3e} ({err / scale:.2e})",
              flush=True)
        assert err <= tol * scale, f"{name}: {err:.3e} > {tol} * {scale:.3e}"


@pytest.mark.parametrize("case", list(CASES))
def test_prefill_backward(case):
    w, tol = CASES[case]
    print(f"[backward] {case}: {w}", flush=True)
    inp, d_o, rb, grads, _ = _run(w)
    nd = _check_routing(w, inp, rb)
    print(f"  support entries inside the tau band that differ: {nd}", flush=True)
    ref = prefill_backward_native(inp["q"], inp["k"], inp["v"], inp["w_s"], d_o,
                                  bs=w.block_size, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma,
                                  window=w.window)
    _compare(grads, ref, tol)


def test_prefill_backward_numpy_oracle():
    """One small case against the numpy writing of the oracle backward."""
    w, tol = CASES["bf16_gqa4_d128"]
    inp, d_o, rb, grads, _ = _run(w)
    ref = prefill_backward(inp["q"], inp["k"], inp["v"], inp["w_s"], d_o, bs=w.block_size,
                           alpha=w.alpha, gamma=w.gamma)
    _compare(grads, ref, tol)


def test_prefill_backward_full_size_8k():
    """The whole 8K prefill workload (B 1, N 8192, H 32 / Hkv 8, d 128, block
    64, bf16), as the benchmark times it: dq, dk, dv and dW_s in full."""
    w = P8K
    print(f"[backward full] {w}", flush=True)
    inp, d_o, rb, grads, _ = _run(w, seed=5)
    nd = _check_routing(w, inp, rb)
    print(f"  support entries inside the tau band that differ: {nd}", flush=True)
    ref = prefill_backward_native(inp["q"], inp["k"], inp["v"], inp["w_s"], d_o,
                                  bs=w.block_size, alpha=w.alpha, gamma=w.gamma)
    _compare(grads, ref, BF16_TOL)


@pytest.mark.parametrize("case", ["bf16_257_tiles_d64", "f32_gqa2_d64"])
def test_prefill_backward_bitwise_reproducible(case):
    w, _ = CASES[case]
    _, _, _, first, backward = _run(w)
    for _ in range(2):
        again = backward()
        torch.cuda.synchronize()
        for name in first:
            assert torch.equal(first[name], again[name]), f"{name} differs between runs"
