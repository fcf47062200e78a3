"""GPU backward of the causal prefill (dash_prefill_backward) against the
fp64 oracle backward (oracle/backward.py, pinned by finite differences).

The forward runs stage by stage on the GPU (its summaries, routing and
output feed the backward, as in training); the oracle recomputes everything
in float64 from the same inputs.  Both must route identically, so the cases
use inputs whose supports have no entry within the parity band of tau.

Tolerance: the GPU backward is float32 arithmetic, so on float32 inputs the
gradients agree to ~1e-5 of their scale; near a support boundary the
gradient of log pbar grows like 1/(x - tau) and inherits the forward's
float32 error in x, hence a bound relative to each tensor's largest entry:
1e-4 for float32 inputs (observed up to 1.2e-5), 1e-2 for bf16 inputs, whose
forward output o, used in delta = dO.o, is rounded to bf16 (observed up to
3.1e-3).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_hierarchical_attention_block_amd as dash
import workloads as W
from gpu_helpers import dev, params, to_dev
from oracle.backward import prefill_backward

pytestmark = pytest.mark.gpu

CASES = {
    "f32_gqa2_d64": (W.get("tiny").replace(n_heads=4, n_kv_heads=2, seq_len=640, gamma=8.0),
                     1e-4),
    "f32_alpha2_sigma_window": (W.get("tiny").replace(n_heads=2, n_kv_heads=1, seq_len=520,
                                                      alpha=2.0, gamma=6.0, sigma=0.5,
                                                      window=2), 1e-4),
    "bf16_gqa4_d128": (W.get("prefill_8k").replace(seq_len=768, n_heads=8, n_kv_heads=2), 1e-2),
    "bf16_bs128_batch2": (W.get("tiny").replace(batch=2, n_heads=4, n_kv_heads=2, seq_len=700,
                                                block_size=128, dtype="bf16", gamma=6.0), 1e-2),
    # 128-key blocks with a two-block branch (the summary-gradient sum starts at tile 2 j + 4)
    "bf16_bs128_window2": (W.get("tiny").replace(n_heads=4, n_kv_heads=2, seq_len=900,
                                                 block_size=128, dtype="bf16", gamma=6.0,
                                                 window=2), 1e-2),
    # one head per KV head (two-wave rows workgroups), ragged tail
    "bf16_mha_d128": (W.get("prefill_8k").replace(seq_len=600, n_heads=2, n_kv_heads=2), 1e-2),
    # eight heads per KV head (two workgroups per tile), window and prior strength
    "bf16_gqa8_window2_sigma": (W.get("prefill_8k").replace(seq_len=640, n_heads=16,
                                                            n_kv_heads=2, window=2, sigma=0.5),
                                1e-2),
}


@pytest.mark.parametrize("case", list(CASES))
def test_prefill_backward(case):
    w, tol = CASES[case]
    print(f"[backward] {case}: {w}", flush=True)
    inp = W.make_prefill(w)
    B, H, Hkv, N, d, bs = w.batch, w.n_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block_size
    rng = np.random.default_rng(4321)
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
    grads = {name: torch.empty(shape, dtype=torch.float32, device=dev())
             for name, shape in (("dq", q.shape), ("dk", k.shape), ("dv", v.shape),
                                 ("dw_s", (d, d)))}
    ws = dash.workspace(dash.dash_prefill_backward_workspace_bytes(p, N), dev())
    dash.dash_prefill_backward(p, q, k, v, o, dO, N, ws_mat, summ, nb, rb, grads["dq"],
                               grads["dk"], grads["dv"], grads["dw_s"], ws)
    torch.cuda.synchronize()

    # the GPU routed exactly like the oracle (no entry near tau)
    ref_f = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["w_s"], bs=bs, alpha=w.alpha,
                           gamma=w.gamma, nb_out=-(-N // bs), want=("o", "tau", "x"),
                           sigma=w.sigma, window=w.window)
    nbo = -(-N // bs)
    bits = rb.support_bits.cpu().numpy().reshape(B, H, N, -1).astype(np.uint32)
    gb = ((bits[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(bool)
    gb = gb.reshape(B, H, N, -1)[..., :nbo].transpose(0, 2, 1, 3).reshape(B * N, H, nbo)
    with np.errstate(invalid="ignore"):
        ob = ref_f["x"] > ref_f["tau"][:, :, None]
    assert np.array_equal(gb, ob), "routing differs from the oracle"

    ref = prefill_backward(inp["q"], inp["k"], inp["v"], inp["w_s"], d_o, bs=bs, alpha=w.alpha,
                           gamma=w.gamma, sigma=w.sigma, window=w.window)
    for name in ("dq", "dk", "dv", "dw_s"):
        g = grads[name].cpu().numpy().astype(np.float64)
        r = ref[name]
        scale = np.abs(r).max()
        err = np.abs(g - r).max()
        print(f"  {name}: max |ref| {scale:.3e}, max err {err:.3e} ({err / scale:.2e})",
              flush=True)
        assert err <= tol * scale, f"{name}: {err:.3e} > {tol} * {scale:.3e}"
