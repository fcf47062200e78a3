"""GPU: prefill of a ragged batch (sequences of different lengths in one
call) against the oracle run on each sequence alone, and against
dash_prefill on each sequence alone (the launch shapes differ with the
length, so the two agree to the parity tolerance, summaries bit for bit).
Rows past a sequence's length and summaries past its last complete block
must stay untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_hierarchical_attention_block_amd as dash
import workloads as W
from gpu_helpers import TOL, dev, params, qbar_dev, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "f32_tiny": (W.get("tiny").replace(batch=4, n_heads=4, n_kv_heads=2, seq_len=700,
                                       gamma=8.0), [700, 1, 64, 333]),
    "bf16_gqa4_d128": (W.get("prefill_8k").replace(batch=3, seq_len=1600),
                       [1600, 129, 1000]),
    "bf16_bs128_window2_qbar": (W.get("prefill_64k").replace(batch=3, seq_len=1500, gamma=2.0,
                                                             window=2, sigma=0.5,
                                                             summary_query=1.0),
                                [256, 1500, 0]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_varlen_prefill(case):
    w, lens = CASES[case]
    print(f"[varlen prefill] {case}: {w} lens={lens}", flush=True)
    inp = W.make_prefill(w)
    p = params(w)
    B, H, Hkv, N, d, bs = w.batch, w.n_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block_size
    q, k, v = (to_dev(inp[x], w.dtype) for x in ("q", "k", "v"))
    ws_mat = torch.from_numpy(inp["w_s"]).to(dev())
    qb = qbar_dev(inp)
    nb = N // bs
    summ = torch.full((B * Hkv * nb * d,), 5.0, dtype=torch.float32, device=dev())
    o = torch.full_like(q, 3.0)
    ws = dash.workspace(dash.dash_prefill_workspace_bytes(p, N), dev())
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev())
    dash.dash_prefill_varlen(p, q, k, v, N, lens_d, ws_mat, summ, nb, o, ws, q_bar=qb)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    gs = summ.cpu().numpy().reshape(B, Hkv, nb, d)
    for b, n in enumerate(lens):
        assert np.all(got[b, :, n:] == 3.0), f"sequence {b}: rows past its length written"
        assert np.all(gs[b, :, n // bs:] == 5.0), f"sequence {b}: summaries past its blocks"
        if n == 0:
            continue
        # the sequence alone through dash_prefill: identical results
        pb = params(w, batch=1)
        qs, ks, vs = (t[b:b + 1, :, :n].contiguous() for t in (q, k, v))
        os_ = torch.empty_like(qs)
        ss = torch.zeros(Hkv * max(n // bs, 1) * d, dtype=torch.float32, device=dev())
        wss = dash.workspace(dash.dash_prefill_workspace_bytes(pb, n), dev())
        dash.dash_prefill(pb, qs, ks, vs, n, ws_mat, ss, max(n // bs, 1), os_, wss, q_bar=qb)
        torch.cuda.synchronize()
        np.testing.assert_allclose(got[b, :, :n], os_.float().cpu().numpy()[0], rtol=0,
                                   atol=TOL[w.dtype])
        np.testing.assert_array_equal(gs[b, :, :n // bs],
                                      ss.cpu().numpy().reshape(Hkv, -1, d)[:, :n // bs])
        # and the oracle on that sequence
        ref = oracle.prefill(inp["q"][b:b + 1, :, :n], inp["k"][b:b + 1, :, :n],
                             inp["v"][b:b + 1, :, :n], inp["w_s"], bs=bs, alpha=w.alpha,
                             gamma=w.gamma, q_bar=inp.get("q_bar"), sigma=w.sigma,
                             window=w.window)
        err = np.abs(got[b, :, :n].transpose(1, 0, 2) - ref["o"]).max()
        assert err <= TOL[w.dtype], f"sequence {b}: max-abs err {err:.3e}"
        np.testing.assert_allclose(gs[b, :, :n // bs], ref["summ"][0], rtol=1e-5, atol=2e-5)
        print(f"  sequence {b} (n={n}) max-abs err {err:.3e}", flush=True)
