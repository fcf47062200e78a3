"""dash_decode_noalloc (the decode step with the library's static device
scratch as workspace, for callers that cannot allocate) against dash_decode
with a caller-allocated workspace: the same kernels, so every output --
attention output, routing result and the completed block's summary -- must
be bitwise equal.  Two calls in a row, the second with a smaller problem
(fewer sequences, shorter caches), so the second reuses scratch the first
left behind.  Collected last (its file name sorts after every other test):
it runs both alone in a fresh process and after the other GPU tests.
"""
import numpy as np
import pytest
import torch

import sparse_hierarchical_attention_block_amd as dash
import workloads as W
from gpu_helpers import dev, params, to_dev

pytestmark = pytest.mark.gpu


def _inputs(w, lens):
    inp = W.make_decode(w, cache_len=lens)
    B, Hkv, d, bs, L = w.batch, w.n_kv_heads, w.head_dim, w.block_size, w.cache_len
    t = {"q": to_dev(inp["q"], w.dtype), "k": to_dev(inp["k_cache"], w.dtype),
         "v": to_dev(inp["v_cache"], w.dtype),
         "lens": torch.from_numpy(np.asarray(lens, np.int32)).to(dev()),
         "w_s": torch.from_numpy(inp["w_s"]).to(dev())}
    nb = -(-L // bs)
    summ = torch.zeros(B * Hkv * nb * d, dtype=torch.float32, device=dev())
    p = params(w)
    dash.dash_summarize(p, t["k"], L, 0, L // bs, t["w_s"], summ, nb)
    t["summ"], t["nb"] = summ, nb
    return p, t


def _step(p, w, t, noalloc):
    L = w.cache_len
    o = torch.empty_like(t["q"])
    summ = t["summ"].clone()
    rb = dash.RouteBuffers(dash.dash_route_sizes_decode(p, L), dev(), bits=True)
    if noalloc:
        dash.dash_decode_noalloc(p, t["q"], t["k"], t["v"], t["lens"], L, t["w_s"], summ,
                                 t["nb"], o, route=rb)
    else:
        ws = dash.workspace(dash.dash_decode_workspace_bytes(p, L), dev())
        dash.dash_decode(p, t["q"], t["k"], t["v"], t["lens"], L, t["w_s"], summ, t["nb"], o,
                         ws, route=rb)
    torch.cuda.synchronize()
    return o, summ, rb


def test_noalloc_decode_matches_decode_two_calls():
    # call 1: 16 sequences x 8K (a 32-pair batch, lengths mixed so that some
    # steps complete a block); call 2: 4 sequences x 2K, a smaller problem
    first = W.get("decode_32k").replace(batch=16, seq_len=8192)
    second = W.get("decode_32k").replace(batch=4, seq_len=2048)
    lens1 = [8192, 8191, 4096, 5000] * 4
    lens2 = [2048, 1500, 640, 2047]
    for w, lens in ((first, lens1), (second, lens2)):
        print(f"[noalloc] batch {w.batch} x {w.seq_len}", flush=True)
        p, t = _inputs(w, lens)
        o_ref, s_ref, r_ref = _step(p, w, t, noalloc=False)
        o, s, r = _step(p, w, t, noalloc=True)
        assert torch.equal(o, o_ref), "outputs differ"
        assert torch.equal(s, s_ref), "summaries differ"
        for name in ("tau", "sel_count", "support_bits"):
            assert torch.equal(getattr(r, name), getattr(r_ref, name)), f"{name} differs"
        cnt = r_ref.sel_count.cpu().numpy()
        idx, idx_ref = r.sel_idx.view(len(cnt), -1).cpu(), r_ref.sel_idx.view(len(cnt), -1).cpu()
        for i, c in enumerate(cnt):
            assert torch.equal(idx[i, :c], idx_ref[i, :c]), "selected blocks differ"


def test_noalloc_rejects_oversized_problem():
    # 64 sequences x 128K with 64 query heads needs ~170 MiB of workspace
    w = W.get("decode_128k").replace(batch=64)
    p = params(w)
    assert dash.dash_decode_workspace_bytes(p, w.seq_len) > 32 << 20
    one = torch.zeros(16, dtype=torch.bfloat16, device=dev())
    with pytest.raises(dash.DashError, match="WORKSPACE_TOO_SMALL"):
        dash._lib._check("dash_decode_noalloc", dash._lib._lib.dash_decode_noalloc(
            __import__("ctypes").byref(p), one.data_ptr(), one.data_ptr(), one.data_ptr(),
            one.data_ptr(), w.seq_len, one.data_ptr(), None, one.data_ptr(),
            w.seq_len // w.block_size, one.data_ptr(), None, None))
