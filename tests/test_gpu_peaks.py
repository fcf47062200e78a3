"""GPU: the measurement helpers that the roofline fractions are stated against.

* dash_peak_stream mode 0 copies its source exactly (a ragged length that is
  not a multiple of the grid's stride);
* modes 1 and 2 fold every 16-byte source vector into exactly one thread's
  value by XOR, so the XOR over all stored vectors equals the XOR over the
  whole source, whatever the split between threads;
* dash_peak_mfma runs `iters` products of one fixed 32x32x16 bf16 tile pair
  per chain; the sum over a wave's accumulators is then 8 * iters times the
  sum over the tile product, sum_k (sum_i A[i,k]) (sum_j B[k,j]), which does
  not depend on how the output elements are spread over the lanes.
"""
import numpy as np
import pytest
import torch

import sparse_hierarchical_attention_block_amd as dash
from gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _xor_all(t):
    v = t.cpu().numpy().view(np.uint32).reshape(-1, 4)
    return np.bitwise_xor.reduce(v, axis=0)


def test_peak_stream_copy():
    g = torch.Generator().manual_seed(11)
    n16 = dash.dash_peak_stream_grid() * 5 + 37
    src = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), generator=g, dtype=torch.int32).to(dev())
    dst = torch.zeros_like(src)
    dash.dash_peak_stream(src, dst, n16 * 16, 0)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("mode", [1, 2])
def test_peak_stream_read_folds_every_vector(mode):
    g = torch.Generator().manual_seed(12 + mode)
    threads = dash.dash_peak_stream_grid()
    for n16 in (threads * 8 * 3 + 5, 100):
        src = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), generator=g,
                            dtype=torch.int32).to(dev())
        dst = torch.full((threads * 4,), -1, dtype=torch.int32, device=dev())
        dash.dash_peak_stream(src, dst, n16 * 16, mode)
        torch.cuda.synchronize()
        assert np.array_equal(_xor_all(dst), _xor_all(src)), (mode, n16)


def test_peak_stream_rejects_bad_mode():
    src = torch.zeros(64, dtype=torch.int32, device=dev())
    dst = torch.zeros(dash.dash_peak_stream_grid() * 4, dtype=torch.int32, device=dev())
    for mode in (3, -1):
        with pytest.raises(Exception):
            dash.dash_peak_stream(src, dst, 256, mode)


def test_peak_mfma_sum_and_flops():
    waves = dash.dash_peak_mfma_grid()
    sink = torch.full((waves,), float("nan"), dtype=torch.float32, device=dev())
    iters = 4
    flops = dash.dash_peak_mfma(iters, sink)
    torch.cuda.synchronize()
    assert flops == waves * iters * 8 * 2.0 * 32 * 32 * 16
    # lane l holds A[l % 32][8 (l // 32) + e] and B[8 (l // 32) + e][l % 32]
    lane = torch.arange(64, dtype=torch.float32)
    e = torch.arange(8, dtype=torch.float32)
    a = (0.001 * (lane[:, None] + e[None, :])).to(torch.bfloat16).double()
    b = (0.002 * (lane[:, None] - e[None, :])).to(torch.bfloat16).double()
    total = 0.0
    for h in range(2):
        rows = slice(32 * h, 32 * h + 32)
        total += float((a[rows].sum(0) * b[rows].sum(0)).sum())
    want = 8 * iters * total
    got = sink.cpu().double().numpy()
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, want, rtol=1e-4, atol=1e-6)
