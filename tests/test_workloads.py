"""Seeded synthetic inputs: determinism, slice regeneration, bf16 rounding."""
import numpy as np
import torch

import workloads as W


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10 ** rng.uniform(-8, 8),
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.3895314e38], np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(W.round_bf16(a), ref)


def test_prefill_is_deterministic_and_sliceable():
    w = W.get("prefill_8k").replace(seq_len=512, batch=2)
    a = W.make_prefill(w)
    b = W.make_prefill(w, batches=[1])
    for key in ("q", "k", "v"):
        np.testing.assert_array_equal(a[key][1:], b[key])
    np.testing.assert_array_equal(W.round_bf16(a["q"]), a["q"])   # bf16-exact values
    np.testing.assert_array_equal(a["w_s"], b["w_s"])


def test_planted_structure():
    w = W.get("prefill_8k").replace(seq_len=1024)
    plan = W.prefill_plan(w, 0, 3)
    assert len(plan) == 1024 // 64
    for t, (u, rel) in enumerate(plan):
        assert abs(np.linalg.norm(u) - 1) < 1e-5
        assert len(rel) <= min(t, 24) and (t < 2 or len(rel) >= 2)
        assert len(set(rel.tolist())) == len(rel) and (rel < t).all()


def test_decode_inputs():
    w = W.get("decode_32k").replace(seq_len=4096, batch=3)
    a = W.make_decode(w)
    b = W.make_decode(w, batches=[2])
    assert a["q"].shape == (3, 32, 128) and a["k_cache"].shape == (3, 8, 4096, 128)
    np.testing.assert_array_equal(a["k_cache"][2], b["k_cache"][0])
    np.testing.assert_array_equal(a["q"][2], b["q"][0])
    assert (a["cache_len"] == 4096).all()
