"""Benchmark of the DashAttention forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_8k]

A step is one fused causal prefill (dash_prefill: Stage 0 summaries, Stage 1
entmax routing, Stage 2 prior-induced sparse attention) over the workload's
synthetic batch, inputs resident in HBM.  ``value`` is prefill tokens/s
(B * N / step time).  The same line carries:
  roofline      the attend kernel (the dominant one): selected-tile MFMA flops
                per launch / its average launch time (HIP events on the stream
                it runs on) against the 2.5 PFLOP/s dense bf16 peak;
  stages        per-stage kernel times (each entry point timed alone);
  decode        one batched decode step (dash_decode) on the 32 x 32K decode
                workload: microseconds per step and selected-KV GB/s against
                the 8 TB/s HBM peak;
  cpu_baseline  the fp64 CPU oracle timed on this host's cores on a bounded
                sample of the same workload, scaled to tokens/s.
Only one GPU is used; --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tok/s + decode step µs at ~75% block sparsity; % HBM/MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3      # vector float32 FMA peak
QT = 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_prefill_8k_traffic.txt")
ATTEND_SRC = os.path.join(ROOT, "sparse_hierarchical_attention_block_amd", "csrc", "attend.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 untimed steps bring the GPU to its steady clock before the timed
    # steps (5 warmup steps of this workload are ~1.5 ms of work, during which
    # the clock is still ramping)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="prefill_8k")
    ap.add_argument("--decode-workload", default="decode_32k")
    ap.add_argument("--alpha", type=float, default=None)
    ap.add_argument("--sigma", type=float, default=None,
                    help="prior strength (default: the workload's, 1)")
    ap.add_argument("--window", type=int, default=None,
                    help="near-diagonal branch in blocks (default: the workload's, 1)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward of the prefill step")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the ragged-batch prefill leg")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--dense", action="store_true",
                    help="also time the in-house dense causal attention (all blocks, zero prior)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="launch one device copy of this many MiB (HBM-counter calibration)")
    return ap.parse_args()


def events_time(fn, steps, warmup, torch):
    """Average milliseconds of fn() over `steps` calls on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def traffic_for_attend(workload):
    """HBM bytes per attend launch from the committed counter summary, or None
    when the counters were taken on another workload or the kernel source
    changed since they were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    src = hashlib.sha256(open(ATTEND_SRC, "rb").read()).hexdigest()
    if kv.get("attend_hip_sha256") != src or kv.get("workload") != workload:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def with_overrides(w, args, alpha=True):
    """The workload with the command line's alpha / sigma / window applied."""
    if alpha and args.alpha is not None:
        w = w.replace(alpha=args.alpha)
    if args.sigma is not None:
        w = w.replace(sigma=args.sigma)
    if args.window is not None:
        w = w.replace(window=args.window)
    return w


def prefill_bench(args, torch, dash, W):
    w = with_overrides(W.get(args.workload), args)
    dev = torch.device("cuda:0")
    inp = W.make_prefill(w)
    B, H, Hkv, N, d, bs, G = w.batch, w.n_heads, w.n_kv_heads, w.seq_len, w.head_dim, \
        w.block_size, w.group
    p = dash.make_params(B, H, Hkv, d, bs, w.alpha, w.gamma, w.dtype, w.sigma, w.window)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(inp[x]).to(dev, tdt) for x in ("q", "k", "v"))
    ws_mat = torch.from_numpy(inp["w_s"]).to(dev)
    nb = N // bs
    summ = torch.zeros(B * Hkv * nb * d, dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    ws = dash.workspace(dash.dash_prefill_workspace_bytes(p, N), dev)
    del inp

    step = lambda: dash.dash_prefill(p, q, k, v, N, ws_mat, summ, nb, o, ws)  # noqa: E731
    ms_step = events_time(step, args.steps, args.warmup, torch)

    # stage-wise launches of the same kernels
    sizes = dash.dash_route_sizes_prefill(p, N)
    rb = dash.RouteBuffers(sizes, dev)
    t_sum = events_time(lambda: dash.dash_summarize(p, k, N, 0, nb, ws_mat, summ, nb),
                        args.steps, 2, torch)
    # Stage 0 pooled by seeded summary queries (same keys, same output size)
    qb = torch.from_numpy(W.summary_query(w.replace(summary_query=1.0))).to(dev)
    summ_q = torch.empty_like(summ)
    t_sum_q = events_time(lambda: dash.dash_summarize(p, k, N, 0, nb, ws_mat, summ_q, nb,
                                                      q_bar=qb), args.steps, 2, torch)
    t_route = events_time(lambda: dash.dash_route(p, q, N, summ, nb, rb), args.steps, 2, torch)
    # the bit-packed mask hand-over: routing that also writes the tile masks,
    # and the lists rebuilt from those masks
    rbm = dash.RouteBuffers(sizes, dev, tile_bits=True)
    t_route_m = events_time(lambda: dash.dash_route(p, q, N, summ, nb, rbm), args.steps, 2,
                            torch)
    t_m2l = events_time(lambda: dash.dash_mask_to_list(p, N, rbm), args.steps, 2, torch)
    o2 = torch.empty_like(q)
    t_att = events_time(lambda: dash.dash_attend(p, q, k, v, N, rb, o2), args.steps, 2, torch)

    # backward of the same step (mean-pooled summaries), from the forward's
    # summaries, routing and output
    t_bwd = None
    if not args.no_backward:
        d_o = torch.randn(q.shape, generator=torch.Generator(device="cpu").manual_seed(7)).to(
            dev, q.dtype)
        grads = [torch.empty(x.shape, dtype=torch.float32, device=dev) for x in (q, k, v)]
        dws = torch.empty((d, d), dtype=torch.float32, device=dev)
        wsb = dash.workspace(dash.dash_prefill_backward_workspace_bytes(p, N), dev)
        t_bwd = events_time(lambda: dash.dash_prefill_backward(p, q, k, v, o2, d_o, N, ws_mat,
                                                               summ, nb, rb, *grads, dws, wsb),
                            max(1, args.steps // 10), 2, torch)
        del grads, wsb

    count = rb.sel_count.view(B, Hkv, -1).cpu().numpy().astype(np.int64)
    n_qt = count.shape[2]
    qt = np.arange(n_qt)
    own_blk = (qt * QT) // bs
    cand = np.maximum(own_blk - (w.window - 1), 0)         # routing candidates per tile
    n_branch = own_blk - cand + 1                           # near-diagonal branch blocks
    cpb = bs // 64
    own_chunks = qt - cand * cpb + 1                       # branch 64-key chunks walked
    chunks = (count * cpb + own_chunks[None, None, :]).sum()
    flops_per_chunk = 4.0 * G * QT * 64 * d                # QK^T + PV for G*64 rows x 64 keys
    att_flops = float(chunks) * flops_per_chunk
    dense_chunks = float(B * Hkv) * (cand * cpb + own_chunks).sum()
    tile_union_density = float((count + n_branch).sum() / (B * Hkv * (cand + n_branch).sum()))
    achieved = att_flops / (t_att * 1e-3) / 1e12
    traffic = traffic_for_attend(w.name)
    res = {
        "workload": w, "ms_step": ms_step, "tok_s": B * N / (ms_step * 1e-3),
        "stages_ms": {"summarize": t_sum, "route": t_route, "attend": t_att,
                      "summarize_qbar": t_sum_q, "route_with_tile_masks": t_route_m,
                      "mask_to_list": t_m2l},
        "attend_flops": att_flops, "attend_tflops": achieved,
        "tile_union_density": tile_union_density,
        "selected_chunk_fraction": float(chunks) / dense_chunks,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    if t_bwd is not None:
        # algorithmic work of the attention backward: the five products S, dP,
        # dQ, dK, dV over the walked chunks = 2.5 x the forward's two
        bwd_flops = 2.5 * att_flops
        bt = bwd_flops / (t_bwd * 1e-3) / 1e12
        # bf16 inputs: the attention products run on bf16 MFMA; float32: vector FMAs
        bound, peak = ("mfma", PEAK_BF16_TFLOPS) if w.dtype == "bf16" else \
            ("alu", PEAK_FP32_TFLOPS)
        res["backward"] = {"ms": round(t_bwd, 4), "attention_gflop": round(bwd_flops / 1e9, 2),
                           "roofline": {"bound": bound, "achieved": round(bt, 2), "peak": peak,
                                        "unit": "TFLOP/s", "frac": round(bt / peak, 4),
                                        "scope": "whole backward, attention products counted"}}
    if args.dense:
        rbd = dash.RouteBuffers(sizes, dev)
        rbd.sel_count.copy_(torch.from_numpy(np.broadcast_to(cand, (B * Hkv, n_qt)).astype(
            np.int32).ravel()))
        idx = np.broadcast_to(np.arange(nb, dtype=np.int32), (B * Hkv * n_qt, nb))
        rbd.sel_idx.copy_(torch.from_numpy(np.ascontiguousarray(idx).ravel()))
        rbd.sel_logp.zero_()
        t_dense = events_time(lambda: dash.dash_attend(p, q, k, v, N, rbd, o2), args.steps, 2,
                              torch)
        res["dense_attend_ms"] = t_dense
        res["dense_tok_s"] = B * N / (t_dense * 1e-3)
        res["dense_tflops"] = dense_chunks * flops_per_chunk / (t_dense * 1e-3) / 1e12
    return res


VARLEN_LENS = (8192, 6144, 3000, 1000)   # a ragged batch of prefill_8k-shaped sequences


def varlen_bench(args, torch, dash, W):
    """dash_prefill_varlen on a ragged batch (sequences of prefill_8k's shape,
    lengths VARLEN_LENS, padded to 8192) against the same sequences run one
    dash_prefill call after another."""
    w = with_overrides(W.get(args.workload), args).replace(batch=len(VARLEN_LENS))
    dev = torch.device("cuda:0")
    inp = W.make_prefill(w)
    B, H, Hkv, N, d, bs = w.batch, w.n_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block_size
    p = dash.make_params(B, H, Hkv, d, bs, w.alpha, w.gamma, w.dtype, w.sigma, w.window)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(inp[x]).to(dev, tdt) for x in ("q", "k", "v"))
    ws_mat = torch.from_numpy(inp["w_s"]).to(dev)
    del inp
    nb = N // bs
    summ = torch.zeros(B * Hkv * nb * d, dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    ws = dash.workspace(dash.dash_prefill_workspace_bytes(p, N), dev)
    lens = torch.tensor(VARLEN_LENS, dtype=torch.int32, device=dev)
    ms = events_time(lambda: dash.dash_prefill_varlen(p, q, k, v, N, lens, ws_mat, summ, nb, o,
                                                      ws), args.steps, args.warmup, torch)
    # one call per sequence, back to back on the same stream
    p1 = dash.make_params(1, H, Hkv, d, bs, w.alpha, w.gamma, w.dtype, w.sigma, w.window)
    parts = []
    for b, n in enumerate(VARLEN_LENS):
        qs, ks, vs = (t[b:b + 1, :, :n].contiguous() for t in (q, k, v))
        parts.append((n, qs, ks, vs, torch.empty_like(qs),
                      torch.zeros(Hkv * max(n // bs, 1) * d, dtype=torch.float32, device=dev),
                      dash.workspace(dash.dash_prefill_workspace_bytes(p1, n), dev)))

    def one_by_one():
        for n, qs, ks, vs, os_, ss, wss in parts:
            dash.dash_prefill(p1, qs, ks, vs, n, ws_mat, ss, max(n // bs, 1), os_, wss)
    ms_seq = events_time(one_by_one, args.steps, args.warmup, torch)
    tokens = sum(VARLEN_LENS)
    return {"workload": f"ragged batch of {w.name} sequences, lengths {list(VARLEN_LENS)} "
                        f"padded to {N}",
            "ms_per_step": round(ms, 4), "tok_s": round(tokens / (ms * 1e-3), 1),
            "one_call_per_sequence_ms": round(ms_seq, 4)}


def decode_bench(args, torch, dash, W):
    w = with_overrides(W.get(args.decode_workload), args, alpha=False)
    dev = torch.device("cuda:0")
    B, H, Hkv, d, bs, L = w.batch, w.n_heads, w.n_kv_heads, w.head_dim, w.block_size, w.seq_len
    p = dash.make_params(B, H, Hkv, d, bs, w.alpha, w.gamma, w.dtype, w.sigma, w.window)
    kc = torch.empty((B, Hkv, L, d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    q = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
    for b0 in range(0, B, 8):
        part = W.make_decode(w, batches=range(b0, min(B, b0 + 8)))
        kc[b0:b0 + 8] = torch.from_numpy(part["k_cache"]).to(dev, torch.bfloat16)
        vc[b0:b0 + 8] = torch.from_numpy(part["v_cache"]).to(dev, torch.bfloat16)
        q[b0:b0 + 8] = torch.from_numpy(part["q"]).to(dev, torch.bfloat16)
        w_s = part["w_s"]
        del part
    ws_mat = torch.from_numpy(w_s).to(dev)
    nb = L // bs
    summ = torch.zeros(B * Hkv * nb * d, dtype=torch.float32, device=dev)
    dash.dash_summarize(p, kc, L, 0, nb, ws_mat, summ, nb)
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    ws = dash.workspace(dash.dash_decode_workspace_bytes(p, L), dev)
    rb = dash.RouteBuffers(dash.dash_route_sizes_decode(p, L), dev)
    step = lambda: dash.dash_decode(p, q, kc, vc, lens, L, ws_mat, summ, nb, o, ws,  # noqa
                                    route=rb)
    ms = events_time(step, args.steps, args.warmup, torch)
    # the same step over a paged cache: every block in its own page, pages in a
    # seeded random order
    nblk = (L + bs - 1) // bs
    gen = torch.Generator(device="cpu").manual_seed(1234)
    perm = torch.randperm(B * nblk, generator=gen).to(dev)
    kp = torch.empty((B * nblk, Hkv, bs, d), dtype=kc.dtype, device=dev)
    vp = torch.empty_like(kp)
    kp[perm] = kc.view(B, Hkv, nblk, bs, d).transpose(1, 2).reshape(B * nblk, Hkv, bs, d)
    vp[perm] = vc.view(B, Hkv, nblk, bs, d).transpose(1, 2).reshape(B * nblk, Hkv, bs, d)
    table = perm.view(B, nblk).to(torch.int32).contiguous()
    op = torch.empty_like(q)
    rbp = dash.RouteBuffers(dash.dash_route_sizes_decode(p, L), dev)
    step_p = lambda: dash.dash_decode_paged(p, q, kp, vp, table, lens, L, ws_mat, summ, nb,  # noqa
                                            op, ws, route=rbp)
    ms_paged = events_time(step_p, args.steps, args.warmup, torch)
    paged_same = bool(torch.equal(op, o))
    del kp, vp

    count = rb.sel_count.cpu().numpy().astype(np.int64)
    own_len = (L - 1) % bs + 1
    own = (L - 1) // bs
    ncand = max(own - (w.window - 1), 0)
    n_branch = own - ncand + 1
    branch_keys = own_len + (n_branch - 1) * bs
    sel_bytes = float(((count * bs + branch_keys) * d * 2 * 2).sum())
    density = float((count + n_branch).sum() / (B * Hkv * (ncand + n_branch)))
    summ_bytes = float(B * Hkv * ncand * d * 4)
    gbs = sel_bytes / (ms * 1e-3) / 1e9
    gbs_p = sel_bytes / (ms_paged * 1e-3) / 1e9
    return {"workload": w, "us_per_step": ms * 1e3, "selected_kv_bytes": sel_bytes,
            "paged": {"us_per_step": round(ms_paged * 1e3, 2), "same_output": paged_same,
                      "roofline_frac": round(gbs_p / PEAK_HBM_GBS, 4)},
            "block_density": density,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "scope": "selected K/V bytes / whole decode step"},
            "all_bytes_gbs": round((sel_bytes + summ_bytes) / (ms * 1e-3) / 1e9, 1)}


def cpu_baseline(args, W, min_seconds=10.0):
    """The CPU oracle on the same workload (all query positions and heads),
    repeated until at least `min_seconds` of CPU work; tokens/s = positions
    processed / seconds (input generation excluded)."""
    import oracle
    w = with_overrides(W.get(args.workload), args)
    inp = W.make_prefill(w)
    threads = oracle.max_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.prefill(inp["q"], inp["k"], inp["v"], inp["w_s"], bs=w.block_size,
                       alpha=w.alpha, gamma=w.gamma, sigma=w.sigma, window=w.window)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= 100:
            break
    return {"value": round(reps * w.batch * w.seq_len / dt, 1), "unit": "tok/s",
            "cores": threads, "kind": "oracle",
            "sample": f"whole workload ({w.batch} x {w.seq_len} positions, {w.n_heads} heads) "
                      f"x {reps} repeats, fp64 C/OpenMP, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_hierarchical_attention_block_amd as dash
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calib_mb:
        n = args.copy_calib_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    pre = prefill_bench(args, torch, dash, W)
    dec = None if args.no_decode else decode_bench(args, torch, dash, W)
    var = None if args.no_varlen else varlen_bench(args, torch, dash, W)
    cpu = None if args.no_cpu else cpu_baseline(args, W)
    w = pre["workload"]
    line = {
        "metric": METRIC,
        "value": round(pre["tok_s"], 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: causal prefill B={w.batch} N={w.seq_len} "
                               f"H={w.n_heads} Hkv={w.n_kv_heads} d={w.head_dim} "
                               f"block={w.block_size} alpha={w.alpha} gamma={w.gamma}"
                               + (f" sigma={w.sigma} window={w.window}"
                                  if (w.sigma, w.window) != (1.0, 1) else ""),
                   "global_batch": w.batch, "seq_len": w.seq_len,
                   "tile_union_block_density": round(pre["tile_union_density"], 4),
                   "parallelism": "single GPU"},
        "roofline": pre["roofline"],
        "stages_ms": {k2: round(v2, 4) for k2, v2 in pre["stages_ms"].items()},
        "attend_gflop": round(pre["attend_flops"] / 1e9, 2),
    }
    if "dense_tok_s" in pre:
        line["dense_attend"] = {"ms": round(pre["dense_attend_ms"], 4),
                                "tok_s": round(pre["dense_tok_s"], 1),
                                "tflops": round(pre["dense_tflops"], 1)}
    if dec is not None:
        dw = dec["workload"]
        line["decode"] = {"workload": f"{dw.name}: batch {dw.batch} x {dw.seq_len} context, "
                                      f"H={dw.n_heads} Hkv={dw.n_kv_heads} block={dw.block_size}"
                                      + (f" sigma={dw.sigma} window={dw.window}"
                                         if (dw.sigma, dw.window) != (1.0, 1) else ""),
                          "us_per_step": round(dec["us_per_step"], 2),
                          "block_density": round(dec["block_density"], 4),
                          "selected_kv_gb": round(dec["selected_kv_bytes"] / 1e9, 4),
                          "roofline": dec["roofline"],
                          "all_bytes_gbs": dec["all_bytes_gbs"],
                          "paged_kv": dec["paged"]}
    if "backward" in pre:
        line["prefill_backward"] = pre["backward"]
    if var is not None:
        line["varlen_prefill"] = var
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
