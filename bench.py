"""Benchmark of the DashAttention forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs ...]

Headline: one fused causal prefill (dash_prefill: Stage 0 summaries, Stage 1
entmax routing, Stage 2 prior-induced sparse attention) of the long-context
workload -- B 1, N 65536, H 32 / Hkv 8, d 128, block 128, bf16, alpha 1.5 --
with inputs resident in HBM.  ``value`` = prefill tokens/s = N / median step
time, where every timed step runs right after a 1 GiB scratch read that
evicts the L2 caches and the 256 MB Infinity Cache (cold cache: none of the
step's inputs is cached, and no dirty line is left to be written back during
the step); the same steps back to back (warm) are reported beside it.

The line also carries
  roofline      the Stage 2 attend kernel (the dominant one): selected-tile
                MFMA flops per launch / its average launch time (HIP events on
                the stream it runs on, the stages launched one after another
                after the same flush), against the 2.5 PFLOP/s dense bf16
                peak, and against the bf16 MFMA rate this GPU attains;
  alpha_sweep   alpha 1.25 / 1.5 / 2 at the same inputs and gamma: step time,
                tokens/s and achieved sparsity (per query and per tile);
  dense         the same attend kernel over every causal block with zero
                prior (the in-house dense causal attention) at the same shape;
  decode        one batched decode step (dash_decode) of 8 sequences x 128K
                context, H 64 / Hkv 8: microseconds per step and selected-KV
                GB/s against 8 TB/s and the measured read-stream rate;
  secondary     the 8K prefill (with its backward and a ragged batch) and the
                32 x 32K decode (contiguous and paged caches);
  measured_peaks  a streaming copy / read and a register-resident MFMA loop;
  cpu_baseline  the fp64 CPU oracle on every 16th query tile of the headline
                workload, extrapolated to the whole by its selected work.
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
FLUSH_BYTES = 1 << 30         # >> 8 x 4 MB L2 + 256 MB Infinity Cache
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sparse_hierarchical_attention_block_amd", "csrc")
ALL_LEGS = ("peaks", "prefill", "sweep", "dense", "decode", "prefill_8k", "backward",
            "varlen", "decode_32k", "cpu")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill_64k")
    ap.add_argument("--decode-workload", default="decode_128k")
    ap.add_argument("--alpha", type=float, default=None)
    ap.add_argument("--sigma", type=float, default=None,
                    help="prior strength (default: the workload's, 1)")
    ap.add_argument("--window", type=int, default=None,
                    help="near-diagonal branch in blocks (default: the workload's, 1)")
    ap.add_argument("--legs", default=",".join(ALL_LEGS),
                    help="comma-separated subset of " + ",".join(ALL_LEGS))
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="launch one device copy of this many MiB (HBM-counter calibration)")
    return ap.parse_args()


# ---------------------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------------------

class Timer:
    """Per-iteration HIP-event timing on torch's current stream (the stream
    every library call below is launched on)."""

    def __init__(self, torch, dash, flush_bytes=FLUSH_BYTES):
        self.torch, self.dash = torch, dash
        self.flush_bytes = flush_bytes
        self.scratch = torch.zeros(flush_bytes // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.empty(dash.dash_peak_stream_grid() * 4, dtype=torch.float32,
                                device="cuda")
        torch.cuda.synchronize()

    def flush(self):
        # one read pass over 1 GiB of scratch (the library's read-stream
        # kernel): every L2 and Infinity Cache line then holds clean scratch
        # data, so the timed work starts with nothing of its own cached and
        # pays for no write-back of the flush
        self.dash.dash_peak_stream(self.scratch, self.sink, self.flush_bytes, 1)

    def run(self, fn, steps, warmup, cold=True, marks=0):
        """Milliseconds of each of `steps` calls of fn (after `warmup` untimed
        ones).  With marks > 0, fn(ev) records marks events ev[0..marks-1]
        between its launches and the result is a [steps, marks + 1] array of
        the intervals between start, the marks and the end."""
        torch = self.torch
        for _ in range(warmup):
            if cold:
                self.flush()
            fn([None] * marks) if marks else fn()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(marks + 2)]
               for _ in range(steps)]
        for i in range(steps):
            if cold:
                self.flush()
            evs[i][0].record()
            if marks:
                fn(evs[i][1:-1])
            else:
                fn()
            evs[i][-1].record()
        torch.cuda.synchronize()
        t = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(marks + 1)] for e in evs])
        return t if marks else t[:, 0]


def stats(t):
    t = np.asarray(t, dtype=np.float64)
    return {"median": float(np.median(t)), "mean": float(t.mean()),
            "p10": float(np.percentile(t, 10)), "p90": float(np.percentile(t, 90))}


def rnd(x, n=4):
    return None if x is None else round(float(x), n)


# ---------------------------------------------------------------------------------------
# committed counter summaries (profiles/*.txt)
# ---------------------------------------------------------------------------------------

def _kv_file(path):
    kv = {}
    if os.path.exists(path):
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    return kv


def counted(kernel_file, sources, workload, key="hbm_bytes_per_launch"):
    """A figure from a committed counter summary (profiles/), or None when the
    counters were taken on another workload or a kernel source has changed
    since they were taken."""
    kv = _kv_file(os.path.join(PROFILES, kernel_file))
    if not kv:
        return None
    h = hashlib.sha256()
    for s in sources:
        h.update(open(os.path.join(CSRC, s), "rb").read())
    if kv.get("source_sha256") != h.hexdigest() or kv.get("workload") != workload:
        return None
    for k, v in kv.items():
        if k == key or k.startswith(key + " "):
            try:
                return float(v)
            except ValueError:
                return None
    return None


# ---------------------------------------------------------------------------------------
# measured ceilings
# ---------------------------------------------------------------------------------------

def peaks_leg(args, torch, dash, tm):
    nbytes = 1 << 30        # copy: 1 GiB in, 1 GiB out
    rbytes = 4 << 30        # reads: 4 GiB, long enough that launch and ramp are ~1 %
    src = torch.ones(rbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    t_copy = tm.run(lambda: dash.dash_peak_stream(src, dst, nbytes, 0), 10, 3, cold=False)
    t_read = tm.run(lambda: dash.dash_peak_stream(src, dst, rbytes, 2), 10, 3, cold=False)
    t_read_alloc = tm.run(lambda: dash.dash_peak_stream(src, dst, rbytes, 1), 10, 3, cold=False)
    sink = torch.empty(dash.dash_peak_mfma_grid(), dtype=torch.float32, device="cuda")
    iters = 20000
    flops = dash.dash_peak_mfma(iters, sink)
    t_mfma = tm.run(lambda: dash.dash_peak_mfma(iters, sink), 10, 3, cold=False)
    del src, dst
    return {"hbm_copy_gbs": round(2 * nbytes / (np.median(t_copy) * 1e-3) / 1e9, 1),
            "hbm_read_gbs": round(rbytes / (np.median(t_read) * 1e-3) / 1e9, 1),
            "hbm_read_allocating_gbs": round(rbytes / (np.median(t_read_alloc) * 1e-3) / 1e9, 1),
            "mfma_bf16_tflops": round(flops / (np.median(t_mfma) * 1e-3) / 1e12, 1),
            "how": "grid-stride 16-byte copy of 1 GiB (read + write bytes) and read of 4 GiB "
                   "(non-temporal loads as in decode; allocating loads beside it); 8 chains of "
                   "v_mfma_f32_32x32x16_bf16 on register operands"}


# ---------------------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------------------

def with_overrides(w, args, alpha=True):
    """The workload with the command line's alpha / sigma / window applied."""
    if alpha and args.alpha is not None:
        w = w.replace(alpha=args.alpha)
    if args.sigma is not None:
        w = w.replace(sigma=args.sigma)
    if args.window is not None:
        w = w.replace(window=args.window)
    return w


def describe_prefill(w):
    return (f"{w.name}: causal prefill B={w.batch} N={w.seq_len} H={w.n_heads} "
            f"Hkv={w.n_kv_heads} d={w.head_dim} block={w.block_size} alpha={w.alpha} "
            f"gamma={w.gamma}" + (f" sigma={w.sigma} window={w.window}"
                                  if (w.sigma, w.window) != (1.0, 1) else ""))


def tile_work(w, count):
    """Per-tile geometry and chunk counts: count [B, Hkv, n_qt] selected blocks."""
    n_qt = count.shape[2]
    qt = np.arange(n_qt)
    own_blk = (qt * QT) // w.block_size
    cand = np.maximum(own_blk - (w.window - 1), 0)          # routing candidates per tile
    n_branch = own_blk - cand + 1                           # near-diagonal branch blocks
    cpb = w.block_size // 64
    own_chunks = qt - cand * cpb + 1                        # branch 64-key chunks walked
    chunks = count * cpb + own_chunks[None, None, :]        # [B, Hkv, n_qt]
    return cand, n_branch, own_chunks, chunks


def popcount32(x, torch):
    """Set bits per int32 element (a torch tensor on the GPU)."""
    table = torch.tensor([bin(i).count("1") for i in range(256)], dtype=torch.int32,
                         device=x.device)
    b = x.contiguous().view(torch.uint8).long()
    return table[b].view(*x.shape, 4).sum(-1)


class PrefillCase:
    """Inputs of one prefill workload on the GPU, and the library calls on them."""

    def __init__(self, w, torch, dash, W):
        self.w, self.torch, self.dash = w, torch, dash
        dev = torch.device("cuda:0")
        inp = W.make_prefill(w)
        B, H, Hkv, N, d, bs = w.batch, w.n_heads, w.n_kv_heads, w.seq_len, w.head_dim, \
            w.block_size
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.q, self.k, self.v = (torch.from_numpy(inp[x]).to(dev, tdt) for x in ("q", "k", "v"))
        self.ws_mat = torch.from_numpy(inp["w_s"]).to(dev)
        del inp
        self.nb = N // bs
        self.summ = torch.zeros(B * Hkv * self.nb * d, dtype=torch.float32, device=dev)
        self.o = torch.empty_like(self.q)
        self.dev = dev
        self.set_alpha(w.alpha)

    def set_alpha(self, alpha):
        w = self.w.replace(alpha=alpha)
        self.w = w
        self.p = self.dash.make_params(w.batch, w.n_heads, w.n_kv_heads, w.head_dim,
                                       w.block_size, w.alpha, w.gamma, w.dtype, w.sigma,
                                       w.window)
        self.sizes = self.dash.dash_route_sizes_prefill(self.p, w.seq_len)
        self.ws = self.dash.workspace(self.dash.dash_prefill_workspace_bytes(self.p, w.seq_len),
                                      self.dev)
        self.rb = self.dash.RouteBuffers(self.sizes, self.dev)

    def step(self):
        self.dash.dash_prefill(self.p, self.q, self.k, self.v, self.w.seq_len, self.ws_mat,
                               self.summ, self.nb, self.o, self.ws)

    def stages(self, ev):
        """The fused step's three kernels launched one by one, events between."""
        d, p, N = self.dash, self.p, self.w.seq_len
        d.dash_summarize(p, self.k, N, 0, self.nb, self.ws_mat, self.summ, self.nb)
        if ev[0] is not None:
            ev[0].record()
        d.dash_route(p, self.q, N, self.summ, self.nb, self.rb)
        if ev[1] is not None:
            ev[1].record()
        d.dash_attend(p, self.q, self.k, self.v, N, self.rb, self.o)

    def counts(self):
        w = self.w
        return self.rb.sel_count.view(w.batch, w.n_kv_heads, -1).cpu().numpy().astype(np.int64)

    def densities(self):
        """(tile-union density, per-query density) of the routing in self.rb:
        visible blocks kept / visible blocks, the near-diagonal branch counted
        as kept.  Per query: the union of the group's heads' supports."""
        torch, w = self.torch, self.w
        B, H, Hkv, G, N, bs = w.batch, w.n_heads, w.n_kv_heads, w.group, w.seq_len, w.block_size
        count = self.counts()
        cand, n_branch, _, _ = tile_work(w, count)
        tile = float((count + n_branch).sum() / (B * Hkv * (cand + n_branch).sum()))
        rbb = self.dash.RouteBuffers(self.sizes, self.dev, bits=True)
        self.dash.dash_route(self.p, self.q, N, self.summ, self.nb, rbb)
        bits = rbb.support_bits.view(B, Hkv, G, N, -1)
        union = bits[:, :, 0]
        for hh in range(1, G):
            union = union | bits[:, :, hh]
        kept = popcount32(union, torch).sum(-1).double()         # [B, Hkv, N]
        pos = torch.arange(N, device=self.dev)
        own = pos // bs
        cand_q = torch.clamp(own - (w.window - 1), min=0)
        branch_q = (own - cand_q + 1).double()
        per_query = float(((kept + branch_q).sum() / (B * Hkv * (cand_q.double() + branch_q)
                                                      .sum())).item())
        del rbb
        return tile, per_query

    def attend_flops(self, count):
        w = self.w
        _, _, _, chunks = tile_work(w, count)
        return float(chunks.sum()) * 4.0 * w.group * QT * 64 * w.head_dim

    def dense_route(self):
        """Route buffers that list every causal candidate with a zero prior."""
        w, torch = self.w, self.torch
        B, Hkv = w.batch, w.n_kv_heads
        n_qt, nb = self.sizes["n_qt"], self.sizes["nb"]
        cand, _, _, _ = tile_work(w, np.zeros((B, Hkv, n_qt), np.int64))
        rbd = self.dash.RouteBuffers(self.sizes, self.dev)
        rbd.sel_count.copy_(torch.from_numpy(np.ascontiguousarray(
            np.broadcast_to(cand, (B * Hkv, n_qt)).astype(np.int32)).ravel()))
        idx = torch.arange(nb, dtype=torch.int32, device=self.dev)
        rbd.sel_idx.view(-1, nb).copy_(idx.expand(B * Hkv * n_qt, nb))
        rbd.sel_logp.zero_()
        dense_chunks = float(B * Hkv) * float((cand * (w.block_size // 64) +
                                               (np.arange(n_qt) - cand * (w.block_size // 64)
                                                + 1)).sum())
        return rbd, dense_chunks * 4.0 * w.group * QT * 64 * w.head_dim


def prefill_leg(args, torch, dash, W, tm, legs):
    w = with_overrides(W.get(args.workload), args)
    case = PrefillCase(w, torch, dash, W)
    N = w.seq_len
    cold = tm.run(case.step, args.steps, args.warmup, cold=True)
    warm = tm.run(case.step, args.steps, 2, cold=False)
    st = tm.run(case.stages, args.steps, 2, cold=True, marks=2)      # [steps, 3]
    count = case.counts()
    flops = case.attend_flops(count)
    tile_density, query_density = case.densities()
    t_att = float(st[:, 2].mean())
    achieved = flops / (t_att * 1e-3) / 1e12
    res = {
        "workload": w, "count": count, "cold": stats(cold), "warm": stats(warm),
        "stages_ms": {"summarize": float(st[:, 0].mean()), "route": float(st[:, 1].mean()),
                      "attend": t_att},
        "attend_flops": flops, "attend_tflops": achieved,
        "tile_union_density": tile_density, "per_query_density": query_density,
    }
    del st
    sweep = []
    if "sweep" in legs:
        for alpha in sorted({1.25, w.alpha, 2.0}):
            if alpha == w.alpha:
                sweep.append({"alpha": alpha, "ms": rnd(res["cold"]["median"]),
                              "tok_s": round(w.batch * N / (res["cold"]["median"] * 1e-3), 1),
                              "tile_union_density": rnd(tile_density),
                              "per_query_density": rnd(query_density),
                              "attend_ms": rnd(t_att), "attend_tflops": round(achieved, 1)})
                continue
            case.set_alpha(alpha)
            n = max(3, args.steps // 4)
            t = tm.run(case.step, n, 1, cold=True)
            sa = tm.run(case.stages, n, 1, cold=True, marks=2)
            fa = case.attend_flops(case.counts())
            td, qd = case.densities()
            sweep.append({"alpha": alpha, "ms": rnd(np.median(t)),
                          "tok_s": round(w.batch * N / (np.median(t) * 1e-3), 1),
                          "tile_union_density": rnd(td), "per_query_density": rnd(qd),
                          "route_ms": rnd(sa[:, 1].mean()), "attend_ms": rnd(sa[:, 2].mean()),
                          "attend_tflops": round(fa / (sa[:, 2].mean() * 1e-3) / 1e12, 1)})
        case.set_alpha(w.alpha)
    res["sweep"] = sweep
    if "dense" in legs:
        rbd, dflops = case.dense_route()
        n = max(3, args.steps // 4)
        td = tm.run(lambda: dash.dash_attend(case.p, case.q, case.k, case.v, N, rbd, case.o),
                    n, 1, cold=True)
        del rbd
        dms = float(np.median(td))
        res["dense"] = {"what": "the same attend kernel over every causal block, zero prior",
                        "ms": rnd(dms), "tok_s": round(w.batch * N / (dms * 1e-3), 1),
                        "tflops": round(dflops / (dms * 1e-3) / 1e12, 1),
                        "sparse_step_speedup": round(dms / res["cold"]["median"], 3)}
    return res


def prefill_small_leg(args, torch, dash, W, tm, legs, name="prefill_8k"):
    """The 8K prefill (its own roofline) and, optionally, its backward."""
    w = with_overrides(W.get(name), args)
    case = PrefillCase(w, torch, dash, W)
    # this workload is ~0.25 ms a step: enough untimed steps to hold the clock
    cold = tm.run(case.step, max(args.steps, 50), max(args.warmup, 50), cold=True)
    warm = tm.run(case.step, max(args.steps, 50), 20, cold=False)
    st = tm.run(case.stages, max(args.steps, 50), 5, cold=True, marks=2)
    count = case.counts()
    flops = case.attend_flops(count)
    t_att = float(st[:, 2].mean())
    out = {"workload": describe_prefill(w),
           "ms_per_step": rnd(np.median(cold)), "warm_ms_per_step": rnd(np.median(warm)),
           "tok_s": round(w.batch * w.seq_len / (np.median(cold) * 1e-3), 1),
           "stages_ms": {"summarize": rnd(st[:, 0].mean()), "route": rnd(st[:, 1].mean()),
                         "attend": rnd(t_att)},
           "attend_roofline": {"bound": "mfma", "achieved": round(flops / (t_att * 1e-3) / 1e12,
                                                                  2),
                               "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                               "frac": rnd(flops / (t_att * 1e-3) / 1e12 / PEAK_BF16_TFLOPS)},
           "tile_union_density": rnd(case.densities()[0])}
    if "backward" in legs:
        d = w.head_dim
        p, q, k, v = case.p, case.q, case.k, case.v
        case.stages([None, None])
        d_o = torch.randn(q.shape, generator=torch.Generator(device="cpu").manual_seed(7)).to(
            case.dev, q.dtype)
        grads = [torch.empty(x.shape, dtype=torch.float32, device=case.dev) for x in (q, k, v)]
        dws = torch.empty((d, d), dtype=torch.float32, device=case.dev)
        wsb = dash.workspace(dash.dash_prefill_backward_workspace_bytes(p, w.seq_len), case.dev)
        tb = tm.run(lambda: dash.dash_prefill_backward(p, q, k, v, case.o, d_o, w.seq_len,
                                                       case.ws_mat, case.summ, case.nb, case.rb,
                                                       *grads, dws, wsb),
                    max(3, args.steps // 2), 2, cold=True)
        bflops = 2.5 * flops      # S, dP, dQ, dK, dV over the walked chunks
        bt = bflops / (np.median(tb) * 1e-3) / 1e12
        bound, peak = ("mfma", PEAK_BF16_TFLOPS) if w.dtype == "bf16" else \
            ("alu", PEAK_FP32_TFLOPS)
        out["backward"] = {"ms": rnd(np.median(tb)), "attention_gflop": round(bflops / 1e9, 2),
                           "workspace_gb": round(wsb.numel() / 1e9, 3),
                           "roofline": {"bound": bound, "achieved": round(bt, 2), "peak": peak,
                                        "unit": "TFLOP/s", "frac": rnd(bt / peak),
                                        "scope": "whole backward, attention products counted"}}
        del grads, wsb
    return out


VARLEN_LENS = (8192, 6144, 3000, 1000)   # a ragged batch of prefill_8k-shaped sequences


def varlen_leg(args, torch, dash, W, tm):
    """dash_prefill_varlen on a ragged batch against the same sequences run one
    dash_prefill call after another."""
    w = with_overrides(W.get("prefill_8k"), args).replace(batch=len(VARLEN_LENS))
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
    steps = max(args.steps, 20)
    t = tm.run(lambda: dash.dash_prefill_varlen(p, q, k, v, N, lens, ws_mat, summ, nb, o, ws),
               steps, 10, cold=True)
    p1 = dash.make_params(1, H, Hkv, d, bs, w.alpha, w.gamma, w.dtype, w.sigma, w.window)
    parts = []
    for b, n in enumerate(VARLEN_LENS):
        qs, ks, vs = (x[b:b + 1, :, :n].contiguous() for x in (q, k, v))
        parts.append((n, qs, ks, vs, torch.empty_like(qs),
                      torch.zeros(Hkv * max(n // bs, 1) * d, dtype=torch.float32, device=dev),
                      dash.workspace(dash.dash_prefill_workspace_bytes(p1, n), dev)))

    def one_by_one():
        for n, qs, ks, vs, os_, ss, wss in parts:
            dash.dash_prefill(p1, qs, ks, vs, n, ws_mat, ss, max(n // bs, 1), os_, wss)
    t_seq = tm.run(one_by_one, steps, 10, cold=True)
    tokens = sum(VARLEN_LENS)
    return {"workload": f"ragged batch of {w.name} sequences, lengths {list(VARLEN_LENS)} "
                        f"padded to {N}",
            "ms_per_step": rnd(np.median(t)), "tok_s": round(tokens / (np.median(t) * 1e-3), 1),
            "one_call_per_sequence_ms": rnd(np.median(t_seq))}


# ---------------------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------------------

def decode_leg(args, torch, dash, W, tm, name, paged=False, peaks=None):
    w = with_overrides(W.get(name), args, alpha=False)
    dev = torch.device("cuda:0")
    B, H, Hkv, d, bs, L = w.batch, w.n_heads, w.n_kv_heads, w.head_dim, w.block_size, w.seq_len
    p = dash.make_params(B, H, Hkv, d, bs, w.alpha, w.gamma, w.dtype, w.sigma, w.window)
    kc = torch.empty((B, Hkv, L, d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    q = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
    for b0 in range(0, B, 4):
        part = W.make_decode(w, batches=range(b0, min(B, b0 + 4)))
        kc[b0:b0 + 4] = torch.from_numpy(part["k_cache"]).to(dev, torch.bfloat16)
        vc[b0:b0 + 4] = torch.from_numpy(part["v_cache"]).to(dev, torch.bfloat16)
        q[b0:b0 + 4] = torch.from_numpy(part["q"]).to(dev, torch.bfloat16)
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
    cold = tm.run(step, max(args.steps, 50), max(args.warmup, 20), cold=True)
    warm = tm.run(step, max(args.steps, 50), 20, cold=False)
    count = rb.sel_count.cpu().numpy().astype(np.int64)
    own_len = (L - 1) % bs + 1
    own = (L - 1) // bs
    ncand = max(own - (w.window - 1), 0)
    n_branch = own - ncand + 1
    branch_keys = own_len + (n_branch - 1) * bs
    sel_bytes = float(((count * bs + branch_keys) * d * 2 * 2).sum())
    density = float((count + n_branch).sum() / (B * Hkv * (ncand + n_branch)))
    summ_bytes = float(B * Hkv * ncand * d * 4)
    ms = float(np.median(cold))
    gbs = sel_bytes / (ms * 1e-3) / 1e9
    out = {"workload": f"{w.name}: batch {B} x {L} context, H={H} Hkv={Hkv} d={d} block={bs} "
                       f"alpha={w.alpha} gamma={w.gamma}"
                       + (f" sigma={w.sigma} window={w.window}"
                          if (w.sigma, w.window) != (1.0, 1) else ""),
           "us_per_step": round(ms * 1e3, 2), "p10_us": round(np.percentile(cold, 10) * 1e3, 2),
           "p90_us": round(np.percentile(cold, 90) * 1e3, 2),
           "warm_us_per_step": round(float(np.median(warm)) * 1e3, 2),
           "block_density": rnd(density), "selected_kv_gb": rnd(sel_bytes / 1e9),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": rnd(gbs / PEAK_HBM_GBS),
                        "scope": "selected K/V bytes / whole decode step (cold cache)"},
           "all_bytes_gbs": round((sel_bytes + summ_bytes) / (ms * 1e-3) / 1e9, 1)}
    if peaks:
        out["roofline"]["frac_of_measured_read"] = rnd(gbs / peaks["hbm_read_gbs"])
    out["roofline"]["traffic"] = counted(f"{w.name}_traffic.txt", ["decode.hip"], w.name,
                                         "hbm_bytes_per_step")
    if paged:
        nblk = (L + bs - 1) // bs
        gen = torch.Generator(device="cpu").manual_seed(1234)
        perm = torch.randperm(B * nblk, generator=gen).to(dev)
        kp = torch.empty((B * nblk, Hkv, bs, d), dtype=kc.dtype, device=dev)
        vp = torch.empty_like(kp)
        kp[perm] = kc.view(B, Hkv, nblk, bs, d).transpose(1, 2).reshape(B * nblk, Hkv, bs, d)
        vp[perm] = vc.view(B, Hkv, nblk, bs, d).transpose(1, 2).reshape(B * nblk, Hkv, bs, d)
        del kc, vc
        table = perm.view(B, nblk).to(torch.int32).contiguous()
        op = torch.empty_like(q)
        rbp = dash.RouteBuffers(dash.dash_route_sizes_decode(p, L), dev)
        step_p = lambda: dash.dash_decode_paged(p, q, kp, vp, table, lens, L, ws_mat, summ,  # noqa
                                                nb, op, ws, route=rbp)
        tp = tm.run(step_p, max(args.steps, 50), 10, cold=True)
        out["paged_kv"] = {"us_per_step": round(float(np.median(tp)) * 1e3, 2),
                           "same_output": bool(torch.equal(op, o)),
                           "roofline_frac": rnd(sel_bytes / (np.median(tp) * 1e-3) / 1e9 /
                                                PEAK_HBM_GBS)}
    return out


# ---------------------------------------------------------------------------------------
# CPU oracle
# ---------------------------------------------------------------------------------------

def cpu_baseline(args, W, count, every=16):
    """The fp64 CPU oracle on every `every`-th query tile of the headline
    workload (all heads), timed on this host's cores; the time of the whole
    workload is extrapolated as summaries + sampled rows x (selected work of
    all tiles / selected work of the sampled tiles), from the GPU routing's
    per-tile chunk counts `count` [B, Hkv, n_qt]."""
    import oracle
    w = with_overrides(W.get(args.workload), args)
    inp = W.make_prefill(w)
    N, bs = w.seq_len, w.block_size
    n_qt = -(-N // QT)
    tiles = np.arange(0, n_qt, every)
    pos = np.concatenate([np.arange(t * QT, min(N, t * QT + QT)) for t in tiles])
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    summ = oracle.summaries(inp["k"], inp["w_s"], bs, N // bs)
    t_summ = time.perf_counter() - t0
    rows_b = np.repeat(np.arange(w.batch), len(pos))
    rows_p = np.tile(pos, w.batch)
    q_rows = np.ascontiguousarray(inp["q"][:, :, pos, :].transpose(0, 2, 1, 3).reshape(
        w.batch * len(pos), w.n_heads, w.head_dim))
    t0 = time.perf_counter()
    oracle.forward_rows(q_rows, rows_b, rows_p, inp["k"], inp["v"], summ, n_heads=w.n_heads,
                        bs=bs, alpha=w.alpha, gamma=w.gamma, sigma=w.sigma, window=w.window)
    t_rows = time.perf_counter() - t0
    _, _, _, chunks = tile_work(w, count)
    work = chunks.sum(axis=(0, 1)).astype(np.float64)
    ratio = float(work.sum() / work[tiles].sum())
    t_full = t_summ + t_rows * ratio
    return {"value": round(w.batch * N / t_full, 1), "unit": "tok/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{w.name} alpha={w.alpha}: every {every}th query tile ({len(tiles)} of "
                      f"{n_qt} tiles, {len(pos)} positions x {w.n_heads} heads) in "
                      f"{t_rows:.1f} s + all summaries in {t_summ:.1f} s, fp64 C/OpenMP; "
                      f"extrapolated x{ratio:.2f} by the selected chunks of all tiles over "
                      f"the sampled ones"}


# ---------------------------------------------------------------------------------------

def headline(line, pre, peaks):
    """The driver-facing keys of the JSON line from the headline prefill leg."""
    w = pre["workload"]
    line.update({
        "value": round(w.batch * w.seq_len / (pre["cold"]["median"] * 1e-3), 1),
        "ms_per_step": rnd(pre["cold"]["median"]),
        "dtype": w.dtype,
        "config": {"workload": describe_prefill(w), "global_batch": w.batch,
                   "seq_len": w.seq_len,
                   "tile_union_block_density": rnd(pre["tile_union_density"]),
                   "per_query_block_density": rnd(pre["per_query_density"]),
                   "parallelism": "single GPU"},
    })
    ach = pre["attend_tflops"]
    line["roofline"] = {
        "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": rnd(ach / PEAK_BF16_TFLOPS),
        "traffic": counted("attend_prefill_64k_traffic.txt", ["attend.hip"], w.name),
        "kernel": "attend_bf16_kernel (Stage 2)",
        "per_launch_gflop": round(pre["attend_flops"] / 1e9, 2)}
    if peaks:
        line["roofline"]["frac_of_measured_mfma"] = rnd(ach / peaks["mfma_bf16_tflops"])
    line["timing"] = {
        "protocol": "per-step HIP events; a 1 GiB scratch read before every cold step",
        "cold_ms": {k2: rnd(v2) for k2, v2 in pre["cold"].items()},
        "warm_ms": {k2: rnd(v2) for k2, v2 in pre["warm"].items()}}
    line["step_roofline"] = {
        "achieved": round(pre["attend_flops"] / (pre["cold"]["median"] * 1e-3) / 1e12, 2),
        "frac": rnd(pre["attend_flops"] / (pre["cold"]["median"] * 1e-3) / 1e12 /
                    PEAK_BF16_TFLOPS),
        "scope": "selected-tile attend flops / whole fused step (summaries + routing + attend)"}
    line["stages_ms"] = {k2: rnd(v2) for k2, v2 in pre["stages_ms"].items()}
    rsrc = ["route_long.hip", "route_common.hpp", "entmax_device.hpp"]
    rbytes = [counted("route_prefill_64k_counters.txt", rsrc, w.name, f"route_long_kernel.{k}")
              for k in ("hbm_read_bytes_per_launch", "hbm_write_bytes_per_launch")]
    t_route = pre["stages_ms"]["route"]
    line["route"] = {
        "ms": rnd(t_route),
        "share_of_step": rnd(t_route / pre["cold"]["median"]),
        "hbm_bytes_counted": None if None in rbytes else sum(rbytes),
        "hbm_gbs": None if None in rbytes else round(sum(rbytes) / (t_route * 1e-3) / 1e9, 1),
        "valu_issue_fraction_counted": counted("route_prefill_64k_counters.txt", rsrc, w.name,
                                               "route_long_kernel.valu_issue_fraction"),
        "bound": "VALU issue (the threshold passes and the summary split; see the counted "
                 "fraction of SIMD cycles), not HBM (see hbm_gbs)"}
    if pre["sweep"]:
        line["alpha_sweep"] = pre["sweep"]
    if "dense" in pre:
        line["dense"] = pre["dense"]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    legs = set(args.legs.split(","))
    unknown = legs - set(ALL_LEGS)
    if unknown:
        print(f"unknown legs {sorted(unknown)}", file=sys.stderr)
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
        del src, dst

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    tm = Timer(torch, dash)
    peaks = None
    if "peaks" in legs:
        peaks = peaks_leg(args, torch, dash, tm)
        log(f"peaks {peaks}")
    line = {"metric": METRIC, "value": None, "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "headline prefill leg not run"}}
    count = None
    if "prefill" in legs:
        pre = prefill_leg(args, torch, dash, W, tm, legs)
        w = pre["workload"]
        log(f"prefill {w.name}: {pre['cold']['median']:.4f} ms cold")
        count = pre["count"]
        torch.cuda.empty_cache()
        headline(line, pre, peaks)
    if "decode" in legs:
        line["decode"] = decode_leg(args, torch, dash, W, tm, args.decode_workload, peaks=peaks)
        log(f"decode {line['decode']['us_per_step']} us")
        torch.cuda.empty_cache()
    secondary = {}
    if "prefill_8k" in legs:
        secondary["prefill_8k"] = prefill_small_leg(args, torch, dash, W, tm, legs)
        log("prefill_8k done")
        torch.cuda.empty_cache()
    if "varlen" in legs:
        secondary["varlen_prefill"] = varlen_leg(args, torch, dash, W, tm)
        torch.cuda.empty_cache()
    if "decode_32k" in legs:
        secondary["decode_32k"] = decode_leg(args, torch, dash, W, tm, "decode_32k", paged=True,
                                             peaks=peaks)
        log("decode_32k done")
        torch.cuda.empty_cache()
    if secondary:
        line["secondary"] = secondary
    if peaks:
        line["measured_peaks"] = peaks
    line["cpu_baseline"] = cpu_baseline(args, W, count) if "cpu" in legs and count is not None \
        else None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
