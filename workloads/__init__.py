"""Seeded synthetic inputs for the DashAttention forward workloads.

This module holds NO arithmetic of the method: it only draws random tensors.
It is shared by the GPU tests, the benchmark and the CPU oracle's tests, and
imports neither the GPU library nor the oracle.

Every tensor is drawn in float32 from ``numpy.random.default_rng`` seeded
with ``SeedSequence([config seed, tensor id, sequence, head])``, so any
(sequence, head) slice can be regenerated on its own.  bf16 workloads round
each value once to bfloat16 (round-to-nearest-even) and keep it as float32:
the oracle and the GPU then see the same numbers.

Planted structure (the reading used for the query-tile workloads): for every
(sequence, KV head, query block t) a seeded unit direction u is drawn; a
uniform count c of "relevant" blocks, capped at the t complete blocks before
the tile, is drawn without replacement from those blocks; every key row of a
relevant block gets + 3u, and the queries of that tile, for every query head
of the group, are q = 3u + 0.1 eps.  Values are N(0, 1) elsewhere.  Decode
workloads plant one direction per (sequence, KV head) -- or per query head
when ``plant_per_head`` is set -- for the single new query.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import json
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

# tensor ids for the seed sequences
_T_Q, _T_K, _T_V, _T_WS, _T_PLANT, _T_EPS, _T_QBAR = 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str             # "prefill" or "decode"
    batch: int
    n_heads: int
    n_kv_heads: int
    seq_len: int          # prefill: N; decode: context length incl. the new token
    head_dim: int
    block_size: int
    dtype: str            # "f32" or "bf16"
    alpha: float
    gamma: float
    seed: int
    planted: bool = True
    count_lo: int = 2     # relevant-block count range (uniform integers) ...
    count_hi: int = 24
    log_uniform: bool = False   # ... or log-uniform in [count_lo, count_hi]
    plant_per_head: bool = False
    max_len: int = 0      # decode cache capacity (0 = seq_len)
    summary_query: float = 0.0  # > 0: Stage 0 summary queries q_bar ~ this * N(0, 1)
    sigma: float = 1.0    # prior strength (Stage 2 bias sigma * log pbar)
    window: int = 1       # near-diagonal branch in blocks

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads

    @property
    def cache_len(self) -> int:
        return self.max_len or self.seq_len

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _gammas():
    path = os.path.join(_HERE, "gammas.json")
    if os.path.exists(path):
        with open(path) as f:
            return json.load(f)
    return {}


def _defaults():
    g = _gammas()
    return {
        # tiny causal prefill + one decode step, fp32, q,k,v ~ N(0,1)
        "tiny": Workload("tiny", "prefill", 1, 2, 2, 1024, 64, 64, "f32", 1.5,
                         g.get("tiny", 8.0), 0, planted=False),
        # causal prefill 8K, GQA 32/8, d 128, block 64, bf16
        "prefill_8k": Workload("prefill_8k", "prefill", 1, 32, 8, 8192, 128, 64, "bf16", 1.5,
                               g.get("prefill_8k", 3.0), 1, count_lo=2, count_hi=24),
        # batched decode: 32 sequences x 32K context
        "decode_32k": Workload("decode_32k", "decode", 32, 32, 8, 32768, 128, 64, "bf16", 1.5,
                               g.get("decode_32k", 1.5), 2, count_lo=16, count_hi=290),
        # long causal prefill 64K, block 128
        "prefill_64k": Workload("prefill_64k", "prefill", 1, 32, 8, 65536, 128, 128, "bf16", 1.5,
                                g.get("prefill_64k", 3.0), 3, count_lo=2, count_hi=24),
        # long-context decode: 8 sequences x 128K, G = 8, log-uniform counts per head
        "decode_128k": Workload("decode_128k", "decode", 8, 64, 8, 131072, 128, 64, "bf16", 1.5,
                                g.get("decode_128k", 2.0), 4, count_lo=1, count_hi=256,
                                log_uniform=True, plant_per_head=True),
    }


WORKLOADS = _defaults()


def get(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.replace(**overrides) if overrides else w


# --------------------------------------------------------------------------
# random draws
# --------------------------------------------------------------------------

def _rng(seed: int, tensor: int, b: int = 0, h: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor, b, h]))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def _cast(w: Workload, a: np.ndarray) -> np.ndarray:
    return round_bf16(a) if w.dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


def w_s(w: Workload) -> np.ndarray:
    """Summary projection W_s = I + 0.01 N(0, 1), float32, row-major [d_in, d_out]."""
    d = w.head_dim
    return (np.eye(d, dtype=np.float32)
            + 0.01 * _rng(w.seed, _T_WS).standard_normal((d, d), dtype=np.float32))


def summary_query(w: Workload):
    """Summary queries q_bar [Hkv, d] float32, drawn as summary_query * N(0, 1)
    (a stand-in for a learned query), or None when the workload has none."""
    if w.summary_query <= 0:
        return None
    return (w.summary_query * _rng(w.seed, _T_QBAR).standard_normal(
        (w.n_kv_heads, w.head_dim), dtype=np.float32)).astype(np.float32)


def _unit(rng: np.random.Generator, d: int) -> np.ndarray:
    u = rng.standard_normal(d).astype(np.float64)
    return (u / np.linalg.norm(u)).astype(np.float32)


def _count(w: Workload, rng: np.random.Generator, cap: int) -> int:
    if cap <= 0:
        return 0
    if w.log_uniform:
        c = int(round(math.exp(rng.uniform(math.log(w.count_lo), math.log(w.count_hi)))))
    else:
        c = int(rng.integers(w.count_lo, w.count_hi + 1))
    return min(max(c, 0), cap)


def prefill_plan(w: Workload, b: int, g: int):
    """Per query block t of sequence b, KV head g: (u [d], relevant block ids)."""
    rng = _rng(w.seed, _T_PLANT, b, g)
    nblk = w.seq_len // w.block_size
    plan = []
    for t in range(-(-w.seq_len // w.block_size)):
        u = _unit(rng, w.head_dim)
        c = _count(w, rng, min(t, nblk))
        rel = np.sort(rng.choice(t, size=c, replace=False)) if c > 0 else np.zeros(0, np.int64)
        plan.append((u, rel))
    return plan


def _pool_map(fn, items):
    workers = min(16, os.cpu_count() or 1, max(len(items), 1))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fn, items))


def make_prefill(w: Workload, batches=None):
    """q [B', H, N, d], k, v [B', Hkv, N, d], w_s [d, d] as float32 arrays, and
    q_bar [Hkv, d] or None."""
    B, H, Hkv, N, d, bs, G = w.batch, w.n_heads, w.n_kv_heads, w.seq_len, w.head_dim, \
        w.block_size, w.group
    batches = list(range(B)) if batches is None else list(batches)
    q = np.empty((len(batches), H, N, d), np.float32)
    k = np.empty((len(batches), Hkv, N, d), np.float32)
    v = np.empty((len(batches), Hkv, N, d), np.float32)

    def unit(item):
        bi, b, g = item
        kk = _rng(w.seed, _T_K, b, g).standard_normal((N, d), dtype=np.float32)
        v[bi, g] = _cast(w, _rng(w.seed, _T_V, b, g).standard_normal((N, d), dtype=np.float32))
        plan = prefill_plan(w, b, g) if w.planted else []
        for u, rel in plan:
            for j in rel:
                kk[j * bs:(j + 1) * bs] += 3.0 * u
        k[bi, g] = _cast(w, kk)
        for hh in range(G):
            h = g * G + hh
            eps = _rng(w.seed, _T_Q, b, h).standard_normal((N, d), dtype=np.float32)
            if plan:
                qq = 0.1 * eps
                for t, (u, _) in enumerate(plan):
                    qq[t * bs:(t + 1) * bs] += 3.0 * u
            else:
                qq = eps
            q[bi, h] = _cast(w, qq)

    _pool_map(unit, [(bi, b, g) for bi, b in enumerate(batches) for g in range(Hkv)])
    return {"q": q, "k": k, "v": v, "w_s": w_s(w), "q_bar": summary_query(w)}


def decode_plan(w: Workload, b: int, g: int):
    """For sequence b, KV head g: list over the group's heads of (u, relevant ids);
    a single shared entry when plants are per KV head."""
    rng = _rng(w.seed, _T_PLANT, b, g)
    L = w.seq_len
    ncand = (L - 1) // w.block_size
    out = []
    for _ in range(w.group if w.plant_per_head else 1):
        u = _unit(rng, w.head_dim)
        c = _count(w, rng, ncand)
        rel = np.sort(rng.choice(ncand, size=c, replace=False)) if c > 0 else np.zeros(0, np.int64)
        out.append((u, rel))
    return out


def make_decode(w: Workload, batches=None, cache_len=None):
    """q [B', H, d]; k_cache, v_cache [B', Hkv, max_len, d]; cache_len [B'] int32;
    w_s; q_bar or None.  The new token's key/value (position cache_len - 1) are in
    the caches."""
    B, H, Hkv, d, bs, G = w.batch, w.n_heads, w.n_kv_heads, w.head_dim, w.block_size, w.group
    Lmax = w.cache_len
    batches = list(range(B)) if batches is None else list(batches)
    if cache_len is None:
        lens = np.full(len(batches), w.seq_len, np.int32)
    else:
        lens = np.asarray(cache_len, np.int32)[batches] if len(cache_len) == B else \
            np.asarray(cache_len, np.int32)
    q = np.empty((len(batches), H, d), np.float32)
    kc = np.empty((len(batches), Hkv, Lmax, d), np.float32)
    vc = np.empty((len(batches), Hkv, Lmax, d), np.float32)

    def unit(item):
        bi, b, g = item
        kk = _rng(w.seed, _T_K, b, g).standard_normal((Lmax, d), dtype=np.float32)
        vc[bi, g] = _cast(w, _rng(w.seed, _T_V, b, g).standard_normal((Lmax, d),
                                                                        dtype=np.float32))
        plans = decode_plan(w, b, g) if w.planted else []
        for u, rel in plans:
            for j in rel:
                kk[j * bs:(j + 1) * bs] += 3.0 * u
        kc[bi, g] = _cast(w, kk)
        for hh in range(G):
            h = g * G + hh
            eps = _rng(w.seed, _T_Q, b, h).standard_normal(d, dtype=np.float32)
            if plans:
                u = plans[hh if w.plant_per_head else 0][0]
                q[bi, h] = _cast(w, 3.0 * u + 0.1 * eps)
            else:
                q[bi, h] = _cast(w, eps)

    _pool_map(unit, [(bi, b, g) for bi, b in enumerate(batches) for g in range(Hkv)])
    return {"q": q, "k_cache": kc, "v_cache": vc, "cache_len": lens, "w_s": w_s(w),
            "q_bar": summary_query(w)}
