"""CPU oracle for the DashAttention forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the GPU library
and never imports it.

The arithmetic lives in ``dash_oracle.c`` (plain C, IEEE double, OpenMP over
query rows), which follows the DashAttention explainer pages (gist.science,
arXiv 2605.18753), "Technical summary": Stage 0 (local chunk summarization),
Stage 1 (entmax chunk routing, w = alpha-entmax(gamma * zbar)) and Stage 2
(prior-induced sparse softmax).  Stage 0 pools a block uniformly, or, given
a summary query q_bar per KV head, by scaled dot-product attention of q_bar
over the block's keys.  This module only marshals numpy arrays; the backward
pass of the prefill is written out in ``oracle/backward.py``.

Parity pins (all in ``tests/test_oracle_*.py``): closed-form sparsemax and
1.5-entmax values, an independent SLSQP solve of the Tsallis-entmax problem,
the alpha -> 1 softmax limit, entmax invariants, exact block means, the Gibbs
variational identity of the prior-induced softmax, brute-force dense attention
equivalences and the masking invariant.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dash_oracle.c")
_LIB = os.path.join(_HERE, "libdash_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile dash_oracle.c with gcc (portable x86-64, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-Wall", "-Wno-unknown-pragmas", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if (not os.path.exists(_LIB)
                or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        fp = ctypes.POINTER(ctypes.c_float)
        ip = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_entmax.restype = ctypes.c_double
        lib.oracle_entmax.argtypes = [dp, ctypes.c_int, ctypes.c_double, ctypes.c_int, dp]
        lib.oracle_summaries.restype = None
        lib.oracle_summaries.argtypes = [fp, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int64, fp, fp,
                                         dp]
        lib.oracle_forward_rows.restype = ctypes.c_int
        lib.oracle_forward_rows.argtypes = [
            fp, ip, ip, ctypes.c_int64, fp, fp, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_int, dp,
            ctypes.c_int64,
            ctypes.c_int64, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.oracle_prefill_backward.restype = ctypes.c_int
        lib.oracle_prefill_backward.argtypes = [
            fp, fp, fp, fp, fp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
            ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_double,
            ctypes.c_int, dp, dp, dp, dp, ctypes.c_int]
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def entmax(x, alpha: float, method: str = "auto"):
    """alpha-entmax of x given in threshold units (x = (alpha-1) * y).

    Returns (p, tau).  method "auto" = exact sort for alpha in {1.5, 2},
    bisection otherwise; "bisect" = bisection for every alpha.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    p = np.empty_like(x)
    tau = _load().oracle_entmax(_ptr(x, ctypes.c_double), int(x.size), float(alpha),
                                0 if method == "auto" else 1, _ptr(p, ctypes.c_double))
    return p, tau


def entmax_of_scores(y, alpha: float, method: str = "auto"):
    """alpha-entmax(y) in the usual parameterisation (x = (alpha-1) * y)."""
    y = np.asarray(y, dtype=np.float64)
    return entmax((alpha - 1.0) * y, alpha, method)


def summaries(k, w_s, bs: int, nblocks: int, q_bar=None):
    """Stage 0 summaries of blocks [0, nblocks): k [B, Hkv, L, d] -> [B, Hkv, nblocks, d].

    ``q_bar`` None pools each block uniformly; a [Hkv, d] array pools it by
    scaled dot-product attention of that head's summary query over the keys."""
    k = np.ascontiguousarray(k, dtype=np.float32)
    w_s = np.ascontiguousarray(w_s, dtype=np.float32)
    B, Hkv, L, d = k.shape
    if q_bar is not None:
        q_bar = np.ascontiguousarray(q_bar, dtype=np.float32)
        if q_bar.shape != (Hkv, d):
            raise ValueError("q_bar must be [Hkv, d]")
    if nblocks * bs > L:
        raise ValueError("summaries requested for incomplete blocks")
    out = np.zeros((B, Hkv, max(nblocks, 0), d), dtype=np.float64)
    if nblocks > 0:
        _load().oracle_summaries(_ptr(k, ctypes.c_float), B, Hkv, L, d, bs, nblocks,
                                 _ptr(w_s, ctypes.c_float), _ptr(q_bar, ctypes.c_float),
                                 _ptr(out, ctypes.c_double))
    return out


def forward_rows(q_rows, row_b, row_pos, k, v, summ, *, n_heads: int, bs: int, alpha: float,
                 gamma: float, causal: bool = True, n_kv: int | None = None,
                 nb_out: int = 0, want=("o", "tau"), threads: int = 0, sigma: float = 1.0,
                 window: int = 1):
    """Stages 1-2 for the given query rows.

    q_rows [nrows, H, d]; row_b / row_pos [nrows]; k, v [B, Hkv, L, d];
    summ [B, Hkv, nb, d] (float64).  ``want`` selects outputs among
    "o", "tau", "x", "p", "pbar"; x/p/pbar need ``nb_out`` columns.
    """
    q_rows = np.ascontiguousarray(q_rows, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    summ = np.ascontiguousarray(summ, dtype=np.float64)
    row_b = np.ascontiguousarray(row_b, dtype=np.int64)
    row_pos = np.ascontiguousarray(row_pos, dtype=np.int64)
    nrows, H, d = q_rows.shape
    B, Hkv, L, d2 = k.shape
    assert d == d2 and H == n_heads and v.shape == k.shape
    if summ.shape[2] == 0:
        summ = np.zeros((B, Hkv, 1, d), dtype=np.float64)
    if n_kv is None:
        n_kv = L
    out = {"o": np.empty((nrows, H, d), dtype=np.float64)}
    if "tau" in want:
        out["tau"] = np.empty((nrows, H), dtype=np.float64)
    for key, shape in (("x", (nrows, H, nb_out)), ("p", (nrows, H, nb_out)),
                       ("pbar", (nrows, Hkv, nb_out))):
        if key in want:
            if nb_out <= 0:
                raise ValueError(f"{key} needs nb_out > 0")
            out[key] = np.empty(shape, dtype=np.float64)
    rc = _load().oracle_forward_rows(
        _ptr(q_rows, ctypes.c_float), _ptr(row_b, ctypes.c_int64), _ptr(row_pos, ctypes.c_int64),
        nrows, _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float), L, n_kv, B, H, Hkv, d, bs,
        float(alpha), float(gamma), float(sigma), int(window), 1 if causal else 0,
        _ptr(summ, ctypes.c_double),
        summ.shape[2], nb_out, _ptr(out["o"], ctypes.c_double),
        _ptr(out.get("tau"), ctypes.c_double), _ptr(out.get("x"), ctypes.c_double),
        _ptr(out.get("p"), ctypes.c_double), _ptr(out.get("pbar"), ctypes.c_double), threads)
    if rc != 0:
        raise ValueError("oracle_forward_rows rejected its arguments")
    return out


def prefill(q, k, v, w_s, *, bs: int, alpha: float, gamma: float, causal: bool = True,
            positions=None, batches=None, nb_out: int = 0, want=("o", "tau"), threads: int = 0,
            q_bar=None, sigma: float = 1.0, window: int = 1):
    """Causal (or non-causal) prefill: q [B, H, N, d], k/v [B, Hkv, N, d].

    Computes the rows (b, i) for b in ``batches`` (default all) and i in
    ``positions`` (default all); results are indexed [row] in b-major order.
    """
    q = np.asarray(q, dtype=np.float32)
    B, H, N, d = q.shape
    batches = np.arange(B) if batches is None else np.asarray(batches)
    positions = np.arange(N) if positions is None else np.asarray(positions)
    nblocks = N // bs
    sub_k = np.asarray(k, dtype=np.float32)[batches]
    sub_v = np.asarray(v, dtype=np.float32)[batches]
    summ = summaries(sub_k, w_s, bs, nblocks, q_bar)
    rb = np.repeat(np.arange(len(batches)), len(positions))
    rp = np.tile(positions, len(batches))
    q_rows = np.ascontiguousarray(np.asarray(q)[batches][:, :, positions, :].transpose(0, 2, 1, 3)
                                  .reshape(len(batches) * len(positions), H, d))
    res = forward_rows(q_rows, rb, rp, sub_k, sub_v, summ, n_heads=H, bs=bs, alpha=alpha,
                       gamma=gamma, causal=causal, n_kv=N, nb_out=nb_out, want=want,
                       threads=threads, sigma=sigma, window=window)
    res["summ"] = summ
    return res


def decode(q, k_cache, v_cache, cache_len, w_s, *, bs: int, alpha: float, gamma: float,
           batches=None, nb_out: int = 0, want=("o", "tau"), threads: int = 0, q_bar=None,
           sigma: float = 1.0, window: int = 1):
    """One decode step: q [B, H, d] is the query at position cache_len[b] - 1
    whose key/value are already in the caches [B, Hkv, max_len, d].  Also
    returns the summary of the block this token completes (None otherwise)."""
    q = np.asarray(q, dtype=np.float32)
    B, H, d = q.shape
    batches = np.arange(B) if batches is None else np.asarray(batches)
    lens = np.asarray(cache_len, dtype=np.int64)[batches]
    sub_k = np.asarray(k_cache, dtype=np.float32)[batches]
    sub_v = np.asarray(v_cache, dtype=np.float32)[batches]
    nblocks = int(lens.max()) // bs
    summ = summaries(sub_k, w_s, bs, nblocks, q_bar)
    res = forward_rows(q[batches], np.arange(len(batches)), lens - 1, sub_k, sub_v, summ,
                       n_heads=H, bs=bs, alpha=alpha, gamma=gamma, causal=True,
                       nb_out=nb_out, want=want, threads=threads, sigma=sigma, window=window)
    res["new_summary"] = [summ[r, :, lens[r] // bs - 1] if lens[r] % bs == 0 else None
                          for r in range(len(batches))]
    return res
