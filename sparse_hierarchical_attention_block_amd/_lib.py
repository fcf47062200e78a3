"""ctypes binding of libdash.so (the C ABI in include/dash.h).

Argument marshalling only: torch tensors provide device memory and the HIP
stream; every step of the computation runs in the library's gfx950 kernels.
Each wrapper checks that tensors live on the GPU, are contiguous and hold at
least the elements the call will touch (the C side cannot inspect device
pointers), then calls the entry point of the same name and raises
``DashError`` on a non-OK status.  There is no fallback: if the library is
not built, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdash.so")

DASH_OK, DASH_ERR_INVALID_ARG, DASH_ERR_UNSUPPORTED, DASH_ERR_WORKSPACE_TOO_SMALL, DASH_ERR_HIP = \
    range(5)
DASH_F32, DASH_BF16 = 0, 1
QUERY_TILE = 64
WS_ALIGN = 256


class DashError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {dash_status_string(status)}")


class dash_params(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("alpha", ctypes.c_float),
                ("gamma", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("sigma", ctypes.c_float), ("window", ctypes.c_int32)]


class dash_route_buf(ctypes.Structure):
    _fields_ = [("tau", ctypes.c_void_p), ("sel_count", ctypes.c_void_p),
                ("sel_idx", ctypes.c_void_p), ("sel_logp", ctypes.c_void_p),
                ("support_bits", ctypes.c_void_p), ("tile_bits", ctypes.c_void_p)]


class dash_route_sizes(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in
                ("n_qt", "nb", "qt", "tau", "sel_count", "sel_idx", "sel_logp", "support_bits",
                 "tile_bits")]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                      "(python -m sparse_hierarchical_attention_block_amd.build)")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.POINTER(dash_params)
_R = ctypes.POINTER(dash_route_buf)
_V = ctypes.c_void_p
_I = ctypes.c_int64
_lib.dash_status_string.restype = ctypes.c_char_p
_lib.dash_status_string.argtypes = [ctypes.c_int]
_lib.dash_version.restype = ctypes.c_char_p
_lib.dash_version.argtypes = []
for _name in ("dash_route_sizes_prefill", "dash_route_sizes_decode"):
    getattr(_lib, _name).restype = ctypes.c_int
    getattr(_lib, _name).argtypes = [_P, _I, ctypes.POINTER(dash_route_sizes)]
for _name in ("dash_prefill_workspace_bytes", "dash_decode_workspace_bytes"):
    getattr(_lib, _name).restype = ctypes.c_int
    getattr(_lib, _name).argtypes = [_P, _I, ctypes.POINTER(ctypes.c_size_t)]
_lib.dash_summarize.restype = ctypes.c_int
_lib.dash_summarize.argtypes = [_P, _V, _I, _I, _I, _V, _V, _V, _I, _V]
_lib.dash_route.restype = ctypes.c_int
_lib.dash_route.argtypes = [_P, _V, _I, _V, _I, _R, _V]
_lib.dash_attend.restype = ctypes.c_int
_lib.dash_attend.argtypes = [_P, _V, _V, _V, _I, _R, _V, _V]
_lib.dash_mask_to_list.restype = ctypes.c_int
_lib.dash_mask_to_list.argtypes = [_P, _I, _R, _V]
_lib.dash_prefill.restype = ctypes.c_int
_lib.dash_prefill.argtypes = [_P, _V, _V, _V, _I, _V, _V, _V, _I, _V, _V, ctypes.c_size_t, _V]
_lib.dash_prefill_backward_workspace_bytes.restype = ctypes.c_int
_lib.dash_prefill_backward_workspace_bytes.argtypes = [_P, _I, ctypes.POINTER(ctypes.c_size_t)]
_lib.dash_prefill_backward.restype = ctypes.c_int
_lib.dash_prefill_backward.argtypes = [_P, _V, _V, _V, _V, _V, _I, _V, _V, _I, _R, _V, _V, _V, _V,
                                       _V, ctypes.c_size_t, _V]
_lib.dash_prefill_varlen.restype = ctypes.c_int
_lib.dash_prefill_varlen.argtypes = [_P, _V, _V, _V, _I, _V, _V, _V, _V, _I, _V, _V,
                                     ctypes.c_size_t, _V]
_lib.dash_decode_paged.restype = ctypes.c_int
_lib.dash_decode_paged.argtypes = [_P, _V, _V, _V, _I, _V, _I, _V, _I, _V, _V, _V, _I, _V, _R, _V,
                                   ctypes.c_size_t, _V]
_lib.dash_decode.restype = ctypes.c_int
_lib.dash_decode.argtypes = [_P, _V, _V, _V, _V, _I, _V, _V, _V, _I, _V, _R, _V, ctypes.c_size_t,
                             _V]
_lib.dash_decode_noalloc.restype = ctypes.c_int
_lib.dash_decode_noalloc.argtypes = [_P, _V, _V, _V, _V, _I, _V, _V, _V, _I, _V, _R, _V]
_lib.dash_peak_stream_grid.restype = ctypes.c_int
_lib.dash_peak_stream_grid.argtypes = [ctypes.POINTER(ctypes.c_int64)]
_lib.dash_peak_stream.restype = ctypes.c_int
_lib.dash_peak_stream.argtypes = [_V, _V, _I, ctypes.c_int32, _V]
_lib.dash_peak_mfma_grid.restype = ctypes.c_int
_lib.dash_peak_mfma_grid.argtypes = [ctypes.POINTER(ctypes.c_int64)]
_lib.dash_peak_mfma.restype = ctypes.c_int
_lib.dash_peak_mfma.argtypes = [_I, _V, ctypes.POINTER(ctypes.c_double), _V]

EXPORTED = ("dash_status_string", "dash_version", "dash_route_sizes_prefill",
            "dash_route_sizes_decode", "dash_prefill_workspace_bytes",
            "dash_decode_workspace_bytes", "dash_summarize", "dash_route", "dash_attend",
            "dash_mask_to_list", "dash_prefill", "dash_prefill_varlen", "dash_decode",
            "dash_decode_paged", "dash_prefill_backward_workspace_bytes",
            "dash_prefill_backward", "dash_decode_noalloc", "dash_peak_stream_grid",
            "dash_peak_stream",
            "dash_peak_mfma_grid", "dash_peak_mfma")


# ---------------------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------------------

def make_params(batch, n_heads, n_kv_heads, head_dim, block_size, alpha, gamma, dtype,
                sigma=1.0, window=1):
    """dtype: "bf16"/"f32", torch dtype, or DASH_* code; sigma: prior strength;
    window: near-diagonal branch in blocks."""
    if dtype in ("bf16", torch.bfloat16):
        code = DASH_BF16
    elif dtype in ("f32", torch.float32):
        code = DASH_F32
    else:
        code = int(dtype)
    return dash_params(int(batch), int(n_heads), int(n_kv_heads), int(head_dim),
                       int(block_size), float(alpha), float(gamma), code, float(sigma),
                       int(window))


def torch_dtype(p: dash_params):
    return torch.bfloat16 if p.dtype == DASH_BF16 else torch.float32


def _check(fn, status):
    if status != DASH_OK:
        raise DashError(fn, status)


def _dev(t, name, numel, dtype=None):
    """Device pointer of a GPU tensor holding >= numel elements."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _opt_dev(t, name, numel, dtype=None):
    """As _dev, or a null pointer for None."""
    return None if t is None else _dev(t, name, numel, dtype)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def dash_status_string(status: int) -> str:
    return _lib.dash_status_string(int(status)).decode()


def dash_version() -> str:
    return _lib.dash_version().decode()


def dash_route_sizes_prefill(p, n):
    out = dash_route_sizes()
    _check("dash_route_sizes_prefill", _lib.dash_route_sizes_prefill(ctypes.byref(p), n,
                                                                     ctypes.byref(out)))
    return {f: getattr(out, f) for f, _ in dash_route_sizes._fields_}


def dash_route_sizes_decode(p, max_len):
    out = dash_route_sizes()
    _check("dash_route_sizes_decode", _lib.dash_route_sizes_decode(ctypes.byref(p), max_len,
                                                                   ctypes.byref(out)))
    return {f: getattr(out, f) for f, _ in dash_route_sizes._fields_}


def dash_prefill_workspace_bytes(p, n) -> int:
    out = ctypes.c_size_t()
    _check("dash_prefill_workspace_bytes",
           _lib.dash_prefill_workspace_bytes(ctypes.byref(p), n, ctypes.byref(out)))
    return out.value


def dash_decode_workspace_bytes(p, max_len) -> int:
    out = ctypes.c_size_t()
    _check("dash_decode_workspace_bytes",
           _lib.dash_decode_workspace_bytes(ctypes.byref(p), max_len, ctypes.byref(out)))
    return out.value


class RouteBuffers:
    """Device tensors of a dash_route_buf (torch supplies the memory)."""

    def __init__(self, sizes, device="cuda", bits=False, tile_bits=False):
        self.sizes = sizes
        self.tau = torch.empty(sizes["tau"], dtype=torch.float32, device=device)
        self.sel_count = torch.empty(sizes["sel_count"], dtype=torch.int32, device=device)
        self.sel_idx = torch.empty(sizes["sel_idx"], dtype=torch.int32, device=device)
        self.sel_logp = torch.empty(sizes["sel_logp"], dtype=torch.float32, device=device)
        self.support_bits = (torch.empty(sizes["support_bits"], dtype=torch.int32, device=device)
                             if bits else None)
        self.tile_bits = (torch.empty(sizes["tile_bits"], dtype=torch.int32, device=device)
                          if tile_bits else None)

    def struct(self):
        s = self.sizes
        return dash_route_buf(
            _dev(self.tau, "tau", s["tau"], torch.float32),
            _dev(self.sel_count, "sel_count", s["sel_count"], torch.int32),
            _dev(self.sel_idx, "sel_idx", s["sel_idx"], torch.int32),
            _dev(self.sel_logp, "sel_logp", s["sel_logp"], torch.float32),
            None if self.support_bits is None else
            _dev(self.support_bits, "support_bits", s["support_bits"], torch.int32),
            None if self.tile_bits is None else
            _dev(self.tile_bits, "tile_bits", s["tile_bits"], torch.int32))


def workspace(nbytes, device="cuda"):
    """A 256-byte aligned uint8 device buffer (torch's caching allocator
    returns at least 512-byte aligned blocks)."""
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    assert ws.data_ptr() % WS_ALIGN == 0
    return ws


# ---------------------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------------------

def dash_summarize(p, k, kv_len, blk_begin, blk_end, w_s, summ, summ_blocks, stream=None,
                   q_bar=None):
    B, Hkv, d = p.batch, p.n_kv_heads, p.head_dim
    _check("dash_summarize", _lib.dash_summarize(
        ctypes.byref(p), _dev(k, "k", B * Hkv * kv_len * d, torch_dtype(p)), kv_len, blk_begin,
        blk_end, _dev(w_s, "w_s", d * d, torch.float32),
        _opt_dev(q_bar, "q_bar", Hkv * d, torch.float32),
        _dev(summ, "summ", B * Hkv * summ_blocks * d, torch.float32), summ_blocks,
        _stream(stream)))


def dash_route(p, q, n, summ, summ_blocks, route: RouteBuffers, stream=None):
    B, H, Hkv, d = p.batch, p.n_heads, p.n_kv_heads, p.head_dim
    if route.sizes != dash_route_sizes_prefill(p, n):
        raise ValueError("route buffers were sized for another problem")
    rb = route.struct()
    _check("dash_route", _lib.dash_route(
        ctypes.byref(p), _dev(q, "q", B * H * n * d, torch_dtype(p)), n,
        _dev(summ, "summ", B * Hkv * summ_blocks * d, torch.float32), summ_blocks,
        ctypes.byref(rb), _stream(stream)))


def dash_attend(p, q, k, v, n, route: RouteBuffers, o, stream=None):
    B, H, Hkv, d = p.batch, p.n_heads, p.n_kv_heads, p.head_dim
    if route.sizes != dash_route_sizes_prefill(p, n):
        raise ValueError("route buffers were sized for another problem")
    rb = route.struct()
    dt = torch_dtype(p)
    _check("dash_attend", _lib.dash_attend(
        ctypes.byref(p), _dev(q, "q", B * H * n * d, dt), _dev(k, "k", B * Hkv * n * d, dt),
        _dev(v, "v", B * Hkv * n * d, dt), n, ctypes.byref(rb), _dev(o, "o", B * H * n * d, dt),
        _stream(stream)))


def dash_mask_to_list(p, n, route: RouteBuffers, stream=None):
    """route.tile_bits -> route.sel_idx / sel_count (prefill layout)."""
    if route.sizes != dash_route_sizes_prefill(p, n):
        raise ValueError("route buffers were sized for another problem")
    if route.tile_bits is None:
        raise ValueError("route buffers hold no tile_bits")
    rb = route.struct()
    _check("dash_mask_to_list", _lib.dash_mask_to_list(ctypes.byref(p), n, ctypes.byref(rb),
                                                       _stream(stream)))


def dash_prefill(p, q, k, v, n, w_s, summ, summ_blocks, o, ws, stream=None, q_bar=None):
    B, H, Hkv, d = p.batch, p.n_heads, p.n_kv_heads, p.head_dim
    dt = torch_dtype(p)
    _check("dash_prefill", _lib.dash_prefill(
        ctypes.byref(p), _dev(q, "q", B * H * n * d, dt), _dev(k, "k", B * Hkv * n * d, dt),
        _dev(v, "v", B * Hkv * n * d, dt), n, _dev(w_s, "w_s", d * d, torch.float32),
        _opt_dev(q_bar, "q_bar", Hkv * d, torch.float32),
        _dev(summ, "summ", B * Hkv * summ_blocks * d, torch.float32), summ_blocks,
        _dev(o, "o", B * H * n * d, dt), _dev(ws, "ws", 0), ws.numel() * ws.element_size(),
        _stream(stream)))


def dash_prefill_varlen(p, q, k, v, n_max, seq_lens, w_s, summ, summ_blocks, o, ws, stream=None,
                        q_bar=None):
    """dash_prefill over a ragged batch: sequence b has seq_lens[b] (int32, on
    the GPU) of the n_max positions of its slices."""
    B, H, Hkv, d = p.batch, p.n_heads, p.n_kv_heads, p.head_dim
    dt = torch_dtype(p)
    _check("dash_prefill_varlen", _lib.dash_prefill_varlen(
        ctypes.byref(p), _dev(q, "q", B * H * n_max * d, dt),
        _dev(k, "k", B * Hkv * n_max * d, dt), _dev(v, "v", B * Hkv * n_max * d, dt), n_max,
        _dev(seq_lens, "seq_lens", B, torch.int32), _dev(w_s, "w_s", d * d, torch.float32),
        _opt_dev(q_bar, "q_bar", Hkv * d, torch.float32),
        _dev(summ, "summ", B * Hkv * summ_blocks * d, torch.float32), summ_blocks,
        _dev(o, "o", B * H * n_max * d, dt), _dev(ws, "ws", 0), ws.numel() * ws.element_size(),
        _stream(stream)))


def dash_decode(p, q, k_cache, v_cache, cache_len, max_len, w_s, summ, summ_blocks, o,
                ws, route: RouteBuffers | None = None, stream=None, q_bar=None):
    B, H, Hkv, d = p.batch, p.n_heads, p.n_kv_heads, p.head_dim
    dt = torch_dtype(p)
    rb = None
    if route is not None:
        if route.sizes != dash_route_sizes_decode(p, max_len):
            raise ValueError("route buffers were sized for another problem")
        rb_struct = route.struct()
        rb = ctypes.byref(rb_struct)
    _check("dash_decode", _lib.dash_decode(
        ctypes.byref(p), _dev(q, "q", B * H * d, dt),
        _dev(k_cache, "k_cache", B * Hkv * max_len * d, dt),
        _dev(v_cache, "v_cache", B * Hkv * max_len * d, dt),
        _dev(cache_len, "cache_len", B, torch.int32), max_len,
        _dev(w_s, "w_s", d * d, torch.float32),
        _opt_dev(q_bar, "q_bar", Hkv * d, torch.float32),
        _dev(summ, "summ", B * Hkv * summ_blocks * d, torch.float32), summ_blocks,
        _dev(o, "o", B * H * d, dt), rb, _dev(ws, "ws", 0), ws.numel() * ws.element_size(),
        _stream(stream)))


def dash_decode_noalloc(p, q, k_cache, v_cache, cache_len, max_len, w_s, summ, summ_blocks, o,
                        route: RouteBuffers | None = None, stream=None, q_bar=None):
    """dash_decode with the library's static device scratch as its workspace
    (for callers that cannot allocate); calls on one GPU must not overlap."""
    B, H, Hkv, d = p.batch, p.n_heads, p.n_kv_heads, p.head_dim
    dt = torch_dtype(p)
    rb = None
    if route is not None:
        if route.sizes != dash_route_sizes_decode(p, max_len):
            raise ValueError("route buffers were sized for another problem")
        rb_struct = route.struct()
        rb = ctypes.byref(rb_struct)
    _check("dash_decode_noalloc", _lib.dash_decode_noalloc(
        ctypes.byref(p), _dev(q, "q", B * H * d, dt),
        _dev(k_cache, "k_cache", B * Hkv * max_len * d, dt),
        _dev(v_cache, "v_cache", B * Hkv * max_len * d, dt),
        _dev(cache_len, "cache_len", B, torch.int32), max_len,
        _dev(w_s, "w_s", d * d, torch.float32),
        _opt_dev(q_bar, "q_bar", Hkv * d, torch.float32),
        _dev(summ, "summ", B * Hkv * summ_blocks * d, torch.float32), summ_blocks,
        _dev(o, "o", B * H * d, dt), rb, _stream(stream)))


def dash_decode_paged(p, q, k_pages, v_pages, block_table, cache_len, max_len, w_s, summ,
                      summ_blocks, o, ws, route: RouteBuffers | None = None, stream=None,
                      q_bar=None):
    """dash_decode over paged caches k_pages / v_pages [num_pages, Hkv, bs, d] and
    block_table [B, max_blocks] int32 (block j of sequence b in page block_table[b, j])."""
    B, H, Hkv, d, bs = p.batch, p.n_heads, p.n_kv_heads, p.head_dim, p.block_size
    dt = torch_dtype(p)
    if k_pages.dim() != 4 or tuple(k_pages.shape[1:]) != (Hkv, bs, d):
        raise ValueError("k_pages must be [num_pages, Hkv, bs, d]")
    if v_pages.shape != k_pages.shape:
        raise ValueError("v_pages must match k_pages")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    num_pages, max_blocks = k_pages.shape[0], block_table.shape[1]
    rb = None
    if route is not None:
        if route.sizes != dash_route_sizes_decode(p, max_len):
            raise ValueError("route buffers were sized for another problem")
        rb_struct = route.struct()
        rb = ctypes.byref(rb_struct)
    _check("dash_decode_paged", _lib.dash_decode_paged(
        ctypes.byref(p), _dev(q, "q", B * H * d, dt),
        _dev(k_pages, "k_pages", num_pages * Hkv * bs * d, dt),
        _dev(v_pages, "v_pages", num_pages * Hkv * bs * d, dt), num_pages,
        _dev(block_table, "block_table", B * max_blocks, torch.int32), max_blocks,
        _dev(cache_len, "cache_len", B, torch.int32), max_len,
        _dev(w_s, "w_s", d * d, torch.float32),
        _opt_dev(q_bar, "q_bar", Hkv * d, torch.float32),
        _dev(summ, "summ", B * Hkv * summ_blocks * d, torch.float32), summ_blocks,
        _dev(o, "o", B * H * d, dt), rb, _dev(ws, "ws", 0), ws.numel() * ws.element_size(),
        _stream(stream)))


def dash_prefill_backward_workspace_bytes(p, n) -> int:
    out = ctypes.c_size_t()
    _check("dash_prefill_backward_workspace_bytes",
           _lib.dash_prefill_backward_workspace_bytes(ctypes.byref(p), n, ctypes.byref(out)))
    return out.value


def dash_prefill_backward(p, q, k, v, o, d_o, n, w_s, summ, summ_blocks, route: RouteBuffers,
                          dq, dk, dv, dw_s, ws, stream=None):
    """Gradients of the causal prefill (mean-pooled summaries) into float32 dq, dk,
    dv, dw_s, from the forward's inputs, output, summaries and routing."""
    B, H, Hkv, d = p.batch, p.n_heads, p.n_kv_heads, p.head_dim
    dt = torch_dtype(p)
    if route.sizes != dash_route_sizes_prefill(p, n):
        raise ValueError("route buffers were sized for another problem")
    rb = route.struct()
    f32 = torch.float32
    _check("dash_prefill_backward", _lib.dash_prefill_backward(
        ctypes.byref(p), _dev(q, "q", B * H * n * d, dt), _dev(k, "k", B * Hkv * n * d, dt),
        _dev(v, "v", B * Hkv * n * d, dt), _dev(o, "o", B * H * n * d, dt),
        _dev(d_o, "d_o", B * H * n * d, dt), n, _dev(w_s, "w_s", d * d, f32),
        _dev(summ, "summ", B * Hkv * summ_blocks * d, f32), summ_blocks, ctypes.byref(rb),
        _dev(dq, "dq", B * H * n * d, f32), _dev(dk, "dk", B * Hkv * n * d, f32),
        _dev(dv, "dv", B * Hkv * n * d, f32), _dev(dw_s, "dw_s", d * d, f32),
        _dev(ws, "ws", 0), ws.numel() * ws.element_size(), _stream(stream)))


# ---------------------------------------------------------------------------------------
# measurement helpers
# ---------------------------------------------------------------------------------------

def dash_peak_stream_grid() -> int:
    """Threads of a dash_peak_stream launch (one 16-byte store each in read mode)."""
    out = ctypes.c_int64()
    _check("dash_peak_stream_grid", _lib.dash_peak_stream_grid(ctypes.byref(out)))
    return out.value


def dash_peak_stream(src, dst, nbytes, mode, stream=None):
    """mode 0: copy nbytes of src into dst; mode 1: read nbytes of src only
    (loads that allocate in the caches); mode 2: the same read with
    non-temporal loads (dst holds 16 bytes per launched thread in modes 1, 2)."""
    need = nbytes if mode == 0 else 16 * dash_peak_stream_grid()
    _check("dash_peak_stream", _lib.dash_peak_stream(
        _dev(src, "src", nbytes // src.element_size()),
        _dev(dst, "dst", need // dst.element_size()), int(nbytes), int(mode), _stream(stream)))


def dash_peak_mfma_grid() -> int:
    """Waves of a dash_peak_mfma launch (one float of sink each)."""
    out = ctypes.c_int64()
    _check("dash_peak_mfma_grid", _lib.dash_peak_mfma_grid(ctypes.byref(out)))
    return out.value


def dash_peak_mfma(iters, sink, stream=None) -> float:
    """Launch the register-resident bf16 MFMA loop; returns its flop count."""
    flops = ctypes.c_double()
    _check("dash_peak_mfma", _lib.dash_peak_mfma(
        int(iters), _dev(sink, "sink", dash_peak_mfma_grid(), torch.float32),
        ctypes.byref(flops), _stream(stream)))
    return flops.value
