"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every symbol include/dash.h declares, and rejects bad arguments before
launching anything."""
import ctypes
import os
import re

import pytest
import torch

import sparse_hierarchical_attention_block_amd as dash
from sparse_hierarchical_attention_block_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(os.path.join(ROOT, "include", "dash.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dash_\w+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 11
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTED)


def test_version_and_status_strings():
    assert "gfx950" in dash.dash_version()
    for code in range(5):
        assert dash.dash_status_string(code).startswith("DASH_")
    assert dash.dash_status_string(99) == "unknown dash_status"


def P(**kw):
    base = dict(batch=1, n_heads=32, n_kv_heads=8, head_dim=128, block_size=64, alpha=1.5,
                gamma=2.0, dtype="bf16")
    base.update(kw)
    return dash.make_params(**base)


def test_params_layout_matches_header():
    # dash_params in include/dash.h: 8 four-byte fields, then sigma and window
    assert ctypes.sizeof(L.dash_params) == 40
    assert L.dash_params.sigma.offset == 32 and L.dash_params.window.offset == 36
    p = P()
    assert p.sigma == 1.0 and p.window == 1


def test_route_sizes():
    s = dash.dash_route_sizes_prefill(P(), 8192)
    assert s["n_qt"] == 128 and s["nb"] == 128 and s["qt"] == 64
    assert s["sel_logp"] == 8 * 128 * 128 * 64 and s["tau"] == 32 * 8192
    assert s["support_bits"] == 32 * 8192 * 4
    s = dash.dash_route_sizes_prefill(P(block_size=128), 1000)
    assert s["n_qt"] == 16 and s["nb"] == 8
    d = dash.dash_route_sizes_decode(P(batch=32), 32768)
    assert d["nb"] == 512 and d["qt"] == 1 and d["sel_idx"] == 32 * 8 * 512
    assert dash.dash_prefill_workspace_bytes(P(), 8192) % 256 == 0
    assert dash.dash_decode_workspace_bytes(P(batch=32), 32768) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(n_heads=30), L.DASH_ERR_INVALID_ARG),          # H % Hkv != 0
    (dict(alpha=1.0), L.DASH_ERR_INVALID_ARG),
    (dict(alpha=2.5), L.DASH_ERR_INVALID_ARG),
    (dict(alpha=float("nan")), L.DASH_ERR_INVALID_ARG),
    (dict(gamma=0.0), L.DASH_ERR_INVALID_ARG),
    (dict(gamma=float("inf")), L.DASH_ERR_INVALID_ARG),
    (dict(dtype=7), L.DASH_ERR_INVALID_ARG),
    (dict(batch=0), L.DASH_ERR_INVALID_ARG),
    (dict(head_dim=96), L.DASH_ERR_UNSUPPORTED),
    (dict(block_size=32), L.DASH_ERR_UNSUPPORTED),
    (dict(n_heads=48, n_kv_heads=4), L.DASH_ERR_UNSUPPORTED),   # G = 12
    (dict(sigma=-0.5), L.DASH_ERR_INVALID_ARG),
    (dict(sigma=float("nan")), L.DASH_ERR_INVALID_ARG),
    (dict(window=0), L.DASH_ERR_INVALID_ARG),
])
def test_bad_params(kw, code):
    out = ctypes.c_size_t()
    p = P(**kw)
    assert L._lib.dash_prefill_workspace_bytes(ctypes.byref(p), 1024, ctypes.byref(out)) == code
    assert L._lib.dash_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, 1024, FAKE, None, FAKE, 16, FAKE,
                               FAKE, 1 << 40, None) == code


def test_null_pointers_and_sizes():
    p = P()
    lib = L._lib
    assert lib.dash_prefill(ctypes.byref(p), None, FAKE, FAKE, 1024, FAKE, None, FAKE, 16, FAKE,
                            FAKE, 1 << 30, None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, -1, FAKE, None, FAKE, 16, FAKE,
                            FAKE, 1 << 30, None) == L.DASH_ERR_INVALID_ARG
    # summary capacity below floor(n / bs)
    assert lib.dash_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, 1024, FAKE, None, FAKE, 15, FAKE,
                            FAKE, 1 << 30, None) == L.DASH_ERR_INVALID_ARG
    # workspace too small / misaligned
    need = dash.dash_prefill_workspace_bytes(p, 1024)
    assert lib.dash_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, 1024, FAKE, None, FAKE, 16, FAKE,
                            FAKE, need - 1, None) == L.DASH_ERR_WORKSPACE_TOO_SMALL
    assert lib.dash_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, 1024, FAKE, None, FAKE, 16, FAKE,
                            FAKE + 8, need, None) == L.DASH_ERR_INVALID_ARG
    # tensors must be 16-byte aligned
    assert lib.dash_prefill(ctypes.byref(p), FAKE + 4, FAKE, FAKE, 1024, FAKE, None, FAKE, 16,
                            FAKE, FAKE, need, None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, 1024, FAKE, FAKE + 8, FAKE, 16,
                            FAKE, FAKE, need, None) == L.DASH_ERR_INVALID_ARG
    # empty problem: nothing to do
    assert lib.dash_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, 0, FAKE, None, FAKE, 0, FAKE,
                            FAKE, 0, None) == L.DASH_OK
    # summarize past the keys / past the summary capacity
    assert lib.dash_summarize(ctypes.byref(p), FAKE, 1000, 0, 16, FAKE, None, FAKE, 16,
                              None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_summarize(ctypes.byref(p), FAKE, 1024, 0, 16, FAKE, None, FAKE, 15,
                              None) == L.DASH_ERR_INVALID_ARG
    # route without buffers
    rb = L.dash_route_buf(FAKE, FAKE, None, FAKE, None, None)
    assert lib.dash_route(ctypes.byref(p), FAKE, 1024, FAKE, 16, ctypes.byref(rb),
                          None) == L.DASH_ERR_INVALID_ARG
    # decode: bad max_len, small summary cache, small workspace
    dneed = dash.dash_decode_workspace_bytes(p, 4096)
    assert lib.dash_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, FAKE, 64, FAKE,
                           None, FAKE, dneed, None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 4096, FAKE, None, FAKE,
                           63, FAKE, None, FAKE, dneed, None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 4096, FAKE, None, FAKE,
                           64, FAKE, None, FAKE, dneed - 1, None) == L.DASH_ERR_WORKSPACE_TOO_SMALL


def test_mask_to_list_argument_checks():
    p = P()
    lib = L._lib
    full = L.dash_route_buf(FAKE, FAKE, FAKE, FAKE, None, FAKE)
    no_bits = L.dash_route_buf(FAKE, FAKE, FAKE, FAKE, None, None)
    no_idx = L.dash_route_buf(FAKE, FAKE, None, FAKE, None, FAKE)
    assert lib.dash_mask_to_list(ctypes.byref(p), 1024, ctypes.byref(no_bits),
                                 None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_mask_to_list(ctypes.byref(p), 1024, ctypes.byref(no_idx),
                                 None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_mask_to_list(ctypes.byref(p), -1, ctypes.byref(full),
                                 None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_mask_to_list(ctypes.byref(p), 1024, None, None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_mask_to_list(ctypes.byref(p), 0, ctypes.byref(full), None) == L.DASH_OK
    assert lib.dash_mask_to_list(ctypes.byref(P(window=0)), 1024, ctypes.byref(full),
                                 None) == L.DASH_ERR_INVALID_ARG
    s = dash.dash_route_sizes_prefill(p, 8192)
    assert s["tile_bits"] == 8 * 128 * 4
    assert dash.dash_route_sizes_decode(P(batch=32), 32768)["tile_bits"] == 32 * 8 * 16


def test_decode_paged_argument_checks():
    p = P()
    lib = L._lib
    need = dash.dash_decode_workspace_bytes(p, 4096)
    # no block table / no pages / table narrower than ceil(max_len / bs)
    assert lib.dash_decode_paged(ctypes.byref(p), FAKE, FAKE, FAKE, 64, None, 64, FAKE, 4096, FAKE,
                                 None, FAKE, 64, FAKE, None, FAKE, need,
                                 None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_decode_paged(ctypes.byref(p), FAKE, FAKE, FAKE, 0, FAKE, 64, FAKE, 4096, FAKE,
                                 None, FAKE, 64, FAKE, None, FAKE, need,
                                 None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_decode_paged(ctypes.byref(p), FAKE, FAKE, FAKE, 64, FAKE, 63, FAKE, 4096, FAKE,
                                 None, FAKE, 64, FAKE, None, FAKE, need,
                                 None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_decode_paged(ctypes.byref(p), FAKE, FAKE, FAKE, 64, FAKE, 64, FAKE, 4096, FAKE,
                                 None, FAKE, 64, FAKE, None, FAKE, need - 1,
                                 None) == L.DASH_ERR_WORKSPACE_TOO_SMALL


def test_prefill_varlen_argument_checks():
    p = P()
    lib = L._lib
    need = dash.dash_prefill_workspace_bytes(p, 1024)
    assert lib.dash_prefill_varlen(ctypes.byref(p), FAKE, FAKE, FAKE, 1024, None, FAKE, None,
                                   FAKE, 16, FAKE, FAKE, need, None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_prefill_varlen(ctypes.byref(p), FAKE, FAKE, FAKE, 1024, FAKE, FAKE, None,
                                   FAKE, 15, FAKE, FAKE, need, None) == L.DASH_ERR_INVALID_ARG
    assert lib.dash_prefill_varlen(ctypes.byref(p), FAKE, FAKE, FAKE, 1024, FAKE, FAKE, None,
                                   FAKE, 16, FAKE, FAKE, need - 1,
                                   None) == L.DASH_ERR_WORKSPACE_TOO_SMALL


def test_binding_rejects_host_tensors():
    p = P(n_heads=2, n_kv_heads=2, head_dim=64)
    t = torch.zeros(2 * 64 * 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        dash.dash_summarize(p, t.bfloat16(), 64, 0, 1, torch.zeros(64 * 64), t, 1)


def test_decode_noalloc_rejects_oversized_problem_before_launch():
    # 64 sequences x 128K, 64 query heads: ~170 MiB of workspace, above the
    # 32 MiB static scratch; rejected on the host, nothing touches a device
    p = P(batch=64, n_heads=64, n_kv_heads=8)
    assert dash.dash_decode_workspace_bytes(p, 131072) > 32 << 20
    st = L._lib.dash_decode_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 131072, FAKE, None,
                                    FAKE, 2048, FAKE, None, None)
    assert st == L.DASH_ERR_WORKSPACE_TOO_SMALL
    st = L._lib.dash_decode_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 0, FAKE, None,
                                    FAKE, 2048, FAKE, None, None)
    assert st == L.DASH_ERR_INVALID_ARG
