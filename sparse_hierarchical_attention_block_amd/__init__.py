"""DashAttention forward pass for AMD Instinct MI355X (gfx950).

The computation lives in ``libdash.so`` (hand-written HIP kernels behind the
C ABI of ``include/dash.h``); this package only binds it.  Importing it fails
loudly when the library has not been built -- there is no CPU fallback.
"""
from ._lib import (  # noqa: F401
    DASH_BF16, DASH_F32, QUERY_TILE, DashError, RouteBuffers, dash_attend, dash_decode,
    dash_decode_noalloc, dash_decode_paged, dash_decode_workspace_bytes, dash_mask_to_list,
    dash_params, dash_peak_mfma, dash_peak_mfma_grid, dash_peak_stream, dash_peak_stream_grid, dash_prefill,
    dash_prefill_backward, dash_prefill_backward_workspace_bytes, dash_prefill_varlen,
    dash_prefill_workspace_bytes, dash_route, dash_route_sizes_decode, dash_route_sizes_prefill,
    dash_status_string, dash_summarize, dash_version, make_params, torch_dtype, workspace)
