// api.cpp -- the C ABI declared in include/dash.h: host-side argument
// validation, workspace carving and kernel launches on the caller's stream.
// Nothing is enqueued when validation fails; no call allocates, frees or
// synchronises; no C++ exception crosses the ABI.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "dash.h"
#include "dash_internal.hpp"

namespace {

using dash::Shape;

constexpr int64_t kQT = DASH_QUERY_TILE;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// The kernels move tensors with 16-byte vector accesses; a null pointer
// passes here (the null checks are separate).
template <typename... P>
bool aligned16(P... ptrs) {
  return ((((uintptr_t)ptrs) % 16 == 0) && ...);
}

dash_status check_params(const dash_params* p, Shape* s) {
  if (!p) return DASH_ERR_INVALID_ARG;
  if (p->batch < 1 || p->n_heads < 1 || p->n_kv_heads < 1) return DASH_ERR_INVALID_ARG;
  if (p->n_heads % p->n_kv_heads != 0) return DASH_ERR_INVALID_ARG;
  if (p->dtype != DASH_F32 && p->dtype != DASH_BF16) return DASH_ERR_INVALID_ARG;
  if (!std::isfinite(p->alpha) || !(p->alpha > 1.0f) || p->alpha > 2.0f) return DASH_ERR_INVALID_ARG;
  if (!std::isfinite(p->gamma) || !(p->gamma > 0.0f)) return DASH_ERR_INVALID_ARG;
  if (!std::isfinite(p->sigma) || !(p->sigma >= 0.0f)) return DASH_ERR_INVALID_ARG;
  if (p->window < 1) return DASH_ERR_INVALID_ARG;
  if (p->head_dim < 1 || p->block_size < 1) return DASH_ERR_INVALID_ARG;
  const int G = p->n_heads / p->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return DASH_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return DASH_ERR_UNSUPPORTED;
  if (p->block_size != 64 && p->block_size != 128) return DASH_ERR_UNSUPPORTED;
  if ((int64_t)p->batch * p->n_heads > (1 << 24)) return DASH_ERR_UNSUPPORTED;
  s->B = p->batch;
  s->H = p->n_heads;
  s->Hkv = p->n_kv_heads;
  s->G = G;
  s->d = p->head_dim;
  s->bs = p->block_size;
  s->alpha = p->alpha;
  s->gamma = p->gamma;
  s->dtype = p->dtype;
  s->sigma = p->sigma;
  s->window = p->window;
  return DASH_OK;
}

dash_status hip_status(hipError_t e) { return e == hipSuccess ? DASH_OK : DASH_ERR_HIP; }

// grid sizes must fit the 32-bit x dimension
bool grid_ok(int64_t blocks) { return blocks >= 0 && blocks < ((int64_t)1 << 31); }

// the attend kernels address one (sequence, KV head)'s keys / values through
// a buffer resource with a 31-bit byte range
bool seq_bytes_ok(const Shape& s, int64_t n) {
  const int64_t elt = s.dtype == DASH_BF16 ? 2 : 4;
  return (n + 64) * s.d * elt < ((int64_t)1 << 31);
}

void prefill_sizes(const Shape& s, int64_t n, dash_route_sizes* r) {
  r->n_qt = (n + kQT - 1) / kQT;
  r->nb = (n + s.bs - 1) / s.bs;
  r->qt = kQT;
  r->tau = (int64_t)s.B * s.H * n;
  r->sel_count = (int64_t)s.B * s.Hkv * r->n_qt;
  r->sel_idx = r->sel_count * r->nb;
  r->sel_logp = r->sel_idx * kQT;
  r->support_bits = (int64_t)s.B * s.H * n * ((r->nb + 31) / 32);
  r->tile_bits = r->sel_count * ((r->nb + 31) / 32);
}

// LDS needed by the pass-based prefill routing kernel, the one with the largest
// buffer (must match launch_route_prefill in route.hip)
bool route_lds_ok(const Shape& s, int64_t n) {
  const int64_t n_qt = (n + kQT - 1) / kQT;
  const int64_t t_max = ((n_qt - 1) * kQT) / s.bs;
  const int64_t pitch = ((t_max > 0 ? t_max : 1) + 15) / 16 * 16 + 4;
  int64_t pp = 64;
  while (pp > 1 && pp * s.G * pitch * 4 > DASH_ROUTE_X_BUDGET) pp >>= 1;
  while (pp * s.G < 16) pp <<= 1;
  while (pp * s.G > 64) pp >>= 1;
  const int64_t lds = (pp * s.G * pitch + pp * s.G) * 4 + (pitch - 4) * 4;
  return lds <= 160 * 1024;
}

struct PrefillLayout {
  size_t off_tau, off_count, off_idx, off_logp, total;
};

PrefillLayout prefill_layout(const Shape& s, int64_t n) {
  dash_route_sizes r;
  prefill_sizes(s, n, &r);
  PrefillLayout L;
  size_t off = 0;
  L.off_tau = off;   off = align_up(off + 4 * (size_t)r.tau);
  L.off_count = off; off = align_up(off + 4 * (size_t)r.sel_count);
  L.off_idx = off;   off = align_up(off + 4 * (size_t)r.sel_idx);
  L.off_logp = off;  off = align_up(off + 4 * (size_t)r.sel_logp);
  L.total = off;
  return L;
}

dash_status check_route_buf(const dash_route_buf* rb) {
  if (!rb || !rb->tau || !rb->sel_count || !rb->sel_idx || !rb->sel_logp)
    return DASH_ERR_INVALID_ARG;
  return DASH_OK;
}

// ---- scratch of dash_decode_noalloc ------------------------------------------------------
// One copy per GPU (a device array, held until the process ends).  Host code
// never passes the array's own name (on the host it is only a stand-in for
// the symbol): its device address is looked up once per device, with that
// device current, and that address is what the kernels receive.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[dash::kMaxDevices];

hipError_t decode_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= dash::kMaxDevices) return hipErrorInvalidDevice;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once,
                 [&slot] { slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch)); });
  if (slot.err != hipSuccess) return slot.err;
  *out = slot.ptr;
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* dash_status_string(dash_status s) {
  switch (s) {
    case DASH_OK: return "DASH_OK";
    case DASH_ERR_INVALID_ARG: return "DASH_ERR_INVALID_ARG: invalid argument";
    case DASH_ERR_UNSUPPORTED: return "DASH_ERR_UNSUPPORTED: configuration not built";
    case DASH_ERR_WORKSPACE_TOO_SMALL: return "DASH_ERR_WORKSPACE_TOO_SMALL: workspace too small";
    case DASH_ERR_HIP: return "DASH_ERR_HIP: HIP runtime error";
  }
  return "unknown dash_status";
}

const char* dash_version(void) { return "dash-mi355x 0.1.0 gfx950"; }

dash_status dash_route_sizes_prefill(const dash_params* p, int64_t n, dash_route_sizes* out) {
  Shape s;
  dash_status st = check_params(p, &s);
  if (st != DASH_OK) return st;
  if (n < 0 || !out) return DASH_ERR_INVALID_ARG;
  prefill_sizes(s, n, out);
  return DASH_OK;
}

dash_status dash_route_sizes_decode(const dash_params* p, int64_t max_len, dash_route_sizes* out) {
  Shape s;
  dash_status st = check_params(p, &s);
  if (st != DASH_OK) return st;
  if (max_len < 1 || !out) return DASH_ERR_INVALID_ARG;
  out->n_qt = 1;
  out->nb = (max_len + s.bs - 1) / s.bs;
  out->qt = 1;
  out->tau = (int64_t)s.B * s.H;
  out->sel_count = (int64_t)s.B * s.Hkv;
  out->sel_idx = out->sel_count * out->nb;
  out->sel_logp = out->sel_idx;
  out->support_bits = (int64_t)s.B * s.H * ((out->nb + 31) / 32);
  out->tile_bits = out->sel_count * ((out->nb + 31) / 32);
  return DASH_OK;
}

dash_status dash_prefill_workspace_bytes(const dash_params* p, int64_t n, size_t* bytes) {
  Shape s;
  dash_status st = check_params(p, &s);
  if (st != DASH_OK) return st;
  if (n < 0 || !bytes) return DASH_ERR_INVALID_ARG;
  *bytes = prefill_layout(s, n).total;
  return DASH_OK;
}

dash_status dash_decode_workspace_bytes(const dash_params* p, int64_t max_len, size_t* bytes) {
  Shape s;
  dash_status st = check_params(p, &s);
  if (st != DASH_OK) return st;
  if (max_len < 1 || !bytes) return DASH_ERR_INVALID_ARG;
  *bytes = dash::decode_layout(s, max_len).total;
  return DASH_OK;
}

dash_status dash_summarize(const dash_params* p, const void* k, int64_t kv_len, int64_t blk_begin,
                           int64_t blk_end, const float* w_s, const float* q_bar, float* summ,
                           int64_t summ_blocks, void* stream) {
  Shape s;
  dash_status st = check_params(p, &s);
  if (st != DASH_OK) return st;
  if (!k || !w_s || !summ) return DASH_ERR_INVALID_ARG;
  if (!aligned16(k, w_s, q_bar, summ)) return DASH_ERR_INVALID_ARG;
  if (blk_begin < 0 || blk_end < blk_begin || kv_len < blk_end * s.bs || summ_blocks < blk_end)
    return DASH_ERR_INVALID_ARG;
  if (!grid_ok((blk_end - blk_begin) * s.B * s.Hkv)) return DASH_ERR_UNSUPPORTED;
  return hip_status(dash::launch_summarize(s, k, kv_len, blk_begin, blk_end, w_s, q_bar, summ,
                                           summ_blocks, (hipStream_t)stream));
}

dash_status dash_route(const dash_params* p, const void* q, int64_t n, const float* summ,
                       int64_t summ_blocks, const dash_route_buf* route, void* stream) {
  Shape s;
  dash_status st = check_params(p, &s);
  if (st != DASH_OK) return st;
  if (n < 0 || !q || !summ) return DASH_ERR_INVALID_ARG;
  if (!aligned16(q, summ)) return DASH_ERR_INVALID_ARG;
  if ((st = check_route_buf(route)) != DASH_OK) return st;
  if (summ_blocks < n / s.bs) return DASH_ERR_INVALID_ARG;
  if (n == 0) return DASH_OK;
  if (!route_lds_ok(s, n)) return DASH_ERR_UNSUPPORTED;
  if (!grid_ok(((n + kQT - 1) / kQT) * s.B * s.Hkv)) return DASH_ERR_UNSUPPORTED;
  return hip_status(dash::launch_route_prefill(s, q, n, summ, summ_blocks, *route,
                                               (hipStream_t)stream));
}

dash_status dash_attend(const dash_params* p, const void* q, const void* k, const void* v,
                        int64_t n, const dash_route_buf* route, void* o, void* stream) {
  Shape s;
  dash_status st = check_params(p, &s);
  if (st != DASH_OK) return st;
  if (n < 0 || !q || !k || !v || !o || !route || !route->sel_count || !route->sel_idx ||
      !route->sel_logp)
    return DASH_ERR_INVALID_ARG;
  if (!aligned16(q, k, v, o)) return DASH_ERR_INVALID_ARG;
  if (n == 0) return DASH_OK;
  if (!grid_ok(((n + kQT - 1) / kQT) * s.B * s.H) || !seq_bytes_ok(s, n))
    return DASH_ERR_UNSUPPORTED;
  return hip_status(dash::launch_attend_prefill(s, q, k, v, n, *route, o, (hipStream_t)stream));
}

dash_status dash_mask_to_list(const dash_params* p, int64_t n, const dash_route_buf* route,
                              void* stream) {
  Shape s;
  dash_status st = check_params(p, &s);
  if (st != DASH_OK) return st;
  if (n < 0 || !route || !route->tile_bits || !route->sel_count || !route->sel_idx)
    return DASH_ERR_INVALID_ARG;
  if (n == 0) return DASH_OK;
  if (!grid_ok(((n + kQT - 1) / kQT) * s.B * s.Hkv)) return DASH_ERR_UNSUPPORTED;
  return hip_status(dash::launch_mask_to_list(s, n, *route, (hipStream_t)stream));
}

// Shared checks and launches of dash_prefill / dash_prefill_varlen (seq_len
// null: every sequence has n positions).
static dash_status prefill_impl(const dash_params* p, const void* q, const void* k, const void* v,
                                int64_t n, const int32_t* seq_len, const float* w_s,
                                const float* q_bar, float* summ, int64_t summ_blocks, void* o,
                                void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  dash_status st = check_params(p, &s);
  if (st != DASH_OK) return st;
  if (n < 0 || !q || !k || !v || !w_s || !summ || !o) return DASH_ERR_INVALID_ARG;
  if (!aligned16(q, k, v, w_s, q_bar, summ, o)) return DASH_ERR_INVALID_ARG;
  if (summ_blocks < n / s.bs) return DASH_ERR_INVALID_ARG;
  if (n == 0) return DASH_OK;
  const PrefillLayout L = prefill_layout(s, n);
  if (!ws || ((uintptr_t)ws % kAlign) != 0) return DASH_ERR_INVALID_ARG;
  if (ws_bytes < L.total) return DASH_ERR_WORKSPACE_TOO_SMALL;
  if (!route_lds_ok(s, n) || !seq_bytes_ok(s, n)) return DASH_ERR_UNSUPPORTED;
  if (!grid_ok(((n + kQT - 1) / kQT) * s.B * s.H) || !grid_ok((n / s.bs) * s.B * s.Hkv))
    return DASH_ERR_UNSUPPORTED;
  char* base = (char*)ws;
  dash_route_buf rb;
  rb.tau = (float*)(base + L.off_tau);
  rb.sel_count = (int32_t*)(base + L.off_count);
  rb.sel_idx = (int32_t*)(base + L.off_idx);
  rb.sel_logp = (float*)(base + L.off_logp);
  rb.support_bits = nullptr;
  rb.tile_bits = nullptr;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e =
      dash::launch_summarize(s, k, n, 0, n / s.bs, w_s, q_bar, summ, summ_blocks, hs, seq_len);
  if (e == hipSuccess) e = dash::launch_route_prefill(s, q, n, summ, summ_blocks, rb, hs, seq_len);
  if (e == hipSuccess) e = dash::launch_attend_prefill(s, q, k, v, n, rb, o, hs, seq_len);
  return hip_status(e);
}

dash_status dash_prefill(const dash_params* p, const void* q, const void* k, const void* v,
                         int64_t n, const float* w_s, const float* q_bar, float* summ,
                         int64_t summ_blocks, void* o, void* ws, size_t ws_bytes, void* stream) {
  return prefill_impl(p, q, k, v, n, nullptr, w_s, q_bar, summ, summ_blocks, o, ws, ws_bytes,
                      stream);
}

dash_status dash_prefill_varlen(const dash_params* p, const void* q, const void* k, const void* v,
                                int64_t n_max, const int32_t* seq_lens, const float* w_s,
                                const float* q_bar, float* summ, int64_t summ_blocks, void* o,
                                void* ws, size_t ws_bytes, void* stream) {
  if (!seq_lens) return DASH_ERR_INVALID_ARG;
  return prefill_impl(p, q, k, v, n_max, seq_lens, w_s, q_bar, summ, summ_blocks, o, ws,
                      ws_bytes, stream);
}

dash_status dash_prefill_backward_workspace_bytes(const dash_params* p, int64_t n,
                                                  size_t* bytes) {
  Shape s;
  dash_status st = check_params(p, &s);
  if (st != DASH_OK) return st;
  if (n < 0 || !bytes) return DASH_ERR_INVALID_ARG;
  *bytes = dash::bwd_layout(s, n).total;
  return DASH_OK;
}

dash_status dash_prefill_backward(const dash_params* p, const void* q, const void* k,
                                  const void* v, const void* o, const void* d_o, int64_t n,
                                  const float* w_s, const float* summ, int64_t summ_blocks,
                                  const dash_route_buf* route, float* dq, float* dk, float* dv,
                                  float* dw_s, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  dash_status st = check_params(p, &s);
  if (st != DASH_OK) return st;
  if (n < 0 || !q || !k || !v || !o || !d_o || !w_s || !summ || !dq || !dk || !dv || !dw_s)
    return DASH_ERR_INVALID_ARG;
  if (!aligned16(q, k, v, o, d_o, w_s, summ, dq, dk, dv, dw_s)) return DASH_ERR_INVALID_ARG;
  if ((st = check_route_buf(route)) != DASH_OK) return st;
  if (summ_blocks < n / s.bs) return DASH_ERR_INVALID_ARG;
  if (n == 0) return DASH_OK;
  const dash::BwdLayout L = dash::bwd_layout(s, n);
  if (!ws || ((uintptr_t)ws % kAlign) != 0) return DASH_ERR_INVALID_ARG;
  if (ws_bytes < L.total) return DASH_ERR_WORKSPACE_TOO_SMALL;
  // the rows kernels address one (sequence, KV head)'s keys and values
  // through a 31-bit buffer range, as the attend kernel does
  if (!grid_ok(n * s.B * s.Hkv) || !grid_ok(((n + kQT - 1) / kQT) * s.B * s.H) ||
      !seq_bytes_ok(s, n))
    return DASH_ERR_UNSUPPORTED;
  return hip_status(dash::launch_prefill_backward(s, q, k, v, o, d_o, n, w_s, summ, summ_blocks,
                                                  *route, dq, dk, dv, dw_s, L, (char*)ws,
                                                  (hipStream_t)stream));
}

// Shared checks and launch of dash_decode / dash_decode_paged (block_table
// null: contiguous caches).
static dash_status decode_impl(const dash_params* p, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* cache_len, int64_t max_len,
                        const float* w_s, const float* q_bar, float* summ, int64_t summ_blocks,
                        void* o, const dash_route_buf* route, void* ws, size_t ws_bytes,
                        void* stream, const int32_t* block_table, int64_t max_blocks,
                        int64_t num_pages) {
  Shape s;
  dash_status st = check_params(p, &s);
  if (st != DASH_OK) return st;
  if (!q || !k_cache || !v_cache || !cache_len || !w_s || !summ || !o || max_len < 1)
    return DASH_ERR_INVALID_ARG;
  if (!aligned16(q, k_cache, v_cache, w_s, q_bar, summ, o)) return DASH_ERR_INVALID_ARG;
  if (summ_blocks < (max_len + s.bs - 1) / s.bs) return DASH_ERR_INVALID_ARG;
  if (route && check_route_buf(route) != DASH_OK) return DASH_ERR_INVALID_ARG;
  const dash::DecodeLayout L = dash::decode_layout(s, max_len);
  if (!ws || ((uintptr_t)ws % kAlign) != 0) return DASH_ERR_INVALID_ARG;
  if (ws_bytes < L.total) return DASH_ERR_WORKSPACE_TOO_SMALL;
  // contiguous caches address one (sequence, KV head) through a 31-bit range
  if ((int64_t)s.G * L.nb * 4 > 160 * 1024 || (!block_table && !seq_bytes_ok(s, max_len)))
    return DASH_ERR_UNSUPPORTED;
  if (!grid_ok(L.n_split) || (int64_t)s.B * s.Hkv > 65535) return DASH_ERR_UNSUPPORTED;
  if (s.dtype == DASH_BF16 && (int64_t)s.B * s.Hkv > dash::kDecodeMaxBg)
    return DASH_ERR_UNSUPPORTED;
  dash_route_buf rb = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  if (route) rb = *route;
  return hip_status(dash::launch_decode(s, q, k_cache, v_cache, cache_len, max_len, w_s, q_bar,
                                        summ, summ_blocks, o, rb, L, (char*)ws,
                                        (hipStream_t)stream, block_table, max_blocks,
                                        num_pages));
}

dash_status dash_decode(const dash_params* p, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* cache_len, int64_t max_len,
                        const float* w_s, const float* q_bar, float* summ, int64_t summ_blocks,
                        void* o, const dash_route_buf* route, void* ws, size_t ws_bytes,
                        void* stream) {
  return decode_impl(p, q, k_cache, v_cache, cache_len, max_len, w_s, q_bar, summ, summ_blocks,
                     o, route, ws, ws_bytes, stream, nullptr, 0, 0);
}

dash_status dash_decode_noalloc(const dash_params* p, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* cache_len, int64_t max_len,
                                const float* w_s, const float* q_bar, float* summ,
                                int64_t summ_blocks, void* o, const dash_route_buf* route,
                                void* stream) {
  Shape s;
  dash_status st = check_params(p, &s);
  if (st != DASH_OK) return st;
  if (max_len < 1) return DASH_ERR_INVALID_ARG;
  if (dash::decode_layout(s, max_len).total > kDecodeScratchBytes)
    return DASH_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (decode_scratch(&ws) != hipSuccess) return DASH_ERR_HIP;
  return decode_impl(p, q, k_cache, v_cache, cache_len, max_len, w_s, q_bar, summ, summ_blocks,
                     o, route, ws, kDecodeScratchBytes, stream, nullptr, 0, 0);
}

dash_status dash_decode_paged(const dash_params* p, const void* q, const void* k_pages,
                              const void* v_pages, int64_t num_pages, const int32_t* block_table,
                              int64_t max_blocks, const int32_t* cache_len, int64_t max_len,
                              const float* w_s, const float* q_bar, float* summ,
                              int64_t summ_blocks, void* o, const dash_route_buf* route,
                              void* ws, size_t ws_bytes, void* stream) {
  if (!p || !block_table || num_pages < 1 || max_len < 1 || p->block_size < 1)
    return DASH_ERR_INVALID_ARG;
  if (max_blocks < (max_len + p->block_size - 1) / p->block_size) return DASH_ERR_INVALID_ARG;
  return decode_impl(p, q, k_pages, v_pages, cache_len, max_len, w_s, q_bar, summ, summ_blocks,
                     o, route, ws, ws_bytes, stream, block_table, max_blocks, num_pages);
}

}  // extern "C"
