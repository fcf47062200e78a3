// abi_driver.cpp -- host-side argument checks of the C ABI (include/dash.h)
// under AddressSanitizer and UndefinedBehaviorSanitizer: every entry point
// is called with arguments it must reject (null or misaligned pointers,
// negative or inconsistent sizes, unsupported shapes, workspaces too small)
// and the sizing helpers with valid and invalid shapes.  No call reaches a
// kernel launch or dereferences a device pointer, so no GPU is needed.
// Exits 0 when every status matches; the sanitizers abort on any error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "dash.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

// never dereferenced: every call below fails its checks first
void* const FAKE = reinterpret_cast<void*>(0x100000);
float* const FF = reinterpret_cast<float*>(0x100000);
int32_t* const FI = reinterpret_cast<int32_t*>(0x100000);

dash_params params(int batch = 1, int heads = 32, int kv_heads = 8, int d = 128, int bs = 64) {
  dash_params p;
  std::memset(&p, 0, sizeof(p));
  p.batch = batch;
  p.n_heads = heads;
  p.n_kv_heads = kv_heads;
  p.head_dim = d;
  p.block_size = bs;
  p.alpha = 1.5f;
  p.gamma = 2.0f;
  p.dtype = DASH_BF16;
  p.sigma = 1.0f;
  p.window = 1;
  return p;
}

void sizing() {
  dash_params p = params();
  dash_route_sizes s;
  expect(dash_route_sizes_prefill(&p, 8192, &s) == DASH_OK && s.n_qt == 128 && s.nb == 128,
         "prefill sizes");
  expect(s.sel_logp == 8LL * 128 * 128 * 64 && s.tau == 32LL * 8192, "prefill size counts");
  expect(dash_route_sizes_prefill(nullptr, 8192, &s) == DASH_ERR_INVALID_ARG, "null params");
  expect(dash_route_sizes_prefill(&p, 8192, nullptr) == DASH_ERR_INVALID_ARG, "null sizes");
  expect(dash_route_sizes_prefill(&p, -1, &s) == DASH_ERR_INVALID_ARG, "negative n");
  dash_params pd = params(32);
  expect(dash_route_sizes_decode(&pd, 32768, &s) == DASH_OK && s.nb == 512 && s.qt == 1,
         "decode sizes");
  expect(dash_route_sizes_decode(&pd, 0, &s) == DASH_ERR_INVALID_ARG, "decode max_len 0");
  size_t bytes = 0;
  expect(dash_prefill_workspace_bytes(&p, 8192, &bytes) == DASH_OK && bytes % 256 == 0,
         "prefill workspace");
  expect(dash_decode_workspace_bytes(&pd, 32768, &bytes) == DASH_OK && bytes > 0,
         "decode workspace");
  expect(dash_prefill_backward_workspace_bytes(&p, 8192, &bytes) == DASH_OK && bytes > 0,
         "backward workspace");
  expect(dash_prefill_workspace_bytes(&p, 8192, nullptr) == DASH_ERR_INVALID_ARG,
         "null workspace out");
}

void bad_params() {
  struct Case {
    dash_params p;
    dash_status code;
    const char* what;
  } cases[14];
  int n = 0;
  auto add = [&](dash_params p, dash_status c, const char* w) { cases[n++] = {p, c, w}; };
  dash_params p = params();
  p.n_heads = 30; add(p, DASH_ERR_INVALID_ARG, "H % Hkv");
  p = params(); p.alpha = 1.0f; add(p, DASH_ERR_INVALID_ARG, "alpha 1");
  p = params(); p.alpha = 2.5f; add(p, DASH_ERR_INVALID_ARG, "alpha 2.5");
  p = params(); p.alpha = std::nanf(""); add(p, DASH_ERR_INVALID_ARG, "alpha NaN");
  p = params(); p.gamma = 0.0f; add(p, DASH_ERR_INVALID_ARG, "gamma 0");
  p = params(); p.gamma = INFINITY; add(p, DASH_ERR_INVALID_ARG, "gamma inf");
  p = params(); p.dtype = 7; add(p, DASH_ERR_INVALID_ARG, "dtype");
  p = params(0); add(p, DASH_ERR_INVALID_ARG, "batch 0");
  p = params(1, 32, 8, 96); add(p, DASH_ERR_UNSUPPORTED, "head_dim 96");
  p = params(1, 32, 8, 128, 32); add(p, DASH_ERR_UNSUPPORTED, "block 32");
  p = params(1, 48, 4); add(p, DASH_ERR_UNSUPPORTED, "G 12");
  p = params(); p.sigma = -0.5f; add(p, DASH_ERR_INVALID_ARG, "sigma < 0");
  p = params(); p.sigma = std::nanf(""); add(p, DASH_ERR_INVALID_ARG, "sigma NaN");
  p = params(); p.window = 0; add(p, DASH_ERR_INVALID_ARG, "window 0");
  for (int i = 0; i < n; ++i) {
    size_t bytes = 0;
    dash_route_sizes s;
    const dash_params& c = cases[i].p;
    expect(dash_prefill_workspace_bytes(&c, 1024, &bytes) == cases[i].code, cases[i].what);
    expect(dash_route_sizes_prefill(&c, 1024, &s) == cases[i].code, cases[i].what);
    expect(dash_decode_workspace_bytes(&c, 1024, &bytes) == cases[i].code, cases[i].what);
    expect(dash_prefill(&c, FAKE, FAKE, FAKE, 1024, FF, nullptr, FF, 16, FAKE, FAKE, 1ull << 40,
                        nullptr) == cases[i].code,
           cases[i].what);
  }
}

void bad_calls() {
  dash_params p = params();
  size_t need = 0;
  dash_prefill_workspace_bytes(&p, 1024, &need);
  expect(dash_prefill(&p, nullptr, FAKE, FAKE, 1024, FF, nullptr, FF, 16, FAKE, FAKE, need,
                      nullptr) == DASH_ERR_INVALID_ARG, "prefill null q");
  expect(dash_prefill(&p, FAKE, FAKE, FAKE, 1024, FF, nullptr, FF, 15, FAKE, FAKE, need,
                      nullptr) == DASH_ERR_INVALID_ARG, "prefill summary capacity");
  expect(dash_prefill(&p, FAKE, FAKE, FAKE, 1024, FF, nullptr, FF, 16, FAKE, FAKE, need - 1,
                      nullptr) == DASH_ERR_WORKSPACE_TOO_SMALL, "prefill workspace size");
  expect(dash_prefill(&p, static_cast<char*>(FAKE) + 4, FAKE, FAKE, 1024, FF, nullptr, FF, 16,
                      FAKE, FAKE, need, nullptr) == DASH_ERR_INVALID_ARG, "prefill alignment");
  expect(dash_prefill(&p, FAKE, FAKE, FAKE, 0, FF, nullptr, FF, 0, FAKE, FAKE, 0, nullptr) ==
             DASH_OK, "empty prefill");
  expect(dash_prefill_varlen(&p, FAKE, FAKE, FAKE, 1024, nullptr, FF, nullptr, FF, 16, FAKE, FAKE,
                             need, nullptr) == DASH_ERR_INVALID_ARG, "varlen without lengths");
  expect(dash_summarize(&p, FAKE, 1000, 0, 16, FF, nullptr, FF, 16, nullptr) ==
             DASH_ERR_INVALID_ARG, "summarize past the keys");
  expect(dash_summarize(&p, FAKE, 1024, 0, 16, FF, nullptr, FF, 15, nullptr) ==
             DASH_ERR_INVALID_ARG, "summarize past the capacity");
  dash_route_buf rb = {FF, FI, nullptr, FF, nullptr, nullptr};
  expect(dash_route(&p, FAKE, 1024, FF, 16, &rb, nullptr) == DASH_ERR_INVALID_ARG,
         "route without sel_idx");
  expect(dash_route(&p, FAKE, 1024, FF, 16, nullptr, nullptr) == DASH_ERR_INVALID_ARG,
         "route without buffers");
  expect(dash_attend(&p, FAKE, FAKE, FAKE, 1024, nullptr, FAKE, nullptr) == DASH_ERR_INVALID_ARG,
         "attend without buffers");
  dash_route_buf no_bits = {FF, FI, FI, FF, nullptr, nullptr};
  expect(dash_mask_to_list(&p, 1024, &no_bits, nullptr) == DASH_ERR_INVALID_ARG,
         "mask_to_list without a mask");
  expect(dash_mask_to_list(&p, -1, &no_bits, nullptr) == DASH_ERR_INVALID_ARG,
         "mask_to_list negative n");
  size_t bneed = 0;
  dash_prefill_backward_workspace_bytes(&p, 1024, &bneed);
  dash_route_buf full = {FF, FI, FI, FF, nullptr, nullptr};
  expect(dash_prefill_backward(&p, FAKE, FAKE, FAKE, FAKE, FAKE, 1024, FF, FF, 16, &full, FF, FF,
                               FF, FF, FAKE, bneed - 1, nullptr) == DASH_ERR_WORKSPACE_TOO_SMALL,
         "backward workspace size");
  expect(dash_prefill_backward(&p, nullptr, FAKE, FAKE, FAKE, FAKE, 1024, FF, FF, 16, &full, FF,
                               FF, FF, FF, FAKE, bneed, nullptr) == DASH_ERR_INVALID_ARG,
         "backward null q");

  size_t dneed = 0;
  dash_decode_workspace_bytes(&p, 4096, &dneed);
  expect(dash_decode(&p, FAKE, FAKE, FAKE, FI, 0, FF, nullptr, FF, 64, FAKE, nullptr, FAKE, dneed,
                     nullptr) == DASH_ERR_INVALID_ARG, "decode max_len 0");
  expect(dash_decode(&p, FAKE, FAKE, FAKE, FI, 4096, FF, nullptr, FF, 63, FAKE, nullptr, FAKE,
                     dneed, nullptr) == DASH_ERR_INVALID_ARG, "decode summary capacity");
  expect(dash_decode(&p, FAKE, FAKE, FAKE, FI, 4096, FF, nullptr, FF, 64, FAKE, nullptr, FAKE,
                     dneed - 1, nullptr) == DASH_ERR_WORKSPACE_TOO_SMALL, "decode workspace");
  expect(dash_decode_paged(&p, FAKE, FAKE, FAKE, 64, nullptr, 64, FI, 4096, FF, nullptr, FF, 64,
                           FAKE, nullptr, FAKE, dneed, nullptr) == DASH_ERR_INVALID_ARG,
         "paged decode without a table");
  expect(dash_decode_paged(&p, FAKE, FAKE, FAKE, 64, FI, 63, FI, 4096, FF, nullptr, FF, 64, FAKE,
                           nullptr, FAKE, dneed, nullptr) == DASH_ERR_INVALID_ARG,
         "paged decode narrow table");
  dash_params big = params(64, 64, 8);
  expect(dash_decode_noalloc(&big, FAKE, FAKE, FAKE, FI, 131072, FF, nullptr, FF, 2048, FAKE,
                             nullptr, nullptr) == DASH_ERR_WORKSPACE_TOO_SMALL,
         "allocation-free decode above its scratch");

  expect(dash_peak_stream(FAKE, FAKE, 15, 0, nullptr) == DASH_ERR_INVALID_ARG, "stream size");
  expect(dash_peak_stream(FAKE, FAKE, 1024, 3, nullptr) == DASH_ERR_INVALID_ARG, "stream mode");
  expect(dash_peak_stream(FAKE, FAKE, 1024, -1, nullptr) == DASH_ERR_INVALID_ARG, "stream mode");
  expect(dash_peak_stream_grid(nullptr) == DASH_ERR_INVALID_ARG, "stream grid out");
  double flops = 0.0;
  expect(dash_peak_mfma(0, FF, &flops, nullptr) == DASH_ERR_INVALID_ARG, "mfma iterations");
  expect(dash_peak_mfma(1, nullptr, &flops, nullptr) == DASH_ERR_INVALID_ARG, "mfma sink");
}

}  // namespace

int main() {
  expect(std::strstr(dash_version(), "gfx950") != nullptr, "version");
  for (int c = 0; c < 5; ++c)
    expect(std::strncmp(dash_status_string(static_cast<dash_status>(c)), "DASH_", 5) == 0,
           "status string");
  sizing();
  bad_params();
  bad_calls();
  if (failures) return 1;
  std::printf("abi driver: ok\n");
  return 0;
}
