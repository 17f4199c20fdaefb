// Host-side checks of librlt's argument validation, sizing and error reporting, built with
// AddressSanitizer on the host code (the device code is compiled as usual and never launched).
// Everything here runs without a GPU: each call either returns a size or rejects its
// arguments before any HIP call, so an out-of-bounds access, use-after-free or leak in that
// host logic is what the sanitizer would report. Prints "abi_asan ok <checks>" and exits 0, or
// names the first failed check and exits 1.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>

#include "rlt.h"

namespace {

int g_checks = 0;
int g_failed = 0;

void expect(bool cond, const char* what, int line) {
  ++g_checks;
  if (!cond) {
    std::fprintf(stderr, "check failed (line %d): %s; last error: %s\n", line, what,
                 rlt_last_error());
    ++g_failed;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// The 140M-class decoder: d = 768, 12 heads of 64, 12 layers, FFN 3072, window 128, one
// memory group per layer, bf16.
rlt_config good() {
  rlt_config c{};
  c.d = 768;
  c.n_heads = 12;
  c.head_dim = 64;
  c.n_layers = 12;
  c.ffn = 3072;
  c.window = 128;
  c.n_groups = 12;
  c.dtype = RLT_BF16;
  c.alpha = 1.0f;
  c.eps = 1e-6f;
  c.version = 5;
  return c;
}

void config_validation() {
  rlt_config c = good();
  EXPECT(rlt_config_check(&c) == RLT_OK);
  EXPECT(rlt_config_check(nullptr) == RLT_ERR_ARG);
  struct Case {
    void (*edit)(rlt_config&);
    rlt_status want;
  };
  const Case cases[] = {
      {[](rlt_config& x) { x.dtype = 7; }, RLT_ERR_DTYPE},
      {[](rlt_config& x) { x.d = 0; }, RLT_ERR_SHAPE},
      {[](rlt_config& x) { x.d = -768; }, RLT_ERR_SHAPE},
      {[](rlt_config& x) { x.head_dim = 48; }, RLT_ERR_SHAPE},
      {[](rlt_config& x) { x.n_heads = 11; }, RLT_ERR_SHAPE},
      {[](rlt_config& x) { x.ffn = 100; }, RLT_ERR_SHAPE},
      {[](rlt_config& x) { x.window = 0; }, RLT_ERR_SHAPE},
      {[](rlt_config& x) { x.window = 2000; }, RLT_ERR_SHAPE},
      {[](rlt_config& x) { x.n_groups = 3; }, RLT_ERR_SHAPE},
      {[](rlt_config& x) { x.n_layers = 1 << 30; }, RLT_ERR_SHAPE},
      {[](rlt_config& x) { x.alpha = NAN; }, RLT_ERR_ARG},
      {[](rlt_config& x) { x.alpha = INFINITY; }, RLT_ERR_ARG},
      {[](rlt_config& x) { x.eps = -1.0f; }, RLT_ERR_ARG},
  };
  for (const Case& k : cases) {
    rlt_config x = good();
    k.edit(x);
    EXPECT(rlt_config_check(&x) == k.want);
    EXPECT(std::strlen(rlt_last_error()) > 0);
    EXPECT(rlt_model_ws_bytes(&x) == 0);
    EXPECT(rlt_state_bytes(&x, 4) == 0);
    EXPECT(rlt_memory_bytes(&x, 4, 16) == 0);
    EXPECT(rlt_parallel_ws_bytes(&x, 4, 16) == 0);
    EXPECT(rlt_bptt_ws_bytes(&x, 4, 16) == 0);
    EXPECT(rlt_head_ws_bytes(&x, 32768) == 0);
    EXPECT(rlt_encode_ws_bytes(&x, 4, 16) == 0);
    EXPECT(rlt_readout_ws_bytes(&x, 32768, 4) == 0);
  }
}

void sizes() {
  const rlt_config c = good();
  const size_t d = 768, L = 12, F = 3072, G = 12, H = 12, hd = 64, W = 128;
  const size_t weights =
      2 * (2 * d * d + L * (6 * d * d + 3 * d * F) + G * 2 * d * d + L * 4 * d * d + d * d);
  const size_t ws = rlt_model_ws_bytes(&c);
  EXPECT(ws >= weights && ws % 256 == 0);
  EXPECT(rlt_memory_bytes(&c, 256, 1024) == 2 * G * 256 * H * 1024 * hd * 2);
  EXPECT(rlt_memory_bytes(&c, 256, 0) == 0);
  EXPECT(rlt_memory_bytes(&c, 256, (int64_t(1) << 20) + 1) == 0);
  EXPECT(rlt_memory_bytes(&c, 0, 16) == 0);
  EXPECT(rlt_state_bytes(&c, 256) >= 2 * L * 256 * H * W * hd * 2);
  EXPECT(rlt_state_bytes(&c, 0) == 0);
  EXPECT(rlt_state_bytes(&c, -1) == 0);
  EXPECT(rlt_state_bytes(&c, (1 << 20) + 1) == 0);
  EXPECT(rlt_parallel_ws_bytes(&c, 16, 8192) >= size_t(16) * 8192 * (d * 4 + (5 * d + F) * 2));
  EXPECT(rlt_parallel_ws_bytes(&c, 16, 0) == 0);
  EXPECT(rlt_parallel_ws_bytes(&c, 0, 8) == 0);
  EXPECT(rlt_bptt_ws_bytes(&c, 4, 64) >= size_t(4) * 64 * L * d * (5 * 4 + 5 * 2));
  EXPECT(rlt_bptt_ws_bytes(&c, 4, 0) == 0);
  const int32_t V = 32768;
  EXPECT(rlt_head_ws_bytes(&c, V) >= size_t(2) * V * d * 2);
  for (int32_t bad : {0, -64, 100, 1000, (1 << 22) + 64}) EXPECT(rlt_head_ws_bytes(&c, bad) == 0);
  EXPECT(rlt_encode_ws_bytes(&c, 16, 1024) == rlt_parallel_ws_bytes(&c, 16, 1024));
  rlt_config f = good();
  f.dtype = RLT_F32;
  EXPECT(rlt_encode_ws_bytes(&f, 16, 1024) == 0);
  EXPECT(rlt_readout_ws_bytes(&c, V, 256) >= size_t(256) * V * 4);
  EXPECT(rlt_readout_ws_bytes(&c, V, 0) == 0);
  EXPECT(rlt_scratch_bytes() > 0 && rlt_scratch_bytes() % 256 == 0);
}

void null_arguments() {
  rlt_config c = good();
  void* out = nullptr;
  EXPECT(rlt_model_create(&c, nullptr, nullptr, 0, nullptr, (rlt_model**)&out) == RLT_ERR_ARG);
  EXPECT(out == nullptr);
  // Weights with one NULL pointer, then a workspace that is too small, then one misaligned:
  // each is rejected before the library reads a weight or touches the device.
  static char fake[1024];
  rlt_weights w;
  const void** slots = reinterpret_cast<const void**>(&w);
  for (size_t i = 0; i < sizeof(w) / sizeof(void*); ++i) slots[i] = fake;
  for (size_t i = 0; i < sizeof(w) / sizeof(void*); ++i) {
    rlt_weights v = w;
    reinterpret_cast<const void**>(&v)[i] = nullptr;
    EXPECT(rlt_model_create(&c, &v, fake, 1u << 30, nullptr, (rlt_model**)&out) == RLT_ERR_ARG);
  }
  EXPECT(rlt_model_create(&c, &w, fake, 1024, nullptr, (rlt_model**)&out) == RLT_ERR_CAPACITY);
  EXPECT(std::strstr(rlt_last_error(), "needs") != nullptr);
  alignas(256) static char aligned_buf[512];
  EXPECT(rlt_model_create(&c, &w, aligned_buf + 16, rlt_model_ws_bytes(&c), nullptr,
                          (rlt_model**)&out) == RLT_ERR_ARG);
  EXPECT(out == nullptr);

  EXPECT(rlt_state_create(nullptr, 4, nullptr, 0, nullptr, (rlt_state**)&out) == RLT_ERR_ARG);
  EXPECT(rlt_memory_create(nullptr, 4, 16, nullptr, 0, (rlt_memory**)&out) == RLT_ERR_ARG);
  EXPECT(rlt_memproj(nullptr, nullptr, nullptr, 0, 1, nullptr) == RLT_ERR_ARG);
  EXPECT(rlt_decoder_step(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == RLT_ERR_ARG);
  EXPECT(rlt_run_sequence(nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr) ==
         RLT_ERR_ARG);
  EXPECT(rlt_run_parallel(nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr, 0, nullptr) ==
         RLT_ERR_ARG);
  EXPECT(rlt_run_parallel_noalloc(nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr) ==
         RLT_ERR_ARG);
  EXPECT(rlt_bptt(nullptr, nullptr, 1, 1, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                  nullptr, nullptr, nullptr, nullptr) == RLT_ERR_ARG);
  EXPECT(rlt_state_export(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr) == RLT_ERR_ARG);
  EXPECT(rlt_state_import(nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr) == RLT_ERR_ARG);
  EXPECT(rlt_state_reset(nullptr, nullptr) == RLT_ERR_ARG);
  EXPECT(rlt_profile_clock(nullptr, nullptr, 0) == RLT_ERR_ARG);
  EXPECT(rlt_head_create(nullptr, 32768, nullptr, nullptr, 0, nullptr, (rlt_head**)&out) ==
         RLT_ERR_ARG);
  EXPECT(rlt_encode(nullptr, nullptr, nullptr, 1, 1, nullptr, nullptr, 0, nullptr) ==
         RLT_ERR_ARG);
  EXPECT(rlt_readout(nullptr, nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, 0, nullptr) == RLT_ERR_ARG);
  EXPECT(rlt_state_position(nullptr) == -1);
  EXPECT(rlt_memory_length(nullptr) == -1);
  EXPECT(std::strstr(rlt_last_error(), "NULL") != nullptr);
  // Destroying a NULL handle does nothing.
  rlt_model_destroy(nullptr);
  rlt_state_destroy(nullptr);
  rlt_memory_destroy(nullptr);
  rlt_head_destroy(nullptr);
}

void thread_local_errors() {
  rlt_config bad = good();
  bad.dtype = 9;
  EXPECT(rlt_config_check(&bad) == RLT_ERR_DTYPE);
  const std::string mine = rlt_last_error();
  std::string other = "unset";
  std::thread th([&] {
    other = rlt_last_error();  // a fresh thread has no error
    rlt_config c = good();
    c.window = 0;
    rlt_config_check(&c);
  });
  th.join();
  EXPECT(other.empty());
  EXPECT(mine == rlt_last_error());  // the other thread's failure did not overwrite it
  EXPECT(rlt_config_check(nullptr) == RLT_ERR_ARG);
  rlt_config ok = good();
  EXPECT(rlt_config_check(&ok) == RLT_OK);
}

}  // namespace

int main() {
  config_validation();
  sizes();
  null_arguments();
  thread_local_errors();
  if (g_failed) {
    std::fprintf(stderr, "abi_asan: %d of %d checks failed\n", g_failed, g_checks);
    return 1;
  }
  std::printf("abi_asan ok %d\n", g_checks);
  return 0;
}
