// Host-side checks of the C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host pass (test_host_sanitized.py builds it with the library's sources and runs it
// on the CPU; no kernel is launched).  It exercises every entry point whose work is host code: un-delay, the
// streaming hand-off with its stop guard, the workspace size rules, context creation where
// no usable device exists, and the argument checks of every call that takes a context.
// Output buffers are sized exactly as include/hta.h documents, so a write past them is
// reported by the sanitizer.  Exit status 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "hta.h"

static int failures = 0;
#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                            \
    }                                                                        \
  } while (0)

static hta_config qwen3_4b(int n_streams) {
  hta_config c{};
  c.n_layers = 36;
  c.hidden = 2560;
  c.n_q_heads = 32;
  c.n_kv_heads = 8;
  c.head_dim = 128;
  c.ffn = 9728;
  c.text_vocab = 151936;
  c.n_codebooks = 8;
  c.codebook_size = 1026;
  c.bos_id = 1024;
  c.eos_id = 1025;
  c.rope_theta = 1e6f;
  c.rms_eps = 1e-6f;
  c.max_seq = 4096;
  c.max_prefill = 512;
  c.precision = HTA_FP8_E4M3;
  c.n_streams = n_streams;
  return c;
}

// Delayed step codes of one utterance: codebook k holds BOS for t < k, EOS from step e + k on
// when codebook 0 emits EOS at step e (e < 0: never), random codes elsewhere.
static std::vector<int32_t> steps_of(std::mt19937& rng, int T, int C, int e) {
  std::vector<int32_t> s((size_t)T * C);
  for (int t = 0; t < T; ++t)
    for (int k = 0; k < C; ++k) {
      int32_t v = (int32_t)(rng() % 1024);
      if (t < k) v = 1024;
      else if (e >= 0 && t >= e + k) v = 1025;
      s[(size_t)t * C + k] = v;
    }
  return s;
}

static void check_undelay_and_stream(std::mt19937& rng) {
  for (int trial = 0; trial < 200; ++trial) {
    const int C = 1 + (int)(rng() % 16);
    const int T = (int)(rng() % 300);
    const int e = (trial % 3 == 0 || T == 0) ? -1 : (int)(rng() % (unsigned)T);
    const std::vector<int32_t> steps = steps_of(rng, T, C, e);
    std::vector<int32_t> frames((size_t)T * C + (T == 0 ? 1 : 0));
    int n = -1;
    const int rc = hta_undelay(T ? steps.data() : frames.data(), T, C, 1025, frames.data(), &n);
    CHECK(rc == HTA_OK);
    CHECK(n >= 0 && n <= T);
    // the same steps pushed through a stream in random pieces, read out in small buffers
    const int chunk = 1 + (int)(rng() % 40);
    const int window = trial % 4 == 0 ? 0 : 2 + (int)(rng() % 60);
    hta_stream* s = nullptr;
    CHECK(hta_stream_create(C, 1024, 1025, chunk, window, 1 + (int)(rng() % 6), &s) == HTA_OK);
    if (!s) continue;
    std::vector<int32_t> got;
    int status = HTA_STREAM_RUNNING;
    for (int t = 0; t < T;) {
      const int piece = 1 + (int)(rng() % 25);
      const int np = piece < T - t ? piece : T - t;
      const int cap = (int)(rng() % 50);
      std::vector<int32_t> out((size_t)cap * C + (cap == 0 ? 1 : 0));
      int nf = -1;
      CHECK(hta_stream_push(s, steps.data() + (size_t)t * C, np, out.data(), cap, &nf, &status) == HTA_OK);
      CHECK(nf >= 0 && nf <= cap);
      got.insert(got.end(), out.begin(), out.begin() + (size_t)nf * C);
      t += np;
    }
    for (int guard = 0; guard < 1000; ++guard) {  // drain, then end the utterance
      const int cap = 1 + (int)(rng() % 50);
      std::vector<int32_t> out((size_t)cap * C);
      int nf = -1;
      CHECK(hta_stream_finish(s, out.data(), cap, &nf) == HTA_OK);
      CHECK(nf >= 0 && nf <= cap);
      got.insert(got.end(), out.begin(), out.begin() + (size_t)nf * C);
      if (nf == 0) break;
    }
    // without the guard the streamed frames are the one-shot un-delay; with it, a prefix
    const size_t ng = got.size() / (size_t)C;
    if (window == 0) CHECK(ng == (size_t)n);
    CHECK(ng <= (size_t)n);
    CHECK(got.empty() || std::memcmp(got.data(), frames.data(), got.size() * sizeof(int32_t)) == 0);
    // pushes after the end are ignored
    int nf = -1;
    int32_t one[16] = {0};
    std::vector<int32_t> out((size_t)4 * C);
    CHECK(hta_stream_push(s, one, 1, out.data(), 4, &nf, nullptr) == HTA_OK);
    hta_stream_destroy(s);
  }
  // argument errors
  hta_stream* s = nullptr;
  CHECK(hta_stream_create(0, 1024, 1025, 4, 0, 1, &s) == HTA_E_ARG);
  CHECK(hta_stream_create(65, 1024, 1025, 4, 0, 1, &s) == HTA_E_ARG);
  CHECK(hta_stream_create(8, 1024, 1025, 0, 0, 1, &s) == HTA_E_ARG);
  CHECK(hta_stream_create(8, 1024, 1025, 4, -1, 1, &s) == HTA_E_ARG);
  CHECK(hta_stream_create(8, 1024, 1025, 4, 0, 1, nullptr) == HTA_E_ARG);
  hta_stream_destroy(nullptr);
  int n = 0;
  int32_t buf[8];
  CHECK(hta_undelay(nullptr, 1, 8, 1025, buf, &n) == HTA_E_ARG);
  CHECK(hta_undelay(buf, 1, 0, 1025, buf, &n) == HTA_E_ARG);
  CHECK(hta_undelay(buf, -1, 8, 1025, buf, &n) == HTA_E_ARG);
}

static void check_workspace_rules() {
  const hta_config base = qwen3_4b(1);
  const size_t one = hta_workspace_bytes(&base);
  CHECK(one > 0);
  for (int m : {2, 16, 128}) {
    const hta_config c = qwen3_4b(m);
    CHECK(hta_workspace_bytes(&c) > one);
  }
  hta_config c = qwen3_4b(129);
  CHECK(hta_workspace_bytes(&c) == 0);
  CHECK(hta_workspace_bytes(nullptr) == 0);
  // shapes the kernels do not take, and sizes whose products do not fit
  const struct { int field; int value; } bad[] = {
      {0, 0}, {1, 100}, {2, 3}, {3, 3}, {4, 96}, {5, 100}, {6, 0}, {7, 17}, {8, 5000},
      {9, 0}, {10, 0}, {11, 1 << 30}, {12, 1 << 30}, {13, 7}, {14, -1}};
  for (const auto& b : bad) {
    hta_config x = qwen3_4b(1);
    switch (b.field) {
      case 0: x.n_layers = b.value; break;
      case 1: x.hidden = b.value; break;
      case 2: x.n_q_heads = b.value; break;
      case 3: x.n_kv_heads = b.value; break;
      case 4: x.head_dim = b.value; break;
      case 5: x.ffn = b.value; break;
      case 6: x.text_vocab = b.value; break;
      case 7: x.n_codebooks = b.value; break;
      case 8: x.codebook_size = b.value; break;
      case 9: x.max_seq = b.value; break;
      case 10: x.max_prefill = b.value; break;
      case 11: x.max_seq = b.value; x.max_prefill = 512; break;
      case 12: x.text_vocab = b.value; break;
      case 13: x.precision = b.value; break;
      case 14: x.n_streams = b.value; break;
    }
    (void)hta_workspace_bytes(&x);  // any answer; the sanitizers watch the arithmetic
  }
}

static void check_null_context() {
  int32_t codes[64] = {0};
  int n = 0;
  float f[8] = {0};
  const void* tensors[1] = {nullptr};
  CHECK(hta_bind_workspace(nullptr, nullptr, 0) == HTA_E_ARG);
  CHECK(hta_load_weights(nullptr, tensors, 1, HTA_SRC_BF16, nullptr) == HTA_E_ARG);
  CHECK(hta_prefill(nullptr, codes, 1) == HTA_E_ARG);
  CHECK(hta_decode_frame(nullptr, codes) == HTA_E_ARG);
  CHECK(hta_decode_frames(nullptr, 1, codes, &n) == HTA_E_ARG);
  CHECK(hta_decode_frames_noalloc(nullptr, 1, codes, &n) == HTA_E_ARG);
  CHECK(hta_set_sampling(nullptr, 1.0f, 1) == HTA_E_ARG);
  CHECK(hta_reset(nullptr, 0) == HTA_E_ARG);
  CHECK(hta_select_stream(nullptr, 0) == HTA_E_ARG);
  CHECK(hta_force_codes(nullptr, codes) == HTA_E_ARG);
  CHECK(hta_read_tap(nullptr, HTA_TAP_STATE, 0, codes, sizeof(codes)) == HTA_E_ARG);
  CHECK(hta_calibrate(nullptr, codes, 1, 1, nullptr, f) == HTA_E_ARG);
  CHECK(hta_layer_step(nullptr, 0, 1, nullptr, nullptr, nullptr) == HTA_E_ARG);
  CHECK(hta_gemm(nullptr, codes, codes, f, 1.0f, 1, 64, 128, f) == HTA_E_ARG);
  CHECK(hta_time_kernels(nullptr, 1, f, 8) == HTA_E_ARG);
  CHECK(hta_set_option(nullptr, HTA_OPT_USE_GRAPH, 1) == HTA_E_ARG);
  hta_destroy(nullptr);
  CHECK(hta_last_error(nullptr) != nullptr);
  CHECK(hta_version() != nullptr && std::strlen(hta_version()) > 0);
}

// Where no usable device exists, hta_create fails with an error code and leaves *out null.
static void check_create_without_device() {
  const hta_config c = qwen3_4b(1);
  hta_ctx* ctx = reinterpret_cast<hta_ctx*>(&failures);  // overwritten on every path
  const int rc = hta_create(&c, nullptr, &ctx);
  CHECK(rc != HTA_OK);
  CHECK(ctx == nullptr);
  CHECK(hta_create(nullptr, nullptr, &ctx) == HTA_E_ARG);
  CHECK(hta_create(&c, nullptr, nullptr) == HTA_E_ARG);
}

int main(int argc, char** argv) {
  std::mt19937 rng(20261203u);
  check_undelay_and_stream(rng);
  check_workspace_rules();
  check_null_context();
  if (argc > 1 && std::strcmp(argv[1], "--no-device") == 0) check_create_without_device();
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host ABI checks passed\n");
  return 0;
}
