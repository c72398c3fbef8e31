// Host-side driver of the C ABI for the sanitizer build (no GPU needed).
//
// Linked with the host code of the library compiled under AddressSanitizer
// and UndefinedBehaviorSanitizer (no device code).  Reads dualar_config
// records from the file argv[1] and, for each, prints one line with what the
// host-side validation returns: the workspace size, dualar_create with NULL
// weights, dualar_create with placeholder weight pointers (16-byte aligned,
// never dereferenced: creation stops at validation or at the device lookup)
// held in layer arrays of exactly the configured lengths, dualar_create_static
// with the same weights, and the last error message.  Then every entry point
// with a NULL context, and every status string.  The test that runs it
// compares the lines with the same calls made on the normal library.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "dualar.h"

namespace {

const void* fake(size_t k) { return (const void*)(uintptr_t)(4096 + 16 * k); }

void fill_layers(std::vector<dualar_layer_weights>& v) {
  size_t k = 0;
  for (auto& l : v) {
    l.attention_norm = fake(k++); l.wq = fake(k++); l.wk = fake(k++); l.wv = fake(k++);
    l.q_norm = fake(k++); l.k_norm = fake(k++); l.wo = fake(k++); l.ffn_norm = fake(k++);
    l.w1 = fake(k++); l.w3 = fake(k++); l.w2 = fake(k++);
  }
}

void one_config(const dualar_config& cfg) {
  const size_t ws = dualar_workspace_bytes(&cfg);
  dualar_ctx_t* h = nullptr;
  const int st_null = dualar_create(&cfg, nullptr, (void*)(uintptr_t)256, ws ? ws : ((size_t)1 << 40), nullptr, &h);
  // the layer arrays hold exactly the configured numbers of entries (a
  // negative or huge count is left at zero entries), so the sanitizer sees
  // any read past them
  const int n = cfg.n_layer >= 0 && cfg.n_layer <= 4096 ? cfg.n_layer : 0;
  const int fn_cfg = cfg.n_fast_layer;
  const int fn = fn_cfg >= 0 && fn_cfg <= 4096 ? fn_cfg : 0;
  std::vector<dualar_layer_weights> slow(n), fast(fn);
  fill_layers(slow);
  fill_layers(fast);
  dualar_weights w{};
  w.tok_embedding = fake(100000); w.codebook_embedding = fake(100001); w.norm = fake(100002);
  w.layers = slow.empty() ? nullptr : slow.data();
  w.fast_layers = fast.empty() ? nullptr : fast.data();
  w.fast_embeddings = fake(100003); w.fast_norm = fake(100004); w.fast_output = fake(100005);
  const int st_fake = dualar_create(&cfg, &w, (void*)(uintptr_t)256, ws ? ws : ((size_t)1 << 40), nullptr, &h);
  const char* e1 = dualar_last_error(nullptr);
  std::string err1 = e1 ? e1 : "(null)";
  const int st_static = dualar_create_static(&cfg, &w, nullptr, &h);
  const char* e2 = dualar_last_error(nullptr);
  printf("ws=%zu null=%d fake=%d static=%d handle=%d err=%s | %s\n", ws, st_null, st_fake, st_static, h != nullptr,
         err1.c_str(), e2 ? e2 : "(null)");
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s <config records>\n", argv[0]);
    return 2;
  }
  // the placeholder weights must never reach a device
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    fprintf(stderr, "a GPU is visible: this driver runs only without one\n");
    return 3;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) {
    perror(argv[1]);
    return 2;
  }
  dualar_config cfg;
  int records = 0;
  while (fread(&cfg, sizeof cfg, 1, f) == 1) {
    one_config(cfg);
    ++records;
  }
  fclose(f);
  dualar_sampling s{1.0f, 1.0f, 1, 0, 0, 1.0f, 0.9f};
  int32_t ids[1] = {0};
  int64_t launches = 0;
  double ms = 0, bytes = 0;
  printf("null-ctx prefill=%d decode=%d fast=%d fast_tf=%d sync=%d reset=%d reset0=%d prof_begin=%d prof_end=%d\n",
         dualar_prefill(nullptr, 1, nullptr, 1, nullptr, &s, nullptr, nullptr, nullptr),
         dualar_decode_frames(nullptr, 1, &s, nullptr, nullptr, nullptr, nullptr),
         dualar_fast_frames(nullptr, 1, 1, nullptr, nullptr, &s, nullptr, nullptr, nullptr),
         dualar_fast_teacher_forced(nullptr, 1, nullptr, nullptr, nullptr), dualar_sync(nullptr, nullptr),
         dualar_reset(nullptr, ids, 1), dualar_reset(nullptr, nullptr, 0), dualar_profile_begin(nullptr, 0),
         dualar_profile_end(nullptr, &launches, &ms, &bytes));
  dualar_destroy(nullptr);
  for (int code = -10; code <= 1; ++code) printf("status %d %s\n", code, dualar_status_string((dualar_status)code));
  printf("records %d\n", records);
  return 0;
}
