// Concurrent host-side calls of the C ABI for a ThreadSanitizer build: every
// thread makes its own invalid call (rejected before any HIP call) many
// times and checks that its thread-local error message names its own
// argument.  Exit status 0 = no mix-up between threads.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "attn_prefill.h"

int main() {
  const int n_threads = 8, iters = 4000;
  std::vector<int> bad(n_threads, 0);
  std::vector<std::thread> pool;
  for (int t = 0; t < n_threads; ++t)
    pool.emplace_back([t, iters, &bad] {
      static char dummy[64];
      static int32_t offsets[2] = {0, 4};
      attn_tensor q = {dummy, ATTN_BF16, 0, 4, 4 * 128, 128};
      attn_tensor o = q;
      attn_seqlens cu = {offsets, 1, 0};
      const int32_t window = -(t + 1000);  // this thread's own invalid window
      char want[32];
      std::snprintf(want, sizeof(want), "%d", (int)window);
      int32_t dims[8];
      for (int i = 0; i < iters; ++i) {
        const int rc = attn_prefill(&q, &q, &q, &o, &cu, 1, 1, 128, 0.1f, window, nullptr);
        const std::string msg = attn_prefill_last_error();
        if (rc != ATTN_ERR_INVALID_ARG || msg.find(want) == std::string::npos) ++bad[t];
        if (attn_prefill_supported_head_dims(dims, 8) < 1) ++bad[t];
        if (std::strlen(attn_prefill_status_string(rc)) == 0) ++bad[t];
      }
    });
  for (auto& th : pool) th.join();
  int total = 0;
  for (int b : bad) total += b;
  std::printf("%s: %d mismatch(es)\n", total ? "FAILED" : "ok", total);
  return total ? 1 : 0;
}
