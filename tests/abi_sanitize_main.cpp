// Host-side C ABI checks for an AddressSanitizer / UndefinedBehaviorSanitizer
// build of the library (host code instrumented, device code as usual).  Every
// call made here is rejected on the host or is an empty batch, so nothing is
// launched and no GPU is needed.  Exit status 0 = every expectation held.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "attn_prefill.h"

static int g_failures = 0;

static void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAIL: %s (last error: %s)\n", what, attn_prefill_last_error());
    ++g_failures;
  }
}

// A descriptor whose data pointer is never dereferenced by the checks.
static attn_tensor tensor(int64_t n_tokens, int64_t heads, int64_t d, int32_t dtype) {
  static char dummy[64];
  attn_tensor t;
  std::memset(&t, 0, sizeof(t));
  t.data = dummy;
  t.dtype = dtype;
  t.n_tokens = n_tokens;
  t.token_stride = heads * d;
  t.head_stride = d;
  return t;
}

int main() {
  const float scale = 0.08838834764831843f;
  static int32_t offsets[4] = {0, 5, 9, 12};
  attn_seqlens cu = {offsets, 3, 0};
  attn_tensor q = tensor(12, 8, 128, ATTN_BF16), k = tensor(12, 2, 128, ATTN_BF16),
              v = tensor(12, 2, 128, ATTN_BF16), o = tensor(12, 8, 128, ATTN_BF16);

  // helpers
  for (int s = -3; s < 8; ++s) expect(attn_prefill_status_string(s) != nullptr, "status string");
  expect(attn_prefill_last_error() != nullptr, "last error");
  int32_t dims[16];
  const int n = attn_prefill_supported_head_dims(dims, 16);
  expect(n > 0 && n <= 16, "head dims count");
  expect(attn_prefill_supported_head_dims(dims, 0) == n, "head dims with cap 0");
  expect(attn_prefill_supported_head_dims(nullptr, 0) == n, "head dims without a buffer");
  expect(attn_prefill_version() > 0, "version");

  // null descriptors and offsets
  expect(attn_prefill(nullptr, &k, &v, &o, &cu, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "null q");
  expect(attn_prefill(&q, &k, &v, &o, nullptr, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "null offsets");
  attn_seqlens cu_null = {nullptr, 3, 0};
  expect(attn_prefill(&q, &k, &v, &o, &cu_null, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "null offset data");
  // arguments outside the contract
  expect(attn_prefill(&q, &k, &v, &o, &cu, 8, 3, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "heads not a multiple of kv heads");
  expect(attn_prefill(&q, &k, &v, &o, &cu, 8, 2, 128, scale, -1, nullptr) ==
             ATTN_ERR_INVALID_ARG, "negative window");
  expect(attn_prefill(&q, &k, &v, &o, &cu, 8, 2, 128, std::nanf(""), 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "NaN scale");
  expect(attn_prefill(&q, &k, &v, &o, &cu, 8, 2, 128,
                      std::numeric_limits<float>::infinity(), 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "infinite scale");
  expect(attn_prefill(&q, &k, &v, &o, &cu, 8, 2, 96, scale, 0, nullptr) != ATTN_OK,
         "head dim without a kernel");
  expect(attn_prefill(&q, &k, &v, &o, &cu, INT32_MAX, 1, 128, scale, 0, nullptr) != ATTN_OK,
         "huge head count");
  attn_tensor q_short = q;
  q_short.token_stride = 8 * 128 - 1;
  expect(attn_prefill(&q_short, &k, &v, &o, &cu, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "token stride too small");
  attn_tensor q_big = q;
  q_big.token_stride = INT64_MAX / 2;
  expect(attn_prefill(&q_big, &k, &v, &o, &cu, 8, 2, 128, scale, 0, nullptr) != ATTN_OK,
         "token stride past the address range");
  attn_tensor k_tok = k;
  k_tok.n_tokens = 11;
  expect(attn_prefill(&q, &k_tok, &v, &o, &cu, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "token counts differ");
  attn_tensor o_fp32 = o;
  o_fp32.dtype = ATTN_FP32;
  expect(attn_prefill(&q, &k, &v, &o_fp32, &cu, 8, 2, 128, scale, 0, nullptr) != ATTN_OK,
         "fp32 output");
  attn_tensor k_fp32 = k;
  k_fp32.dtype = ATTN_FP32;
  expect(attn_prefill(&q, &k_fp32, &v, &o, &cu, 8, 2, 128, scale, 0, nullptr) != ATTN_OK,
         "fp32 keys");
  attn_tensor q_res = q;
  q_res.reserved = 1;
  expect(attn_prefill(&q_res, &k, &v, &o, &cu, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "reserved field set");
  attn_seqlens cu_zero = {offsets, 0, 0};
  expect(attn_prefill(&q, &k, &v, &o, &cu_zero, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "no sequences");
  expect(attn_prefill(&q, &k, &v, &q, &cu, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "output aliases q");

  // chunked, paged and the general entry point
  expect(attn_prefill_chunked(&q, &k, &v, &o, &cu, nullptr, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "chunked without key offsets");
  expect(attn_prefill_paged(&q, &k, &v, &o, &cu, nullptr, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "paged without a table");
  static int32_t table[6] = {0, 1, 0, 1, 0, 1};
  static int32_t klen[3] = {5, 4, 3};
  attn_paged_kv paged = {table, klen, 2, 48};
  expect(attn_prefill_paged(&q, &k, &v, &o, &cu, &paged, 8, 2, 128, scale, 0, nullptr) != ATTN_OK,
         "page size not a multiple of the key tile");
  paged.page_size = 64;
  paged.table_stride = 0;
  expect(attn_prefill_paged(&q, &k, &v, &o, &cu, &paged, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "empty table rows");
  paged.table_stride = 2;
  expect(attn_prefill_ex(&q, &k, &v, &o, &cu, &cu, &paged, 8, 2, 128, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "history and pages together");
  expect(attn_prefill_ex(&q, &k, &v, &o, &cu, nullptr, nullptr, 8, 2, 320, 200, scale, 0,
                         nullptr) != ATTN_OK, "head pair without a kernel");
  expect(attn_prefill_ex_ws(&q, &k, &v, &o, &cu, nullptr, nullptr, 8, 2, 128, 128, scale, 0,
                            nullptr, 1024, nullptr) != ATTN_OK, "null workspace with a size");

  // decode
  attn_tensor qd = tensor(3, 8, 128, ATTN_BF16), od = tensor(3, 8, 128, ATTN_BF16);
  expect(attn_decode(&qd, &k, &v, &od, nullptr, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "decode without key offsets");
  expect(attn_decode(&qd, &k, &v, &od, &cu, 8, 2, 128, scale, -5, nullptr) ==
             ATTN_ERR_INVALID_ARG, "decode negative window");
  expect(attn_decode_paged(&qd, &k, &v, &od, nullptr, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "decode paged without a table");
  expect(attn_decode_ws(&qd, &k, &v, &od, &cu, 8, 2, 128, scale, 0, nullptr, 4096, nullptr) !=
             ATTN_OK, "decode null workspace with a size");
  expect(attn_decode_paged_ws(&qd, &k, &v, &od, nullptr, 8, 2, 128, scale, 0, nullptr, 0,
                              nullptr) == ATTN_ERR_INVALID_ARG, "decode paged ws without a table");
  expect(attn_decode_noalloc(&qd, &k, &v, &od, nullptr, 8, 2, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "no-alloc decode without key offsets");
  expect(attn_decode_noalloc(&qd, &k, &v, &od, &cu, 8, 2, 128, scale, -5, nullptr) ==
             ATTN_ERR_INVALID_ARG, "no-alloc decode negative window");
  expect(attn_decode_noalloc(&qd, &k, &v, &od, &cu, 8, 3, 128, scale, 0, nullptr) ==
             ATTN_ERR_INVALID_ARG, "no-alloc decode heads not a multiple of KV heads");

  // workspace sizes at the edges of their arguments
  const int64_t big[] = {-1, 0, 1, 63, 64, 65, 1 << 20, INT32_MAX, INT64_MAX / 4, INT64_MAX};
  for (int64_t t : big)
    for (int64_t keys : big) {
      (void)attn_prefill_workspace_size(t, keys, 1, 4, 1, 128, 128, 0);
      (void)attn_prefill_workspace_size(t, keys, INT32_MAX, INT32_MAX, 1, 128, 128, 1000);
      (void)attn_prefill_workspace_size(t, keys, 3, 32, 8, 64, 64, INT32_MAX);
    }
  for (int64_t s : big) {
    (void)attn_decode_workspace_size(s, 32, 8, 128);
    (void)attn_decode_workspace_size(s, INT32_MAX, 1, 128);
    (void)attn_decode_workspace_size(s, -4, -1, 128);
  }
  expect(attn_prefill_workspace_size(8192, 8192, 1, 32, 8, 96, 96, 0) == 0,
         "no workspace for a head size without a split");

  // empty batches return before any HIP call
  static int32_t zeros[4] = {0, 0, 0, 0};
  attn_seqlens cu_empty = {zeros, 3, 0};
  attn_tensor q0 = tensor(0, 8, 128, ATTN_BF16), k0 = tensor(0, 2, 128, ATTN_BF16),
              v0 = tensor(0, 2, 128, ATTN_BF16), o0 = tensor(0, 8, 128, ATTN_BF16);
  expect(attn_prefill(&q0, &k0, &v0, &o0, &cu_empty, 8, 2, 128, scale, 0, nullptr) == ATTN_OK,
         "empty batch");

  std::printf("%s: %d failure(s)\n", g_failures ? "FAILED" : "ok", g_failures);
  return g_failures ? 1 : 0;
}
