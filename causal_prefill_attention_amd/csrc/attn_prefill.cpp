// C ABI of the prefill-attention library: argument checks, dispatch, errors.
//
// Every check runs on the host before the first HIP call, so a bad argument
// never reaches the device and every error path is testable without a GPU.
// Nothing is allocated and nothing synchronises (unless the debug variable
// ATTN_PREFILL_VALIDATE=1 asks for a host check of cu_seqlens).
#include "attn_prefill.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <functional>
#include <queue>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "prefill_params.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

const int32_t kHeadDims[] = {64, 128, 256, 512};

bool head_dim_supported(int32_t d) {
  for (int32_t x : kHeadDims)
    if (x == d) return true;
  return false;
}

int64_t elem_bytes(int32_t dtype) { return dtype == ATTN_FP32 ? 4 : 2; }

bool dtype_known(int32_t dtype) {
  return dtype == ATTN_BF16 || dtype == ATTN_FP16 || dtype == ATTN_FP32;
}

// Byte range [lo, hi) touched by a tensor of n_heads x head_dim per token.
struct Extent {
  uintptr_t lo, hi;
};

// Elements from a tensor's first to one past its last element,
// (T - 1) * token_stride + (H - 1) * head_stride + d, or -1 if that does not
// fit in int64.
int64_t span_elems(int64_t T, int64_t ts, int64_t H, int64_t hs, int64_t d) {
  int64_t a, b, s;
  if (__builtin_mul_overflow(T - 1, ts, &a) || __builtin_mul_overflow(H - 1, hs, &b) ||
      __builtin_add_overflow(a, b, &s) || __builtin_add_overflow(s, d, &s))
    return -1;
  return s;
}

Extent extent_of(const attn_tensor* t, int32_t n_heads, int32_t head_dim) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(t->data);
  const int64_t span =
      span_elems(t->n_tokens, t->token_stride, n_heads, t->head_stride, head_dim);
  int64_t bytes;
  if (span < 0 || __builtin_mul_overflow(span, elem_bytes(t->dtype), &bytes))
    return {lo, UINTPTR_MAX};  // (check_tensor rejects such tensors first)
  return {lo, lo + (uintptr_t)bytes};
}

bool overlaps(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

// Checks one tensor descriptor; `what` names it in messages.
int check_tensor(const attn_tensor* t, const char* what, int32_t n_heads, int32_t head_dim) {
  if (t == nullptr) return fail(ATTN_ERR_INVALID_ARG, "%s: descriptor is NULL", what);
  if (!dtype_known(t->dtype))
    return fail(ATTN_ERR_INVALID_ARG, "%s: unknown dtype code %d", what, (int)t->dtype);
  if (t->reserved != 0)
    return fail(ATTN_ERR_INVALID_ARG, "%s: reserved field must be 0", what);
  if (t->n_tokens < 0)
    return fail(ATTN_ERR_INVALID_ARG, "%s: n_tokens %lld < 0", what, (long long)t->n_tokens);
  if (t->n_tokens > INT32_MAX)
    return fail(ATTN_ERR_INVALID_ARG, "%s: n_tokens %lld exceeds int32 offsets", what,
                (long long)t->n_tokens);
  if (t->n_tokens == 0) return ATTN_OK;
  if (t->data == nullptr) return fail(ATTN_ERR_INVALID_ARG, "%s: data is NULL", what);
  if (t->token_stride < 0 || t->head_stride < 0)
    return fail(ATTN_ERR_INVALID_ARG, "%s: negative stride", what);
  // Head vectors must not overlap: token-major or head-major nesting.
  const int64_t T = t->n_tokens, H = n_heads, d = head_dim;
  const int64_t ts = t->token_stride, hs = t->head_stride;
  // (once the span fits in int64, every product and sum below does too)
  const int64_t span = span_elems(T, ts, H, hs, d);
  int64_t span_bytes;
  if (span < 0 || __builtin_mul_overflow(span, (int64_t)elem_bytes(t->dtype), &span_bytes))
    return fail(ATTN_ERR_INVALID_ARG,
                "%s: strides (token %lld, head %lld) put the tensor past the address range",
                what, (long long)ts, (long long)hs);
  const bool token_major = (H == 1 || hs >= d) && (T == 1 || ts >= (H - 1) * hs + d);
  const bool head_major = (T == 1 || ts >= d) && (H == 1 || hs >= (T - 1) * ts + d);
  if (!token_major && !head_major)
    return fail(ATTN_ERR_INVALID_ARG,
                "%s: strides (token %lld, head %lld) overlap head vectors of %d x %d",
                what, (long long)ts, (long long)hs, (int)H, (int)d);
  const int64_t eb = elem_bytes(t->dtype);
  if ((reinterpret_cast<uintptr_t>(t->data) & 15u) != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: data pointer is not 16-byte aligned", what);
  // (unsigned products: the residue mod 16 survives wrap-around)
  if (((uint64_t)ts * (uint64_t)eb) % 16 != 0 || ((uint64_t)hs * (uint64_t)eb) % 16 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: strides are not multiples of 16 bytes", what);
  return ATTN_OK;
}

int read_offsets(const attn_seqlens* cu, std::vector<int32_t>& host, hipStream_t stream,
                 const char* what) {
  host.resize((size_t)cu->n_seqs + 1);
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess)
    e = hipMemcpy(host.data(), cu->data, host.size() * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess)
    return fail(ATTN_ERR_HIP, "ATTN_PREFILL_VALIDATE: reading %s failed: %s", what,
                hipGetErrorString(e));
  return ATTN_OK;
}

int check_offsets(const std::vector<int32_t>& host, int64_t n_tokens, const char* what) {
  if (host[0] != 0) return fail(ATTN_ERR_INVALID_ARG, "%s[0] = %d, expected 0", what, host[0]);
  for (size_t i = 1; i < host.size(); ++i)
    if (host[i] < host[i - 1])
      return fail(ATTN_ERR_INVALID_ARG, "%s decreases at index %zu", what, i);
  if (host.back() != n_tokens)
    return fail(ATTN_ERR_INVALID_ARG, "%s[n_seqs] = %d, expected %lld", what, host.back(),
                (long long)n_tokens);
  return ATTN_OK;
}

// Debug-only host check of the device offsets (ATTN_PREFILL_VALIDATE=1).
int debug_validate_offsets(const attn_seqlens* cu_q, int64_t n_q, const attn_seqlens* cu_k,
                           int64_t n_k, hipStream_t stream) {
  std::vector<int32_t> hq, hk;
  int rc;
  if ((rc = read_offsets(cu_q, hq, stream, "cu_seqlens")) != ATTN_OK) return rc;
  if ((rc = check_offsets(hq, n_q, "cu_seqlens")) != ATTN_OK) return rc;
  if (cu_k == nullptr) return ATTN_OK;
  if ((rc = read_offsets(cu_k, hk, stream, "cu_seqlens_k")) != ATTN_OK) return rc;
  if ((rc = check_offsets(hk, n_k, "cu_seqlens_k")) != ATTN_OK) return rc;
  for (size_t s = 0; s + 1 < hq.size(); ++s)
    if (hq[s + 1] - hq[s] > hk[s + 1] - hk[s])
      return fail(ATTN_ERR_INVALID_ARG, "sequence %zu has %d queries but only %d keys", s,
                  hq[s + 1] - hq[s], hk[s + 1] - hk[s]);
  return ATTN_OK;
}

int check_seqlens(const attn_seqlens* cu, const char* what) {
  if (cu == nullptr) return fail(ATTN_ERR_INVALID_ARG, "%s is NULL", what);
  if (cu->n_seqs < 1) return fail(ATTN_ERR_INVALID_ARG, "%s: n_seqs %d < 1", what, (int)cu->n_seqs);
  if (cu->data == nullptr) return fail(ATTN_ERR_INVALID_ARG, "%s data is NULL", what);
  if (cu->max_seqlen < 0)
    return fail(ATTN_ERR_INVALID_ARG, "%s: max_seqlen %d < 0", what, (int)cu->max_seqlen);
  return ATTN_OK;
}

// Checks shared by the paged entry points (prefill and decode).
int check_paged(const attn_paged_kv* paged, int64_t Tk, int tile, int64_t n_queries,
                int64_t* n_pages) {
  if (paged->block_table == nullptr || paged->seqlens_k == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "paged: block_table and seqlens_k must be set");
  if (paged->table_stride < 1)
    return fail(ATTN_ERR_INVALID_ARG, "paged: table_stride %d < 1", (int)paged->table_stride);
  if (paged->page_size < 1)
    return fail(ATTN_ERR_INVALID_ARG, "paged: page_size %d < 1", (int)paged->page_size);
  if (paged->page_size % tile != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "paged: page_size %d is not a multiple of %d",
                (int)paged->page_size, tile);
  if ((int64_t)paged->table_stride * paged->page_size > INT32_MAX)
    return fail(ATTN_ERR_UNSUPPORTED, "paged: table_stride * page_size exceeds int32");
  if (Tk % paged->page_size != 0)
    return fail(ATTN_ERR_INVALID_ARG, "paged: k has %lld token slots, not a multiple of "
                "page_size %d", (long long)Tk, (int)paged->page_size);
  *n_pages = Tk / paged->page_size;
  if (n_queries > 0 && *n_pages == 0)
    return fail(ATTN_ERR_INVALID_ARG, "q has %lld tokens but k and v have none",
                (long long)n_queries);
  return ATTN_OK;
}

// Debug-only host check of a paged cache's device metadata.
int debug_validate_paged(const attn_seqlens* cu_q, int64_t n_q, const attn_paged_kv* pg,
                         int64_t n_pages, hipStream_t stream) {
  std::vector<int32_t> hq;
  int rc;
  if ((rc = read_offsets(cu_q, hq, stream, "cu_seqlens")) != ATTN_OK) return rc;
  if ((rc = check_offsets(hq, n_q, "cu_seqlens")) != ATTN_OK) return rc;
  const size_t n_seqs = hq.size() - 1;
  std::vector<int32_t> lens(n_seqs), table(n_seqs * (size_t)pg->table_stride);
  hipError_t e = hipMemcpy(lens.data(), pg->seqlens_k, lens.size() * sizeof(int32_t),
                           hipMemcpyDeviceToHost);
  if (e == hipSuccess)
    e = hipMemcpy(table.data(), pg->block_table, table.size() * sizeof(int32_t),
                  hipMemcpyDeviceToHost);
  if (e != hipSuccess)
    return fail(ATTN_ERR_HIP, "ATTN_PREFILL_VALIDATE: reading the paged metadata failed: %s",
                hipGetErrorString(e));
  const int64_t cap = (int64_t)pg->table_stride * pg->page_size;
  for (size_t s = 0; s < n_seqs; ++s) {
    if (lens[s] < 0 || lens[s] > cap)
      return fail(ATTN_ERR_INVALID_ARG, "seqlens_k[%zu] = %d outside [0, %lld]", s, lens[s],
                  (long long)cap);
    if (hq[s + 1] - hq[s] > lens[s])
      return fail(ATTN_ERR_INVALID_ARG, "sequence %zu has %d queries but only %d keys", s,
                  hq[s + 1] - hq[s], lens[s]);
    const int used = (lens[s] + pg->page_size - 1) / pg->page_size;
    for (int b = 0; b < used; ++b) {
      const int32_t page = table[s * (size_t)pg->table_stride + b];
      if (page < 0 || page >= n_pages)
        return fail(ATTN_ERR_INVALID_ARG, "block_table[%zu][%d] = %d outside [0, %lld)", s, b,
                    page, (long long)n_pages);
    }
  }
  return ATTN_OK;
}

// All entry points: cu_k == nullptr and paged == nullptr means the keys are
// the queries' own tokens (no history); cu_k gives packed keys with a
// history; paged gives keys in a paged cache.
// Compute units of the current device (0 if the query fails).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return n;
}

// Keys of each query tile split across workgroups when the grid would not
// fill the chip: the 128-d and 64-d kernels only, planned from the shapes
// the host knows (the offsets stay on the device).  max_keys bounds any
// sequence's key count.  piece_tiles == 0: no split.
struct SplitPlan {
  int32_t piece_tiles = 0;
  int32_t max_pieces = 1;
  int64_t bytes = 0;
};

// Finishing time of workgroups of the given costs on `cus` CUs, taken in
// grid order (the order the hardware dispatches them), each by the CU that
// frees up first.
double list_makespan(const std::vector<double>& jobs, int64_t cus) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int64_t i = 0; i < cus; ++i) free_at.push(0.0);
  double end = 0.0;
  for (double j : jobs) {
    const double t = free_at.top() + j;
    free_at.pop();
    free_at.push(t);
    end = std::max(end, t);
  }
  return end;
}

SplitPlan plan_prefill_split_uncached(int64_t T, int64_t max_keys, int64_t n_seqs,
                                      int32_t n_q_heads, int32_t head_dim, int32_t head_dim_v,
                                      int32_t window) {
  SplitPlan sp;
  if (head_dim != head_dim_v || (head_dim != 128 && head_dim != 64) || T <= 0) return sp;
  const int64_t bm = attnp::prefill_min_block_m(head_dim);
  const int64_t tile = attnp::prefill_kv_tile(head_dim);
  const int64_t slots = (T + bm - 1) / bm + n_seqs;
  const int64_t grid = slots * n_q_heads;
  const int64_t cus = device_cus();
  if (cus <= 0 || grid >= 2 * cus) return sp;  // enough workgroups already
  const int64_t max_nt = (max_keys + tile - 1) / tile + 1;  // +1: window alignment
  auto finish = [&](int32_t c, int64_t pieces) {
    sp.piece_tiles = c;
    sp.max_pieces = (int32_t)pieces;
    sp.bytes = slots * pieces * n_q_heads * attnp::prefill_partial_floats(head_dim, (int)bm) * 4;
    return sp;
  };
  if (n_seqs == 1 && T <= max_keys && grid <= 16384) {
    // One sequence: every query tile's key tiles are known (the keys are a
    // history of max_keys - T followed by the T queries).  Compare the
    // finishing time of whole tiles with that of pieces, both in grid order
    // (heaviest query tile first, its pieces next, heads innermost), in
    // units of one key tile's time: 2.5 more per workgroup (prologue and
    // epilogue), 12 more per piece of a split tile (a CU's share of HBM
    // time to write its fp32 partial and read it back in the merge) and 0.5
    // per empty grid piece.  Measured: 4 query heads over 8192 tokens run
    // fastest with 48-tile pieces at half the unsplit time, and 2048 tokens
    // over 32 heads run slower with any split; the model gives both.
    const int64_t hist = max_keys - T;
    std::vector<int64_t> nts;  // grid order: the last query tile first
    for (int64_t q0 = ((T - 1) / bm) * bm; q0 >= 0; q0 -= bm) {
      const int64_t kv_hi = hist + std::min(T, q0 + bm);
      const int64_t kv_lo = window > 0 ? std::max<int64_t>(0, hist + q0 - window + 1) : 0;
      nts.push_back(std::max<int64_t>(1, (kv_hi - (kv_lo - kv_lo % tile) + tile - 1) / tile));
    }
    std::vector<double> jobs;
    for (int64_t nt : nts)
      for (int32_t h = 0; h < n_q_heads; ++h) jobs.push_back((double)nt + 2.5);
    const double whole = list_makespan(jobs, cus);
    double best = 0.85 * whole;  // split only for a clear gain
    int32_t best_c = 0;
    int64_t best_mp = 1;
    for (int32_t c : {4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128}) {
      int64_t mp = 1, n_jobs = 0;
      for (int64_t nt : nts) {
        mp = std::max(mp, (nt + c - 1) / c);
        n_jobs += (nt + c - 1) / c * n_q_heads;
      }
      if (mp < 2) break;                // no tile is split at this length or above
      if (n_jobs > 16 * cus) continue;  // pieces this short cost more than they save
      jobs.clear();
      for (int64_t nt : nts) {
        const int64_t n = (nt + c - 1) / c;
        for (int64_t i = 0; i < mp; ++i)
          for (int32_t h = 0; h < n_q_heads; ++h)
            jobs.push_back(i >= n ? 0.5
                                  : (double)std::min<int64_t>(c, nt - i * c) + 2.5 +
                                        (n > 1 ? 12.0 : 0.0));
      }
      const double t = list_makespan(jobs, cus);
      if (t < best) {
        best = t;
        best_c = c;
        best_mp = mp;
      }
    }
    if (best_c == 0) return sp;
    return finish(best_c, best_mp);
  }
  // Several sequences (lengths unknown here): split only a grid with fewer
  // workgroups than CUs, into about two pieces per query tile on average.
  if (grid >= cus) return sp;
  const int64_t want = (2 * cus + grid - 1) / grid;
  int64_t c = (max_nt + 2 * want - 1) / (2 * want);
  if (c < 8) c = 8;
  const int64_t pieces = (max_nt + c - 1) / c;
  if (pieces < 2 || c > INT32_MAX) return sp;
  return finish((int32_t)c, pieces);
}

// The plan of the last call on this thread is kept: a serving loop repeats
// the same shapes, and one plan costs up to ~0.1 ms of host time.
SplitPlan plan_prefill_split(int64_t T, int64_t max_keys, int64_t n_seqs, int32_t n_q_heads,
                             int32_t head_dim, int32_t head_dim_v, int32_t window) {
  struct Key {
    int64_t T, max_keys, n_seqs;
    int32_t n_q_heads, head_dim, head_dim_v, window;
    int dev;
    bool operator==(const Key& o) const {
      return T == o.T && max_keys == o.max_keys && n_seqs == o.n_seqs &&
             n_q_heads == o.n_q_heads && head_dim == o.head_dim && head_dim_v == o.head_dim_v &&
             window == o.window && dev == o.dev;
    }
  };
  thread_local Key last_key{-1, -1, -1, 0, 0, 0, 0, -1};
  thread_local SplitPlan last_plan;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const Key key{T, max_keys, n_seqs, n_q_heads, head_dim, head_dim_v, window, dev};
  if (key == last_key) return last_plan;
  last_plan =
      plan_prefill_split_uncached(T, max_keys, n_seqs, n_q_heads, head_dim, head_dim_v, window);
  last_key = key;
  return last_plan;
}

int run_prefill(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                const attn_tensor* out, const attn_seqlens* cu_q, const attn_seqlens* cu_k,
                const attn_paged_kv* paged, int32_t n_q_heads, int32_t n_kv_heads,
                int32_t head_dim, int32_t head_dim_v, float scale, int32_t sliding_window,
                void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  g_last_error.clear();
  if (n_q_heads < 1 || n_kv_heads < 1)
    return fail(ATTN_ERR_INVALID_ARG, "n_q_heads (%d) and n_kv_heads (%d) must be >= 1",
                (int)n_q_heads, (int)n_kv_heads);
  if (n_q_heads % n_kv_heads != 0)
    return fail(ATTN_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                (int)n_q_heads, (int)n_kv_heads);
  if (head_dim < 1) return fail(ATTN_ERR_INVALID_ARG, "head_dim %d < 1", (int)head_dim);
  if (head_dim_v < 1)
    return fail(ATTN_ERR_INVALID_ARG, "head_dim_v %d < 1", (int)head_dim_v);
  if (head_dim_v == head_dim ? !head_dim_supported(head_dim)
                             : !(head_dim == 320 && head_dim_v == 256))
    return fail(ATTN_ERR_UNSUPPORTED,
                "no kernel for head_dim %d / head_dim_v %d (supported: 64, 128, 256 and 512 "
                "for both, or 320 for q/k with 256 for v/out)",
                (int)head_dim, (int)head_dim_v);
  if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale is not finite");
  if (sliding_window < 0)
    return fail(ATTN_ERR_INVALID_ARG, "sliding_window %d < 0 (0 = off)", (int)sliding_window);
  int rc;
  if ((rc = check_tensor(q, "q", n_q_heads, head_dim)) != ATTN_OK) return rc;
  if ((rc = check_tensor(k, "k", n_kv_heads, head_dim)) != ATTN_OK) return rc;
  if ((rc = check_tensor(v, "v", n_kv_heads, head_dim_v)) != ATTN_OK) return rc;
  if ((rc = check_tensor(out, "out", n_q_heads, head_dim_v)) != ATTN_OK) return rc;
  if (q->dtype != ATTN_BF16 && q->dtype != ATTN_FP32)
    return fail(ATTN_ERR_UNSUPPORTED, "q dtype must be BF16 or FP32");
  if (k->dtype != v->dtype) return fail(ATTN_ERR_UNSUPPORTED, "k and v dtypes differ");
  if (k->dtype != ATTN_BF16 && k->dtype != ATTN_FP16)
    return fail(ATTN_ERR_UNSUPPORTED, "k/v dtype must be BF16 or FP16");
  if (out->dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "out dtype must be BF16");
  const int64_t T = q->n_tokens;
  const int64_t Tk = k->n_tokens;
  if (cu_k == nullptr && paged == nullptr) {
    if (k->n_tokens != T || v->n_tokens != T || out->n_tokens != T)
      return fail(ATTN_ERR_INVALID_ARG, "n_tokens differ: q %lld k %lld v %lld out %lld",
                  (long long)T, (long long)k->n_tokens, (long long)v->n_tokens,
                  (long long)out->n_tokens);
  } else {
    if (out->n_tokens != T)
      return fail(ATTN_ERR_INVALID_ARG, "n_tokens differ: q %lld out %lld", (long long)T,
                  (long long)out->n_tokens);
    if (v->n_tokens != Tk)
      return fail(ATTN_ERR_INVALID_ARG, "n_tokens differ: k %lld v %lld", (long long)Tk,
                  (long long)v->n_tokens);
  }
  if ((rc = check_seqlens(cu_q, "cu_seqlens")) != ATTN_OK) return rc;
  int64_t n_pages = 0;
  if (paged != nullptr &&
      (rc = check_paged(paged, Tk, attnp::prefill_kv_tile(head_dim), T, &n_pages)) != ATTN_OK)
    return rc;
  if (cu_k != nullptr) {
    if ((rc = check_seqlens(cu_k, "cu_seqlens_k")) != ATTN_OK) return rc;
    if (cu_k->n_seqs != cu_q->n_seqs)
      return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens has %d sequences, cu_seqlens_k %d",
                  (int)cu_q->n_seqs, (int)cu_k->n_seqs);
    if (T > 0 && Tk == 0)
      return fail(ATTN_ERR_INVALID_ARG, "q has %lld tokens but k and v have none",
                  (long long)T);
  }
  // K and V tiles are read through buffer resources with a 32-bit range and
  // 32-bit offsets, one resource per tile of up to 64 rows.
  for (const attn_tensor* t : {k, v}) {
    if (Tk > 1 && t->token_stride * elem_bytes(t->dtype) * 64 > (int64_t)INT32_MAX)
      return fail(ATTN_ERR_UNSUPPORTED,
                  "%s: token stride of %lld bytes is too large (at most 32 MiB - 1 B)",
                  t == k ? "k" : "v", (long long)(t->token_stride * elem_bytes(t->dtype)));
  }
  if (T == 0) return ATTN_OK;  // nothing to compute or write
  const Extent eo = extent_of(out, n_q_heads, head_dim_v);
  if (overlaps(eo, extent_of(q, n_q_heads, head_dim)) ||
      overlaps(eo, extent_of(k, n_kv_heads, head_dim)) ||
      overlaps(eo, extent_of(v, n_kv_heads, head_dim_v)))
    return fail(ATTN_ERR_INVALID_ARG, "out overlaps q, k or v");

  if (workspace_bytes > 0 && workspace == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "workspace is NULL but workspace_bytes is %zu",
                workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
    return fail(ATTN_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  SplitPlan sp;
  if (workspace_bytes > 0) {
    const int64_t max_keys =
        paged != nullptr ? (int64_t)paged->table_stride * paged->page_size : Tk;
    sp = plan_prefill_split(T, max_keys, cu_q->n_seqs, n_q_heads, head_dim, head_dim_v,
                            sliding_window);
    if (sp.bytes > (int64_t)workspace_bytes) sp = SplitPlan();  // too small: no split
  }
  if (sp.piece_tiles > 0) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(workspace);
    const Extent ew = {lo, lo + (uintptr_t)sp.bytes};
    if (overlaps(ew, eo) || overlaps(ew, extent_of(q, n_q_heads, head_dim)) ||
        overlaps(ew, extent_of(k, n_kv_heads, head_dim)) ||
        overlaps(ew, extent_of(v, n_kv_heads, head_dim_v)))
      return fail(ATTN_ERR_INVALID_ARG, "workspace overlaps q, k, v or out");
  }

  const int bm = attnp::prefill_min_block_m(head_dim);
  const int64_t slots = (T + bm - 1) / bm + cu_q->n_seqs;
  const int64_t blocks = slots * n_q_heads * sp.max_pieces;
  if (slots > INT32_MAX || blocks * 1024 >= ((int64_t)1 << 32))
    return fail(ATTN_ERR_UNSUPPORTED, "grid of %lld workgroups is too large",
                (long long)blocks);

  const char* dbg = getenv("ATTN_PREFILL_VALIDATE");
  if (dbg != nullptr && dbg[0] == '1') {
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    rc = paged != nullptr ? debug_validate_paged(cu_q, T, paged, n_pages, st)
                          : debug_validate_offsets(cu_q, T, cu_k, Tk, st);
    if (rc != ATTN_OK) return rc;
  }

  attnp::PrefillParams p;
  p.q = q->data;
  p.k = k->data;
  p.v = v->data;
  p.out = out->data;
  p.cu_seqlens = cu_q->data;
  p.cu_seqlens_k = cu_k != nullptr ? cu_k->data : cu_q->data;
  p.q_ts = q->token_stride;
  p.q_hs = q->head_stride;
  p.k_ts = k->token_stride;
  p.k_hs = k->head_stride;
  p.v_ts = v->token_stride;
  p.v_hs = v->head_stride;
  p.o_ts = out->token_stride;
  p.o_hs = out->head_stride;
  p.n_tokens = (int32_t)T;
  p.n_tokens_k = (int32_t)Tk;
  p.n_seqs = cu_q->n_seqs;
  p.n_q_heads = n_q_heads;
  p.group = n_q_heads / n_kv_heads;
  p.window = sliding_window;
  p.tile_slots = 0;  // set by the launcher
  p.block_table = paged != nullptr ? paged->block_table : nullptr;
  p.seqlens_k = paged != nullptr ? paged->seqlens_k : nullptr;
  p.table_stride = paged != nullptr ? paged->table_stride : 0;
  p.page_size = paged != nullptr ? paged->page_size : 0;
  p.n_pages = (int32_t)n_pages;
  const float log2e = 1.4426950408889634f;
  if (scale == 0.f) {
    p.score_mult = 1.f;  // Q is zeroed, every visible score is 0
    p.q_mult = 0.f;
  } else {
    p.score_mult = fabsf(scale) * log2e;
    p.q_mult = scale < 0.f ? -1.f : 1.f;
  }
  p.piece_tiles = sp.piece_tiles;
  p.max_pieces = sp.max_pieces;
  p.partial = sp.piece_tiles > 0 ? static_cast<float*>(workspace) : nullptr;
  // A causal grid of at most one workgroup per CU finishes with its
  // heaviest query tile, which sees twice the keys of the average one;
  // folded, every workgroup pairs a sequence's row block r with block
  // nb - 1 - r: 32-row blocks of four query heads of a KV head (64 rows
  // each per workgroup) for the 64-d and 128-d kernel, 64-row blocks of one
  // head (128 rows per workgroup) for the 512-d kernel.  Sum over sequences
  // of ceil(len / rows) is at most ceil(T / rows) + n_seqs - 1.
  // ATTN_PREFILL_FOLD=0 / =1 turns folding off / on wherever the shape
  // allows it (for tests of both grids on one shape).
  p.fold = 0;
  int64_t fold_rows = 0, fold_units = 0;
  if (sp.piece_tiles == 0 && sliding_window == 0 && head_dim == head_dim_v) {
    if ((head_dim == 64 || head_dim == 128) && p.group % 4 == 0) {
      fold_rows = 64;
      fold_units = n_q_heads / 4;
    } else if (head_dim == 512) {
      fold_rows = 128;
      fold_units = n_q_heads;
    }
  }
  if (fold_rows > 0) {
    const char* force = getenv("ATTN_PREFILL_FOLD");
    if (force != nullptr && (force[0] == '0' || force[0] == '1')) {
      p.fold = force[0] == '1';
    } else {
      const int64_t pairs = (T + fold_rows - 1) / fold_rows + cu_q->n_seqs - 1;
      const int64_t cus = device_cus();
      if (cus > 0 && pairs * fold_units <= cus) p.fold = 1;
    }
  }
  const hipError_t e = attnp::launch_prefill(p, head_dim, head_dim_v, (attnp::DType)q->dtype,
                                             (attnp::DType)k->dtype,
                                             reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(ATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

// Debug-only host check of decode metadata: every sequence has >= 1 key.
int debug_validate_decode(int64_t n_seqs, const attn_seqlens* cu_k, int64_t Tk,
                          const attn_paged_kv* pg, int64_t n_pages, hipStream_t stream) {
  std::vector<int32_t> lens((size_t)n_seqs);
  int rc;
  if (cu_k != nullptr) {
    std::vector<int32_t> hk;
    if ((rc = read_offsets(cu_k, hk, stream, "cu_seqlens_k")) != ATTN_OK) return rc;
    if ((rc = check_offsets(hk, Tk, "cu_seqlens_k")) != ATTN_OK) return rc;
    for (int64_t s = 0; s < n_seqs; ++s) lens[s] = hk[s + 1] - hk[s];
  } else {
    std::vector<int32_t> table((size_t)n_seqs * pg->table_stride);
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess)
      e = hipMemcpy(lens.data(), pg->seqlens_k, lens.size() * sizeof(int32_t),
                    hipMemcpyDeviceToHost);
    if (e == hipSuccess)
      e = hipMemcpy(table.data(), pg->block_table, table.size() * sizeof(int32_t),
                    hipMemcpyDeviceToHost);
    if (e != hipSuccess)
      return fail(ATTN_ERR_HIP, "ATTN_PREFILL_VALIDATE: reading the paged metadata failed: %s",
                  hipGetErrorString(e));
    const int64_t cap = (int64_t)pg->table_stride * pg->page_size;
    for (int64_t s = 0; s < n_seqs; ++s) {
      if (lens[s] > cap)
        return fail(ATTN_ERR_INVALID_ARG, "seqlens_k[%lld] = %d exceeds %lld", (long long)s,
                    lens[s], (long long)cap);
      const int used = (lens[s] + pg->page_size - 1) / pg->page_size;
      for (int b = 0; b < used; ++b) {
        const int32_t page = table[s * (size_t)pg->table_stride + b];
        if (page < 0 || page >= n_pages)
          return fail(ATTN_ERR_INVALID_ARG, "block_table[%lld][%d] = %d outside [0, %lld)",
                      (long long)s, b, page, (long long)n_pages);
      }
    }
  }
  for (int64_t s = 0; s < n_seqs; ++s)
    if (lens[s] < 1)
      return fail(ATTN_ERR_INVALID_ARG, "sequence %lld has %d keys (decode needs >= 1)",
                  (long long)s, lens[s]);
  return ATTN_OK;
}

// Decode work units (sequence, KV head, block of 32 query heads) and the
// split of each unit's keys into ranges: as many as keep every workgroup of
// the launch resident at once (one per CU: the kernel's LDS admits one), at
// most kMaxSplits.
int64_t decode_units(int64_t n_seqs, int32_t n_q_heads, int32_t n_kv_heads) {
  const int64_t group = n_q_heads / n_kv_heads;
  return n_seqs * n_kv_heads * ((group + 31) / 32);
}
int decode_preferred_splits(int64_t units) {
  const int64_t cus = device_cus();
  if (units <= 0 || 2 * units > cus) return 1;
  const int64_t s = cus / units;
  return (int)(s < attnp::kMaxSplits ? s : attnp::kMaxSplits);
}

// Both decode entry points: exactly one of cu_k and paged is set; a
// workspace (may be NULL) lets the keys of a sequence be split across
// workgroups.
int run_decode(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
               const attn_tensor* out, const attn_seqlens* cu_k, const attn_paged_kv* paged,
               int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
               int32_t sliding_window, void* workspace, size_t workspace_bytes,
               attn_stream_t stream) {
  g_last_error.clear();
  if (n_q_heads < 1 || n_kv_heads < 1)
    return fail(ATTN_ERR_INVALID_ARG, "n_q_heads (%d) and n_kv_heads (%d) must be >= 1",
                (int)n_q_heads, (int)n_kv_heads);
  if (n_q_heads % n_kv_heads != 0)
    return fail(ATTN_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                (int)n_q_heads, (int)n_kv_heads);
  if (head_dim < 1) return fail(ATTN_ERR_INVALID_ARG, "head_dim %d < 1", (int)head_dim);
  if (head_dim != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "no decode kernel for head_dim %d (supported: 128)",
                (int)head_dim);
  if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale is not finite");
  if (sliding_window < 0)
    return fail(ATTN_ERR_INVALID_ARG, "sliding_window %d < 0 (0 = off)", (int)sliding_window);
  int rc;
  if ((rc = check_tensor(q, "q", n_q_heads, head_dim)) != ATTN_OK) return rc;
  if ((rc = check_tensor(k, "k", n_kv_heads, head_dim)) != ATTN_OK) return rc;
  if ((rc = check_tensor(v, "v", n_kv_heads, head_dim)) != ATTN_OK) return rc;
  if ((rc = check_tensor(out, "out", n_q_heads, head_dim)) != ATTN_OK) return rc;
  if (q->dtype != ATTN_BF16 && q->dtype != ATTN_FP32)
    return fail(ATTN_ERR_UNSUPPORTED, "q dtype must be BF16 or FP32");
  if (k->dtype != v->dtype) return fail(ATTN_ERR_UNSUPPORTED, "k and v dtypes differ");
  if (k->dtype != ATTN_BF16 && k->dtype != ATTN_FP16)
    return fail(ATTN_ERR_UNSUPPORTED, "k/v dtype must be BF16 or FP16");
  if (out->dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "out dtype must be BF16");
  const int64_t n_seqs = q->n_tokens;  // one query token per sequence
  const int64_t Tk = k->n_tokens;
  if (out->n_tokens != n_seqs)
    return fail(ATTN_ERR_INVALID_ARG, "n_tokens differ: q %lld out %lld", (long long)n_seqs,
                (long long)out->n_tokens);
  if (v->n_tokens != Tk)
    return fail(ATTN_ERR_INVALID_ARG, "n_tokens differ: k %lld v %lld", (long long)Tk,
                (long long)v->n_tokens);
  if (n_seqs == 0) return ATTN_OK;  // no sequence, nothing to compute or write
  int64_t n_pages = 0;
  if (cu_k != nullptr) {
    if ((rc = check_seqlens(cu_k, "cu_seqlens_k")) != ATTN_OK) return rc;
    if (cu_k->n_seqs != n_seqs)
      return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens_k has %d sequences, q has %lld tokens",
                  (int)cu_k->n_seqs, (long long)n_seqs);
    if (n_seqs > 0 && Tk == 0)
      return fail(ATTN_ERR_INVALID_ARG, "q has %lld tokens but k and v have none",
                  (long long)n_seqs);
  } else if ((rc = check_paged(paged, Tk, attnp::decode_kv_tile(), n_seqs, &n_pages)) !=
             ATTN_OK) {
    return rc;
  }
  for (const attn_tensor* t : {k, v}) {
    if (Tk > 1 && t->token_stride * elem_bytes(t->dtype) * 64 > (int64_t)INT32_MAX)
      return fail(ATTN_ERR_UNSUPPORTED,
                  "%s: token stride of %lld bytes is too large (at most 32 MiB - 1 B)",
                  t == k ? "k" : "v", (long long)(t->token_stride * elem_bytes(t->dtype)));
  }
  const Extent eo = extent_of(out, n_q_heads, head_dim);
  if (overlaps(eo, extent_of(q, n_q_heads, head_dim)) ||
      overlaps(eo, extent_of(k, n_kv_heads, head_dim)) ||
      overlaps(eo, extent_of(v, n_kv_heads, head_dim)))
    return fail(ATTN_ERR_INVALID_ARG, "out overlaps q, k or v");
  const int64_t group = n_q_heads / n_kv_heads;
  if (workspace_bytes > 0 && workspace == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "workspace is NULL but workspace_bytes is %zu",
                workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
    return fail(ATTN_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  const int64_t units = decode_units(n_seqs, n_q_heads, n_kv_heads);
  int n_splits = decode_preferred_splits(units);
  const int64_t split_bytes = units * (int64_t)attnp::decode_partial_floats(head_dim) * 4;
  const int64_t fit = split_bytes > 0 ? (int64_t)(workspace_bytes / (size_t)split_bytes) : 0;
  if (n_splits > fit) n_splits = (int)fit;
  if (n_splits < 2) n_splits = 1;
  // the merge kernel of a split batch runs 8 workgroups per unit; the decode
  // grid is rounded up to a multiple of 32
  const int64_t blocks = n_splits > 1 && n_splits < 8 ? units * 8 : units * n_splits;
  if ((blocks + 31) * 256 >= ((int64_t)1 << 32))
    return fail(ATTN_ERR_UNSUPPORTED, "grid of %lld workgroups is too large", (long long)blocks);
  if (n_splits > 1) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(workspace);
    const Extent ew = {lo, lo + (uintptr_t)(n_splits * split_bytes)};
    if (overlaps(ew, eo) || overlaps(ew, extent_of(q, n_q_heads, head_dim)) ||
        overlaps(ew, extent_of(k, n_kv_heads, head_dim)) ||
        overlaps(ew, extent_of(v, n_kv_heads, head_dim)))
      return fail(ATTN_ERR_INVALID_ARG, "workspace overlaps q, k, v or out");
  }
  const char* dbg = getenv("ATTN_PREFILL_VALIDATE");
  if (dbg != nullptr && dbg[0] == '1') {
    if ((rc = debug_validate_decode(n_seqs, cu_k, Tk, paged, n_pages,
                                    reinterpret_cast<hipStream_t>(stream))) != ATTN_OK)
      return rc;
  }

  attnp::DecodeParams p;
  p.q = q->data;
  p.k = k->data;
  p.v = v->data;
  p.out = out->data;
  p.cu_seqlens_k = cu_k != nullptr ? cu_k->data : nullptr;
  p.block_table = paged != nullptr ? paged->block_table : nullptr;
  p.seqlens_k = paged != nullptr ? paged->seqlens_k : nullptr;
  p.q_ts = q->token_stride;
  p.q_hs = q->head_stride;
  p.k_ts = k->token_stride;
  p.k_hs = k->head_stride;
  p.v_ts = v->token_stride;
  p.v_hs = v->head_stride;
  p.o_ts = out->token_stride;
  p.o_hs = out->head_stride;
  p.n_seqs = (int32_t)n_seqs;
  p.n_q_heads = n_q_heads;
  p.n_kv_heads = n_kv_heads;
  p.group = (int32_t)group;
  p.window = sliding_window;
  p.n_tokens_k = (int32_t)Tk;
  p.table_stride = paged != nullptr ? paged->table_stride : 0;
  p.page_size = paged != nullptr ? paged->page_size : 0;
  p.n_pages = (int32_t)n_pages;
  const float log2e = 1.4426950408889634f;
  if (scale == 0.f) {
    p.score_mult = 1.f;
    p.q_mult = 0.f;
  } else {
    p.score_mult = fabsf(scale) * log2e;
    p.q_mult = scale < 0.f ? -1.f : 1.f;
  }
  p.n_splits = n_splits;
  p.partial = n_splits > 1 ? static_cast<float*>(workspace) : nullptr;
  const hipError_t e = attnp::launch_decode(p, head_dim, (attnp::DType)q->dtype,
                                            (attnp::DType)k->dtype,
                                            reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(ATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                const attn_tensor* out, const attn_seqlens* cu_seqlens_k, int32_t n_q_heads,
                int32_t n_kv_heads, int32_t head_dim, float scale, int32_t sliding_window,
                attn_stream_t stream) {
  if (cu_seqlens_k == nullptr) {
    g_last_error.clear();
    return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens_k is NULL");
  }
  return run_decode(q, k, v, out, cu_seqlens_k, nullptr, n_q_heads, n_kv_heads, head_dim, scale,
                    sliding_window, nullptr, 0, stream);
}

int attn_decode_ws(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                   const attn_tensor* out, const attn_seqlens* cu_seqlens_k, int32_t n_q_heads,
                   int32_t n_kv_heads, int32_t head_dim, float scale, int32_t sliding_window,
                   void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  if (cu_seqlens_k == nullptr) {
    g_last_error.clear();
    return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens_k is NULL");
  }
  return run_decode(q, k, v, out, cu_seqlens_k, nullptr, n_q_heads, n_kv_heads, head_dim, scale,
                    sliding_window, workspace, workspace_bytes, stream);
}

size_t attn_decode_workspace_size(int64_t n_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t head_dim) {
  if (n_seqs < 1 || n_seqs > INT32_MAX || n_q_heads < 1 || n_kv_heads < 1 ||
      n_q_heads % n_kv_heads != 0 || head_dim != 128)
    return 0;
  const int64_t units = decode_units(n_seqs, n_q_heads, n_kv_heads);
  const int n_splits = decode_preferred_splits(units);
  if (n_splits < 2) return 0;
  return (size_t)(units * n_splits * (int64_t)attnp::decode_partial_floats(head_dim) * 4);
}

int attn_decode_noalloc(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                        const attn_tensor* out, const attn_seqlens* cu_seqlens_k,
                        int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                        int32_t sliding_window, attn_stream_t stream) {
  g_last_error.clear();
  if (cu_seqlens_k == nullptr) return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens_k is NULL");
  // the split attn_decode_ws makes with its preferred workspace (0: none);
  // shapes outside the contract give 0 here and are rejected by run_decode
  const size_t need = q != nullptr ? attn_decode_workspace_size(q->n_tokens, n_q_heads,
                                                                n_kv_heads, head_dim)
                                   : 0;
  if (need > attnp::kDecodeScratchBytes)
    return fail(ATTN_ERR_UNSUPPORTED,
                "this batch's key split needs %zu bytes of scratch, beyond the %zu bytes of "
                "the static decode scratch; use attn_decode_ws with a workspace",
                need, attnp::kDecodeScratchBytes);
  void* ptr = nullptr;
  if (need > 0) {
    const hipError_t e = attnp::decode_static_scratch(&ptr);
    if (e != hipSuccess)
      return fail(ATTN_ERR_HIP, "static decode scratch lookup failed: %s", hipGetErrorString(e));
  }
  return run_decode(q, k, v, out, cu_seqlens_k, nullptr, n_q_heads, n_kv_heads, head_dim, scale,
                    sliding_window, ptr, need, stream);
}

int attn_decode_paged(const attn_tensor* q, const attn_tensor* k_pool, const attn_tensor* v_pool,
                      const attn_tensor* out, const attn_paged_kv* paged, int32_t n_q_heads,
                      int32_t n_kv_heads, int32_t head_dim, float scale, int32_t sliding_window,
                      attn_stream_t stream) {
  if (paged == nullptr) {
    g_last_error.clear();
    return fail(ATTN_ERR_INVALID_ARG, "paged is NULL");
  }
  return run_decode(q, k_pool, v_pool, out, nullptr, paged, n_q_heads, n_kv_heads, head_dim,
                    scale, sliding_window, nullptr, 0, stream);
}

int attn_decode_paged_ws(const attn_tensor* q, const attn_tensor* k_pool,
                         const attn_tensor* v_pool, const attn_tensor* out,
                         const attn_paged_kv* paged, int32_t n_q_heads, int32_t n_kv_heads,
                         int32_t head_dim, float scale, int32_t sliding_window, void* workspace,
                         size_t workspace_bytes, attn_stream_t stream) {
  if (paged == nullptr) {
    g_last_error.clear();
    return fail(ATTN_ERR_INVALID_ARG, "paged is NULL");
  }
  return run_decode(q, k_pool, v_pool, out, nullptr, paged, n_q_heads, n_kv_heads, head_dim,
                    scale, sliding_window, workspace, workspace_bytes, stream);
}

int attn_prefill(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                 const attn_tensor* out, const attn_seqlens* cu_seqlens,
                 int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                 int32_t sliding_window, attn_stream_t stream) {
  return run_prefill(q, k, v, out, cu_seqlens, nullptr, nullptr, n_q_heads, n_kv_heads,
                     head_dim, head_dim, scale, sliding_window, nullptr, 0, stream);
}

int attn_prefill_chunked(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                         const attn_tensor* out, const attn_seqlens* cu_seqlens_q,
                         const attn_seqlens* cu_seqlens_k, int32_t n_q_heads,
                         int32_t n_kv_heads, int32_t head_dim, float scale,
                         int32_t sliding_window, attn_stream_t stream) {
  if (cu_seqlens_k == nullptr) {
    g_last_error.clear();
    return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens_k is NULL");
  }
  return run_prefill(q, k, v, out, cu_seqlens_q, cu_seqlens_k, nullptr, n_q_heads, n_kv_heads,
                     head_dim, head_dim, scale, sliding_window, nullptr, 0, stream);
}

int attn_prefill_paged(const attn_tensor* q, const attn_tensor* k_pool,
                       const attn_tensor* v_pool, const attn_tensor* out,
                       const attn_seqlens* cu_seqlens_q, const attn_paged_kv* paged,
                       int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                       int32_t sliding_window, attn_stream_t stream) {
  if (paged == nullptr) {
    g_last_error.clear();
    return fail(ATTN_ERR_INVALID_ARG, "paged is NULL");
  }
  return run_prefill(q, k_pool, v_pool, out, cu_seqlens_q, nullptr, paged, n_q_heads,
                     n_kv_heads, head_dim, head_dim, scale, sliding_window, nullptr, 0, stream);
}

int attn_prefill_ex(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                    const attn_tensor* out, const attn_seqlens* cu_seqlens_q,
                    const attn_seqlens* cu_seqlens_k, const attn_paged_kv* paged,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim_qk,
                    int32_t head_dim_v, float scale, int32_t sliding_window,
                    attn_stream_t stream) {
  if (cu_seqlens_k != nullptr && paged != nullptr) {
    g_last_error.clear();
    return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens_k and paged are both set");
  }
  return run_prefill(q, k, v, out, cu_seqlens_q, cu_seqlens_k, paged, n_q_heads, n_kv_heads,
                     head_dim_qk, head_dim_v, scale, sliding_window, nullptr, 0, stream);
}

int attn_prefill_ex_ws(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                       const attn_tensor* out, const attn_seqlens* cu_seqlens_q,
                       const attn_seqlens* cu_seqlens_k, const attn_paged_kv* paged,
                       int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim_qk,
                       int32_t head_dim_v, float scale, int32_t sliding_window, void* workspace,
                       size_t workspace_bytes, attn_stream_t stream) {
  if (cu_seqlens_k != nullptr && paged != nullptr) {
    g_last_error.clear();
    return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens_k and paged are both set");
  }
  return run_prefill(q, k, v, out, cu_seqlens_q, cu_seqlens_k, paged, n_q_heads, n_kv_heads,
                     head_dim_qk, head_dim_v, scale, sliding_window, workspace, workspace_bytes,
                     stream);
}

size_t attn_prefill_workspace_size(int64_t n_tokens_q, int64_t max_keys, int32_t n_seqs,
                                   int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim_qk,
                                   int32_t head_dim_v, int32_t sliding_window) {
  // (token counts beyond int32 offsets are outside every entry point's contract)
  if (n_tokens_q < 1 || n_tokens_q > INT32_MAX || max_keys < 0 || max_keys > INT32_MAX ||
      n_seqs < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0 ||
      sliding_window < 0)
    return 0;
  const SplitPlan sp = plan_prefill_split(n_tokens_q, max_keys, n_seqs, n_q_heads, head_dim_qk,
                                          head_dim_v, sliding_window);
  return sp.piece_tiles > 0 ? (size_t)sp.bytes : 0;
}

const char* attn_prefill_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG: argument outside the contract";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: no kernel for this configuration";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: HIP launch or runtime error";
    default: return "unknown status";
  }
}

const char* attn_prefill_last_error(void) { return g_last_error.c_str(); }

int attn_prefill_supported_head_dims(int32_t* dims, int32_t cap) {
  const int n = (int)(sizeof(kHeadDims) / sizeof(kHeadDims[0]));
  for (int i = 0; i < n && i < cap && dims != nullptr; ++i) dims[i] = kHeadDims[i];
  return n;
}

int attn_prefill_version(void) { return 100; }

}  // extern "C"
