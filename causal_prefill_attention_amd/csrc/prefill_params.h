// Internal interface between the C ABI host code and the HIP kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace attnp {

enum DType : int32_t { kBF16 = 0, kFP16 = 1, kFP32 = 2 };

// Everything one launch needs; passed to the kernel by value.  Strides are
// in elements of the tensor's own dtype.
struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const int32_t* cu_seqlens;    // device, n_seqs + 1 query offsets
  const int32_t* cu_seqlens_k;  // device, n_seqs + 1 key offsets (may equal cu_seqlens)
  int64_t q_ts, q_hs;         // token / head strides
  int64_t k_ts, k_hs;
  int64_t v_ts, v_hs;
  int64_t o_ts, o_hs;
  int32_t n_tokens;           // Tq: tokens of q and out (query offsets clamp into [0, Tq])
  int32_t n_tokens_k;         // Tk: tokens of k and v (key offsets clamp into [0, Tk])
  int32_t n_seqs;
  int32_t n_q_heads;
  int32_t group;              // n_q_heads / n_kv_heads
  int32_t window;             // 0 = off
  int32_t tile_slots;         // q-tile slots in the grid (set by the launcher)
  float score_mult;           // log2(e) * |scale|, or 1 when scale == 0
  float q_mult;               // +1, -1 or 0: sign of scale folded into Q
  // Paged K/V (page_size > 0): k and v are pools of n_pages * page_size token
  // slots; key position j of sequence s is slot j % page_size of page
  // block_table[s * table_stride + j / page_size]; seqlens_k[s] keys.
  const int32_t* block_table;
  const int32_t* seqlens_k;
  int32_t table_stride;
  int32_t page_size;          // 0 = packed K/V (cu_seqlens_k)
  int32_t n_pages;
  // Keys split across workgroups (128-d and 64-d kernels, piece_tiles > 0):
  // the key tiles of each query tile are cut into pieces of piece_tiles
  // tiles, one workgroup each; a query tile of more than one piece writes
  // fp32 partial results (running max, sum, unnormalised output) to
  // `partial` and prefill_merge combines them.
  int32_t piece_tiles = 0;    // 0 = every query tile in one workgroup
  int32_t max_pieces = 1;     // grid pieces per query-tile slot
  float* partial = nullptr;   // [slot][piece][head] blocks of prefill_partial_floats
  // Folded grid (64-d and 128-d, four query heads per workgroup, causal
  // without a window, no key split): a workgroup's two wave groups take the
  // 32-row query blocks r and nb - 1 - r of one sequence instead of two
  // adjacent ones, which evens out the causal work of a grid of about one
  // workgroup per CU.
  int32_t fold = 0;
};

// fp32 values of one partial block: running max and sum of each of bm rows,
// then bm x head_dim output values (row-major: value d of row r at
// 2 * bm + r * head_dim + d).
constexpr int64_t prefill_partial_floats(int head_dim, int bm) {
  return (int64_t)bm * (2 + head_dim);
}

// Smallest number of query rows per workgroup any launch uses (the grid has
// at most ceil(T / this) + n_seqs tile slots per query head).
int prefill_min_block_m(int head_dim);

// Keys per K/V tile; a paged cache's page_size must be a multiple of it.
int prefill_kv_tile(int head_dim);

// The wide-head (256-d) prefill kernel: rows per workgroup, and its launcher.
int prefill_wide_block_m();
hipError_t launch_prefill_wide(const PrefillParams& p, int head_dim_qk, int head_dim_v,
                               DType q_dtype, DType kv_dtype, hipStream_t stream);

// The 512-d prefill kernel (head columns split across the four waves): rows
// per workgroup, and its launcher.
int prefill_d512_block_m();
hipError_t launch_prefill_d512(const PrefillParams& p, DType q_dtype, DType kv_dtype,
                               hipStream_t stream);

// One decode step: one query token per sequence (the sequence's next
// position) against its keys.  Passed to the decode kernel by value.
struct DecodeParams {
  const void* q;               // [n_seqs, n_q_heads, d]
  const void* k;               // packed [Tk, n_kv_heads, d] or a paged pool
  const void* v;
  void* out;                   // [n_seqs, n_q_heads, d] bf16
  const int32_t* cu_seqlens_k; // packed: n_seqs + 1 key offsets (device)
  const int32_t* block_table;  // paged: [n_seqs * table_stride] (device)
  const int32_t* seqlens_k;    // paged: [n_seqs] key counts (device)
  int64_t q_ts, q_hs;
  int64_t k_ts, k_hs;
  int64_t v_ts, v_hs;
  int64_t o_ts, o_hs;
  int32_t n_seqs;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t group;               // n_q_heads / n_kv_heads
  int32_t window;              // 0 = off
  int32_t n_tokens_k;          // Tk of packed K/V (offsets clamp into [0, Tk])
  int32_t table_stride;
  int32_t page_size;           // 0 = packed
  int32_t n_pages;
  float score_mult;
  float q_mult;
  // Split of each sequence's keys across n_splits workgroups (1 = none).
  // With n_splits > 1 every workgroup writes its unnormalised partial
  // result to `partial` and a second kernel merges them into out.
  int32_t n_splits;
  float* partial;  // [n_seqs][n_kv_heads][hblocks][n_splits][32 + 32 + 32 * d] fp32
};

// Floats of one split's partial result (max, sum and 32 x head_dim values).
constexpr int decode_partial_floats(int head_dim) { return 64 + 32 * head_dim; }
// Most key ranges one decode unit is split into.
constexpr int kMaxSplits = 64;

// The decode split's static scratch (attn_decode_noalloc): room for 256
// partial blocks of a 128-d unit, the most the preferred split of any batch
// uses on a device of up to 256 compute units.
constexpr size_t kDecodeScratchBytes = 256 * (size_t)decode_partial_floats(128) * 4;
// Device address of the current device's static decode scratch (looked up
// once per device).
hipError_t decode_static_scratch(void** ptr);

// Launches the decode kernel (head_dim 128, q bf16/fp32, kv bf16/fp16).
hipError_t launch_decode(const DecodeParams& p, int head_dim, DType q_dtype, DType kv_dtype,
                         hipStream_t stream);

// Keys per decode tile; a paged cache's page_size must be a multiple of it.
int decode_kv_tile();

// Launches the kernel for (head_dim, q dtype, kv dtype) on `stream`; picks
// the workgroup size and sets p.tile_slots.  Returns hipErrorInvalidValue if
// no instantiation exists.
hipError_t launch_prefill(const PrefillParams& p, int head_dim_qk, int head_dim_v,
                          DType q_dtype, DType kv_dtype, hipStream_t stream);

}  // namespace attnp
