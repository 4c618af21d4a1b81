/*
 * attn_prefill.h -- C ABI of the MI355X (gfx950) causal prefill-attention
 * library (libattn_prefill.so).  Plain C: no C++ or torch types cross it.
 *
 * Operation (one call = one layer's prefill attention over a packed batch):
 *
 *   for every sequence s, query token i of s, query head h:
 *     g        = h / (n_q_heads / n_kv_heads)          (consecutive GQA groups)
 *     visible  = { j in s : j <= i  and  (W == 0  or  j >= i - W + 1) }
 *     out[i,h] = sum_{j in visible} softmax_j(scale * q[i,h] . k[j,g]) * v[j,g]
 *
 * Sources on the pages:
 *   - causal bound kv_end = min(q_pos + 1, seq_len) and online softmax: the
 *     fused MLA prefill kernel in atlas PR #69 (its fix and re-audit commits);
 *   - scale passed by the caller, sliding window passed as a width with
 *     0 = off, head_dim explicit so that a 128-d head is never read with a
 *     256-d stride: the cache-skip MLA prefill fix in atlas PR #69;
 *   - the window keeps the W most recent keys (an exact recent ring): m40-llm
 *     AGENTS.md, "Current Progress";
 *   - packed variable-length prefill over cumulative offsets, GQA, FP16
 *     storage with FP32 compute, Q in FP32 and K/V in FP16: m40-llm
 *     AGENTS.md, "Project Snapshot" and the varlen-batch task under
 *     "Current Tasks";
 *   - fail loudly instead of falling back to a kernel of another head size:
 *     the ensure! guard commits of atlas PR #69.
 *
 * Layouts.  Every tensor is [n_tokens, n_heads, head_dim] addressed as
 *   data + token * token_stride + head * head_stride + c      (c < head_dim)
 * in ELEMENTS of the tensor's dtype; the head_dim axis is contiguous.  Token-
 * major ([T, H, d]) and head-major ([H, T, d]) layouts are both accepted.
 * Sequences are packed back to back along the token axis; sequence s owns
 * tokens [cu_seqlens[s], cu_seqlens[s+1]).
 *
 * Precision.  Both contractions run on the matrix cores in the K/V storage
 * type with fp32 accumulation, so that K and V enter them exactly as stored
 * (the pages' FP16 storage with FP32 compute): bf16 K/V use the bf16 MFMA,
 * fp16 K/V the fp16 MFMA.  Q (bf16 or fp32) and the softmax probabilities
 * are rounded to that type (round to nearest even) -- with fp16 K/V, q must
 * lie within the fp16 range (|q| <= 65504); softmax statistics are fp32; out
 * is bf16 (RNE).
 *
 * Ownership and ordering.  The caller owns every buffer; the library keeps
 * no pointer after the call returns and allocates nothing.  The call is
 * asynchronous on `stream` (NULL = the null stream): it performs no host
 * synchronisation, no device-to-host copy and no host read of cu_seqlens,
 * so it may be captured in a HIP graph.  `out` must not overlap q, k or v.
 *
 * Errors.  Every argument check runs on the host before any HIP call; a
 * failing check returns its status and leaves a message for
 * attn_prefill_last_error().  There is no fallback to another head size,
 * dtype or to the CPU.  cu_seqlens lives on the device and is not read by
 * the host: the kernel clamps every offset into [0, n_tokens] and treats a
 * negative-length sequence as empty, so malformed offsets give wrong output
 * but no out-of-bounds access.  Setting ATTN_PREFILL_VALIDATE=1 in the
 * environment adds a debug-only host check of cu_seqlens that synchronises
 * the stream (never use it when timing or capturing).
 *
 * Grid shape.  For causal calls without a window whose grid would have at
 * most one workgroup per compute unit, each workgroup pairs a sequence's
 * query block r with block nb - 1 - r (nb blocks; 32 rows of four query
 * heads for head_dim 64 and 128, 64 rows of one head for head_dim 512), so
 * that every workgroup sees about the same number of keys; the output is
 * bitwise the same as with the plain grid.  ATTN_PREFILL_FOLD=0 or =1 in
 * the environment turns this off, or on wherever the head size and
 * grouping allow it (for tests of both grids).
 */
#ifndef ATTN_PREFILL_H
#define ATTN_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define ATTN_OK 0
#define ATTN_ERR_INVALID_ARG 1 /* argument outside the contract            */
#define ATTN_ERR_UNSUPPORTED 2 /* valid, but no kernel for it (head_dim,   */
                               /* dtype pair, alignment, grid size)        */
#define ATTN_ERR_HIP 3         /* launch or runtime error from HIP         */

/* element types */
#define ATTN_BF16 0
#define ATTN_FP16 1
#define ATTN_FP32 2

/* Same type as hipStream_t; declared here so that the header needs no HIP
 * include. */
typedef struct ihipStream_t* attn_stream_t;

/* One device tensor [n_tokens, n_heads, head_dim] (n_heads and head_dim are
 * the call's arguments).  Strides are in elements and must be >= 0; the
 * head vectors of different (token, head) pairs must not overlap.  data must
 * be 16-byte aligned and token_stride / head_stride must be multiples of
 * 16 bytes, else ATTN_ERR_UNSUPPORTED.  For k and v, 64 token strides must
 * span less than 2 GiB (token_stride * element size < 32 MiB), else
 * ATTN_ERR_UNSUPPORTED. */
typedef struct {
  void* data;           /* device pointer, caller-owned; may be NULL if
                           n_tokens == 0                                   */
  int32_t dtype;        /* q: BF16 | FP32;  k, v: BF16 | FP16 (equal);
                           out: BF16                                       */
  int32_t reserved;     /* must be 0                                       */
  int64_t n_tokens;     /* T; must agree across q, k, v and out            */
  int64_t token_stride; /* elements between consecutive tokens             */
  int64_t head_stride;  /* elements between consecutive heads              */
} attn_tensor;

/* Packed sequence offsets. */
typedef struct {
  const int32_t* data;  /* DEVICE int32[n_seqs + 1]: data[0] = 0,
                           non-decreasing, data[n_seqs] = n_tokens         */
  int32_t n_seqs;       /* >= 1                                            */
  int32_t max_seqlen;   /* optional hint (0 = unknown); unused today       */
} attn_seqlens;

/* Causal (optionally sliding-window) prefill attention, see above.
 *   n_q_heads >= 1, n_kv_heads >= 1, n_q_heads % n_kv_heads == 0
 *   head_dim: one of attn_prefill_supported_head_dims() (64, 128, 256, 512)
 *   scale: finite (0 and negative values allowed), applied to q.k before
 *          masking and softmax
 *   sliding_window: 0 = off, W > 0 = the W most recent keys including the
 *          query itself, < 0 = ATTN_ERR_INVALID_ARG
 * Returns ATTN_OK or an error status. */
int attn_prefill(const attn_tensor* q, const attn_tensor* k,
                 const attn_tensor* v, const attn_tensor* out,
                 const attn_seqlens* cu_seqlens, int32_t n_q_heads,
                 int32_t n_kv_heads, int32_t head_dim, float scale,
                 int32_t sliding_window, attn_stream_t stream);

/* Chunked prefill against a KV history.  A later prefill chunk attends to
 * every earlier token of its sequence, not only to the chunk (the
 * multi-chunk fix in atlas PR #69: later chunks use kv_len =
 * seq_len_start + n).  Sequence s has Lq = cu_seqlens_q[s+1] - cu_seqlens_q[s]
 * new queries in q / out and Lk = cu_seqlens_k[s+1] - cu_seqlens_k[s] >= Lq
 * keys and values in k / v: its history followed by the chunk's own tokens.
 * The queries are the sequence's last Lq positions, so local query i has
 * position p = Lk - Lq + i and sees the keys j <= p (and j >= p - W + 1 for
 * a window W > 0); with Lq == Lk this is attn_prefill.
 *   q, out: n_tokens = Tq (packed by cu_seqlens_q)
 *   k, v:   n_tokens = Tk (packed by cu_seqlens_k); Tk = 0 with Tq > 0 is
 *           ATTN_ERR_INVALID_ARG
 *   cu_seqlens_q, cu_seqlens_k: device offsets with the same n_seqs
 * Other arguments, layouts, precision, ownership and errors as for
 * attn_prefill.  Offsets are not read by the host; the kernel clamps them
 * into [0, Tq] and [0, Tk], and a query left without a visible key (only
 * possible with Lq > Lk, outside the contract) gets an all-zero row.
 * ATTN_PREFILL_VALIDATE=1 also checks Lq <= Lk per sequence. */
int attn_prefill_chunked(const attn_tensor* q, const attn_tensor* k,
                         const attn_tensor* v, const attn_tensor* out,
                         const attn_seqlens* cu_seqlens_q,
                         const attn_seqlens* cu_seqlens_k, int32_t n_q_heads,
                         int32_t n_kv_heads, int32_t head_dim, float scale,
                         int32_t sliding_window, attn_stream_t stream);

/* A paged K/V cache.  k and v are pools of token slots, n_tokens =
 * n_pages * page_size, page p holding slots [p * page_size, (p+1) *
 * page_size) of the usual [n_tokens, n_kv_heads, head_dim] descriptor.  Key
 * position j of sequence s is slot j % page_size of page
 * block_table[s * table_stride + j / page_size] (the paged MLA prefill in
 * atlas PR #69 reads every key through a page-table lookup; m40-llm
 * AGENTS.md, "Current Progress", addresses the cache per sequence and
 * position). */
typedef struct {
  const int32_t* block_table;  /* DEVICE int32[n_seqs * table_stride]: pages */
  const int32_t* seqlens_k;    /* DEVICE int32[n_seqs]: keys per sequence
                                  (history + the chunk's own tokens)       */
  int32_t table_stride;        /* entries per sequence row, >= 1           */
  int32_t page_size;           /* slots per page: a multiple of 64         */
} attn_paged_kv;

/* Chunked prefill whose keys and values are read from a paged cache: as
 * attn_prefill_chunked with sequence s's Lk = seqlens_k[s] keys at the
 * positions the block table maps (the chunk's own K/V must already be in
 * the cache).  q and out are packed by cu_seqlens_q; k_pool and v_pool are
 * the pools above (same dtype, same n_tokens).  page_size not a multiple
 * of 64 is ATTN_ERR_UNSUPPORTED; n_tokens not a multiple of page_size, an
 * empty pool with Tq > 0, table_stride < 1 or a NULL table pointer is
 * ATTN_ERR_INVALID_ARG.  The device metadata is not read by the host: the
 * kernel clamps seqlens_k into [0, table_stride * page_size] and every page
 * number into [0, n_pages), so bad metadata gives wrong output but stays in
 * bounds; ATTN_PREFILL_VALIDATE=1 checks it on the host. */
int attn_prefill_paged(const attn_tensor* q, const attn_tensor* k_pool,
                       const attn_tensor* v_pool, const attn_tensor* out,
                       const attn_seqlens* cu_seqlens_q,
                       const attn_paged_kv* paged, int32_t n_q_heads,
                       int32_t n_kv_heads, int32_t head_dim, float scale,
                       int32_t sliding_window, attn_stream_t stream);

/* The general prefill entry point: separate head sizes for the score
 * contraction (q, k: head_dim_qk) and for the values (v, out: head_dim_v),
 * with the key layout of attn_prefill (cu_seqlens_k and paged both NULL),
 * attn_prefill_chunked (cu_seqlens_k set) or attn_prefill_paged (paged
 * set; both set is ATTN_ERR_INVALID_ARG).  Supported pairs: (64, 64),
 * (128, 128), (256, 256), (512, 512) and (320, 256), the absorbed MLA
 * prefill of atlas PR #69 (q = [q_absorbed | q_rope] against the
 * compressed cache row
 * [kv_latent | k_rope], v = the kv_latent part of the same row -- a view of
 * k with the same token stride -- and scale 1/sqrt(320)); others are
 * ATTN_ERR_UNSUPPORTED. */
int attn_prefill_ex(const attn_tensor* q, const attn_tensor* k,
                    const attn_tensor* v, const attn_tensor* out,
                    const attn_seqlens* cu_seqlens_q,
                    const attn_seqlens* cu_seqlens_k, const attn_paged_kv* paged,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim_qk,
                    int32_t head_dim_v, float scale, int32_t sliding_window,
                    attn_stream_t stream);

/* attn_prefill_ex with a caller-provided workspace.  When a call has fewer
 * (query tile, head) pairs than about two per compute unit (a few long
 * sequences, or few query heads), the 64-key tiles each query tile sees are
 * cut into pieces of equal length computed by separate workgroups: a query
 * tile of more than one piece writes per-row running max, softmax sum and
 * unnormalised output (fp32) to the workspace, and a second kernel on the
 * same stream rescales the pieces to their common max and writes out, the
 * online-softmax combination applied across workgroups.  The result equals
 * attn_prefill_ex up to fp32 rounding order.  Splitting applies to head
 * sizes (64, 64) and (128, 128); other sizes, calls that already fill the
 * chip and workspaces smaller than attn_prefill_workspace_size() asks for
 * run exactly as attn_prefill_ex.
 *   workspace: device memory, 16-byte aligned, owned by the caller, not
 *              read before it is written, not overlapping q, k, v or out;
 *              may be NULL when workspace_bytes == 0
 * Calls that share a workspace on different streams race.  Other arguments
 * and errors as for attn_prefill_ex. */
int attn_prefill_ex_ws(const attn_tensor* q, const attn_tensor* k,
                       const attn_tensor* v, const attn_tensor* out,
                       const attn_seqlens* cu_seqlens_q,
                       const attn_seqlens* cu_seqlens_k,
                       const attn_paged_kv* paged, int32_t n_q_heads,
                       int32_t n_kv_heads, int32_t head_dim_qk,
                       int32_t head_dim_v, float scale, int32_t sliding_window,
                       void* workspace, size_t workspace_bytes,
                       attn_stream_t stream);

/* Workspace bytes with which attn_prefill_ex_ws splits a call on the
 * current device; 0 when it would not split.  n_tokens_q = q->n_tokens;
 * max_keys bounds any sequence's key count: k->n_tokens for packed or
 * chunked keys, table_stride * page_size for a paged cache.  For a single
 * sequence the library compares the finishing time of whole query tiles
 * with that of pieces (it knows every tile's key count) and splits only for
 * a clear gain; for several sequences it splits only grids with fewer
 * workgroups than compute units.  Planning a single sequence takes up to a
 * few hundred microseconds of host time; the plan of the last shape is kept
 * per thread, so repeated calls cost about a microsecond.  Call it once the
 * device is initialised (it reads the device's compute-unit count). */
size_t attn_prefill_workspace_size(int64_t n_tokens_q, int64_t max_keys,
                                   int32_t n_seqs, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t head_dim_qk,
                                   int32_t head_dim_v, int32_t sliding_window);

/* Decode: one new query token per sequence (the batched last-token step).
 * Sequence s's query q[s] sits at position Lk - 1 of its Lk keys and sees
 * all of them (with a window W > 0 the last W).  This is
 * attn_prefill_chunked with one query per sequence, computed by a kernel
 * that puts the query heads sharing a KV head on the MFMA columns and
 * splits each sequence's keys across four waves.
 *   q, out: n_tokens = n_seqs ([n_seqs, heads, head_dim], any strides)
 *   k, v:   packed keys, n_tokens = Tk, sequence s owning
 *           [cu_seqlens_k[s], cu_seqlens_k[s+1]); cu_seqlens_k->n_seqs must
 *           equal q->n_tokens
 *   head_dim: 128 only (else ATTN_ERR_UNSUPPORTED)
 * A sequence with no key (outside the contract) gets a zero row.  Other
 * arguments, precision, ownership and errors as for attn_prefill. */
int attn_decode(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                const attn_tensor* out, const attn_seqlens* cu_seqlens_k,
                int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                float scale, int32_t sliding_window, attn_stream_t stream);

/* Decode against a paged cache: as attn_decode with sequence s's
 * Lk = seqlens_k[s] keys read through the block table (attn_paged_kv
 * above; the table has q->n_tokens rows, page_size a multiple of 64). */
int attn_decode_paged(const attn_tensor* q, const attn_tensor* k_pool,
                      const attn_tensor* v_pool, const attn_tensor* out,
                      const attn_paged_kv* paged, int32_t n_q_heads,
                      int32_t n_kv_heads, int32_t head_dim, float scale,
                      int32_t sliding_window, attn_stream_t stream);

/* Decode with a caller-provided workspace.  When a batch has fewer
 * (sequence, KV head, 32-query-head block) units than half the compute
 * units, each unit's keys are split into up to 64 contiguous ranges computed
 * by separate workgroups; each writes its running max, softmax denominator
 * and unnormalised output (fp32) to the workspace, and a second kernel on
 * the same stream merges the ranges by rescaling each to the common max
 * (the online-softmax combination used within a kernel, applied across
 * workgroups).  The result equals attn_decode up to fp32 rounding order.
 *   workspace: device memory, 16-byte aligned, owned by the caller, not
 *              read before it is written, not overlapping q, k, v or out;
 *              may be NULL when workspace_bytes == 0 (then no split: the
 *              same kernel and result as attn_decode)
 *   workspace_bytes: its size; the number of ranges is reduced to what
 *              fits, so any size is valid
 * Calls that share a workspace on different streams race.  Other arguments
 * and errors as for attn_decode / attn_decode_paged. */
int attn_decode_ws(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                   const attn_tensor* out, const attn_seqlens* cu_seqlens_k,
                   int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                   float scale, int32_t sliding_window, void* workspace,
                   size_t workspace_bytes, attn_stream_t stream);
int attn_decode_paged_ws(const attn_tensor* q, const attn_tensor* k_pool,
                         const attn_tensor* v_pool, const attn_tensor* out,
                         const attn_paged_kv* paged, int32_t n_q_heads,
                         int32_t n_kv_heads, int32_t head_dim, float scale,
                         int32_t sliding_window, void* workspace,
                         size_t workspace_bytes, attn_stream_t stream);

/* Workspace bytes with which attn_decode_ws / attn_decode_paged_ws use
 * their preferred split on the current device for a batch of n_seqs
 * sequences; 0 when that batch would not be split or the arguments are not
 * a supported decode shape. */
size_t attn_decode_workspace_size(int64_t n_seqs, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim);

/* Decode that allocates nothing, for callers that cannot call hipMalloc:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The same operation, arguments and result as attn_decode_ws
 * given attn_decode_workspace_size() bytes of workspace (the same split of
 * the keys, bitwise the same output), with the split's partial results kept
 * in a static device array of the library instead of a caller workspace:
 * 4,259,840 bytes (256 partial blocks of 16,640 bytes), which every GPU the
 * library runs on holds from the first split call on that device until the
 * process ends.  A batch whose split would need more (only possible on a
 * device of more than 256 compute units) is rejected with
 * ATTN_ERR_UNSUPPORTED and a message naming both sizes; attn_decode_ws
 * serves it.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (on different streams, or from different
 * threads) race; calls on one stream are ordered.  Nothing in the array
 * needs clearing between calls: each split call writes every partial it
 * reads.  Other arguments, precision and errors as for attn_decode. */
int attn_decode_noalloc(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                        const attn_tensor* out, const attn_seqlens* cu_seqlens_k,
                        int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                        float scale, int32_t sliding_window, attn_stream_t stream);

/* Static description of a status code (never NULL). */
const char* attn_prefill_status_string(int status);

/* Detail message of the calling thread's last failing call ("" if none).
 * The pointer stays valid until the thread's next call into the library. */
const char* attn_prefill_last_error(void);

/* Writes up to `cap` supported head_dim values into `dims` (may be NULL when
 * cap == 0) and returns how many exist. */
int attn_prefill_supported_head_dims(int32_t* dims, int32_t cap);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int attn_prefill_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PREFILL_H */
