// Decode attention forward for gfx950 (CDNA4): one new query token per
// sequence against the sequence's keys -- the batched last-token GQA step of
// the m40-llm AGENTS.md page ("Current Progress", decode plans over mixed KV
// lengths) and the next-token position of the causal bound kv_end =
// min(q_pos + 1, seq_len) of the fused MLA prefill (atlas PR #69).
//
//   for sequence s with L keys (packed by cu_seqlens_k, or L = seqlens_k[s]
//   read through a block table), KV head g and its query heads h:
//     out[s,h] = sum_{j visible} softmax_j(scale * q[s,h] . k[j,g]) v[j,g]
//   where the query sits at position L - 1: every key j < L is visible, or
//   with a window W > 0 the keys j >= L - W.  L = 0 leaves a zero row.
//
// Design (ours, for CDNA4):
//   * One workgroup per (sequence, KV head, block of 32 query heads): the
//     query heads that share a KV head are the 32 columns of the MFMA, so
//     Sᵀ = K Qᵀ and Oᵀ += Vᵀ Pᵀ run on the 32x32x16 MFMA of the K/V storage
//     type (bf16 or fp16, K and V as stored) exactly as in the prefill
//     kernel, with heads in place of query tokens (MQA with
//     32 query heads fills the columns; smaller groups leave some empty).
//   * Four waves, one per SIMD, split the key range into contiguous slices
//     of 64-key tiles and stream their slice independently: each tile is
//     loaded with coalesced 16-byte loads into registers one tile ahead and
//     stored into the wave's own LDS slice with the
//     16-byte chunks of row r at position (chunk ^ (r & 15)); K operands are
//     read back row-wise, Vᵀ operands with the transposing LDS read
//     ds_read_b64_tr_b16 (four keys of one column per lane per read).
//   * The online softmax is the prefill kernel's (base 2, lazy max); at the
//     end the four waves' (max, sum, Oᵀ) are merged through LDS and each wave
//     normalises and stores one 32-wide block of head_dim.
//   * Rows of a tile past the key count read as zero through the buffer
//     range, so padded keys are masked finite values.
//   * The grid visits the sequences longest first (each workgroup ranks the
//     batch's tile counts in LDS, up to 256 sequences), so that uneven
//     lengths do not leave CUs idle at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "prefill_params.h"

namespace attnp {
namespace {

using namespace dev;

typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kDWave = 64;
constexpr int kDWaves = 4;                 // one per SIMD
constexpr int kDThreads = kDWave * kDWaves;
constexpr int kDBN = 64;                   // keys per tile
constexpr int kDHeads = 32;                // query heads per workgroup (MFMA columns)
constexpr float kDLazy = 8.0f;             // lazy-max threshold, log2 units
constexpr int kDSortMax = 256;             // largest batch ranked by length

template <int HDIM, class QT, class KVT, bool PAGED>
__global__ __launch_bounds__(kDThreads, 1) void decode_fwd_kernel(DecodeParams p) {
  static_assert(HDIM == 128, "decode is instantiated for 128-d heads");
  constexpr int CPR = HDIM / 8;            // 16-byte chunks per row
  constexpr int DCH = HDIM / 16;           // score k-steps
  constexpr int DBLK = HDIM / 32;          // output row blocks
  constexpr int TILE = kDBN * HDIM;        // elements of one K (or V) tile
  constexpr int LOADS = kDBN * CPR / kDWave;  // 16-byte chunks per lane per tile
  static_assert(DBLK == kDWaves, "one output block per wave");
  typedef typename QT::T qelem;
  typedef typename KVT::T kvelem;
  typedef typename OpOf<KVT>::T OP;  // operand type of both products
  typedef typename OP::v8 opv8;

  // Per wave: K tile then V tile (rows of HDIM, chunks swizzled).
  // After the key loop the same memory holds the merge buffers.
  __shared__ __attribute__((aligned(16))) uint16_t smem[kDWaves * 2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & (kDWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kDWave);
  const int col = lane & 31;    // head column
  const int half = lane >> 5;

  const int hblocks = (p.group + kDHeads - 1) / kDHeads;
  const int per_seq = hblocks * p.n_kv_heads;  // units of one sequence
  const int bid = dispatch_index(blockIdx.x);
  const int split = bid % p.n_splits;
  const int order = bid / p.n_splits;
  if (order >= p.n_seqs * per_seq) return;  // past the work (uniform)
  const int rank = order / per_seq;
  const int sub = order - rank * per_seq;
  const int hb = sub % hblocks;
  const int g = sub / hblocks;

  // keys of sequence i (clamped into the key buffer or the table row) and
  // the 64-key tiles they take with the window
  auto seq_keys = [&](int i, int* start) -> int {
    if (PAGED) {
      *start = 0;
      return min(max(p.seqlens_k[i], 0), p.table_stride * p.page_size);
    }
    const int a = min(max(p.cu_seqlens_k[i], 0), p.n_tokens_k);
    const int b = min(max(p.cu_seqlens_k[i + 1], 0), p.n_tokens_k);
    *start = a;
    return max(b - a, 0);
  };
  auto seq_tiles = [&](int keys) -> int {
    const int lo = p.window > 0 ? max(0, keys - p.window) : 0;
    return keys > 0 ? (keys - (lo - lo % kDBN) + kDBN - 1) / kDBN : 0;
  };

  // ---- longest sequences first.  Units of uneven length taken in
  // sequence order leave CUs idle at the end (a third of the time for
  // lengths spread evenly over 512..8191); the grid therefore visits the
  // sequences in decreasing order of tiles (ties by index) when the batch
  // is small enough to rank in LDS, else in sequence order.
  int s = rank;
  if (p.n_seqs <= kDSortMax) {
    __shared__ int wts[kDSortMax];
    __shared__ int pick;
    for (int i = tid; i < p.n_seqs; i += kDThreads) {
      int st;
      wts[i] = seq_tiles(seq_keys(i, &st));
    }
    __syncthreads();
    for (int i = tid; i < p.n_seqs; i += kDThreads) {
      const int wi = wts[i];
      int r = 0;
      for (int j = 0; j < p.n_seqs; ++j) {
        const int wj = wts[j];
        r += (wj > wi || (wj == wi && j < i)) ? 1 : 0;
      }
      if (r == rank) pick = i;  // ranks are a permutation: exactly one match
    }
    __syncthreads();
    s = pick;
  }
  s = __builtin_amdgcn_readfirstlane(s);
  const int unit = s * per_seq + sub;  // the merge kernel's unit numbering

  int kstart = 0;
  int L = seq_keys(s, &kstart);
  kstart = __builtin_amdgcn_readfirstlane(kstart);
  L = __builtin_amdgcn_readfirstlane(L);
  const int kv_lo = p.window > 0 ? max(0, L - p.window) : 0;
  const int kv_start = kv_lo - kv_lo % kDBN;
  const int n_t = seq_tiles(L);
  // this workgroup's contiguous share of the tiles, then this wave's
  const int g_begin = split * n_t / p.n_splits;
  const int g_cnt = (split + 1) * n_t / p.n_splits - g_begin;
  const int t_begin = __builtin_amdgcn_readfirstlane(g_begin + wave * g_cnt / kDWaves);
  const int t_end = __builtin_amdgcn_readfirstlane(g_begin + (wave + 1) * g_cnt / kDWaves);

  const int hcol = hb * kDHeads + col;     // head index inside the group
  const bool hvalid = hcol < p.group;
  const int head = g * p.group + (hvalid ? hcol : 0);

  // ---- tile loads: lane moves chunk (lane % CPR) of rows 4i + lane / CPR
  const kvelem* kbase = static_cast<const kvelem*>(p.k) + (int64_t)g * p.k_hs;
  const kvelem* vbase = static_cast<const kvelem*>(p.v) + (int64_t)g * p.v_hs;
  const int k_row_bytes = (int)(p.k_ts * (int64_t)sizeof(kvelem));
  const int v_row_bytes = (int)(p.v_ts * (int64_t)sizeof(kvelem));
  auto tile_slot = [&](int kv0) -> int64_t {
    if (!PAGED) return (int64_t)kstart + kv0;
    const int* row = p.block_table + (int64_t)s * p.table_stride;
    const int idx = __builtin_amdgcn_readfirstlane(kv0 / p.page_size);
    const int page = min(max(row[idx], 0), p.n_pages - 1);
    return (int64_t)page * p.page_size + (kv0 - idx * p.page_size);
  };
  u32x4_t kr[LOADS], vr[LOADS];
  auto gload = [&](int kv0) {
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(L - kv0, kDBN)));
    const int64_t slot = tile_slot(kv0);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<kvelem*>(kbase + slot * p.k_ts), 0, rows * k_row_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<kvelem*>(vbase + slot * p.v_ts), 0, rows * v_row_bytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int row = i * (kDWave / CPR) + lane / CPR;
      const int ch = lane % CPR;
      kr[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, row * k_row_bytes + 16 * ch, 0, 0);
      vr[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, row * v_row_bytes + 16 * ch, 0, 0);
    }
  };
  uint16_t* const kt = smem + wave * 2 * TILE;
  uint16_t* const vt = kt + TILE;
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int row = i * (kDWave / CPR) + lane / CPR;
      const int pos = (lane % CPR) ^ (row & 15);
      *reinterpret_cast<u32x4_t*>(kt + row * HDIM + 8 * pos) = kv_to_op(OP(), KVT(), kr[i]);
      *reinterpret_cast<u32x4_t*>(vt + row * HDIM + 8 * pos) = kv_to_op(OP(), KVT(), vr[i]);
    }
  };

  // ---- per-wave state
  f32x16_t o[DBLK];
#pragma unroll
  for (int c = 0; c < DBLK; ++c) o[c] = (f32x16_t){};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float cmul = p.score_mult;

  // first tile in flight before Q, so that the two latencies overlap
  if (t_begin < t_end) gload(kv_start + t_begin * kDBN);

  // ---- Qᵀ operand: lane holds q[s, head, 16c + 8*half .. +7], zeroed for a
  // column past the group (head is clamped to a real head, so every load is
  // in bounds and none waits behind a branch)
  opv8 qf[DCH];
  {
    const qelem* qp = static_cast<const qelem*>(p.q) + (int64_t)s * p.q_ts +
                      (int64_t)head * p.q_hs;
    load_q_op<DCH, OP>(qp, half, hvalid ? p.q_mult : 0.f, qf);
  }

  for (int t = t_begin; t < t_end; ++t) {
    const int kv0 = kv_start + t * kDBN;
    lstore();  // tile t: registers -> this wave's LDS slice
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (t + 1 < t_end) gload(kv0 + kDBN);  // tile t+1 in flight meanwhile

    // Sᵀ = K Qᵀ: keys on M (two 32-key blocks), heads on N
    f32x16_t sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = (f32x16_t){};
      const int row = 32 * kb + col;
#pragma unroll
      for (int c = 0; c < DCH; ++c) {
        const int pos = (2 * c + half) ^ (row & 15);
        const opv8 a = *reinterpret_cast<const opv8*>(kt + row * HDIM + 8 * pos);
        sc[kb] = OP::mfma(a, qf[c], sc[kb]);
      }
    }
    // mask the window start and the key count (first and last tiles only)
    if (kv0 < kv_lo || kv0 + kDBN > L) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key < kv_lo || key >= L) sc[kb][r] = -INFINITY;
        }
    }
    // online softmax (lazy max, base 2) into the Pᵀ operand
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    mx = pair_max(mx);
    const bool raise = (mx - m_run) * cmul > kDLazy;
    const bool any = __ballot(raise) != 0ull;
    const float m_new = any ? fmaxf(m_run, mx) : m_run;
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2((m_run - m_new) * cmul);
    const float neg_mc = (m_new == -INFINITY) ? 0.f : -m_new * cmul;
    m_run = m_new;
    opv8 pf[4];
    float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      u32x4_t u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(fmaf(sc[kq >> 1][8 * (kq & 1) + 2 * e], cmul, neg_mc));
        const float p1 = fast_exp2(fmaf(sc[kq >> 1][8 * (kq & 1) + 2 * e + 1], cmul, neg_mc));
        const typename OP::v2 pb = OP::cvt2(p0, p1);
        u[e] = __builtin_bit_cast(uint32_t, pb);
        l4[e] = OP::sum2(pb, l4[e]);
      }
      pf[kq] = __builtin_bit_cast(opv8, u);
    }
    l_run = l_run * alpha + ((l4[0] + l4[1]) + (l4[2] + l4[3]));
    if (any) {
#pragma unroll
      for (int c = 0; c < DBLK; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
    }

    // Oᵀ += Vᵀ Pᵀ.  MFMA k-index 8*half + e of step kq is key
    // 16*kq + 8*(e / 4) + 4*half + e % 4 (the Sᵀ accumulator's order): two
    // transposing reads give keys +0..3 and +8..11 (+4*half) of column d.
    const int grp = (lane >> 4) & 1;   // 16-column half of the 32-row block
    const int j = lane & 15;
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
#pragma unroll
      for (int c = 0; c < DBLK; ++c) {
        s16x4_t part[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = 16 * kq + 8 * r + 4 * half + (j >> 2);
          const int d = 32 * c + 16 * grp + 4 * (j & 3);
          const int pos = (d >> 3) ^ (row & 15);
          part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t*)(vt + row * HDIM + 8 * pos + (d & 7)));
        }
        u32x4_t u;
        u[0] = __builtin_bit_cast(u32x2_t, part[0])[0];
        u[1] = __builtin_bit_cast(u32x2_t, part[0])[1];
        u[2] = __builtin_bit_cast(u32x2_t, part[1])[0];
        u[3] = __builtin_bit_cast(u32x2_t, part[1])[1];
        o[c] = OP::mfma(__builtin_bit_cast(opv8, u), pf[kq], o[c]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge the four waves' partial results through LDS
  __syncthreads();
  float* const cw = reinterpret_cast<float*>(smem);  // [wave][c][r][lane]
  float* const mw = cw + kDWaves * DBLK * 16 * kDWave;  // [wave][col]
  float* const lw = mw + kDWaves * 32;
#pragma unroll
  for (int c = 0; c < DBLK; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) cw[((wave * DBLK + c) * 16 + r) * kDWave + lane] = o[c][r];
  const float l_tot = pair_sum(l_run);
  if (half == 0) {
    mw[wave * 32 + col] = m_run;
    lw[wave * 32 + col] = l_tot;
  }
  __syncthreads();
  float mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < kDWaves; ++w) mx = fmaxf(mx, mw[w * 32 + col]);
  float wt[kDWaves];
  float den = 0.f;
#pragma unroll
  for (int w = 0; w < kDWaves; ++w) {
    const float mwv = mw[w * 32 + col];
    wt[w] = (mwv == -INFINITY) ? 0.f : fast_exp2((mwv - mx) * cmul);
    den += wt[w] * lw[w * 32 + col];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;  // no visible key: zero row
  const int c = wave;                             // this wave's output block
  if (p.n_splits > 1) {
    // unnormalised partial of this split: max (raw score units), sum and
    // values relative to that max; merged by decode_merge_kernel
    float* part = p.partial + ((int64_t)unit * p.n_splits + split) * decode_partial_floats(HDIM);
    if (wave == 0 && half == 0) {
      part[col] = mx;
      part[32 + col] = den;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < kDWaves; ++w)
        acc += wt[w] * cw[((w * DBLK + c) * 16 + r) * kDWave + lane];
      const int d = 32 * c + 8 * (r >> 2) + 4 * half + (r & 3);
      part[64 + d * 32 + col] = acc;
    }
    return;
  }
  if (hvalid) {
    uint16_t* op = static_cast<uint16_t*>(p.out) + (int64_t)s * p.o_ts + (int64_t)head * p.o_hs;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kDWaves; ++w)
          acc += wt[w] * cw[((w * DBLK + c) * 16 + 4 * rb + i) * kDWave + lane];
        v[i] = acc * inv;
      }
      u32x2_t pk;
      pk[0] = pack_bf16x2(v[0], v[1]);
      pk[1] = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<u32x2_t*>(op + 32 * c + 8 * rb + 4 * half) = pk;
    }
  }
}

// Merges the n_splits partials of one (sequence, KV head, head block):
// out = sum_i o_i 2^((m_i - M) c) / sum_i l_i 2^((m_i - M) c), M = max_i m_i.
// Workgroup (unit, slab) handles 16 of the head_dim values of the unit's 32
// heads: thread (col, pair) reads the split partials of two values, and a
// wave's 32 columns read 128 contiguous bytes per value.
constexpr int kMergeSlab = 16;
constexpr int kMergeChunk = 16;  // splits combined per round of loads

template <int HDIM>
__global__ __launch_bounds__(kDThreads) void decode_merge_kernel(DecodeParams p) {
  constexpr int SLABS = HDIM / kMergeSlab;
  constexpr int PF = decode_partial_floats(HDIM);
  const int hblocks = (p.group + kDHeads - 1) / kDHeads;
  const int wid = blockIdx.x / SLABS;
  const int slab = blockIdx.x % SLABS;
  const int hb = wid % hblocks;
  const int g = (wid / hblocks) % p.n_kv_heads;
  const int s = wid / (hblocks * p.n_kv_heads);
  const int col = threadIdx.x & 31;
  const int d = slab * kMergeSlab + 2 * (threadIdx.x >> 5);
  const int hcol = hb * kDHeads + col;
  if (hcol >= p.group) return;
  const int head = g * p.group + hcol;
  const float* base = p.partial + (int64_t)wid * p.n_splits * PF;
  const int n = p.n_splits;
  // Splits in chunks of kMergeChunk, every load of a chunk issued before any
  // is used (one memory latency per chunk), combined online: the sums so far
  // are rescaled to the chunk's new max.  With n <= kMergeChunk this is the
  // single combination relative to the overall max.
  float mx = -INFINITY, den = 0.f, a0 = 0.f, a1 = 0.f;
  for (int i0 = 0; i0 < n; i0 += kMergeChunk) {
    float m[kMergeChunk], l[kMergeChunk], v0[kMergeChunk], v1[kMergeChunk];
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) {
      const float* part = base + (int64_t)(i0 + j) * PF;
      const bool in = i0 + j < n;
      m[j] = in ? part[col] : -INFINITY;
      l[j] = in ? part[32 + col] : 0.f;
      v0[j] = in ? part[64 + d * 32 + col] : 0.f;
      v1[j] = in ? part[64 + (d + 1) * 32 + col] : 0.f;
    }
    float cm = mx;
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) cm = fmaxf(cm, m[j]);
    // (the sums are still zero while mx = -inf)
    const float r = mx == -INFINITY ? 0.f : fast_exp2((mx - cm) * p.score_mult);
    den *= r;
    a0 *= r;
    a1 *= r;
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) {
      const float w = m[j] == -INFINITY ? 0.f : fast_exp2((m[j] - cm) * p.score_mult);
      den += w * l[j];
      a0 += w * v0[j];
      a1 += w * v1[j];
    }
    mx = cm;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint16_t* op = static_cast<uint16_t*>(p.out) + (int64_t)s * p.o_ts + (int64_t)head * p.o_hs;
  *reinterpret_cast<uint32_t*>(op + d) = pack_bf16x2(a0 * inv, a1 * inv);
}

template <class QT, class KVT>
hipError_t launch_decode_one(const DecodeParams& p, hipStream_t stream) {
  const int64_t hblocks = (p.group + kDHeads - 1) / kDHeads;
  const uint64_t units = (uint64_t)p.n_seqs * (uint64_t)p.n_kv_heads * (uint64_t)hblocks;
  const uint64_t blocks = dispatch_grid(units * (uint64_t)p.n_splits);
  if (p.page_size > 0)
    hipLaunchKernelGGL((decode_fwd_kernel<128, QT, KVT, true>), dim3((uint32_t)blocks),
                       dim3(kDThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_fwd_kernel<128, QT, KVT, false>), dim3((uint32_t)blocks),
                       dim3(kDThreads), 0, stream, p);
  if (p.n_splits > 1)
    hipLaunchKernelGGL((decode_merge_kernel<128>), dim3((uint32_t)(units * (128 / kMergeSlab))),
                       dim3(kDThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int decode_kv_tile() { return kDBN; }

hipError_t launch_decode(const DecodeParams& p, int head_dim, DType q_dtype, DType kv_dtype,
                         hipStream_t stream) {
  if (head_dim != 128) return hipErrorInvalidValue;
  if (q_dtype == kBF16 && kv_dtype == kBF16) return launch_decode_one<BF16, BF16>(p, stream);
  if (q_dtype == kBF16 && kv_dtype == kFP16) return launch_decode_one<BF16, FP16>(p, stream);
  if (q_dtype == kFP32 && kv_dtype == kBF16) return launch_decode_one<FP32, BF16>(p, stream);
  if (q_dtype == kFP32 && kv_dtype == kFP16) return launch_decode_one<FP32, FP16>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attnp
