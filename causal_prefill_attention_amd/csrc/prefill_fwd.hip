// Causal / sliding-window prefill attention forward for gfx950 (CDNA4).
//
// What is computed (one workgroup = one query tile of one query head, or
// of four query heads that share a KV head):
//   out[i,h] = sum_j softmax_j(scale * q[i,h] . k[j,g]) v[j,g],
//   j visible iff j <= i (causal bound kv_end = min(q_pos + 1, seq_len), atlas
//   PR #69 fused MLA prefill) and, for a window W > 0, j >= i - W + 1 (the W
//   most recent keys, m40-llm AGENTS.md "Current Progress").  With a KV
//   history (chunked prefill: a later chunk attends to every earlier token,
//   kv_len = seq_len_start + n in atlas PR #69) the sequence has Lk keys and
//   Lq <= Lk queries, the queries being its last Lq positions: i above is
//   the query's key position Lk - Lq + (local query index).  The softmax is
//   evaluated online over key tiles with a running max and running sum (the
//   fused MLA prefill kernel's recurrence in atlas PR #69), in base 2 with
//   log2(e) folded into the score multiplier.
//
// Design (ours, for CDNA4 -- the pages' GB10 / M40 kernels are prior art):
//   * 8 waves per workgroup, two per SIMD, 32 query rows per wave, 256 rows
//     per workgroup (256 of one head, or 64 of each of four heads sharing a
//     KV head), 64-key tiles.  The waves form two groups (A = waves 0-3,
//     B = waves 4-7; wave w and w + 4 share a SIMD) that run in anti-phase:
//     in each barrier-delimited slot one group issues its matrix work
//     [P(j-1) V(j-1), then S(j) = K(j) Q^T] while the other runs the softmax
//     of its previous tile on the vector ALU, so the SIMD's matrix core and
//     vector ALU are fed by different waves.  K(j) and V(j-1) stay in LDS for
//     both slots; group A stages the next K tiles (in its softmax slot) and
//     group B the next V tiles (after its matrix work) into the other LDS
//     buffers.
//   * Q enters through LDS: each wave loads its 32 rows whole (a lane per
//     16-byte chunk, several rows per load instruction), rounds them into
//     its own LDS slice and reads the MFMA operand layout back.
//   * Folded grids (causal, no window, about one workgroup per CU): group A
//     takes a sequence's 32-row block r and group B its mirror nb - 1 - r,
//     so every workgroup sees about the same number of keys.
//   * Both contractions run on the 32x32x16 MFMA of the K/V storage type
//     (bf16 K/V: v_mfma_f32_32x32x16_bf16; fp16 K/V: ..._f16, so keys and
//     values enter the products as stored) with fp32 accumulation; Q and P
//     are rounded to that type.
//     Scores are formed transposed, S^T = K Q^T (keys on the MFMA M axis,
//     queries on N), so every lane owns one query column: the per-query max
//     and sum reduce 16 values in-lane plus one lane-pair exchange
//     (v_permlane32_swap), and the softmax row scale is one scalar per lane.
//   * The S^T accumulator, rounded to the operand type, is directly the B operand of
//     O^T += V^T P^T.  The key order inside each 16-key MFMA step follows the
//     accumulator layout; V^T is written into LDS in that permuted order.
//   * The running max moves lazily and is not taken on the common tile: the
//     probabilities are formed against the running reference m_run, and
//     only when a lane's sum of them exceeds a cap (2^32 for bf16 operands,
//     2^15 for fp16 ones, so that every probability stays in the operand's
//     range), or on a row's first visible tile, does the wave take the
//     tile's max, move m_run to it, rescale O and l and form the
//     probabilities again (a rare wave-uniform branch).  l sums the rounded
//     probabilities with v_dot2 so it matches what P.V uses.
//   * Masks are applied only to tiles that straddle the diagonal or the
//     window edge.  Every wave runs every tile of its workgroup; a tile none
//     of its rows can see is fully masked and adds exact zeros.
//   * The epilogue stages each wave's normalised 32 x HDIM bf16 tile in its
//     own LDS slice and stores whole rows, one 16-byte chunk per lane.
//   * K/V tiles are read with buffer loads whose range covers only the
//     tile's valid rows: keys past the tile's last query or the sequence read
//     as zero with no branch and no vector address arithmetic.
//   * Varlen: the grid covers an upper bound of q-tile slots; each workgroup
//     decodes its (sequence, tile) from cu_seqlens with a wave-wide scan, so
//     the host never reads the offsets.  Each sequence's tiles run heaviest
//     (last) first.  Offsets are clamped into [0, T].
//   * Every global address is token * token_stride + head * head_stride in
//     64-bit elements with head_dim explicit: a 128-d head is never read or
//     written with another head size's extent (the HDIM=256-on-128 overread
//     fixed in atlas PR #69).
#include <hip/hip_runtime.h>
#include <climits>
#include <stdint.h>

#include "device_common.h"
#include "prefill_params.h"
#include "prefill_work.h"

namespace attnp {
namespace {

using namespace dev;

constexpr int kWave = 64;
constexpr int kWaves = 8;      // two groups of four, one wave of each per SIMD
constexpr int kThreads = kWave * kWaves;
constexpr int kBN = 64;        // keys per KV tile: two 32-key MFMA blocks
constexpr int kKB = kBN / 32;
constexpr int kKT = kBN / 16;  // 16-key MFMA k-steps of the P.V contraction
constexpr int kBM = 32 * kWaves;  // query rows per workgroup

template <int HDIM>
struct Cfg {
  static_assert(HDIM % 32 == 0, "head_dim must be a multiple of 32");
  static constexpr int KSTR = HDIM + 8;  // K row pitch in LDS (16-bit elements)
  static constexpr int VSTR = kBN + 8;   // V^T row pitch in LDS (16-bit elements)
  static constexpr int K_ELEMS = kBN * KSTR;
  static constexpr int V_ELEMS = HDIM * VSTR;
  static constexpr int DCH = HDIM / 16;   // MFMA k-steps of the Q.K contraction
  static constexpr int DBLK = HDIM / 32;  // 32-wide output column blocks
  static constexpr int OCTS = HDIM / 8;   // 16-byte chunks per row
  // Group A's 256 threads stage K, group B's stage V.
  static constexpr int STAGERS = kThreads / 2;
  static constexpr int K_TOTAL = kBN * OCTS;         // 16-byte K chunks per tile
  static constexpr int V_TOTAL = (kBN / 4) * OCTS;   // 4-key x 8-d V units per tile
  static constexpr int K_CHUNKS = (K_TOTAL + STAGERS - 1) / STAGERS;  // per thread
  static constexpr int V_UNITS = (V_TOTAL + STAGERS - 1) / STAGERS;   // per thread
  static constexpr int NPV = DBLK * (kBN / 16);  // P.V MFMAs per tile
  static constexpr int NS = DCH * (kBN / 32);    // score MFMAs per tile
};

// ---------------------------------------------------------------- element io

// ------------------------------------------------------------------ kernel
// Key range of one query tile: 64-key tiles [kv_start, kv_start + 64 n) up
// to the tile's last visible key (kv_hi), from the window start on.
struct KeyRange {
  int hist, kv_hi, kv_start, n_tiles;
};
template <int BM>
__device__ __forceinline__ KeyRange key_range(const PrefillParams& p, const Work& w) {
  KeyRange r;
  // Queries are the last len of the sequence's klen positions: local query
  // i sits at key position hist + i (hist = 0 without a KV history).
  r.hist = w.klen - w.len;
  const int q_end = min(w.len, w.q0 + BM);
  // the tile's last query sees keys < hist + q_end
  r.kv_hi = min(max(r.hist + q_end, 0), w.klen);
  const int kv_lo = p.window > 0 ? min(max(0, r.hist + w.q0 - p.window + 1), r.kv_hi) : 0;
  r.kv_start = kv_lo - kv_lo % kBN;
  // at least one (then fully masked) tile keeps the slot schedule uniform
  // when no key is visible, which only malformed offsets produce
  r.n_tiles = max(1, (r.kv_hi - r.kv_start + kBN - 1) / kBN);
  return r;
}

// SPLIT: the workgroup runs piece (blockIdx / heads) % max_pieces of its
// query tile's key tiles; a tile of more than one piece leaves fp32
// partials for prefill_merge_kernel instead of its output.
// HP: query heads per workgroup.  With HP = 4 (the heads of one group of
// four sharing a KV head) the workgroup covers 64 rows of each of the four
// heads: wave w runs head 4 * group_index + w % 4 on rows 32 * (w / 4) ..
// +31 of the tile, so every K/V tile staged in LDS serves four heads and a
// query tile's causal diagonal spans one key tile instead of four.
// FOLD (HP = 4, causal without a window): group A runs the 32-row block r
// of the sequence and group B its mirror nb - 1 - r, so a workgroup's work
// no longer grows with its position in the sequence.  Both see key tiles
// from 0; group B, the later block, sees at least as many, and group A
// stops its matrix and softmax work after its own last key tile (it keeps
// staging K and passing the barriers), leaving the SIMDs to group B.
template <int HDIM, class QT, class KVT, bool PAGED, bool SPLIT, int HP, bool FOLD>
__global__ __launch_bounds__(kThreads, 1) void prefill_fwd_kernel(PrefillParams p) {
  static_assert(HP == 1 || (HP == 4 && !SPLIT), "head packing is for unsplit tiles");
  static_assert(!FOLD || HP == 4, "folded grids pack four heads");
  constexpr int BMQ = FOLD ? 32 : kBM / HP;  // query rows per head (per group when folded)
  using C = Cfg<HDIM>;
  typedef typename QT::T qelem;
  typedef typename KVT::T kvelem;
  typedef typename OpOf<KVT>::T OP;  // operand type of both products
  typedef typename OP::v8 opv8;
  // K stages [2][kBN][KSTR], V^T stages [2][HDIM][VSTR] (operand bits), then
  // one 32-row slice per wave (Q on the way in, O on the way out).
  constexpr int QSTR = HDIM + 8;  // slice row pitch (16-bit elements)
  __shared__ __attribute__((aligned(16)))
  uint16_t smem[2 * C::K_ELEMS + 2 * C::V_ELEMS + kWaves * 32 * QSTR];
  uint16_t* const kstage0 = smem;
  uint16_t* const vstage0 = smem + 2 * C::K_ELEMS;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  uint16_t* const slice = smem + 2 * C::K_ELEMS + 2 * C::V_ELEMS + wave * 32 * QSTR;
  const int group = wave >> 2;                                   // 0 = A, 1 = B
  const int n_units = p.n_q_heads / HP;       // workgroups per tile slot (and piece)
  // (unsplit grids run in dispatch order: dispatch_index)
  const int bid = SPLIT ? (int)blockIdx.x : dispatch_index(blockIdx.x);
  const int unit = bid / n_units;             // slot, or slot * max_pieces + piece
  const int hbase = (bid - unit * n_units) * HP;
  const int head = hbase + (HP == 1 ? 0 : (wave & (HP - 1)));  // wave-uniform
  const int slot = SPLIT ? unit / p.max_pieces : unit;
  const int piece = SPLIT ? unit - slot * p.max_pieces : 0;
  Work w = decode_work<BMQ, PAGED, FOLD>(p, slot);
  if (!w.valid) return;  // uniform across the workgroup
  w.start = __builtin_amdgcn_readfirstlane(w.start);
  w.len = __builtin_amdgcn_readfirstlane(w.len);
  w.q0 = __builtin_amdgcn_readfirstlane(w.q0);
  w.q0_b = __builtin_amdgcn_readfirstlane(w.q0_b);
  w.kstart = __builtin_amdgcn_readfirstlane(w.kstart);
  w.seq = __builtin_amdgcn_readfirstlane(w.seq);
  w.klen = __builtin_amdgcn_readfirstlane(w.klen);

  const int kvh = hbase / p.group;  // the same for every head of the workgroup
  // Folded: the key range is group B's (the mirror block, kv_start 0); group
  // A's tiles are its first n_a (none when the two blocks coincide).
  Work wb = w;
  wb.q0 = w.q0_b;
  const KeyRange kr = key_range<BMQ>(p, wb);
  const bool a_live = !FOLD || w.q0 != w.q0_b;
  const int n_a = FOLD ? (a_live ? key_range<BMQ>(p, w).n_tiles : 0) : kr.n_tiles;
  const int hist = kr.hist;
  const int kv_hi = kr.kv_hi;
  int kv_start = kr.kv_start;
  int n_tiles = kr.n_tiles;
  int n_pieces = 1;
  if (SPLIT) {
    // at most max_pieces pieces (the grid's and the workspace's bound); the
    // last one takes every remaining tile
    n_pieces = min((n_tiles + p.piece_tiles - 1) / p.piece_tiles, p.max_pieces);
    if (piece >= n_pieces) return;  // uniform: this tile has fewer pieces
    kv_start += piece * p.piece_tiles * kBN;
    n_tiles = piece == n_pieces - 1 ? n_tiles - piece * p.piece_tiles : p.piece_tiles;
  }

  const int col = lane & 31;   // query column of this lane
  const int half = lane >> 5;  // which 8-wide half of each 16-wide k-step
  // first row of this wave (a folded idle group A gets rows past the sequence)
  const int wq0 = FOLD ? (group == 0 ? (a_live ? w.q0 : w.len) : w.q0_b)
                       : w.q0 + (HP == 1 ? wave : wave / HP) * 32;
  const int wq_last = min(wq0 + 31, w.len - 1);
  const bool wave_live = wq0 < w.len;
  const int myq = wq0 + col;
  const int mypos = hist + myq;  // key position of this lane's query

  // ---- Q^T operand: lane holds q[myq, 16c + 8*half .. +7], read with
  // whole-row loads through the wave's own LDS slice (QRows).
  opv8 qf[C::DCH];
  const qelem* const qhead = static_cast<const qelem*>(p.q) + (int64_t)head * p.q_hs;
  QRows<HDIM, qelem> qrows;
  auto q_issue = [&]() { qrows.issue(qhead, p.q_ts, w.start, wq0, w.len - wq0, lane); };
  auto q_finish = [&]() {
    qrows.template finish<OP>(w.len - wq0, p.q_mult, slice, QSTR, lane, qf);
  };

  // ---- K/V tile movement (K by group A, V by group B).  Per-sequence bases
  // are wave-uniform; each tile is read through a buffer resource covering
  // only its valid rows.
  const kvelem* kseq = static_cast<const kvelem*>(p.k) + (int64_t)w.kstart * p.k_ts +
                       (int64_t)kvh * p.k_hs;
  const kvelem* vseq = static_cast<const kvelem*>(p.v) + (int64_t)w.kstart * p.v_ts +
                       (int64_t)kvh * p.v_hs;
  // Token slot of key position kv0 (a tile start, a multiple of kBN): packed
  // keys are contiguous; in a paged cache the whole tile sits in the page
  // that the block table names (page_size is a multiple of kBN), one scalar
  // table read per tile, the page number clamped into the pool.
  auto tile_slot = [&](int kv0) -> int64_t {
    if (!PAGED) return kv0;
    const int* row = p.block_table + (int64_t)w.seq * p.table_stride;
    const int idx = __builtin_amdgcn_readfirstlane(kv0 / p.page_size);
    const int page = min(max(row[idx], 0), p.n_pages - 1);
    return (int64_t)page * p.page_size + (kv0 - idx * p.page_size);
  };
  const int k_row_bytes = (int)(p.k_ts * (int64_t)sizeof(kvelem));
  const int v_row_bytes = (int)(p.v_ts * (int64_t)sizeof(kvelem));

  const int stid = tid & (C::STAGERS - 1);  // index inside the staging group
  u32x4_t kst[C::K_CHUNKS];
  u32x4_t vst[C::V_UNITS][4];

  auto rows_of = [&](int kv0) {
    // (readfirstlane keeps the descriptor scalar: a VALU min/max here would
    // force a waterfall loop around every buffer load)
    return __builtin_amdgcn_readfirstlane(max(0, min(kv_hi - kv0, kBN)));
  };
  auto gload_k = [&](int kv0) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<kvelem*>(kseq + tile_slot(kv0) * p.k_ts), 0, rows_of(kv0) * k_row_bytes,
        kRsrcWord3);
#pragma unroll
    for (int i = 0; i < C::K_CHUNKS; ++i) {
      const int chunk = stid + i * C::STAGERS;
      if (C::K_TOTAL % C::STAGERS == 0 || chunk < C::K_TOTAL)
        kst[i] = __builtin_amdgcn_raw_buffer_load_b128(
            r, (chunk / C::OCTS) * k_row_bytes + 16 * (chunk % C::OCTS), 0, 0);
    }
  };
  auto gload_v = [&](int kv0) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<kvelem*>(vseq + tile_slot(kv0) * p.v_ts), 0, rows_of(kv0) * v_row_bytes,
        kRsrcWord3);
#pragma unroll
    for (int u = 0; u < C::V_UNITS; ++u) {
      const int unit = stid + u * C::STAGERS;
      const int kq = unit % (kBN / 4);
      const int oct = unit / (kBN / 4);
      if (C::V_TOTAL % C::STAGERS == 0 || unit < C::V_TOTAL) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vst[u][i] = __builtin_amdgcn_raw_buffer_load_b128(
              r, (4 * kq + i) * v_row_bytes + 16 * oct, 0, 0);
      }
    }
  };
  // K row-major into stage `st`.
  auto store_k = [&](int st) {
    uint16_t* ks = kstage0 + st * C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::K_CHUNKS; ++i) {
      const int chunk = stid + i * C::STAGERS;
      if (C::K_TOTAL % C::STAGERS == 0 || chunk < C::K_TOTAL)
        *reinterpret_cast<u32x4_t*>(ks + (chunk / C::OCTS) * C::KSTR + 8 * (chunk % C::OCTS)) =
            kv_to_op(OP(), KVT(), kst[i]);
    }
  };
  // V transposed into stage `st` with the key order of the S^T accumulator:
  // inside each 16-key group, LDS positions 4..7 hold keys 8..11 and
  // positions 8..11 hold keys 4..7.
  auto store_v = [&](int st) {
    uint16_t* vs = vstage0 + st * C::V_ELEMS;
#pragma unroll
    for (int u = 0; u < C::V_UNITS; ++u) {
      const int unit = stid + u * C::STAGERS;
      if (C::V_TOTAL % C::STAGERS != 0 && unit >= C::V_TOTAL) continue;
      const int kq = unit % (kBN / 4);
      const int oct = unit / (kBN / 4);
      const int qq = kq & 3;
      const int pos = 16 * (kq >> 2) + 4 * (((qq & 1) << 1) | (qq >> 1));
      u32x4_t r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = kv_to_op(OP(), KVT(), vst[u][i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // element j of keys (i, i+1) -> one dword (v_perm_b32)
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        u32x2_t out;
        out[0] = __builtin_amdgcn_perm(r[1][j >> 1], r[0][j >> 1], sel);
        out[1] = __builtin_amdgcn_perm(r[3][j >> 1], r[2][j >> 1], sel);
        *reinterpret_cast<u32x2_t*>(vs + (8 * oct + j) * C::VSTR + pos) = out;
      }
    }
  };

  // ---- per-wave state
  f32x16_t o[C::DBLK];
#pragma unroll
  for (int c = 0; c < C::DBLK; ++c) o[c] = (f32x16_t){};
  f32x16_t s[kKB];
  opv8 pf[kKT];
  float m_run = -INFINITY;  // running (lazy) max of raw scores
  float l_run = 0.f;        // this lane's share of the running sum
  const float cmul = p.score_mult;

  // Whether every key of the tile at kv0 is visible to every row of this wave.
  auto tile_full = [&](int kv0) {
    return (kv0 + kBN - 1 <= hist + wq0) &&
           (p.window == 0 || kv0 >= hist + wq_last - p.window + 1);
  };

  // S^T = K Q^T for the tile in K stage `st`.
  auto scores = [&](int st) {
    const uint16_t* ks = kstage0 + st * C::K_ELEMS;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) s[kb] = (f32x16_t){};
#pragma unroll
    for (int c = 0; c < C::DCH; ++c) {
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        const opv8 a = *reinterpret_cast<const opv8*>(
            ks + (32 * kb + col) * C::KSTR + 16 * c + 8 * half);
        s[kb] = OP::mfma(a, qf[c], s[kb]);
      }
    }
  };
  // O^T += V^T P^T for the tile in V stage `st`.
  auto pv = [&](int st) {
    const uint16_t* vs = vstage0 + st * C::V_ELEMS;
#pragma unroll
    for (int c = 0; c < C::DBLK; ++c) {
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) {
        const opv8 a = *reinterpret_cast<const opv8*>(
            vs + (32 * c + col) * C::VSTR + 16 * kt + 8 * half);
        o[c] = OP::mfma(a, pf[kt], o[c]);
      }
    }
  };
  // Matrix slot of tile j when both P(j-1)V(j-1) and S(j) are needed, as one
  // straight-line block: the NPV P.V MFMAs (DBLK accumulator chains), then
  // the NS score MFMAs, with every LDS operand read kAhead MFMAs ahead
  // (across the boundary between the two products, too).
  auto matrix_fused = [&](int kst_i, int vst_i) {
    const uint16_t* ks = kstage0 + kst_i * C::K_ELEMS;
    const uint16_t* vs = vstage0 + vst_i * C::V_ELEMS;
    constexpr int NPV = C::NPV, N = C::NPV + C::NS;
    // operand i < NPV: V^T for P.V step i (kt-major over the output blocks);
    // i >= NPV: K for score step i - NPV (d-chunk-major over the key blocks)
    auto operand = [&](int i) -> opv8 {
      if (i >= NPV) {
        const int c = (i - NPV) / kKB, kb = (i - NPV) % kKB;
        return *reinterpret_cast<const opv8*>(ks + (32 * kb + col) * C::KSTR + 16 * c +
                                              8 * half);
      }
      const int kt = i / C::DBLK, c = i % C::DBLK;
      return *reinterpret_cast<const opv8*>(vs + (32 * c + col) * C::VSTR + 16 * kt +
                                            8 * half);
    };
    constexpr int kAhead = N < 8 ? N : 8;
    opv8 buf[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) buf[i] = operand(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const opv8 a = buf[i % kAhead];
      if (i + kAhead < N) buf[i % kAhead] = operand(i + kAhead);
      if (i >= NPV) {
        const int c = (i - NPV) / kKB, kb = (i - NPV) % kKB;
        s[kb] = OP::mfma(a, qf[c], c == 0 ? (f32x16_t){} : s[kb]);
      } else {
        const int kt = i / C::DBLK, c = i % C::DBLK;
        o[c] = OP::mfma(a, pf[kt], o[c]);
      }
    }
    // pin the order: kAhead LDS reads, then (MFMA, LDS read) pairs, then the
    // last kAhead MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < N - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
  };
  // Mask (boundary tiles only), then the lazy online softmax into the P
  // operand (lazy_softmax), and the rare rescale of O.
  auto softmax = [&](int kv0) {
    if (!tile_full(kv0)) {
      // Element r of key block kb holds key kv0 + 4*half + off, with the
      // compile-time offset off = 32*kb + 8*(r/4) + r%4.  The key is visible
      // when off <= hi (causal) and, with a window, off >= lo.
      const int hi = mypos - kv0 - 4 * half;
      // (lo <= 0 bounds nothing since off >= 0: the subtraction only runs where it
      // cannot overflow; no branch, the same code with and without a window)
      const int lo = (p.window > 0 && p.window <= hi) ? hi - p.window + 1 : INT_MIN;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
          if (off > hi || off < lo) s[kb][r] = -INFINITY;
        }
    }
    lazy_softmax<OP, kKT>(
        [&](int kt, int i) { return s[kt >> 1][8 * (kt & 1) + i]; }, cmul, m_run, l_run, pf, [&](float alpha) {
#pragma unroll
          for (int c = 0; c < C::DBLK; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
        });
  };

  // ---- prologue: group A holds its Q operand, K(0) is in stage 0 and K(1)
  // in flight; group B's Q and V(0) are in flight (B needs its Q only in
  // slot 1, so it finishes it during A's first matrix slot).
  // (The K/V loads go first: issuing Q first made hipcc keep about 30 more
  // registers live across the tile loops.)
  if (group == 0) {
    gload_k(kv_start);
    q_issue();
    q_finish();
    store_k(0);
    if (n_tiles > 1) gload_k(kv_start + kBN);
  } else {
    gload_v(kv_start);
    q_issue();
  }
  __syncthreads();

  // ---- ping-pong slots.  Each barrier ends a slot.  In slot 2j group A
  // runs its matrix work for tile j (P(j-1)V(j-1), then S(j)) while group B
  // runs softmax(j-1); in slot 2j+1 group A runs softmax(j) while group B
  // runs its matrix work for tile j.  Tile j uses K stage j&1 and V stage
  // j&1, both resident through slots 2j and 2j+1 and free during slots
  // 2j-2 and 2j-1, when they are written.  Group A stages K and group B
  // stages V, each at the end of its slot 2j-1 (A: softmax slot, B: matrix
  // slot, after its MFMAs are issued): store the tile loaded two slots
  // earlier, then issue the loads of the next one, so every load has two
  // slots to arrive.  Both groups pass the same 2n + 1 barriers after the
  // prologue's; group B's last P.V (slot 2n + 1) runs after the last one,
  // beside group A's epilogue: from then on the waves only read the V stage
  // and write their own slices.  Every wave runs every tile: a tile none of
  // its rows can see is fully masked and contributes exact zeros.
  if (group == 0) {
    // Group A computes tiles [0, n_a) (n_a = n_tiles unless folded) and
    // stages K for all n_tiles: K(j + 1) stored and K(j + 2) issued in
    // the slot after tile j's matrix slot.
    auto stage_after = [&](int j) {
      if (j + 1 < n_tiles) {
        store_k((j + 1) & 1);
        if (j + 2 < n_tiles) gload_k(kv_start + (j + 2) * kBN);
      }
    };
    // prologue (before the loop): K(0) stored, K(1) in flight
    if (!FOLD || n_a > 0) scores(0);
    __syncthreads();
    if (!FOLD || n_a > 0) softmax(kv_start);
    stage_after(0);
    __syncthreads();
    const int n_full = FOLD ? max(n_a, 1) : n_tiles;
    for (int j = 1; j < n_full; ++j) {
      matrix_fused(j & 1, (j - 1) & 1);
      __syncthreads();
      softmax(kv_start + j * kBN);
      stage_after(j);
      __syncthreads();
    }
    if (FOLD) {
      // Folded: A's last P.V in tile n_a's matrix slot, then K staging only.
      int j = n_full;
      if (n_a > 0 && n_a < n_tiles) {
        pv((n_a - 1) & 1);
        __syncthreads();
        stage_after(n_a);
        __syncthreads();
        j = n_a + 1;
      }
      for (; j < n_tiles; ++j) {
        __syncthreads();
        stage_after(j);
        __syncthreads();
      }
    }
    if (!FOLD || n_a == n_tiles) pv((n_tiles - 1) & 1);
    __syncthreads();
  } else {
    q_finish();
    __syncthreads();
    // V(0) was loaded before the first barrier
    scores(0);
    store_v(0);
    if (n_tiles > 1) gload_v(kv_start + kBN);
    __syncthreads();
    softmax(kv_start);
    __syncthreads();
    for (int j = 1; j < n_tiles; ++j) {
      const int kv0 = kv_start + j * kBN;
      matrix_fused(j & 1, (j - 1) & 1);
      store_v(j & 1);
      if (j + 1 < n_tiles) gload_v(kv0 + kBN);
      __syncthreads();
      softmax(kv0);
      __syncthreads();
    }
    pv((n_tiles - 1) & 1);
  }

  const float l_tot = pair_sum(l_run);
  if (SPLIT && n_pieces > 1) {
    // partial of this piece: running max (raw score units), sum, and O
    // relative to that max, for every row of the tile (rows past the
    // sequence are written too and never read)
    float* part = p.partial + (int64_t)blockIdx.x * prefill_partial_floats(HDIM, kBM);
    const int row = wave * 32 + col;
    if (half == 0) {
      part[row] = m_run;
      part[kBM + row] = l_tot;
    }
    // row-major: the lane's four consecutive columns per (block, row group)
    f32x4_t* po = reinterpret_cast<f32x4_t*>(part + 2 * kBM + row * HDIM);
#pragma unroll
    for (int c = 0; c < C::DBLK; ++c)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        po[8 * c + 2 * rb + half] = (f32x4_t){o[c][4 * rb], o[c][4 * rb + 1], o[c][4 * rb + 2],
                                              o[c][4 * rb + 3]};
    return;
  }

  // ---- epilogue: O / l -> bf16, rows of this sequence only.  The wave's
  // 32 x HDIM tile goes through its own LDS slice so that every global
  // store writes whole 2*HDIM-byte rows.
  if (wave_live) {
    constexpr int OSTR = QSTR;
    uint16_t* ob = slice;
    // rows past the sequence are never stored; a row without any visible
    // key (malformed offsets only) is written as zeros
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int c = 0; c < C::DBLK; ++c) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        u32x2_t pk;
        pk[0] = pack_bf16x2(o[c][4 * rb] * inv, o[c][4 * rb + 1] * inv);
        pk[1] = pack_bf16x2(o[c][4 * rb + 2] * inv, o[c][4 * rb + 3] * inv);
        *reinterpret_cast<u32x2_t*>(ob + col * OSTR + 32 * c + 8 * rb + 4 * half) = pk;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    constexpr int CPR = HDIM / 8;          // 16-byte chunks per row
    constexpr int RPI = kWave / CPR;       // rows per store instruction
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = RPI * i + lane / CPR;
      const int ch = lane % CPR;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ob + row * OSTR + 8 * ch);
      if (wq0 + row < w.len)
        *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p.out) +
                                    (int64_t)(w.start + wq0 + row) * p.o_ts +
                                    (int64_t)head * p.o_hs + 8 * ch) = v;
    }
  }
}

// Combines the pieces of every split query tile: per row,
// out = sum_i o_i 2^((m_i - M) c) / sum_i l_i 2^((m_i - M) c), M = max_i m_i
// (the online-softmax combination, across workgroups).  One workgroup per
// (slot, head, group of kMergeRows rows); thread (row, chunk) handles four
// consecutive columns of a row, so a wave reads contiguous rows of the
// partials and writes contiguous bf16 output, and every thread makes one
// pass (two rounds of independent loads).  Tiles of one piece wrote their
// output directly.
template <int HDIM>
constexpr int merge_rows() { return 256 / (HDIM / 4); }

template <int HDIM, bool PAGED>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillParams p) {
  constexpr int CH = HDIM / 4;        // 16-byte chunks of a row of partials
  constexpr int RPP = merge_rows<HDIM>();  // rows per workgroup
  constexpr int RB = kBM / RPP;       // row groups per query tile
  constexpr int64_t PF = prefill_partial_floats(HDIM, kBM);
  const int rb = blockIdx.x % RB;
  const int sh = blockIdx.x / RB;
  const int slot = sh / p.n_q_heads;
  const int head = sh - slot * p.n_q_heads;
  Work w = decode_work<kBM, PAGED>(p, slot);
  if (!w.valid) return;
  const int n_pieces =
      min((key_range<kBM>(p, w).n_tiles + p.piece_tiles - 1) / p.piece_tiles, p.max_pieces);
  if (n_pieces <= 1) return;
  const float* base =
      p.partial + ((int64_t)slot * p.max_pieces * p.n_q_heads + head) * PF;
  const int64_t step = (int64_t)p.n_q_heads * PF;  // next piece of the same tile
  const int chunk = threadIdx.x % CH;
  const int row = rb * RPP + threadIdx.x / CH;
  if (w.q0 + row < w.len) {
    float mx = -INFINITY;
    for (int i = 0; i < n_pieces; ++i) mx = fmaxf(mx, base[i * step + row]);
    float den = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < n_pieces; ++i) {
      const float* part = base + i * step;
      const float m = part[row];
      const float wt = m == -INFINITY ? 0.f : fast_exp2((m - mx) * p.score_mult);
      den += wt * part[kBM + row];
      const f32x4_t o = reinterpret_cast<const f32x4_t*>(part + 2 * kBM + row * HDIM)[chunk];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += wt * o[e];
    }
    // a row without any visible key (malformed offsets only) is written as zeros
    const float inv = den > 0.f ? 1.f / den : 0.f;
    u32x2_t v;
    v[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    v[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.out) +
                                (int64_t)(w.start + w.q0 + row) * p.o_ts +
                                (int64_t)head * p.o_hs + 4 * chunk) = v;
  }
}

template <int HDIM, class QT, class KVT, bool PAGED>
void launch_paged_or_not(PrefillParams p, uint64_t slots, hipStream_t stream) {
  if (p.piece_tiles == 0 && p.group % 4 == 0) {
    // four heads of one KV head per workgroup, 64 rows each (or, folded,
    // two mirrored 32-row blocks: ceil(ceil(n / 32) / 2) = ceil(n / 64)
    // pairs for n tokens, the same slot count)
    constexpr int bm = kBM / 4;
    const uint64_t slots4 = (uint64_t)((p.n_tokens + bm - 1) / bm + p.n_seqs);
    p.tile_slots = (int32_t)slots4;
    const dim3 grid((uint32_t)dispatch_grid(slots4 * (uint64_t)(p.n_q_heads / 4)));
    if (p.fold && p.window == 0)
      hipLaunchKernelGGL((prefill_fwd_kernel<HDIM, QT, KVT, PAGED, false, 4, true>), grid,
                         dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((prefill_fwd_kernel<HDIM, QT, KVT, PAGED, false, 4, false>), grid,
                         dim3(kThreads), 0, stream, p);
    return;
  }
  if (p.piece_tiles > 0) {
    const uint64_t blocks = slots * (uint64_t)p.max_pieces * (uint64_t)p.n_q_heads;
    hipLaunchKernelGGL((prefill_fwd_kernel<HDIM, QT, KVT, PAGED, true, 1, false>),
                       dim3((uint32_t)blocks), dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL((prefill_merge_kernel<HDIM, PAGED>),
                       dim3((uint32_t)(slots * (uint64_t)p.n_q_heads *
                                       (uint64_t)(kBM / merge_rows<HDIM>()))),
                       dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL((prefill_fwd_kernel<HDIM, QT, KVT, PAGED, false, 1, false>),
                       dim3((uint32_t)dispatch_grid(slots * (uint64_t)p.n_q_heads)),
                       dim3(kThreads), 0, stream, p);
  }
}

template <int HDIM, class QT, class KVT>
hipError_t launch_one(PrefillParams p, hipStream_t stream) {
  const int64_t slots = (p.n_tokens + kBM - 1) / kBM + p.n_seqs;
  p.tile_slots = (int32_t)slots;
  if (p.page_size > 0)
    launch_paged_or_not<HDIM, QT, KVT, true>(p, (uint64_t)slots, stream);
  else
    launch_paged_or_not<HDIM, QT, KVT, false>(p, (uint64_t)slots, stream);
  return hipGetLastError();
}

template <int HDIM>
hipError_t launch_dtypes(const PrefillParams& p, DType q_dtype, DType kv_dtype,
                         hipStream_t stream) {
  if (q_dtype == kBF16 && kv_dtype == kBF16) return launch_one<HDIM, BF16, BF16>(p, stream);
  if (q_dtype == kBF16 && kv_dtype == kFP16) return launch_one<HDIM, BF16, FP16>(p, stream);
  if (q_dtype == kFP32 && kv_dtype == kBF16) return launch_one<HDIM, FP32, BF16>(p, stream);
  if (q_dtype == kFP32 && kv_dtype == kFP16) return launch_one<HDIM, FP32, FP16>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace

int prefill_min_block_m(int head_dim) {
  if (head_dim == 512) return prefill_d512_block_m();
  return head_dim >= 256 ? prefill_wide_block_m() : kBM;
}

int prefill_kv_tile(int /*head_dim*/) { return kBN; }

hipError_t launch_prefill(const PrefillParams& p, int head_dim_qk, int head_dim_v,
                          DType q_dtype, DType kv_dtype, hipStream_t stream) {
  if (head_dim_qk == 128 && head_dim_v == 128)
    return launch_dtypes<128>(p, q_dtype, kv_dtype, stream);
  if (head_dim_qk == 64 && head_dim_v == 64) return launch_dtypes<64>(p, q_dtype, kv_dtype, stream);
  if (head_dim_qk == 512 && head_dim_v == 512)
    return launch_prefill_d512(p, q_dtype, kv_dtype, stream);
  if (head_dim_qk >= 256)
    return launch_prefill_wide(p, head_dim_qk, head_dim_v, q_dtype, kv_dtype, stream);
  return hipErrorInvalidValue;
}

}  // namespace attnp
