// Causal / sliding-window prefill attention for 512-wide heads on gfx950
// (CDNA4): the 512-dim path that the atlas page guards for head sizes above
// 256 ("Project Snapshot" of the HDIM-templated prefill kernels).  Same
// operation, inputs, masks and results as the 128-d kernel: causal bound
// kv_end = min(q_pos + 1, seq_len) of the fused MLA prefill (atlas PR #69),
// the W most recent keys for a window (m40-llm AGENTS.md, "Current
// Progress"), KV histories and paged caches as in the chunked and paged MLA
// prefill of atlas PR #69.
//
// Design (ours, for CDNA4): a 512-d head would need 256 fp32 accumulator
// and 128 Q operand registers in one 32-row wave, beyond the budget of two
// waves per SIMD.  The head is split into two column halves instead, laid
// over the 128-d kernel's ping-pong:
//   * Eight waves in two groups, A (waves 0-3) and B (4-7), each group 64
//     query rows (128 per workgroup): wave w of a group runs the 32-row
//     block (w >> 1) & 1 on columns [256 h, 256 h + 256), h = w & 1, of Q,
//     K, V and out.  Waves w and w + 4 -- one SIMD -- read the same column
//     half of every K/V tile.
//   * Per 32-key tile a wave forms partial scores Sᵀ_h = K_h Q_hᵀ from its
//     half (16 MFMAs, 32x32x16 in the K/V storage type) and writes them to
//     LDS; in the group's next slot it adds its partner's (same rows, other
//     half: the two sums are the same fp32 numbers, a + b = b + a), runs the
//     online softmax (both partners take the same decisions on the same
//     scores) and later accumulates Oᵀ_h += Vᵀ_h Pᵀ for its 256 output
//     columns (16 MFMAs).  No MFMA work is repeated.
//   * The groups run in anti-phase as in the 128-d kernel: in one slot
//     group A issues its MFMAs (the partial scores of tile j, then P.V of
//     tile j - 1) while group B adds partials and runs its softmax, and the
//     next slot the other way round.
//   * K and V tiles go straight from memory into LDS (buffer loads to LDS,
//     one 1 KiB row per instruction, 16-byte chunk c of row r at position
//     c ^ (r & 15) for K, c ^ 2 (r & 7) for V, so that the K operand reads
//     (16 rows, 16 bytes each) and the transposing Vᵀ reads (4 rows, 32
//     bytes each, per 16 lanes) meet no bank twice), with no staging
//     registers: group A issues them after the operand reads of its matrix
//     slot and waits for them at the end of its softmax slot, so that no
//     wave has a load to LDS in flight while it reads operands (hipcc
//     waits for such a load before any LDS read it cannot prove disjoint).  Vᵀ operands come from the
//     transposing LDS read ds_read_b64_tr_b16.  LDS: two K and two V
//     stages (128 KiB) and the partial scores of the eight waves (32 KiB).
//   * Folded grids (causal, no window, about one workgroup per CU): group A
//     takes a sequence's 64-row block r and group B its mirror nb - 1 - r.
#include <hip/hip_runtime.h>
#include <climits>
#include <stdint.h>

#include "device_common.h"
#include "prefill_params.h"
#include "prefill_work.h"

namespace attnp {
namespace {

using namespace dev;

typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kGWave = 64;
constexpr int kGWaves = 8;                  // two groups of four
constexpr int kGThreads = kGWave * kGWaves;
constexpr int kGD = 512;                    // head size
constexpr int kGHalf = kGD / 2;             // columns per wave
constexpr int kGBM = 128;                   // query rows per workgroup (64 per group)
constexpr int kGBN = 32;                    // keys per tile: one 32-key score block
constexpr int kGKQ = kGBN / 16;             // 16-key P.V steps per tile
constexpr int kGTile = kGBN * kGD;          // elements of one K or V stage

// FOLD: group A runs the 64-row block r of a sequence and group B its
// mirror nb - 1 - r (causal, no window); group B, the later block, sees at
// least as many key tiles, and group A stops its matrix and softmax work
// after its own last key tile (it keeps moving K and passing the barriers).
template <class QT, class KVT, bool PAGED, bool FOLD>
__global__ __launch_bounds__(kGThreads, 1) void prefill_d512_kernel(PrefillParams p) {
  constexpr int DCH = kGHalf / 16;   // score k-steps per half
  constexpr int DBLK = kGHalf / 32;  // output blocks per half
  constexpr int BMG = kGBM / 2;      // query rows per group
  typedef typename QT::T qelem;
  typedef typename KVT::T kvelem;
  typedef typename OpOf<KVT>::T OP;  // operand type of both products
  typedef typename OP::v8 opv8;

  // K stages 0, 1 then V stages 0, 1 ([32 rows][512] operand elements), then
  // the partial scores [wave][r/4][lane]
  __shared__ __attribute__((aligned(16))) uint16_t kvs[4 * kGTile];
  __shared__ __attribute__((aligned(16))) f32x4_t xch[kGWaves * 4 * kGWave];

  const int tid = threadIdx.x;
  const int lane = tid & (kGWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kGWave);
  const int group = wave >> 2;      // 0 = A (moves K), 1 = B (moves V)
  const int blk = (wave >> 1) & 1;  // 32-row block of the group
  const int hf = wave & 1;          // column half
  const int col = lane & 31;        // query column of this lane
  const int half = lane >> 5;
  const int bid = dispatch_index(blockIdx.x);
  const int slot = bid / p.n_q_heads;
  const int head = bid - slot * p.n_q_heads;
  Work w = decode_work<FOLD ? BMG : kGBM, PAGED, FOLD>(p, slot);
  if (!w.valid) return;  // uniform across the workgroup
  w.start = __builtin_amdgcn_readfirstlane(w.start);
  w.len = __builtin_amdgcn_readfirstlane(w.len);
  w.q0 = __builtin_amdgcn_readfirstlane(w.q0);
  w.q0_b = __builtin_amdgcn_readfirstlane(w.q0_b);
  w.kstart = __builtin_amdgcn_readfirstlane(w.kstart);
  w.seq = __builtin_amdgcn_readfirstlane(w.seq);
  w.klen = __builtin_amdgcn_readfirstlane(w.klen);

  const int kvh = head / p.group;
  const int hist = w.klen - w.len;  // queries are the last len key positions
  // key range of the workgroup: the whole 128-row tile, or, folded, group
  // B's block (which starts at key 0 and ends last)
  const int qb = FOLD ? w.q0_b : w.q0;
  const int q_end = min(w.len, qb + (FOLD ? BMG : kGBM));
  const int kv_hi = min(max(hist + q_end, 0), w.klen);
  const int kv_lo = p.window > 0 ? min(max(0, hist + w.q0 - p.window + 1), kv_hi) : 0;
  const int kv_start = kv_lo - kv_lo % kGBN;
  const int n_tiles = max(1, (kv_hi - kv_start + kGBN - 1) / kGBN);
  const bool a_live = !FOLD || w.q0 != w.q0_b;
  int n_a = n_tiles;
  if (FOLD) {
    const int a_hi = min(max(hist + min(w.len, w.q0 + BMG), 0), w.klen);
    n_a = a_live ? max(1, (a_hi + kGBN - 1) / kGBN) : 0;
  }
  // first row of this wave (a folded idle group A gets rows past the sequence)
  const int wq0 = (FOLD ? (group == 0 ? (a_live ? w.q0 : w.len) : w.q0_b) : w.q0 + BMG * group) +
                  32 * blk;
  const int wq_last = min(wq0 + 31, w.len - 1);
  const int myq = wq0 + col;
  const int mypos = hist + myq;
  const int d0 = kGHalf * hf;  // first column of this wave's half

  // ---- K and V tiles straight into LDS (group A's waves): wave i moves
  // rows 8i .. 8i + 7, one row per load, lane l the chunk that goes to
  // position l of the row
  const kvelem* const kseq =
      static_cast<const kvelem*>(p.k) + (int64_t)w.kstart * p.k_ts + (int64_t)kvh * p.k_hs;
  const kvelem* const vseq =
      static_cast<const kvelem*>(p.v) + (int64_t)w.kstart * p.v_ts + (int64_t)kvh * p.v_hs;
  const int k_row_bytes = (int)(p.k_ts * (int64_t)sizeof(kvelem));
  const int v_row_bytes = (int)(p.v_ts * (int64_t)sizeof(kvelem));
  auto tile_slot = [&](int kv0) -> int64_t {
    if (!PAGED) return kv0;
    const int* row = p.block_table + (int64_t)w.seq * p.table_stride;
    const int idx = __builtin_amdgcn_readfirstlane(kv0 / p.page_size);
    const int page = min(max(row[idx], 0), p.n_pages - 1);
    return (int64_t)page * p.page_size + (kv0 - idx * p.page_size);
  };
  // buffer resource of the K or V tile at kv0: rows past the last visible
  // key read as zero (buffer range)
  auto tile_rsrc = [&](int kv0, bool vtile) {
    const kvelem* const src = vtile ? vseq : kseq;
    const int64_t src_ts = vtile ? p.v_ts : p.k_ts;
    const int row_bytes = vtile ? v_row_bytes : k_row_bytes;
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(kv_hi - kv0, kGBN)));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<kvelem*>(src + tile_slot(kv0) * src_ts),
                                             0, rows * row_bytes, kRsrcWord3);
  };
  auto move = [&](__amdgpu_buffer_rsrc_t r, int st, bool vtile) {
    const int row_bytes = vtile ? v_row_bytes : k_row_bytes;
    uint16_t* stage = kvs + (2 * (vtile ? 1 : 0) + st) * kGTile;
    // (offsets formed here from an opaque copy of the lane index rather than
    // kept live across the tile loop)
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < kGBN / 4; ++i) {
      const int row = (kGBN / 4) * (wave & 3) + i;
      const int key = vtile ? 2 * (row & 7) : (row & 15);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(stage + row * kGD), 16,
          row * row_bytes + 16 * (ln ^ key), 0, 0, 0);
    }
  };
  // the loads this wave issued have reached LDS (before the barrier that
  // publishes them)
  auto landed = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  const uint16_t* const kst0 = kvs;
  const uint16_t* const vst0 = kvs + 2 * kGTile;

  // ---- Qᵀ operand of this wave's half: lane holds q[myq, d0 + 16c + 8*half ..]
  opv8 qf[DCH];
  const qelem* const qrow = static_cast<const qelem*>(p.q) +
                            (int64_t)(w.start + (myq < w.len ? myq : 0)) * p.q_ts +
                            (int64_t)head * p.q_hs + d0;
  const float qmul = myq < w.len ? p.q_mult : 0.f;

  // ---- per-wave state (the two waves of a block keep the same m and l)
  f32x16_t o[DBLK];
#pragma unroll
  for (int c = 0; c < DBLK; ++c) o[c] = (f32x16_t){};
  f32x16_t sc;
  opv8 pf[kGKQ];
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float cmul = p.score_mult;
  f32x4_t* const xw = xch + wave * 4 * kGWave;              // this wave's partial
  const f32x4_t* const xp = xch + (wave ^ 1) * 4 * kGWave;  // its partner's

  // LDS operand addresses.  For a lane's fixed row only the low bits of the
  // k-step index meet the swizzle, so each lane keeps a few base addresses
  // per operand and the rest of every address is an immediate offset.
  //   K, score step c (0..15), row col: chunk 32 hf + 2c + half at position
  //     chunk ^ (col & 15), element col*512 + 256 hf + 8 (half ^ (col & 1)) +
  //     16 ((c & 7) ^ y) + 128 (c >> 3), y = (col >> 1) & 7.
  //   V, P.V step kq, output block c (0..7), read r: row 16 kq + 8 r + t
  //     (t = 4 half + j / 4, j = lane & 15), columns d0 + 32 c + 16 g +
  //     4 (j & 3) (g = bit 4 of the lane): chunk 32 hf + 4c + 2g + (j & 3) / 2
  //     at position chunk ^ 2t, element kq*8192 + r*4096 + t*512 + 256 hf +
  //     16 (g ^ (t & 1)) + 8 ((j & 3) / 2) + 4 (j & 1) + 32 ((c & 3) ^ k) +
  //     128 (c >> 2), k = t / 2.
  // (The bases are formed again at every tile from an opaque copy of the
  // lane index, a few vector instructions, rather than kept live across the
  // tile loop: the loop holds 216 registers of Q, O, S and P already.)
  auto k_bases = [&](int* kaddr) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int cl = ln & 31, hl = ln >> 5, y = (cl >> 1) & 7;
    const int kb = cl * kGD + 256 * hf + 8 * (hl ^ (cl & 1));
#pragma unroll
    for (int c = 0; c < 8; ++c) kaddr[c] = kb + 16 * (c ^ y);
  };
  auto v_bases = [&](int* vaddr) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int g = (ln >> 4) & 1, j = ln & 15, hl = ln >> 5;
    const int t = 4 * hl + (j >> 2);
    const int vb = t * kGD + 256 * hf + 16 * (g ^ (t & 1)) + 8 * ((j & 3) >> 1) + 4 * (j & 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) vaddr[c] = vb + 32 * (c ^ (t >> 1));
  };

  // partial Sᵀ_h = K_h Q_hᵀ of the tile in K stage st
  auto scores = [&](int st) {
    const uint16_t* kt = kst0 + st * kGTile;
    int kaddr[8];
    k_bases(kaddr);
    sc = (f32x16_t){};
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
      const opv8 a = *reinterpret_cast<const opv8*>(kt + kaddr[c & 7] + 128 * (c >> 3));
      sc = OP::mfma(a, qf[c], sc);
    }
  };
  auto publish = [&]() {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      xw[r4 * kGWave + lane] = (f32x4_t){sc[4 * r4], sc[4 * r4 + 1], sc[4 * r4 + 2],
                                         sc[4 * r4 + 3]};
  };
  // Oᵀ_h += Vᵀ_h Pᵀ for the tile in V stage st.  MFMA k-index 8*half + e of
  // step kq is key 16*kq + 8*(e / 4) + 4*half + e % 4 (the Sᵀ accumulator's
  // order): two transposing reads give keys +0..3 and +8..11 (+4*half).
  auto pv = [&](int st) {
    const uint16_t* vt = vst0 + st * kGTile;
    int vaddr[4];
    v_bases(vaddr);
#pragma unroll
    for (int kq = 0; kq < kGKQ; ++kq) {
#pragma unroll
      for (int c = 0; c < DBLK; ++c) {
        s16x4_t part[2];
#pragma unroll
        for (int r = 0; r < 2; ++r)
          part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t*)(vt + kq * 8192 + 4096 * r +
                                                           vaddr[c & 3] + 128 * (c >> 2)));
        u32x4_t u;
        u[0] = __builtin_bit_cast(u32x2_t, part[0])[0];
        u[1] = __builtin_bit_cast(u32x2_t, part[0])[1];
        u[2] = __builtin_bit_cast(u32x2_t, part[1])[0];
        u[3] = __builtin_bit_cast(u32x2_t, part[1])[1];
        o[c] = OP::mfma(__builtin_bit_cast(opv8, u), pf[kq], o[c]);
      }
    }
  };
  // Matrix slot of tile j when both P(j-1)V(j-1) and S(j) are due, as one
  // straight-line block: the 16 P.V MFMAs (P dies with them), then the 16
  // partial-score MFMAs, every LDS operand read kAhead MFMAs ahead (a Vᵀ
  // operand is two transposing reads), the order pinned.
  auto matrix = [&](int kst_i, int vst_i) {
    const uint16_t* kt = kst0 + kst_i * kGTile;
    const uint16_t* vt = vst0 + vst_i * kGTile;
    constexpr int NPV = kGKQ * DBLK, N = NPV + DCH;
    int kaddr[8], vaddr[4];
    v_bases(vaddr);
    k_bases(kaddr);
    auto operand = [&](int i) -> opv8 {
      if (i >= NPV) {
        const int c = i - NPV;
        return *reinterpret_cast<const opv8*>(kt + kaddr[c & 7] + 128 * (c >> 3));
      }
      const int kq = i / DBLK, c = i % DBLK;
      s16x4_t part[2];
#pragma unroll
      for (int r = 0; r < 2; ++r)
        part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(vt + kq * 8192 + 4096 * r +
                                                         vaddr[c & 3] + 128 * (c >> 2)));
      u32x4_t u;
      u[0] = __builtin_bit_cast(u32x2_t, part[0])[0];
      u[1] = __builtin_bit_cast(u32x2_t, part[0])[1];
      u[2] = __builtin_bit_cast(u32x2_t, part[1])[0];
      u[3] = __builtin_bit_cast(u32x2_t, part[1])[1];
      return __builtin_bit_cast(opv8, u);
    };
    constexpr int kAhead = 4;
    static_assert(kAhead < NPV && kAhead < DCH, "look-ahead within each product");
    opv8 buf[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) buf[i] = operand(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const opv8 a = buf[i % kAhead];
      if (i + kAhead < N) buf[i % kAhead] = operand(i + kAhead);
      if (i < NPV) {
        o[i % DBLK] = OP::mfma(a, pf[i / DBLK], o[i % DBLK]);
      } else {
        const int c = i - NPV;
        sc = OP::mfma(a, qf[c], c == 0 ? (f32x16_t){} : sc);
      }
    }
    // pin the order: the first kAhead operands' reads, then (MFMA, the reads
    // of the operand kAhead further on) pairs, then the last kAhead MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);
#pragma unroll
    for (int i = 0; i < NPV - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int i = NPV - kAhead; i < N - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
  };
  // End of a matrix slot: the partial written, then the barrier, without
  // waiting for this wave's K/V loads to LDS still in flight (they are waited
  // for at the end of the next slot, before the stage is read).
  auto end_matrix_slot = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
  };

  // own partial plus the partner's (both read back: the scores leave the
  // registers after the matrix slot), masks, online softmax
  auto softmax = [&](int kv0) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4_t a = xw[r4 * kGWave + lane];
      const f32x4_t b = xp[r4 * kGWave + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[4 * r4 + e] = a[e] + b[e];
    }
    const bool full = (kv0 + kGBN - 1 <= hist + wq0) &&
                      (p.window == 0 || kv0 >= hist + wq_last - p.window + 1);
    if (!full) {
      // key = kv0 + 4*half + off, off = 8*(r/4) + r%4 (compile-time): visible
      // when off <= hi and, with a window, off >= lo (lo <= 0 bounds nothing
      // since off >= 0; the subtraction only runs where it cannot overflow)
      const int hi = mypos - kv0 - 4 * half;
      const int lo = (p.window > 0 && p.window <= hi) ? hi - p.window + 1 : INT_MIN;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        if (off > hi || off < lo) sc[r] = -INFINITY;
      }
    }
    lazy_softmax<OP, kGKQ>(
        [&](int kt, int i) { return sc[8 * kt + i]; }, cmul, m_run, l_run, pf, [&](float alpha) {
#pragma unroll
          for (int c = 0; c < DBLK; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
        });
  };

  // ---- prologue: K(0) and K(1) (group A) or V(0) (group B) in LDS, Q in
  // registers
  if (group == 0) move(tile_rsrc(kv_start, false), 0, false);
  load_q_op<DCH, OP>(qrow, half, qmul, qf);
  landed();
  __syncthreads();

  // ---- ping-pong slots (the 128-d kernel's schedule).  In slot 2j group A
  // runs its matrix work for tile j (P(j-1)V(j-1), then partial S(j)) while
  // group B adds partials and runs softmax(j-1); in slot 2j+1 the other way
  // round.  K(j) (stage j&1) is read in slots 2j and 2j+1, V(j) (stage j&1)
  // in slots 2j+2 and 2j+3.  Group A alone moves the tiles: after the last
  // operand read of its matrix slot 2j it issues K(j+1) (into the stage
  // K(j-1) left) and V(j) (into the stage V(j-2) left), and waits for them
  // before the barrier that ends its softmax slot 2j+1; no wave has a load
  // to LDS in flight while it reads operands.  A wave's partial is written
  // in its matrix slot and read by its partner in the next slot.  Both
  // groups pass the same 2n + 1 barriers after the prologue's; group B's
  // last P.V and group A's epilogue run after the last one.
  if (group == 0) {
    // K(j + 1) and V(j) after the reads of matrix slot 2j
    // (both descriptors first: any spilled value they need is reloaded, and
    // waited for, before the first load to LDS is in flight)
    auto move_after = [&](int j) {
      const bool k_next = j + 1 < n_tiles;
      const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kv_start + (k_next ? j + 1 : j) * kGBN, false);
      const __amdgpu_buffer_rsrc_t rv = tile_rsrc(kv_start + j * kGBN, true);
      if (k_next) move(rk, (j + 1) & 1, false);
      move(rv, j & 1, true);
    };
    if (!FOLD || n_a > 0) scores(0);
    move_after(0);
    if (!FOLD || n_a > 0) publish();
    end_matrix_slot();
    if (!FOLD || n_a > 0) softmax(kv_start);
    landed();
    __syncthreads();
    const int n_full = FOLD ? max(n_a, 1) : n_tiles;
    for (int j = 1; j < n_full; ++j) {
      matrix(j & 1, (j - 1) & 1);
      move_after(j);
      publish();
      end_matrix_slot();
      softmax(kv_start + j * kGBN);
      landed();
      __syncthreads();
    }
    if (FOLD) {
      // Folded: A's last P.V in tile n_a's matrix slot, then moves only.
      int j = n_full;
      if (n_a > 0 && n_a < n_tiles) {
        pv((n_a - 1) & 1);
        move_after(n_a);
        end_matrix_slot();
        landed();
        __syncthreads();
        j = n_a + 1;
      }
      for (; j < n_tiles; ++j) {
        move_after(j);
        end_matrix_slot();
        landed();
        __syncthreads();
      }
    }
    if (!FOLD || n_a == n_tiles) pv((n_tiles - 1) & 1);
    __syncthreads();
  } else {
    __syncthreads();
    scores(0);
    publish();
    end_matrix_slot();
    softmax(kv_start);
    __syncthreads();
    for (int j = 1; j < n_tiles; ++j) {
      matrix(j & 1, (j - 1) & 1);
      publish();
      end_matrix_slot();
      softmax(kv_start + j * kGBN);
      __syncthreads();
    }
    pv((n_tiles - 1) & 1);
  }

  // ---- epilogue: O_h / l -> bf16, 4 consecutive columns per lane and block
  const float l_tot = pair_sum(l_run);
  if (myq < w.len) {
    // a row without any visible key (malformed offsets only) is written as zeros
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = static_cast<uint16_t*>(p.out) + (int64_t)(w.start + myq) * p.o_ts +
                   (int64_t)head * p.o_hs + d0;
#pragma unroll
    for (int c = 0; c < DBLK; ++c)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        u32x2_t pk;
        pk[0] = pack_bf16x2(o[c][4 * rb] * inv, o[c][4 * rb + 1] * inv);
        pk[1] = pack_bf16x2(o[c][4 * rb + 2] * inv, o[c][4 * rb + 3] * inv);
        *reinterpret_cast<u32x2_t*>(op + 32 * c + 8 * rb + 4 * half) = pk;
      }
  }
}

template <class QT, class KVT, bool PAGED>
void launch_d512_grid(const PrefillParams& p, uint64_t blocks, hipStream_t stream) {
  if (p.fold && p.window == 0)
    hipLaunchKernelGGL((prefill_d512_kernel<QT, KVT, PAGED, true>), dim3((uint32_t)blocks),
                       dim3(kGThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_d512_kernel<QT, KVT, PAGED, false>), dim3((uint32_t)blocks),
                       dim3(kGThreads), 0, stream, p);
}

template <class QT, class KVT>
hipError_t launch_d512_one(PrefillParams p, hipStream_t stream) {
  // (folded: ceil(ceil(n / 64) / 2) = ceil(n / 128) pairs for n tokens)
  const int64_t slots = (p.n_tokens + kGBM - 1) / kGBM + p.n_seqs;
  p.tile_slots = (int32_t)slots;
  const uint64_t blocks = dispatch_grid((uint64_t)slots * (uint64_t)p.n_q_heads);
  if (p.page_size > 0)
    launch_d512_grid<QT, KVT, true>(p, blocks, stream);
  else
    launch_d512_grid<QT, KVT, false>(p, blocks, stream);
  return hipGetLastError();
}

}  // namespace

int prefill_d512_block_m() { return kGBM; }

hipError_t launch_prefill_d512(const PrefillParams& p, DType q_dtype, DType kv_dtype,
                               hipStream_t stream) {
  if (q_dtype == kBF16 && kv_dtype == kBF16) return launch_d512_one<BF16, BF16>(p, stream);
  if (q_dtype == kBF16 && kv_dtype == kFP16) return launch_d512_one<BF16, FP16>(p, stream);
  if (q_dtype == kFP32 && kv_dtype == kBF16) return launch_d512_one<FP32, BF16>(p, stream);
  if (q_dtype == kFP32 && kv_dtype == kFP16) return launch_d512_one<FP32, FP16>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace attnp
