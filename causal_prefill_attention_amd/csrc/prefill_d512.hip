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
// and 128 Q operand registers in one 32-row wave, beyond one wave's
// budget.  The head is split by columns instead, and the split is laid over
// the 128-d kernel's ping-pong:
//   * Eight waves in two groups, A (waves 0-3) and B (4-7), each group one
//     32-row query block (64 rows per workgroup).  Wave w of a group owns
//     columns [128w, 128w + 128) of Q, K, V and out, so waves w and w + 4 --
//     one SIMD -- share that column slice of every K/V tile.
//   * Per 32-key tile a wave forms partial scores Sᵀ_w = K_w Q_wᵀ from its
//     columns (8 MFMAs, 32x32x16 in the K/V storage type) and writes them to its group's LDS
//     exchange; in the group's next slot every wave sums the four partials
//     in the same order (so all four hold the same fp32 scores), runs the
//     same online softmax, and later accumulates Oᵀ_w += Vᵀ_w Pᵀ for its 128
//     output columns (8 MFMAs).  No MFMA work is repeated.
//   * The groups run in anti-phase as in the 128-d kernel: in one slot group
//     A issues its MFMAs (P.V of the previous tile, then the partial scores
//     of this one) while group B runs its exchange and softmax, and the
//     next slot the other way round, so the matrix core of each SIMD is fed
//     by one wave while the vector ALU works for the other.
//   * Group A stages the K column slices and group B the V slices through
//     registers into two LDS stages (rows of 128 elements, 16-byte chunks of row
//     r at position chunk ^ (r & 15)); Vᵀ operands come from the transposing
//     LDS read ds_read_b64_tr_b16.  LDS: 128 KiB of K/V stages and 32 KiB of
//     exchange.
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
constexpr int kGSlices = 4;                 // column slices (one wave per group each)
constexpr int kGSlice = 512 / kGSlices;     // 128 columns per slice
constexpr int kGBM = 64;                    // query rows per workgroup (32 per group)
constexpr int kGBN = 32;                    // keys per tile: one 32-key score block
constexpr int kGKQ = kGBN / 16;             // 16-key P.V steps per tile

template <class QT, class KVT, bool PAGED>
__global__ __launch_bounds__(kGThreads, 1) void prefill_d512_kernel(PrefillParams p) {
  constexpr int CPR = kGSlice / 8;            // 16-byte chunks per slice row
  constexpr int DCH = kGSlice / 16;           // score k-steps per slice
  constexpr int DBLK = kGSlice / 32;          // output blocks per slice
  constexpr int TILE = kGBN * kGSlice;        // elements of one K or V slice tile
  constexpr int LOADS = kGBN * CPR / kGWave;  // 16-byte chunks per lane per tile
  typedef typename QT::T qelem;
  typedef typename KVT::T kvelem;
  typedef typename OpOf<KVT>::T OP;  // operand type of both products
  typedef typename OP::v8 opv8;

  // [stage][slice][K, V][TILE] operand elements, then the exchange [group][slice][r/4][lane]
  __shared__ __attribute__((aligned(16))) uint16_t kvs[2 * kGSlices * 2 * TILE];
  __shared__ __attribute__((aligned(16))) f32x4_t xch[2 * kGSlices * 4 * kGWave];

  const int tid = threadIdx.x;
  const int lane = tid & (kGWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kGWave);
  const int group = wave >> 2;  // 0 = A (stages K), 1 = B (stages V)
  const int sl = wave & 3;      // column slice
  const int col = lane & 31;    // query column of this lane
  const int half = lane >> 5;
  const int bid = dispatch_index(blockIdx.x);
  const int slot = bid / p.n_q_heads;
  const int head = bid - slot * p.n_q_heads;
  Work w = decode_work<kGBM, PAGED>(p, slot);
  if (!w.valid) return;  // uniform across the workgroup
  w.start = __builtin_amdgcn_readfirstlane(w.start);
  w.len = __builtin_amdgcn_readfirstlane(w.len);
  w.q0 = __builtin_amdgcn_readfirstlane(w.q0);
  w.kstart = __builtin_amdgcn_readfirstlane(w.kstart);
  w.seq = __builtin_amdgcn_readfirstlane(w.seq);
  w.klen = __builtin_amdgcn_readfirstlane(w.klen);

  const int kvh = head / p.group;
  const int hist = w.klen - w.len;  // queries are the last len key positions
  const int q_end = min(w.len, w.q0 + kGBM);
  const int kv_hi = min(max(hist + q_end, 0), w.klen);
  const int kv_lo = p.window > 0 ? min(max(0, hist + w.q0 - p.window + 1), kv_hi) : 0;
  const int kv_start = kv_lo - kv_lo % kGBN;
  const int n_tiles = max(1, (kv_hi - kv_start + kGBN - 1) / kGBN);
  const int wq0 = w.q0 + 32 * group;  // this group's query block
  const int wq_last = min(wq0 + 31, w.len - 1);
  const int myq = wq0 + col;
  const int mypos = hist + myq;
  const int d0 = sl * kGSlice;  // first column of this wave's slice

  // ---- K (group A) or V (group B) slice tiles: lane moves chunk
  // (lane % CPR) of rows 4i + lane / CPR
  const kvelem* src = group == 0
      ? static_cast<const kvelem*>(p.k) + (int64_t)w.kstart * p.k_ts + (int64_t)kvh * p.k_hs + d0
      : static_cast<const kvelem*>(p.v) + (int64_t)w.kstart * p.v_ts + (int64_t)kvh * p.v_hs + d0;
  const int64_t src_ts = group == 0 ? p.k_ts : p.v_ts;
  const int row_bytes = (int)(src_ts * (int64_t)sizeof(kvelem));
  auto tile_slot = [&](int kv0) -> int64_t {
    if (!PAGED) return kv0;
    const int* row = p.block_table + (int64_t)w.seq * p.table_stride;
    const int idx = __builtin_amdgcn_readfirstlane(kv0 / p.page_size);
    const int page = min(max(row[idx], 0), p.n_pages - 1);
    return (int64_t)page * p.page_size + (kv0 - idx * p.page_size);
  };
  u32x4_t st_regs[LOADS];
  auto gload = [&](int kv0) {
    // rows past the last visible key read as zero (buffer range)
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(kv_hi - kv0, kGBN)));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<kvelem*>(src + tile_slot(kv0) * src_ts), 0, rows * row_bytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int row = i * (kGWave / CPR) + lane / CPR;
      st_regs[i] = __builtin_amdgcn_raw_buffer_load_b128(r, row * row_bytes + 16 * (lane % CPR),
                                                         0, 0);
    }
  };
  auto kslice = [&](int st) { return kvs + ((st * kGSlices + sl) * 2 + 0) * TILE; };
  auto vslice = [&](int st) { return kvs + ((st * kGSlices + sl) * 2 + 1) * TILE; };
  auto lstore = [&](int st) {  // group A: K stage st; group B: V stage st
    uint16_t* dst = group == 0 ? kslice(st) : vslice(st);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int row = i * (kGWave / CPR) + lane / CPR;
      const int pos = (lane % CPR) ^ (row & 15);
      *reinterpret_cast<u32x4_t*>(dst + row * kGSlice + 8 * pos) = kv_to_op(OP(), KVT(), st_regs[i]);
    }
  };

  // ---- Qᵀ operand of this wave's slice: lane holds q[myq, d0 + 16c + 8*half ..]
  opv8 qf[DCH];
  const qelem* const qrow = static_cast<const qelem*>(p.q) +
                            (int64_t)(w.start + (myq < w.len ? myq : 0)) * p.q_ts +
                            (int64_t)head * p.q_hs + d0;
  const float qmul = myq < w.len ? p.q_mult : 0.f;

  // ---- per-wave state (the four waves of a group keep the same m and l)
  f32x16_t o[DBLK];
#pragma unroll
  for (int c = 0; c < DBLK; ++c) o[c] = (f32x16_t){};
  opv8 pf[kGKQ];
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float cmul = p.score_mult;
  f32x4_t* const xg = xch + group * kGSlices * 4 * kGWave;  // this group's exchange
  f32x4_t* const xw = xg + sl * 4 * kGWave;                   // this wave's partial

  // partial Sᵀ = K_w Q_wᵀ of the tile in K stage st, to the exchange
  auto scores = [&](int st) {
    const uint16_t* kt = kslice(st);
    f32x16_t sc = (f32x16_t){};
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
      const int pos = (2 * c + half) ^ (col & 15);
      const opv8 a = *reinterpret_cast<const opv8*>(kt + col * kGSlice + 8 * pos);
      sc = OP::mfma(a, qf[c], sc);
    }
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      xw[r4 * kGWave + lane] = (f32x4_t){sc[4 * r4], sc[4 * r4 + 1], sc[4 * r4 + 2],
                                         sc[4 * r4 + 3]};
  };
  // Oᵀ_w += Vᵀ_w Pᵀ for the tile in V stage st.  MFMA k-index 8*half + e of
  // step kq is key 16*kq + 8*(e / 4) + 4*half + e % 4 (the Sᵀ accumulator's
  // order): two transposing reads give keys +0..3 and +8..11 (+4*half).
  auto pv = [&](int st) {
    const uint16_t* vt = vslice(st);
    const int grp16 = (lane >> 4) & 1;  // 16-column half of the 32-row block
    const int j = lane & 15;
#pragma unroll
    for (int kq = 0; kq < kGKQ; ++kq) {
#pragma unroll
      for (int c = 0; c < DBLK; ++c) {
        s16x4_t part[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = 16 * kq + 8 * r + 4 * half + (j >> 2);
          const int d = 32 * c + 16 * grp16 + 4 * (j & 3);
          const int pos = (d >> 3) ^ (row & 15);
          part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t*)(vt + row * kGSlice + 8 * pos +
                                                           (d & 7)));
        }
        u32x4_t u;
        u[0] = __builtin_bit_cast(u32x2_t, part[0])[0];
        u[1] = __builtin_bit_cast(u32x2_t, part[0])[1];
        u[2] = __builtin_bit_cast(u32x2_t, part[1])[0];
        u[3] = __builtin_bit_cast(u32x2_t, part[1])[1];
        o[c] = OP::mfma(__builtin_bit_cast(opv8, u), pf[kq], o[c]);
      }
    }
  };
  // the group's four partials summed in slice order, masks, online softmax
  auto softmax = [&](int kv0) {
    f32x16_t sc;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4_t acc = xg[r4 * kGWave + lane];
#pragma unroll
      for (int v = 1; v < kGSlices; ++v) acc += xg[(v * 4 + r4) * kGWave + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[4 * r4 + e] = acc[e];
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

  // ---- prologue: K(0) stored (group A), V(0) in flight (group B), Q loaded
  // once the first tile's loads are issued
  gload(kv_start);
  load_q_op<DCH, OP>(qrow, half, qmul, qf);
  if (group == 0) {
    lstore(0);
    if (n_tiles > 1) gload(kv_start + kGBN);
  }
  __syncthreads();

  // ---- ping-pong slots (the 128-d kernel's schedule).  In slot 2j group A
  // runs its matrix work for tile j (P(j-1)V(j-1), then partial S(j) to its
  // exchange) while group B runs softmax(j-1) from its exchange; in slot
  // 2j+1 the other way round.  K(j) (stage j&1) is read in slots 2j and
  // 2j+1, V(j) (stage j&1) in slots 2j+2 and 2j+3.  Group A writes K(j+1)
  // in its softmax slot 2j+1, group B writes V(j) after its matrix work in
  // slot 2j+1; each load has two slots to arrive.  A group's exchange is
  // written in its matrix slot and read in its next slot, after the
  // barrier.  Both groups pass the same 2n + 2 barriers after the prologue.
  if (group == 0) {
    scores(0);
    __syncthreads();
    softmax(kv_start);
    if (n_tiles > 1) {
      lstore(1);
      if (n_tiles > 2) gload(kv_start + 2 * kGBN);
    }
    __syncthreads();
    for (int j = 1; j < n_tiles; ++j) {
      const int kv0 = kv_start + j * kGBN;
      pv((j - 1) & 1);
      scores(j & 1);
      __syncthreads();
      softmax(kv0);
      if (j + 1 < n_tiles) {
        lstore((j + 1) & 1);
        if (j + 2 < n_tiles) gload(kv0 + 2 * kGBN);
      }
      __syncthreads();
    }
    pv((n_tiles - 1) & 1);
    __syncthreads();
    __syncthreads();
  } else {
    __syncthreads();
    // V(0) was loaded before the first barrier
    scores(0);
    lstore(0);
    if (n_tiles > 1) gload(kv_start + kGBN);
    __syncthreads();
    softmax(kv_start);
    __syncthreads();
    for (int j = 1; j < n_tiles; ++j) {
      const int kv0 = kv_start + j * kGBN;
      pv((j - 1) & 1);
      scores(j & 1);
      lstore(j & 1);
      if (j + 1 < n_tiles) gload(kv0 + kGBN);
      __syncthreads();
      softmax(kv0);
      __syncthreads();
    }
    pv((n_tiles - 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O_w / l -> bf16, 4 consecutive columns per lane and block
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

template <class QT, class KVT>
hipError_t launch_d512_one(PrefillParams p, hipStream_t stream) {
  const int64_t slots = (p.n_tokens + kGBM - 1) / kGBM + p.n_seqs;
  p.tile_slots = (int32_t)slots;
  const uint64_t blocks = dispatch_grid((uint64_t)slots * (uint64_t)p.n_q_heads);
  if (p.page_size > 0)
    hipLaunchKernelGGL((prefill_d512_kernel<QT, KVT, true>), dim3((uint32_t)blocks),
                       dim3(kGThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_d512_kernel<QT, KVT, false>), dim3((uint32_t)blocks),
                       dim3(kGThreads), 0, stream, p);
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
