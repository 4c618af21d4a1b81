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
// budget.  Instead the four waves of a workgroup (one per SIMD) share the
// same 32 query rows and split the head dimension: wave w owns columns
// [128w, 128w + 128) of Q, K, V and out.
//   * Per 64-key tile, wave w forms the partial scores Sᵀ_w = K_w Q_wᵀ from
//     its 128 columns (16 MFMAs, 32x32x16 bf16), the four partials are
//     summed through LDS in a fixed order (so every wave holds the same fp32
//     scores), every wave runs the same online softmax (the same P, running
//     max and sum in all four), and wave w accumulates Oᵀ_w += Vᵀ_w Pᵀ for
//     its 128 output columns (16 MFMAs).  No MFMA work is repeated.
//   * A wave only ever reads its own columns of K and V, so it stages them
//     privately: coalesced 16-byte loads one tile ahead into registers, bf16
//     conversion, a store into its own LDS slice with 16-byte chunks of row
//     r at position (chunk ^ (r & 15)); K operands are read row-wise, Vᵀ
//     operands with ds_read_b64_tr_b16 (four keys of one column per lane, in
//     the Sᵀ accumulator's key order).
//   * Two barriers per tile fence the 32 KiB score exchange (16-byte LDS
//     writes and reads); LDS holds four 32 KiB K/V slices plus the
//     exchange, 160 KiB in all.
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
constexpr int kGWaves = 4;                  // one per SIMD, one column slice each
constexpr int kGThreads = kGWave * kGWaves;
constexpr int kGHead = 512;                 // head size of q, k, v and out
constexpr int kGSlice = kGHead / kGWaves;   // 128 columns per wave
constexpr int kGBM = 32;                    // query rows per workgroup
constexpr int kGBN = 64;                    // keys per tile
constexpr float kGLazy = 8.0f;              // lazy-max threshold, log2 units

template <class QT, class KVT, bool PAGED>
__global__ __launch_bounds__(kGThreads, 1) void prefill_d512_kernel(PrefillParams p) {
  constexpr int CPR = kGSlice / 8;          // 16-byte chunks per slice row
  constexpr int DCH = kGSlice / 16;         // score k-steps per wave
  constexpr int DBLK = kGSlice / 32;        // output blocks per wave
  constexpr int TILE = kGBN * kGSlice;      // elements of one K (or V) slice tile
  constexpr int LOADS = kGBN * CPR / kGWave;  // 16-byte chunks per lane per tile
  typedef typename QT::T qelem;
  typedef typename KVT::T kvelem;

  // per wave: K slice tile then V slice tile (bf16, rows of 128, swizzled)
  __shared__ __attribute__((aligned(16))) uint16_t kvs[kGWaves * 2 * TILE];
  // partial scores of every wave: [wave][kb][r / 4][lane] x 4 floats
  __shared__ __attribute__((aligned(16))) f32x4_t xch[kGWaves * 2 * 4 * kGWave];

  const int tid = threadIdx.x;
  const int lane = tid & (kGWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kGWave);
  const int col = lane & 31;   // query column of this lane
  const int half = lane >> 5;
  const int slot = blockIdx.x / p.n_q_heads;
  const int head = blockIdx.x - slot * p.n_q_heads;
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
  const int q_last = min(w.q0 + kGBM - 1, w.len - 1);
  const int myq = w.q0 + col;
  const int mypos = hist + myq;
  const int d0 = wave * kGSlice;  // first column of this wave's slice

  // ---- K/V slice tiles: lane moves chunk (lane % CPR) of rows 4i + lane / CPR
  const kvelem* kbase = static_cast<const kvelem*>(p.k) + (int64_t)w.kstart * p.k_ts +
                        (int64_t)kvh * p.k_hs + d0;
  const kvelem* vbase = static_cast<const kvelem*>(p.v) + (int64_t)w.kstart * p.v_ts +
                        (int64_t)kvh * p.v_hs + d0;
  const int k_row_bytes = (int)(p.k_ts * (int64_t)sizeof(kvelem));
  const int v_row_bytes = (int)(p.v_ts * (int64_t)sizeof(kvelem));
  auto tile_slot = [&](int kv0) -> int64_t {
    if (!PAGED) return kv0;
    const int* row = p.block_table + (int64_t)w.seq * p.table_stride;
    const int idx = __builtin_amdgcn_readfirstlane(kv0 / p.page_size);
    const int page = min(max(row[idx], 0), p.n_pages - 1);
    return (int64_t)page * p.page_size + (kv0 - idx * p.page_size);
  };
  u32x4_t kr[LOADS], vr[LOADS];
  auto gload = [&](int kv0) {
    // rows past the last visible key read as zero (buffer range)
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(kv_hi - kv0, kGBN)));
    const int64_t ts = tile_slot(kv0);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<kvelem*>(kbase + ts * p.k_ts), 0, rows * k_row_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<kvelem*>(vbase + ts * p.v_ts), 0, rows * v_row_bytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int row = i * (kGWave / CPR) + lane / CPR;
      const int ch = lane % CPR;
      kr[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, row * k_row_bytes + 16 * ch, 0, 0);
      vr[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, row * v_row_bytes + 16 * ch, 0, 0);
    }
  };
  uint16_t* const kt = kvs + wave * 2 * TILE;
  uint16_t* const vt = kt + TILE;
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int row = i * (kGWave / CPR) + lane / CPR;
      const int pos = (lane % CPR) ^ (row & 15);
      *reinterpret_cast<u32x4_t*>(kt + row * kGSlice + 8 * pos) = kv_to_bf16(KVT(), kr[i]);
      *reinterpret_cast<u32x4_t*>(vt + row * kGSlice + 8 * pos) = kv_to_bf16(KVT(), vr[i]);
    }
  };

  // first tile in flight before Q, so that the two latencies overlap
  gload(kv_start);

  // ---- Qᵀ operand of this wave's slice: lane holds q[myq, d0 + 16c + 8*half ..]
  bf16x8_t qf[DCH];
  {
    const qelem* qrow = static_cast<const qelem*>(p.q) +
                        (int64_t)(w.start + (myq < w.len ? myq : 0)) * p.q_ts +
                        (int64_t)head * p.q_hs + d0;
    load_q_operand<DCH>(qrow, half, myq < w.len ? p.q_mult : 0.f, qf);
  }

  // ---- per-wave state (m_run and l_run are the same in all four waves)
  f32x16_t o[DBLK];
#pragma unroll
  for (int c = 0; c < DBLK; ++c) o[c] = (f32x16_t){};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float cmul = p.score_mult;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  f32x4_t* const xw = xch + wave * 2 * 4 * kGWave;

  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = kv_start + t * kGBN;
    lstore();  // tile t: registers -> this wave's slice (read by this wave only)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (t + 1 < n_tiles) gload(kv0 + kGBN);  // tile t+1 in flight meanwhile

    // partial Sᵀ = K_w Q_wᵀ: keys on M (two 32-key blocks), queries on N
    f32x16_t sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = (f32x16_t){};
      const int row = 32 * kb + col;
#pragma unroll
      for (int c = 0; c < DCH; ++c) {
        const int pos = (2 * c + half) ^ (row & 15);
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kt + row * kGSlice + 8 * pos);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], sc[kb], 0, 0, 0);
      }
    }
    // exchange: every wave finished reading the previous tile's partials
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        xw[(kb * 4 + r4) * kGWave + lane] = (f32x4_t){sc[kb][4 * r4], sc[kb][4 * r4 + 1],
                                                      sc[kb][4 * r4 + 2], sc[kb][4 * r4 + 3]};
    __syncthreads();
    // full scores, summed in wave order 0..3 in every wave
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4_t acc = xch[(kb * 4 + r4) * kGWave + lane];
#pragma unroll
        for (int v = 1; v < kGWaves; ++v) acc += xch[((v * 2 + kb) * 4 + r4) * kGWave + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[kb][4 * r4 + e] = acc[e];
      }

    // mask the causal diagonal, the window start and the key count
    const bool full = (kv0 + kGBN - 1 <= hist + w.q0) &&
                      (p.window == 0 || kv0 >= hist + q_last - p.window + 1);
    if (!full) {
      // key = kv0 + 4*half + off, off = 32*kb + 8*(r/4) + r%4 (compile-time):
      // visible when off <= hi and, with a window, off >= lo
      const int hi = mypos - kv0 - 4 * half;
      // (lo <= 0 bounds nothing since off >= 0: the subtraction only runs where it
      // cannot overflow; no branch, the same code with and without a window)
      const int lo = (p.window > 0 && p.window <= hi) ? hi - p.window + 1 : INT_MIN;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
          if (off > hi || off < lo) sc[kb][r] = -INFINITY;
        }
    }
    // online softmax (lazy max, base 2) into the bf16 Pᵀ operand
    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], sc[kb][r]);
    float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    mx = pair_max(mx);
    const bool raise = (mx - m_run) * cmul > kGLazy;
    const bool any = __ballot(raise) != 0ull;
    const float m_new = any ? fmaxf(m_run, mx) : m_run;
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2((m_run - m_new) * cmul);
    const float neg_mc = (m_new == -INFINITY) ? 0.f : -m_new * cmul;
    m_run = m_new;
    bf16x8_t pf[4];
    float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      u32x4_t u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(fmaf(sc[kq >> 1][8 * (kq & 1) + 2 * e], cmul, neg_mc));
        const float p1 = fast_exp2(fmaf(sc[kq >> 1][8 * (kq & 1) + 2 * e + 1], cmul, neg_mc));
        // (the converted pair feeds the dot product directly; see the 128-d kernel)
        const bf16x2_t pb = __builtin_convertvector((f32x2_t){p0, p1}, bf16x2_t);
        u[e] = __builtin_bit_cast(uint32_t, pb);
        l4[e] = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, l4[e], false);
      }
      pf[kq] = __builtin_bit_cast(bf16x8_t, u);
    }
    l_run = l_run * alpha + ((l4[0] + l4[1]) + (l4[2] + l4[3]));
    if (any) {
#pragma unroll
      for (int c = 0; c < DBLK; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
    }

    // Oᵀ_w += Vᵀ_w Pᵀ.  MFMA k-index 8*half + e of step kq is key
    // 16*kq + 8*(e / 4) + 4*half + e % 4 (the Sᵀ accumulator's order): two
    // transposing reads give keys +0..3 and +8..11 (+4*half) of column d.
    const int grp = (lane >> 4) & 1;  // 16-column half of the 32-row block
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
              (__attribute__((address_space(3))) s16x4_t*)(vt + row * kGSlice + 8 * pos +
                                                           (d & 7)));
        }
        u32x4_t u;
        u[0] = __builtin_bit_cast(u32x2_t, part[0])[0];
        u[1] = __builtin_bit_cast(u32x2_t, part[0])[1];
        u[2] = __builtin_bit_cast(u32x2_t, part[1])[0];
        u[3] = __builtin_bit_cast(u32x2_t, part[1])[1];
        o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, u), pf[kq],
                                                       o[c], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
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
  const uint64_t blocks = (uint64_t)slots * (uint64_t)p.n_q_heads;
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
