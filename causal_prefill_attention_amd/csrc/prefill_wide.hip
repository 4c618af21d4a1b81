// Causal / sliding-window prefill attention for wide heads on gfx950
// (CDNA4): head_dim 256, and q/k head size 320 with v/out head size 256 (the
// absorbed MLA prefill of atlas PR #69: [q_absorbed | q_rope] against the
// compressed cache row [kv_latent | k_rope], values = kv_latent, scale
// 1/sqrt(320)).  Same operation, inputs, masks and results as the
// 128-d kernel (causal bound kv_end = min(q_pos + 1, seq_len) of the fused
// MLA prefill in atlas PR #69; the W most recent keys for a window,
// m40-llm AGENTS.md "Current Progress"; KV histories and paged caches as
// in the chunked and paged MLA prefill of atlas PR #69); the head sizes of
// the HDIM-templated prefill kernels on the atlas page other than 128.
//
// Design: a 256-d head needs 128 fp32 accumulator registers and 64 Q
// operand registers per 32-row wave, more than the two-waves-per-SIMD
// budget of the 128-d kernel allows.  Here one wave per SIMD (4 waves, 128
// query rows per workgroup) owns up to 512 registers and runs, per 64-key
// tile, Sᵀ = K Qᵀ (32 MFMAs), the online softmax and Oᵀ += Vᵀ Pᵀ (32
// MFMAs); the MFMA chains of one tile overlap the softmax and staging of
// the wave through the matrix core's queue.  All four waves stage both K
// (row-major) and Vᵀ (key order of the Sᵀ accumulator) of the next tile
// through registers into two LDS stages, K and V at different points of the
// tile so that their staging registers are not live together; one barrier
// per tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "prefill_params.h"
#include "prefill_work.h"

namespace attnp {
namespace {

using namespace dev;

constexpr int kXWave = 64;
constexpr int kXWaves = 4;                 // one per SIMD
constexpr int kXThreads = kXWave * kXWaves;
constexpr int kXBN = 64;                   // keys per tile
constexpr int kXKB = kXBN / 32;
constexpr int kXKT = kXBN / 16;
constexpr int kXBM = 32 * kXWaves;         // query rows per workgroup
// Softmax of the 320/256 instance: a max pass on every tile, the running max
// moving when a tile's max exceeds it by more than 2^kXLazy (log2 units).
// The 256-d instance uses lazy_softmax (no max pass on most tiles, 2%
// faster); in the 320/256 instance its second exponent pass spills
// registers and costs 5%.
constexpr float kXLazy = 8.0f;

// DQK: head size of q and k (score contraction), DV: of v and out.
template <int DQK, int DV>
struct WideCfg {
  static_assert(DQK % 16 == 0 && DV % 32 == 0, "head sizes");
  static constexpr int KSTR = DQK + 8;
  static constexpr int VSTR = kXBN + 8;
  static constexpr int K_ELEMS = kXBN * KSTR;
  static constexpr int V_ELEMS = DV * VSTR;
  static constexpr int DCH = DQK / 16;
  static constexpr int DBLK = DV / 32;
  static constexpr int OCTS = DQK / 8;   // 16-byte chunks per K row
  static constexpr int VOCTS = DV / 8;   // 16-byte chunks per V row
  static constexpr int K_TOTAL = kXBN * OCTS;
  static constexpr int V_TOTAL = (kXBN / 4) * VOCTS;
  static constexpr int K_CHUNKS = K_TOTAL / kXThreads;
  // K staging: KTPR threads per row, each with KCPP 16-byte chunks of a row
  // in each of KPASS row passes
  static constexpr int KTPR = 8;
  static constexpr int KROWS = kXThreads / KTPR;
  static constexpr int KPASS = kXBN / KROWS;
  static constexpr int KCPP = OCTS / KTPR;
  static_assert(OCTS % KTPR == 0 && KPASS * KCPP == K_CHUNKS, "K staging map");
  static constexpr int V_UNITS = V_TOTAL / kXThreads;
  static_assert(K_CHUNKS * kXThreads == K_TOTAL && V_UNITS * kXThreads == V_TOTAL,
                "every thread stages the same share");
};

template <int DQK, int DV, class QT, class KVT, bool PAGED>
__global__ __launch_bounds__(kXThreads, 1) void prefill_wide_kernel(PrefillParams p) {
  using C = WideCfg<DQK, DV>;
  typedef typename QT::T qelem;
  typedef typename KVT::T kvelem;
  typedef typename OpOf<KVT>::T OP;  // operand type of both products
  typedef typename OP::v8 opv8;
  constexpr int kStage = 2 * C::K_ELEMS + 2 * C::V_ELEMS;
  constexpr int kOut = kXWaves * 32 * (DV + 8);
  __shared__ __attribute__((aligned(16))) uint16_t smem[kStage > kOut ? kStage : kOut];
  uint16_t* const kstage0 = smem;
  uint16_t* const vstage0 = smem + 2 * C::K_ELEMS;

  const int tid = threadIdx.x;
  const int lane = tid & (kXWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kXWave);
  const int bid = dispatch_index(blockIdx.x);
  const int slot = bid / p.n_q_heads;
  const int head = bid - slot * p.n_q_heads;
  Work w = decode_work<kXBM, PAGED>(p, slot);
  if (!w.valid) return;  // uniform across the workgroup
  w.start = __builtin_amdgcn_readfirstlane(w.start);
  w.len = __builtin_amdgcn_readfirstlane(w.len);
  w.q0 = __builtin_amdgcn_readfirstlane(w.q0);
  w.kstart = __builtin_amdgcn_readfirstlane(w.kstart);
  w.seq = __builtin_amdgcn_readfirstlane(w.seq);
  w.klen = __builtin_amdgcn_readfirstlane(w.klen);

  const int kvh = head / p.group;
  const int hist = w.klen - w.len;  // queries are the last len key positions
  const int q_end = min(w.len, w.q0 + kXBM);
  const int kv_hi = min(max(hist + q_end, 0), w.klen);
  const int kv_lo = p.window > 0 ? min(max(0, hist + w.q0 - p.window + 1), kv_hi) : 0;
  const int kv_start = kv_lo - kv_lo % kXBN;
  const int n_tiles = max(1, (kv_hi - kv_start + kXBN - 1) / kXBN);

  const int col = lane & 31;
  const int half = lane >> 5;
  const int wq0 = w.q0 + wave * 32;
  const int wq_last = min(wq0 + 31, w.len - 1);
  const bool wave_live = wq0 < w.len;
  const int myq = wq0 + col;
  const int mypos = hist + myq;

  // ---- Qᵀ operand: lane holds q[myq, 16c + 8*half .. +7]
  opv8 qf[C::DCH];  // loaded once the first tile's loads are in flight
  const qelem* const qrow = static_cast<const qelem*>(p.q) +
                            (int64_t)(w.start + (myq < w.len ? myq : 0)) * p.q_ts +
                            (int64_t)head * p.q_hs;
  const float qmul = myq < w.len ? p.q_mult : 0.f;

  // ---- K/V tile movement (every thread stages a share of both)
  const kvelem* kseq = static_cast<const kvelem*>(p.k) + (int64_t)w.kstart * p.k_ts +
                       (int64_t)kvh * p.k_hs;
  const kvelem* vseq = static_cast<const kvelem*>(p.v) + (int64_t)w.kstart * p.v_ts +
                       (int64_t)kvh * p.v_hs;
  const int k_row_bytes = (int)(p.k_ts * (int64_t)sizeof(kvelem));
  const int v_row_bytes = (int)(p.v_ts * (int64_t)sizeof(kvelem));
  auto tile_slot = [&](int kv0) -> int64_t {
    if (!PAGED) return kv0;
    const int* row = p.block_table + (int64_t)w.seq * p.table_stride;
    const int idx = __builtin_amdgcn_readfirstlane(kv0 / p.page_size);
    const int page = min(max(row[idx], 0), p.n_pages - 1);
    return (int64_t)page * p.page_size + (kv0 - idx * p.page_size);
  };
  auto rows_of = [&](int kv0) {
    return __builtin_amdgcn_readfirstlane(max(0, min(kv_hi - kv0, kXBN)));
  };
  u32x4_t kst[C::K_CHUNKS];
  u32x4_t vst[C::V_UNITS][4];
  const int k_row = tid / C::KTPR, k_oct = tid % C::KTPR;
  auto gload_k = [&](int kv0) {
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<kvelem*>(kseq + tile_slot(kv0) * p.k_ts), 0, rows_of(kv0) * k_row_bytes,
        kRsrcWord3);
    // thread t loads chunks (t % KTPR) + KTPR i of rows t / KTPR + KROWS pass:
    // every KTPR lanes read 128 contiguous bytes of a row, and one offset
    // register serves all of a thread's chunks (the rest are immediates)
#pragma unroll
    for (int pass = 0; pass < C::KPASS; ++pass)
#pragma unroll
      for (int i = 0; i < C::KCPP; ++i)
        kst[pass * C::KCPP + i] = __builtin_amdgcn_raw_buffer_load_b128(
            rk, (k_row + C::KROWS * pass) * k_row_bytes + 16 * (k_oct + C::KTPR * i), 0, 0);
  };
  auto gload_v = [&](int kv0) {
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<kvelem*>(vseq + tile_slot(kv0) * p.v_ts), 0, rows_of(kv0) * v_row_bytes,
        kRsrcWord3);
#pragma unroll
    for (int u = 0; u < C::V_UNITS; ++u) {
      const int unit = tid + u * kXThreads;
      const int kq = unit % (kXBN / 4);
      const int oct = unit / (kXBN / 4);  // < VOCTS
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vst[u][i] = __builtin_amdgcn_raw_buffer_load_b128(
            rv, (4 * kq + i) * v_row_bytes + 16 * oct, 0, 0);
    }
  };
  // K row-major; Vᵀ in the Sᵀ accumulator's key order (inside each 16-key
  // group, positions 4..7 hold keys 8..11 and positions 8..11 keys 4..7).
  auto store_k = [&](int st) {
    uint16_t* ks = kstage0 + st * C::K_ELEMS + k_row * C::KSTR + 8 * k_oct;
#pragma unroll
    for (int pass = 0; pass < C::KPASS; ++pass)
#pragma unroll
      for (int i = 0; i < C::KCPP; ++i)
        *reinterpret_cast<u32x4_t*>(ks + C::KROWS * pass * C::KSTR + 8 * C::KTPR * i) =
            kv_to_op(OP(), KVT(), kst[pass * C::KCPP + i]);
  };
  auto store_v = [&](int st) {
    uint16_t* vs = vstage0 + st * C::V_ELEMS;
#pragma unroll
    for (int u = 0; u < C::V_UNITS; ++u) {
      const int unit = tid + u * kXThreads;
      const int kq = unit % (kXBN / 4);
      const int oct = unit / (kXBN / 4);
      const int qq = kq & 3;
      const int pos = 16 * (kq >> 2) + 4 * (((qq & 1) << 1) | (qq >> 1));
      u32x4_t r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = kv_to_op(OP(), KVT(), vst[u][i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
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
  f32x16_t s[kXKB];
  opv8 pf[kXKT];
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float cmul = p.score_mult;

  auto tile_full = [&](int kv0) {
    return (kv0 + kXBN - 1 <= hist + wq0) &&
           (p.window == 0 || kv0 >= hist + wq_last - p.window + 1);
  };
  // The two products, every LDS operand read kAhead MFMAs ahead with the
  // order pinned: with one wave per SIMD nothing else hides the read
  // latency from the matrix core.
  constexpr int kAhead = 4;
  auto scores = [&](int st) {
    const uint16_t* ks = kstage0 + st * C::K_ELEMS;
    constexpr int N = C::DCH * kXKB;
    auto operand = [&](int i) -> opv8 {
      const int c = i / kXKB, kb = i % kXKB;
      return *reinterpret_cast<const opv8*>(ks + (32 * kb + col) * C::KSTR + 16 * c + 8 * half);
    };
    opv8 buf[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) buf[i] = operand(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const opv8 a = buf[i % kAhead];
      if (i + kAhead < N) buf[i % kAhead] = operand(i + kAhead);
      const int c = i / kXKB, kb = i % kXKB;
      s[kb] = OP::mfma(a, qf[c], c == 0 ? (f32x16_t){} : s[kb]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < N - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
  };
  auto pv = [&](int st) {
    const uint16_t* vs = vstage0 + st * C::V_ELEMS;
    constexpr int N = kXKT * C::DBLK;
    auto operand = [&](int i) -> opv8 {
      const int kt = i / C::DBLK, c = i % C::DBLK;
      return *reinterpret_cast<const opv8*>(vs + (32 * c + col) * C::VSTR + 16 * kt + 8 * half);
    };
    opv8 buf[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) buf[i] = operand(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const opv8 a = buf[i % kAhead];
      if (i + kAhead < N) buf[i % kAhead] = operand(i + kAhead);
      const int kt = i / C::DBLK, c = i % C::DBLK;
      o[c] = OP::mfma(a, pf[kt], o[c]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < N - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
  };
  auto softmax = [&](int kv0) {
    if (!tile_full(kv0)) {
#pragma unroll
      for (int kb = 0; kb < kXKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = key <= mypos && (p.window == 0 || key > mypos - p.window);
          if (!vis) s[kb][r] = -INFINITY;
        }
    }
    auto rescale = [&](float alpha) {
#pragma unroll
      for (int c = 0; c < C::DBLK; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
    };
    if constexpr (DQK <= 256) {
      lazy_softmax<OP, kXKT>([&](int kt, int i) { return s[kt >> 1][8 * (kt & 1) + i]; },
                             cmul, m_run, l_run, pf, rescale);
      return;
    }
    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < kXKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], s[kb][r]);
    float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    mx = pair_max(mx);
    const bool raise = (mx - m_run) * cmul > kXLazy;
    const bool any = __ballot(raise) != 0ull;
    const float m_new = any ? fmaxf(m_run, mx) : m_run;
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2((m_run - m_new) * cmul);
    const float neg_mc = (m_new == -INFINITY) ? 0.f : -m_new * cmul;
    m_run = m_new;
    float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < kXKT; ++kt) {
      u32x4_t u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(fmaf(s[kt >> 1][8 * (kt & 1) + 2 * e], cmul, neg_mc));
        const float p1 = fast_exp2(fmaf(s[kt >> 1][8 * (kt & 1) + 2 * e + 1], cmul, neg_mc));
        // (the converted pair feeds the dot product directly; see the 128-d kernel)
        const typename OP::v2 pb = OP::cvt2(p0, p1);
        u[e] = __builtin_bit_cast(uint32_t, pb);
        l4[e] = OP::sum2(pb, l4[e]);
      }
      pf[kt] = __builtin_bit_cast(opv8, u);
    }
    l_run = l_run * alpha + ((l4[0] + l4[1]) + (l4[2] + l4[3]));
    if (any) rescale(alpha);
  };

  // ---- tile loop: tile j in stage j & 1.  Tile j + 1 moves in during
  // iteration j -- K loaded at its start and stored after the softmax, V
  // loaded then and stored after P.V -- so the K and V staging registers are
  // never live at once; stage (j+1) & 1 last held tile j - 1, which every
  // wave finished before the previous barrier.  One barrier per tile.
  gload_k(kv_start);
  gload_v(kv_start);
  load_q_op<C::DCH, OP>(qrow, half, qmul, qf);
  store_k(0);
  store_v(0);
  __syncthreads();
  for (int j = 0; j < n_tiles; ++j) {
    const int kv0 = kv_start + j * kXBN;
    const bool more = j + 1 < n_tiles;
    if (more) gload_k(kv0 + kXBN);
    scores(j & 1);
    softmax(kv0);
    if (more) {
      store_k((j + 1) & 1);
      gload_v(kv0 + kXBN);
    }
    pv(j & 1);
    if (more) store_v((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O / l -> bf16 via the wave's LDS slice, whole rows stored
  const float l_tot = pair_sum(l_run);
  if (wave_live) {
    constexpr int OSTR = DV + 8;
    uint16_t* ob = smem + wave * 32 * OSTR;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int c = 0; c < C::DBLK; ++c)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        u32x2_t pk;
        pk[0] = pack_bf16x2(o[c][4 * rb] * inv, o[c][4 * rb + 1] * inv);
        pk[1] = pack_bf16x2(o[c][4 * rb + 2] * inv, o[c][4 * rb + 3] * inv);
        *reinterpret_cast<u32x2_t*>(ob + col * OSTR + 32 * c + 8 * rb + 4 * half) = pk;
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    constexpr int CPR = DV / 8;
    constexpr int RPI = kXWave / CPR > 0 ? kXWave / CPR : 1;  // rows per store round
    constexpr int LPR = CPR / (kXWave / RPI);                  // chunks per lane per row
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = RPI * i + lane / (CPR / LPR);
#pragma unroll
      for (int k = 0; k < LPR; ++k) {
        const int ch = (lane % (CPR / LPR)) * LPR + k;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ob + row * OSTR + 8 * ch);
        if (wq0 + row < w.len)
          *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p.out) +
                                      (int64_t)(w.start + wq0 + row) * p.o_ts +
                                      (int64_t)head * p.o_hs + 8 * ch) = v;
      }
    }
  }
}

template <int DQK, int DV, class QT, class KVT>
hipError_t launch_wide_one(PrefillParams p, hipStream_t stream) {
  const int64_t slots = (p.n_tokens + kXBM - 1) / kXBM + p.n_seqs;
  p.tile_slots = (int32_t)slots;
  const uint64_t blocks = dispatch_grid((uint64_t)slots * (uint64_t)p.n_q_heads);
  if (p.page_size > 0)
    hipLaunchKernelGGL((prefill_wide_kernel<DQK, DV, QT, KVT, true>), dim3((uint32_t)blocks),
                       dim3(kXThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_wide_kernel<DQK, DV, QT, KVT, false>), dim3((uint32_t)blocks),
                       dim3(kXThreads), 0, stream, p);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_wide_dtypes(const PrefillParams& p, DType q_dtype, DType kv_dtype,
                              hipStream_t stream) {
  if (q_dtype == kBF16 && kv_dtype == kBF16) return launch_wide_one<DQK, DV, BF16, BF16>(p, stream);
  if (q_dtype == kBF16 && kv_dtype == kFP16) return launch_wide_one<DQK, DV, BF16, FP16>(p, stream);
  if (q_dtype == kFP32 && kv_dtype == kBF16) return launch_wide_one<DQK, DV, FP32, BF16>(p, stream);
  if (q_dtype == kFP32 && kv_dtype == kFP16) return launch_wide_one<DQK, DV, FP32, FP16>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace

int prefill_wide_block_m() { return kXBM; }

hipError_t launch_prefill_wide(const PrefillParams& p, int head_dim_qk, int head_dim_v,
                               DType q_dtype, DType kv_dtype, hipStream_t stream) {
  if (head_dim_qk == 256 && head_dim_v == 256)
    return launch_wide_dtypes<256, 256>(p, q_dtype, kv_dtype, stream);
  if (head_dim_qk == 320 && head_dim_v == 256)
    return launch_wide_dtypes<320, 256>(p, q_dtype, kv_dtype, stream);
  return hipErrorInvalidValue;
}

}  // namespace attnp
