// Causal / sliding-window prefill attention forward for gfx950 (CDNA4).
//
// What is computed (one workgroup = one query tile of one query head):
//   out[i,h] = sum_j softmax_j(scale * q[i,h] . k[j,g]) v[j,g],
//   j visible iff j <= i (causal bound kv_end = min(q_pos + 1, seq_len), atlas
//   PR #69 fused MLA prefill) and, for a window W > 0, j >= i - W + 1 (the W
//   most recent keys, m40-llm AGENTS.md "Current Progress").  The softmax is
//   evaluated online over key tiles with a running max and running sum (the
//   fused MLA prefill kernel's recurrence in atlas PR #69), in base 2 with
//   log2(e) folded into the score multiplier.
//
// Design (ours, for CDNA4 -- the pages' GB10 / M40 kernels are prior art):
//   * Both contractions use v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//   * Scores are formed transposed, S^T = K Q^T (keys on the MFMA M axis,
//     queries on N), so every lane owns ONE query column: the per-query max
//     and sum reduce 16 values in-lane plus one lane-pair exchange
//     (v_permlane32_swap), and the softmax row scale is one scalar per lane.
//   * The S^T accumulator, rounded to bf16, is directly the B operand of
//     O^T += V^T P^T.  The key order inside each 16-key MFMA step follows the
//     accumulator layout; V^T is written into LDS in that permuted order.
//   * K is staged row-major in LDS, V transposed (V^T), both padded so that
//     the 16-byte operand reads are bank-conflict free; the next tile is
//     fetched into registers while the current one is consumed (two LDS
//     stages, one barrier per tile).
//   * Varlen: the grid covers an upper bound of q-tile slots; each workgroup
//     decodes its (sequence, tile) from cu_seqlens with a wave-wide scan, so
//     the host never reads the offsets.  Each sequence's tiles run heaviest
//     (last) first.  Offsets are clamped into [0, T].
//   * Every global address is token * token_stride + head * head_stride in
//     64-bit elements with head_dim explicit: a 128-d head is never read or
//     written with another head size's extent (the HDIM=256-on-128 overread
//     fixed in atlas PR #69).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "prefill_params.h"

namespace attnp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kBM = 128;  // query rows per workgroup: 32 per wave
constexpr int kBN = 64;   // keys per KV tile: two 32-key MFMA blocks

template <int HDIM>
struct Cfg {
  static_assert(HDIM % 32 == 0, "head_dim must be a multiple of 32");
  static constexpr int KSTR = HDIM + 8;  // K row pitch in LDS (bf16 elements)
  static constexpr int VSTR = kBN + 8;   // V^T row pitch in LDS (bf16 elements)
  static constexpr int K_ELEMS = kBN * KSTR;
  static constexpr int V_ELEMS = HDIM * VSTR;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int DCH = HDIM / 16;   // MFMA k-steps of the Q.K contraction
  static constexpr int DBLK = HDIM / 32;  // 32-wide output column blocks
  static constexpr int OCTS = HDIM / 8;   // 16-byte chunks per row
  static constexpr int K_CHUNKS = kBN * OCTS / kThreads;
  static constexpr int V_UNITS = (kBN / 4) * OCTS / kThreads;  // 4 keys x 8 d
  static_assert(K_CHUNKS * kThreads == kBN * OCTS, "K tile split");
  static_assert(V_UNITS * kThreads == (kBN / 4) * OCTS, "V tile split");
};

// ---------------------------------------------------------------- element io
struct BF16 { typedef uint16_t T; };
struct FP16 { typedef _Float16 T; };
struct FP32 { typedef float T; };

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t r = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Eight consecutive elements as float.
__device__ __forceinline__ void load8f(const uint16_t* p, float* f) {
  const u32x4_t u = load16(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8f(const float* p, float* f) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = a[i];
    f[4 + i] = b[i];
  }
}

// Raw 16-byte K/V chunk -> eight bf16 (identity for bf16 storage).
__device__ __forceinline__ u32x4_t kv_to_bf16(BF16, u32x4_t raw) { return raw; }
__device__ __forceinline__ u32x4_t kv_to_bf16(FP16, u32x4_t raw) {
  const f16x8_t h = __builtin_bit_cast(f16x8_t, raw);
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2((float)h[2 * i], (float)h[2 * i + 1]);
  return r;
}

// Value of the other half-wave's lane (l <-> l ^ 32) combined with ours.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------- work decode
struct Work {
  int start;  // first token of the sequence in the packed batch
  int len;    // sequence length
  int q0;     // first local query row of this tile
  bool valid;
};

// Maps a q-tile slot to (sequence, tile).  Slots enumerate sequences in
// order; inside a sequence the last (most expensive causal) tile comes
// first.  Every lane of the wave computes the same answer.
__device__ Work decode_work(const PrefillParams& p, int slot) {
  const int lane = threadIdx.x & (kWave - 1);
  int base = 0;
  for (int s0 = 0; s0 < p.n_seqs; s0 += kWave) {
    const int s = s0 + lane;
    int a = 0, b = 0;
    if (s < p.n_seqs) {
      a = min(max(p.cu_seqlens[s], 0), p.n_tokens);
      b = min(max(p.cu_seqlens[s + 1], 0), p.n_tokens);
    }
    const int len = max(b - a, 0);
    const int nt = (len + kBM - 1) / kBM;
    int incl = nt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    const int total = __shfl(incl, kWave - 1, kWave);
    if (slot < base + total) {
      const unsigned long long hit = __ballot(base + incl > slot);
      const int src = __ffsll((long long)hit) - 1;
      const int excl = __shfl(incl - nt, src, kWave);
      Work w;
      w.start = __shfl(a, src, kWave);
      w.len = __shfl(len, src, kWave);
      const int ntiles = __shfl(nt, src, kWave);
      const int rank = slot - base - excl;  // 0 = heaviest tile
      w.q0 = (ntiles - 1 - rank) * kBM;
      w.valid = true;
      return w;
    }
    base += total;
  }
  Work w{0, 0, 0, false};
  return w;
}

// ------------------------------------------------------------------ kernel
template <int HDIM, class QT, class KVT>
__global__ __launch_bounds__(kThreads, 2) void prefill_fwd_kernel(PrefillParams p) {
  using C = Cfg<HDIM>;
  typedef typename QT::T qelem;
  typedef typename KVT::T kvelem;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int slot = blockIdx.x / p.n_q_heads;
  const int head = blockIdx.x - slot * p.n_q_heads;
  const Work w = decode_work(p, slot);
  if (!w.valid) return;  // uniform across the workgroup

  const int kvh = head / p.group;
  const int q_end = min(w.len, w.q0 + kBM);
  const int kv_hi = q_end;  // last query of the tile sees keys < q_end
  const int kv_lo = p.window > 0 ? max(0, w.q0 - p.window + 1) : 0;
  const int kv_start = kv_lo - kv_lo % kBN;
  const int n_tiles = (kv_hi - kv_start + kBN - 1) / kBN;

  const int col = lane & 31;   // query column of this lane inside the wave
  const int half = lane >> 5;  // which 8-wide half of each 16-wide k-step
  const int wq0 = w.q0 + wave * 32;
  const int wq_last = min(wq0 + 31, w.len - 1);
  const bool wave_live = wq0 < w.len;
  const int myq = wq0 + col;

  // ---- Q^T operand: lane holds q[myq, 16c + 8*half .. +7] for every c.
  bf16x8_t qf[C::DCH];
  {
    const bool ok = myq < w.len;
    const qelem* qp = static_cast<const qelem*>(p.q) +
                      (int64_t)(w.start + (ok ? myq : 0)) * p.q_ts + (int64_t)head * p.q_hs;
#pragma unroll
    for (int c = 0; c < C::DCH; ++c) {
      float f[8];
      if (ok) {
        load8f(qp + 16 * c + 8 * half, f);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = 0.f;
      }
      u32x4_t u;
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(f[2 * e] * p.q_mult, f[2 * e + 1] * p.q_mult);
      qf[c] = __builtin_bit_cast(bf16x8_t, u);
    }
  }

  const kvelem* kbase = static_cast<const kvelem*>(p.k) + (int64_t)kvh * p.k_hs;
  const kvelem* vbase = static_cast<const kvelem*>(p.v) + (int64_t)kvh * p.v_hs;

  u32x4_t kst[C::K_CHUNKS];
  u32x4_t vst[C::V_UNITS][4];

  // Global -> registers for the tile starting at local key kv0.  Keys at or
  // past kv_hi (beyond the tile's last query, or the sequence) read as zero.
  auto gload = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < C::K_CHUNKS; ++i) {
      const int chunk = tid + i * kThreads;
      const int row = chunk / C::OCTS;
      const int oct = chunk % C::OCTS;
      const int key = kv0 + row;
      kst[i] = (u32x4_t){0u, 0u, 0u, 0u};
      if (key < kv_hi) kst[i] = load16(kbase + (int64_t)(w.start + key) * p.k_ts + 8 * oct);
    }
#pragma unroll
    for (int u = 0; u < C::V_UNITS; ++u) {
      const int unit = tid + u * kThreads;
      const int kq = unit & 15;
      const int oct = unit >> 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kv0 + 4 * kq + i;
        vst[u][i] = (u32x4_t){0u, 0u, 0u, 0u};
        if (key < kv_hi) vst[u][i] = load16(vbase + (int64_t)(w.start + key) * p.v_ts + 8 * oct);
      }
    }
  };

  // Registers -> LDS stage.  K row-major; V transposed with the key order of
  // the S^T accumulator: inside each 16-key group, LDS positions 4..7 hold
  // keys 8..11 and positions 8..11 hold keys 4..7.
  auto lds_store = [&](int stage) {
    uint16_t* ks = smem + stage * C::STAGE;
    uint16_t* vs = ks + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::K_CHUNKS; ++i) {
      const int chunk = tid + i * kThreads;
      const int row = chunk / C::OCTS;
      const int oct = chunk % C::OCTS;
      *reinterpret_cast<u32x4_t*>(ks + row * C::KSTR + 8 * oct) = kv_to_bf16(KVT(), kst[i]);
    }
#pragma unroll
    for (int u = 0; u < C::V_UNITS; ++u) {
      const int unit = tid + u * kThreads;
      const int kq = unit & 15;
      const int oct = unit >> 4;
      const int qq = kq & 3;
      const int pos = 16 * (kq >> 2) + 4 * (((qq & 1) << 1) | (qq >> 1));
      u32x4_t r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = kv_to_bf16(KVT(), vst[u][i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int dw = j >> 1;
        u32x2_t out;
        if (j & 1) {
          out[0] = (r[0][dw] >> 16) | (r[1][dw] & 0xffff0000u);
          out[1] = (r[2][dw] >> 16) | (r[3][dw] & 0xffff0000u);
        } else {
          out[0] = (r[0][dw] & 0xffffu) | (r[1][dw] << 16);
          out[1] = (r[2][dw] & 0xffffu) | (r[3][dw] << 16);
        }
        *reinterpret_cast<u32x2_t*>(vs + (8 * oct + j) * C::VSTR + pos) = out;
      }
    }
  };

  gload(kv_start);
  lds_store(0);
  __syncthreads();

  f32x16_t o[C::DBLK];
#pragma unroll
  for (int c = 0; c < C::DBLK; ++c) o[c] = (f32x16_t){};
  float m_run = -INFINITY;  // running max of raw scores q.k
  float l_run = 0.f;        // this lane's share of the running sum
  const float cmul = p.score_mult;

  for (int it = 0; it < n_tiles; ++it) {
    const int kv0 = kv_start + it * kBN;
    const bool more = it + 1 < n_tiles;
    if (more) gload(kv0 + kBN);
    const uint16_t* ks = smem + (it & 1) * C::STAGE;
    const uint16_t* vs = ks + C::K_ELEMS;

    const bool skip = !wave_live || kv0 > wq_last ||
                      (p.window > 0 && kv0 + kBN - 1 < wq0 - p.window + 1);
    if (!skip) {
      // ---- S^T = K Q^T for keys kv0 .. kv0+63 (two 32-key blocks).
      f32x16_t s[2] = {(f32x16_t){}, (f32x16_t){}};
#pragma unroll
      for (int c = 0; c < C::DCH; ++c) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
              ks + (32 * kb + col) * C::KSTR + 16 * c + 8 * half);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[kb], 0, 0, 0);
        }
      }
      // ---- mask (only tiles that straddle the diagonal or the window edge)
      const bool full = (kv0 + kBN - 1 <= wq0) &&
                        (p.window == 0 || kv0 >= wq_last - p.window + 1);
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool vis = key <= myq && (p.window == 0 || key > myq - p.window);
            if (!vis) s[kb][r] = -INFINITY;
          }
        }
      }
      // ---- online softmax (base 2): running max m, sum l, rescale O.
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      }
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * cmul);
      const float neg_mc = -m_use * cmul;
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < C::DBLK; ++c) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
      }
      bf16x8_t pf[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        u32x4_t u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(fmaf(s[kt >> 1][8 * (kt & 1) + 2 * e], cmul, neg_mc));
          const float p1 = fast_exp2(fmaf(s[kt >> 1][8 * (kt & 1) + 2 * e + 1], cmul, neg_mc));
          l_run += p0 + p1;
          u[e] = pack_bf16x2(p0, p1);
        }
        pf[kt] = __builtin_bit_cast(bf16x8_t, u);
      }
      m_run = m_new;
      // ---- O^T += V^T P^T
#pragma unroll
      for (int c = 0; c < C::DBLK; ++c) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
              vs + (32 * c + col) * C::VSTR + 16 * kt + 8 * half);
          o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kt], o[c], 0, 0, 0);
        }
      }
    }
    if (more) lds_store((it + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O / l -> bf16, rows of this sequence only.
  const float l_tot = pair_sum(l_run);
  if (wave_live && myq < w.len) {
    const float inv = 1.f / l_tot;
    uint16_t* op = static_cast<uint16_t*>(p.out) + (int64_t)(w.start + myq) * p.o_ts +
                   (int64_t)head * p.o_hs;
#pragma unroll
    for (int c = 0; c < C::DBLK; ++c) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int d = 32 * c + 8 * rb + 4 * half;
        u32x2_t pk;
        pk[0] = pack_bf16x2(o[c][4 * rb] * inv, o[c][4 * rb + 1] * inv);
        pk[1] = pack_bf16x2(o[c][4 * rb + 2] * inv, o[c][4 * rb + 3] * inv);
        *reinterpret_cast<u32x2_t*>(op + d) = pk;
      }
    }
  }
}

template <int HDIM, class QT, class KVT>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
  const uint64_t blocks = (uint64_t)p.tile_slots * (uint64_t)p.n_q_heads;
  hipLaunchKernelGGL((prefill_fwd_kernel<HDIM, QT, KVT>), dim3((uint32_t)blocks),
                     dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int prefill_block_m(int /*head_dim*/) { return kBM; }

hipError_t launch_prefill(const PrefillParams& p, int head_dim, DType q_dtype,
                          DType kv_dtype, hipStream_t stream) {
  if (head_dim == 128) {
    if (q_dtype == kBF16 && kv_dtype == kBF16) return launch_one<128, BF16, BF16>(p, stream);
    if (q_dtype == kBF16 && kv_dtype == kFP16) return launch_one<128, BF16, FP16>(p, stream);
    if (q_dtype == kFP32 && kv_dtype == kBF16) return launch_one<128, FP32, BF16>(p, stream);
    if (q_dtype == kFP32 && kv_dtype == kFP16) return launch_one<128, FP32, FP16>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace attnp
