// Device helpers shared by the prefill and decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnp {
namespace dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;

// Dispatch order.  Workgroup b of a grid goes to XCD b mod 8, and an XCD
// starts its workgroups in order, four at a time (one per shader engine),
// each four once all four engines have a free CU; so the four that start
// together should take equally long.  A grid in dispatch order is a whole
// number of rounds of 32 workgroups (dispatch_grid), and workgroup b runs
// linear index dispatch_index(b): in each round, the k-th workgroup on XCD
// x runs index 4q + k, q = x in even rounds and x ^ 6 in odd ones.  With 8
// (or 16) workgroups per work item (prefill: per query tile slot; decode:
// per sequence or per split unit) the four are parts of one item, an XCD
// keeps the same parts in every round (with 8 per item: the KV heads its
// L2 holds), and over two rounds every XCD gets as much work.  Indices past
// the work exit at once.
__device__ __forceinline__ int dispatch_index(unsigned b) {
  const unsigned q = (b & 7u) ^ (6u * ((b >> 5) & 1u));
  return (int)((b & ~31u) | (q << 2) | ((b >> 3) & 3u));
}
inline uint64_t dispatch_grid(uint64_t n) { return (n + 31) & ~(uint64_t)31; }

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

// ------------------------------------------------------ MFMA operand types
// The matrix products run in the K/V storage type: bf16 K/V on the bf16
// MFMA, fp16 K/V on the fp16 MFMA, so that keys and values enter both
// products exactly as stored (the pages keep K/V in FP16 and compute in
// FP32: m40-llm AGENTS.md "Project Snapshot").  Q and the probabilities P
// are rounded (to nearest even) to that type; accumulation is fp32.
struct OpBF16 {
  typedef bf16x8_t v8;
  typedef bf16x2_t v2;
  static __device__ __forceinline__ f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ v2 cvt2(float a, float b) {
    return __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  }
  // acc + x.x + x.y
  static __device__ __forceinline__ float sum2(v2 x, float acc) {
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(x, ones, acc, false);
  }
};

struct OpFP16 {
  typedef f16x8_t v8;
  typedef f16x2_t v2;
  static __device__ __forceinline__ f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ v2 cvt2(float a, float b) {
    return __builtin_convertvector((f32x2_t){a, b}, f16x2_t);
  }
  static __device__ __forceinline__ float sum2(v2 x, float acc) {
    const f16x2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(x, ones, acc, false);
  }
};

// Operand type of each K/V storage type.
template <class KVT> struct OpOf;
template <> struct OpOf<BF16> { typedef OpBF16 T; };
template <> struct OpOf<FP16> { typedef OpFP16 T; };

// Raw 16-byte K/V chunk -> eight operand elements: the identity when the
// operand type is the storage type.
__device__ __forceinline__ u32x4_t kv_to_op(OpBF16, BF16, u32x4_t raw) { return raw; }
__device__ __forceinline__ u32x4_t kv_to_op(OpFP16, FP16, u32x4_t raw) { return raw; }

// Eight floats -> the operand register of type OP.
template <class OP>
__device__ __forceinline__ typename OP::v8 to_op8(const float* f, float mult) {
  u32x4_t u;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    u[e] = __builtin_bit_cast(uint32_t, OP::cvt2(f[2 * e] * mult, f[2 * e + 1] * mult));
  return __builtin_bit_cast(typename OP::v8, u);
}

// The Qᵀ MFMA operand of one lane in operand type OP: chunk c holds the
// eight elements at 16c + 8*half of the query row at qp, times mult (+-1
// carries the sign of the scale, 0 blanks a lane without a query; qp must
// still point at a real row).  Every load is issued before any is used and
// none sits behind a branch, so the row costs one memory latency.
template <int DCH, class OP, class T>
__device__ __forceinline__ void load_q_op(const T* qp, int half, float mult,
                                          typename OP::v8* qf) {
  float f[DCH][8];
#pragma unroll
  for (int c = 0; c < DCH; ++c) load8f(qp + 16 * c + 8 * half, f[c]);
#pragma unroll
  for (int c = 0; c < DCH; ++c) qf[c] = to_op8<OP>(f[c], mult);
}

// Reads the Qᵀ MFMA operands of one wave's 32 query rows back from the
// wave's own LDS slice (32 rows of `pitch` elements): lane (col, half) takes
// its operand chunks of row col.  The slice is the wave's own, and LDS
// operations of one wave complete in order, so a wave-level fence suffices.
template <int HDIM, class OP>
__device__ __forceinline__ void read_q_operand(const uint16_t* slice, int pitch, int lane,
                                               typename OP::v8* qf) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int col = lane & 31, half = lane >> 5;
#pragma unroll
  for (int c = 0; c < HDIM / 16; ++c)
    qf[c] = *reinterpret_cast<const typename OP::v8*>(slice + col * pitch + 16 * c + 8 * half);
}

// The Qᵀ MFMA operands of one wave's 32 query rows, loaded through the
// wave's own LDS slice, in two steps so that other work can run while the
// loads are in flight.  issue() reads whole rows with 16-byte loads, one
// lane per 16-byte chunk (RPI rows per instruction), so that every load
// instruction touches a few whole cache lines; row r of the wave is token
// tok0 + row0 + r of qhead (token stride q_ts elements), and a row at or
// past nvalid reads token tok0 instead (a real row, blanked later).
// finish() multiplies each chunk by its row's multiplier (mult, or 0 for a
// row at or past nvalid), rounds it to the operand type, writes it to the
// slice (the wave's own: no other wave may write it meanwhile) and reads the
// operands back.
template <int HDIM, class T>
struct QRows {
  static constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int CPR = HDIM / EPC;           // chunks per row
  static_assert(CPR <= 64 && 64 % CPR == 0, "a load instruction covers whole rows");
  static constexpr int RPI = 64 / CPR;             // rows per load instruction
  static constexpr int NI = 32 / RPI;              // load instructions per wave
  u32x4_t raw[NI];

  __device__ __forceinline__ void issue(const T* qhead, int64_t q_ts, int tok0, int row0,
                                        int nvalid, int lane) {
    const int rr = lane / CPR, ch = lane % CPR;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = RPI * i + rr;
      const int tok = tok0 + (r < nvalid ? row0 + r : 0);
      raw[i] = load16(qhead + (int64_t)tok * q_ts + EPC * ch);
    }
  }

  template <class OP>
  __device__ __forceinline__ void finish(int nvalid, float mult, uint16_t* slice, int pitch,
                                         int lane, typename OP::v8* qf) const {
    const int rr = lane / CPR, ch = lane % CPR;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = RPI * i + rr;
      const float m = r < nvalid ? mult : 0.f;
      uint16_t* dst = slice + r * pitch + EPC * ch;
      if constexpr (EPC == 8) {  // 16-bit elements (bf16)
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = __uint_as_float(raw[i][e] << 16);
          f[2 * e + 1] = __uint_as_float(raw[i][e] & 0xffff0000u);
        }
        *reinterpret_cast<typename OP::v8*>(dst) = to_op8<OP>(f, m);
      } else {  // fp32
        u32x2_t u;
        u[0] = __builtin_bit_cast(uint32_t, OP::cvt2(__uint_as_float(raw[i][0]) * m,
                                                     __uint_as_float(raw[i][1]) * m));
        u[1] = __builtin_bit_cast(uint32_t, OP::cvt2(__uint_as_float(raw[i][2]) * m,
                                                     __uint_as_float(raw[i][3]) * m));
        *reinterpret_cast<u32x2_t*>(dst) = u;
      }
    }
    read_q_operand<HDIM, OP>(slice, pitch, lane, qf);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float pair_max(float x);

// Lazy online softmax.  A lane's sum of one tile's probabilities against the
// running reference m_run may reach this cap before m_run moves to the
// running max, so no probability exceeds it: 2^15 keeps fp16 operands in
// range; bf16 operands (the fp32 exponent range) and the fp32 sums and
// accumulators keep full relative precision far beyond 2^32.
template <class OP> constexpr float lazy_sum_cap() { return 4294967296.0f; }
template <> constexpr float lazy_sum_cap<OpFP16>() { return 32768.0f; }

// One tile of the online softmax in base 2 (scores in raw units times cmul =
// |scale| log2 e).  The lane holds 8 * NKT masked scores, score(kt, i) for
// MFMA k-step kt and i < 8, and fills the P operand pf[kt] with their
// probabilities rounded to the operand type.  Common case: the
// probabilities are taken against the running reference m_run with no max
// pass.  When a lane's sum of them exceeds the cap, or on a row's first
// visible tile (m_run = -inf), the wave (uniformly) takes the tile's max
// over both half-waves, moves m_run to the running max, calls rescale(alpha)
// for the caller's O accumulators and forms the probabilities again.  l_run
// accumulates the rounded probabilities (v_dot2), the values the P.V
// product uses.
template <class OP, int NKT, class ScoreAt, class Rescale>
__device__ __forceinline__ void lazy_softmax(const ScoreAt& score, float cmul, float& m_run,
                                             float& l_run, typename OP::v8* pf,
                                             const Rescale& rescale) {
  auto exp_tile = [&](float neg_mc) {
    float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      u32x4_t u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(fmaf(score(kt, 2 * e), cmul, neg_mc));
        const float p1 = fast_exp2(fmaf(score(kt, 2 * e + 1), cmul, neg_mc));
        // The dot product takes the converted pair itself: bit-casting an
        // element of `u` back to a pair made hipcc (ROCm 7.2) feed the same
        // register to every v_dot2c of the group.
        const typename OP::v2 pb = OP::cvt2(p0, p1);
        u[e] = __builtin_bit_cast(uint32_t, pb);
        l4[e] = OP::sum2(pb, l4[e]);
      }
      pf[kt] = __builtin_bit_cast(typename OP::v8, u);
    }
    return (l4[0] + l4[1]) + (l4[2] + l4[3]);
  };
  float lt = exp_tile(m_run == -INFINITY ? 0.f : -m_run * cmul);
  // (a NaN sum fails the comparison and takes the slow path too)
  const bool raise = !(lt <= lazy_sum_cap<OP>()) || m_run == -INFINITY;
  if (__ballot(raise) != 0ull) {  // wave-uniform, rare
    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 8; ++i) m4[i & 3] = fmaxf(m4[i & 3], score(kt, i));
    const float mx = pair_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
    const float m_new = fmaxf(m_run, mx);
    // O and l are still zero while m_run = -inf
    const float alpha = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_new) * cmul);
    lt = exp_tile(m_new == -INFINITY ? 0.f : -m_new * cmul);
    m_run = m_new;
    l_run *= alpha;
    rescale(alpha);
  }
  l_run += lt;
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

}  // namespace dev
}  // namespace attnp
