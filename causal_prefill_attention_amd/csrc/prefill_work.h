// Work decode shared by the prefill kernels: q-tile slot -> (sequence, tile).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "prefill_params.h"

namespace attnp {
namespace dev {

constexpr int kWorkWave = 64;

// ------------------------------------------------------------- work decode
struct Work {
  int start;   // first query token of the sequence in the packed q / out
  int len;     // number of queries (new tokens) of the sequence
  int kstart;  // first key token of the sequence in the packed k / v (unpaged)
  int klen;    // number of keys: the history followed by the new tokens
  int q0;      // first local query row of this tile
  int seq;     // sequence index (the block-table row of a paged cache)
  bool valid;
  int q0_b;    // folded grids: first local row of the second (mirrored) block
};

// Maps a q-tile slot to (sequence, tile).  Slots enumerate sequences in
// order; inside a sequence the last (most expensive causal) tile comes
// first.  Query and key offsets are clamped into [0, T].  Every lane of the
// wave computes the same answer.  With a paged cache the key count comes
// from seqlens_k, clamped to the table row's capacity.
// FOLD: a slot is a pair of BM-row blocks of one sequence, block r and its
// mirror nb - 1 - r (nb blocks in the sequence), so that every pair sees
// about the same number of causal keys; rank 0 (the first block with the
// last, the heaviest pair) comes first.  q0 is block r, q0_b the mirror;
// they coincide for the middle block of an odd nb.
template <int BM, bool PAGED, bool FOLD = false>
__device__ Work decode_work(const PrefillParams& p, int slot) {
  const int lane = threadIdx.x & (kWorkWave - 1);
  int base = 0;
  for (int s0 = 0; s0 < p.n_seqs; s0 += kWorkWave) {
    const int s = s0 + lane;
    // every lane reads a real entry (n_seqs >= 1) with no branch, so the
    // offsets cost one memory latency; lanes past the batch then drop theirs
    const int sc = min(s, p.n_seqs - 1);
    int a = min(max(p.cu_seqlens[sc], 0), p.n_tokens);
    int b = min(max(p.cu_seqlens[sc + 1], 0), p.n_tokens);
    int ka = 0, kb;
    if (PAGED) {
      kb = min(max(p.seqlens_k[sc], 0), p.table_stride * p.page_size);
    } else {
      ka = min(max(p.cu_seqlens_k[sc], 0), p.n_tokens_k);
      kb = min(max(p.cu_seqlens_k[sc + 1], 0), p.n_tokens_k);
    }
    if (s >= p.n_seqs) a = b = ka = kb = 0;
    const int len = max(b - a, 0);
    const int nb = (len + BM - 1) / BM;  // BM-row blocks
    const int nt = FOLD ? (nb + 1) / 2 : nb;
    int incl = nt;
#pragma unroll
    for (int off = 1; off < kWorkWave; off <<= 1) {
      const int y = __shfl_up(incl, off, kWorkWave);
      if (lane >= off) incl += y;
    }
    const int total = __shfl(incl, kWorkWave - 1, kWorkWave);
    if (slot < base + total) {
      const unsigned long long hit = __ballot(base + incl > slot);
      const int src = __ffsll((long long)hit) - 1;
      const int excl = __shfl(incl - nt, src, kWorkWave);
      Work w;
      w.start = __shfl(a, src, kWorkWave);
      w.len = __shfl(len, src, kWorkWave);
      w.kstart = __shfl(ka, src, kWorkWave);
      w.klen = __shfl(max(kb - ka, 0), src, kWorkWave);
      const int ntiles = __shfl(nt, src, kWorkWave);
      const int rank = slot - base - excl;  // 0 = heaviest tile (or pair)
      if (FOLD) {
        w.q0 = rank * BM;
        w.q0_b = (__shfl(nb, src, kWorkWave) - 1 - rank) * BM;
      } else {
        w.q0 = (ntiles - 1 - rank) * BM;
        w.q0_b = w.q0;
      }
      w.seq = s0 + src;
      w.valid = true;
      return w;
    }
    base += total;
  }
  Work w{0, 0, 0, 0, 0, 0, false, 0};
  return w;
}


}  // namespace dev
}  // namespace attnp
