// Chunk planning for the scan, as a device function of one 256-thread block:
// sanitised cu_seqlens (clamped to [0, T] and made non-decreasing) and the
// chunk table, each sequence's chunks in scan order (the chunk the scan
// starts in first).  Its own kernel runs it (plan_chunks), and a GEMM launch
// that precedes the scan can host it as one extra block.
#pragma once

#include "common.h"

namespace r2l {

struct PlanArgs {
  const int32_t* cu;
  int nseq, Tn, Lc, max_chunks, l2r;
  int32_t* cu_clean;
  ChunkDesc* chunks;
  int32_t* n_chunks;
  int* zero;   // n_zero ints cleared on the way (counters of later kernels)
  int n_zero;
  int hosted;  // (host side) set by a launch that ran the planning as an extra block
};

// Exclusive block-wide scan of one value per thread (256 threads), max or
// sum: a shuffle scan inside each wave, then the earlier waves' totals from
// LDS (two barriers instead of a barrier per step).
template <bool MAX>
R2L_DEV int block_exclusive_scan(int v, int* buf) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  auto op = [](int a, int b) { return MAX ? max(a, b) : a + b; };   // values are >= 0: 0 is neutral for both
  int x = v;   // inclusive scan within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(x, off, 64);
    if (lane >= off) x = op(x, o);
  }
  if (lane == 63) buf[w] = x;
  __syncthreads();
  int pre = 0;
  for (int k = 0; k < w; ++k) pre = op(pre, buf[k]);
  const int below = __shfl_up(x, 1, 64);
  const int excl = lane > 0 ? op(pre, below) : pre;
  __syncthreads();   // buf is reused by the next scan
  return excl;
}

constexpr int kLongestFirstMaxSeq = 256;

// buf: 256 ints of LDS (only the first four are used)
R2L_DEV void plan_chunks_block(const PlanArgs& p, int* buf) {
  const int tid = threadIdx.x;
  const int nseq = p.nseq, Tn = p.Tn, Lc = p.Lc, max_chunks = p.max_chunks;
  for (int i = tid; i < p.n_zero; i += 256) p.zero[i] = 0;
  const int n1 = nseq + 1;
  const int per = (n1 + 255) / 256;
  const int qa = min(tid * per, n1), qb = min(qa + per, n1);
  auto clampT = [&](int v) { return v < 0 ? 0 : (v > Tn ? Tn : v); };
  // sanitised offsets: clamp into [0, T], then running maximum
  int m = 0;
  for (int q = qa; q < qb; ++q) m = max(m, clampT(p.cu[q]));
  int run = block_exclusive_scan<true>(m, buf);
  for (int q = qa; q < qb; ++q) {
    run = max(run, clampT(p.cu[q]));
    p.cu_clean[q] = run;
  }
  __syncthreads();
  // chunk counts and each sequence's first table index
  const int ps = (nseq + 255) / 256;
  const int sa = min(tid * ps, nseq), sb = min(sa + ps, nseq);
  // (and the number of 16-token state slots of the chunks: only the last
  // chunk of a sequence can be partial)
  int cnt = 0, slots = 0;
  for (int q = sa; q < sb; ++q) {
    const int len = p.cu_clean[q + 1] - p.cu_clean[q];
    const int nc = (len + Lc - 1) / Lc;
    cnt += nc;
    slots += nc > 0 ? (nc - 1) * ((Lc + 15) / 16) + (len - (nc - 1) * Lc + 15) / 16 : 0;
  }
  int base = block_exclusive_scan<false>(cnt, buf);
  int slot = block_exclusive_scan<false>(slots, buf);
  if (tid == 255) *p.n_chunks = min(base + cnt, max_chunks);
  // When Lc covers the token count every non-empty sequence is one chunk
  // and no chunk refers to another, so the table lists them longest first
  // (ties in sequence order): the scans launch their blocks in table order,
  // and the longest sequences then start first, a greedy longest-first
  // schedule over the CUs.  (Quadratic in the sequence count, so only for a
  // few hundred sequences; chunked tables keep sequence order, since a
  // chunk's carry reads the summaries of its sequence's earlier entries.)
  const bool longest_first = Lc >= Tn && nseq <= kLongestFirstMaxSeq;
  for (int q = sa; q < sb; ++q) {
    const int slo = p.cu_clean[q], send = p.cu_clean[q + 1];
    const int nc = (send - slo + Lc - 1) / Lc;
    if (longest_first && nc == 1) {
      const int len = send - slo;
      int rank = 0;
      for (int q2 = 0; q2 < nseq; ++q2) {
        const int l2 = p.cu_clean[q2 + 1] - p.cu_clean[q2];
        rank += l2 > len || (l2 == len && q2 < q);
      }
      base = rank;
    }
    for (int j = 0; j < nc; ++j) {
      if (base + j >= max_chunks) break;
      ChunkDesc d;
      if (p.l2r) {          // cut from the sequence start, leftmost first
        d.lo = slo + j * Lc;
        d.hi = min(send, d.lo + Lc);
      } else {              // cut from the sequence end, rightmost first
        d.hi = send - j * Lc;
        d.lo = max(slo, d.hi - Lc);
      }
      d.seq_lo = slo;
      d.seq_end = send;
      d.first = base;
      d.j = j;
      d.n_in_seq = nc;
      d.slot0 = slot;
      slot += (d.hi - d.lo + 15) / 16;
      p.chunks[base + j] = d;
    }
    base += nc;
  }
}

}  // namespace r2l
