// Internal helpers shared by the HIP kernels of libr2l.so (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define R2L_DEV __device__ __forceinline__

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- activation-type conversions ------------------------------------------
R2L_DEV float to_f32(float v) { return v; }
R2L_DEV float to_f32(bf16 v) { return (float)v; }
template <typename T> R2L_DEV T from_f32(float v);
template <> R2L_DEV float from_f32<float>(float v) { return v; }
template <> R2L_DEV bf16 from_f32<bf16>(float v) { return (bf16)v; }  // v_cvt_pk_bf16_f32, RNE

// ---- pointwise functions ----------------------------------------------------
// 2^x on the transcendental unit (v_exp_f32).
R2L_DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// sigmoid(v) = 1 / (1 + e^-v); e^-v via 2^(-v log2 e).
R2L_DEV float sigmoid_fast(float v) { return __builtin_amdgcn_rcpf(1.0f + exp2_fast(-v * kLog2e)); }
R2L_DEV float silu_fast(float v) { return v * sigmoid_fast(v); }
// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(w), w = e^-|v| in (0, 1].
// log1p(w): below w = 2^-5 the alternating series to the w^6 term (truncation
// under w^7/7, i.e. ~1e-10 relative); above, log2(1 + w) ln 2 on the
// transcendental unit (rounding 1 + w costs at most 2^-19 of w there).
R2L_DEV float softplus_f(float v) {
  const float w = exp2_fast(-fabsf(v) * kLog2e);
  float ser = fmaf(w, -1.0f / 6.0f, 0.2f);
  ser = fmaf(w, ser, -0.25f);
  ser = fmaf(w, ser, 1.0f / 3.0f);
  ser = fmaf(w, ser, -0.5f);
  ser = fmaf(w, ser, 1.0f) * w;
  const float lg = __builtin_amdgcn_logf(1.0f + w) * kLn2;
  return fmaxf(v, 0.0f) + (w < 0.03125f ? ser : lg);
}

// ---- wave / lane helpers ------------------------------------------------------
R2L_DEV int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
R2L_DEV int lane_id() { return threadIdx.x & 63; }

R2L_DEV float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Bijective remap of a 1D block index so that each of the 8 XCDs (which
// receive blocks round-robin) works on a contiguous range of logical tiles:
// tiles that share operands then share that XCD's L2.
R2L_DEV int xcd_remap(int bid, int nblocks) {
  const int q = nblocks >> 3, r = nblocks & 7;
  const int xcd = bid & 7, pos = bid >> 3;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + pos;
}

// Sequence lookup on a (possibly malformed) cu_seqlens: returns the end of
// the sequence containing token t, clamped into [t+1, n_tokens].
R2L_DEV int seq_end_of(const int32_t* cu, int nseq, int t, int n_tokens) {
  int lo = 0, hi = nseq;  // find the last q in [0, nseq) with cu[q] <= t
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  int e = cu[lo + 1];
  e = e < t + 1 ? t + 1 : e;
  return e > n_tokens ? n_tokens : e;
}

// The start of the sequence containing token t, clamped into [0, t].
R2L_DEV int seq_start_of(const int32_t* cu, int nseq, int t) {
  int lo = 0, hi = nseq;  // the last q in [0, nseq) with cu[q] <= t
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  const int s = cu[lo];
  return s > t ? t : (s < 0 ? 0 : s);
}

// ---- chunk table used by the scan ----------------------------------------------
// One time chunk of one sequence; chunks of a sequence are stored contiguously
// in scan order: the rightmost first (j = 0) for the right-to-left scan, the
// leftmost first for the left-to-right one.
struct ChunkDesc {
  int lo, hi;        // token range [lo, hi)
  int seq_lo, seq_end;
  int first;         // table index of the sequence's rightmost chunk
  int j;             // position counted from the right (0 = rightmost)
  int n_in_seq;      // number of chunks of this sequence
  int slot0;         // first 16-token state slot of this chunk (scan backward)
};
