// Anti-causal depthwise conv1d + bias + SiLU, optionally fused with x_proj
// ("Bifocal Diffusion Language Models", §3.4 steps 1-2: the Mamba-1 block's
// causal conv run over the flipped sequence is, in the original order, a
// conv that looks at a token and the K-1 tokens to its right):
//   u[t,e] = SiLU(b[e] + sum_{j=0}^{K-1} w[e,K-1-j] * x[t+j,e]),
// with x past the end of t's sequence taken as 0.  With L2R (the left-to-
// right control of §4.4, Table 4) the taps look left instead: x[t-j], with
// x before the start of t's sequence taken as 0.
#include <type_traits>

#include "kernels.h"

namespace r2l {

// ---------------------------------------------------------------------------
// delta split (see kernels.h): RP = the dt_rank padded to the scan's k-steps
// of 32 (1, 2, 4 or 8 of them); beyond 8 the scan computes dt on the VALU.
// ---------------------------------------------------------------------------
int delta_split_width(int R) {
  const int ks = (R + 31) / 32;
  return ks > 8 ? 0 : 32 * (ks <= 1 ? 1 : ks <= 2 ? 2 : ks <= 4 ? 4 : 8);
}

// columns [col, col + V) of one x_proj output row (col % V == 0, RP % V == 0)
template <int V>
R2L_DEV void split_store(bf16* __restrict__ ds, long row, int col, int R, int RP, const float* v) {
  if (col >= RP) return;
  bf16 hi[V], lo[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const bool in = col + i < R;
    hi[i] = (bf16)(in ? v[i] : 0.0f);
    lo[i] = (bf16)(in ? v[i] - (float)hi[i] : 0.0f);
  }
  bf16* p = ds + row * 2L * RP + col;
  if constexpr (V == 4) {
    *(bf16x4*)p = bf16x4{hi[0], hi[1], hi[2], hi[3]};
    *(bf16x4*)(p + RP) = bf16x4{lo[0], lo[1], lo[2], lo[3]};
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      p[i] = hi[i];
      p[RP + i] = lo[i];
    }
  }
}

__global__ __launch_bounds__(256) void split_delta_kernel(long n, int P, int R, int RP, const float* __restrict__ xdbl,
                                                          bf16* __restrict__ ds) {
  // one thread per (row, column < RP)
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const long row = i / RP;
    const int col = (int)(i % RP);
    const float v = col < R ? xdbl[row * P + col] : 0.0f;
    split_store<1>(ds, row, col, R, RP, &v);
  }
}

hipError_t split_delta(int Tn, int P, int R, const float* xdbl, bf16* dsplit, hipStream_t st) {
  const int RP = delta_split_width(R);
  if (Tn <= 0 || RP == 0) return hipSuccess;
  const long n = (long)Tn * RP;
  const long want = (n + 255) / 256;
  hipLaunchKernelGGL(split_delta_kernel, dim3((unsigned)(want < 4096 ? want : 4096)), dim3(256), 0, st, n, P, R,
                     RP, xdbl, dsplit);
  return hipGetLastError();
}

constexpr int KC = 4;  // d_conv (§4.1)

// ---------------------------------------------------------------------------
// Standalone conv: block = 64 channels x 32 tokens; wave w handles 8 tokens,
// lane = channel, so every load/store instruction touches 64 consecutive
// channels of one token row.
// ---------------------------------------------------------------------------
template <typename T, bool L2R>
__global__ __launch_bounds__(256) void conv_silu_kernel(int Tn, int E, const T* __restrict__ x,
                                                        long ld_x, const T* __restrict__ cw,
                                                        const T* __restrict__ cb, T* __restrict__ u,
                                                        const int32_t* __restrict__ cu, int nseq) {
  const int lane = lane_id();
  const int e = blockIdx.y * 64 + lane;
  // a wave owns 8 consecutive tokens of 64 channels (the token index is
  // wave-uniform, so the sequence lookups are too)
  const int t0 = __builtin_amdgcn_readfirstlane(blockIdx.x * 32 + wave_id() * 8);
  if (t0 >= Tn) return;
  float wt[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) wt[k] = to_f32(cw[(long)e * KC + k]);
  const float b = to_f32(cb[e]);
  // rows t0 .. t0+10 (R2L) or t0-3 .. t0+7 (L2R), all loads first
  constexpr int NR = 8 + KC - 1;
  const int rbase = L2R ? t0 - (KC - 1) : t0;
  float xv[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = rbase + i;
    xv[i] = row >= 0 && row < Tn ? to_f32(x[(long)row * ld_x + e]) : 0.0f;
  }
  // the current sequence [sl, se); looked up again only past its end
  int sl = seq_start_of(cu, nseq, t0), se = seq_end_of(cu, nseq, t0, Tn);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + i;
    if (t >= Tn) break;
    if (t >= se) {
      sl = seq_start_of(cu, nseq, t);
      se = seq_end_of(cu, nseq, t, Tn);
    }
    float c = b;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const int row = L2R ? t - j : t + j;     // rbase + (L2R ? i + KC - 1 - j : i + j)
      const float xr = xv[L2R ? i + KC - 1 - j : i + j];
      if (L2R ? row >= sl : row < se) c = fmaf(wt[KC - 1 - j], xr, c);
    }
    u[(long)t * E + e] = from_f32<T>(silu_fast(c));
  }
}

// The same for bf16 with 16-byte channel groups (E and ld_x multiples of 8;
// x, u, taps and bias 16-byte aligned): a lane owns 8 consecutive channels,
// so a wave covers 8 tokens of 512 channels and every load and store
// instruction moves 1 KB of one token row in 16-byte pieces.  The
// arithmetic per (token, channel) is the kernel's above, in the same order,
// so both give the same bits.
template <bool L2R>
__global__ __launch_bounds__(256) void conv_silu16_kernel(int Tn, int E, const bf16* __restrict__ x, long ld_x,
                                                          const bf16* __restrict__ cw, const bf16* __restrict__ cb,
                                                          bf16* __restrict__ u, const int32_t* __restrict__ cu,
                                                          int nseq) {
  const int lane = lane_id();
  const int e = (blockIdx.y * 64 + lane) * 8;   // the lane's first channel
  const int t0 = __builtin_amdgcn_readfirstlane(blockIdx.x * 32 + wave_id() * 8);
  if (t0 >= Tn) return;
  const bool on = e < E;                        // lanes past the channels load and store nothing
  float wt[8][KC], b[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    b[c] = 0.0f;
#pragma unroll
    for (int k = 0; k < KC; ++k) wt[c][k] = 0.0f;
  }
  if (on) {
    // taps of channels e + 2q and e + 2q + 1 in one 16-byte piece
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8 tv = *(const bf16x8*)(cw + (long)e * KC + 8 * q);
#pragma unroll
      for (int k = 0; k < 8; ++k) wt[2 * q + k / KC][k % KC] = (float)tv[k];
    }
    const bf16x8 bv = *(const bf16x8*)(cb + e);
#pragma unroll
    for (int c = 0; c < 8; ++c) b[c] = (float)bv[c];
  }
  // rows t0 .. t0+10 (R2L) or t0-3 .. t0+7 (L2R), all loads first
  constexpr int NR = 8 + KC - 1;
  const int rbase = L2R ? t0 - (KC - 1) : t0;
  bf16x8 xv[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = rbase + i;
    xv[i] = on && row >= 0 && row < Tn ? *(const bf16x8*)(x + (long)row * ld_x + e) : bf16x8{};
  }
  int sl = seq_start_of(cu, nseq, t0), se = seq_end_of(cu, nseq, t0, Tn);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + i;
    if (t >= Tn) break;
    if (t >= se) {
      sl = seq_start_of(cu, nseq, t);
      se = seq_end_of(cu, nseq, t, Tn);
    }
    bf16x8 o;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float acc = b[c];
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const int row = L2R ? t - j : t + j;
        const float xr = (float)xv[L2R ? i + KC - 1 - j : i + j][c];
        if (L2R ? row >= sl : row < se) acc = fmaf(wt[c][KC - 1 - j], xr, acc);
      }
      o[c] = from_f32<bf16>(silu_fast(acc));
    }
    if (on) *(bf16x8*)(u + (long)t * E + e) = o;
  }
}

template <typename T>
hipError_t conv_silu(int Tn, int E, const T* x, long ld_x, const T* conv_w, const T* conv_b, T* u,
                     const int32_t* cu, int nseq, bool l2r, hipStream_t st) {
  if (Tn <= 0) return hipSuccess;
  if constexpr (std::is_same<T, bf16>::value) {
    auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    if (E % 8 == 0 && ld_x % 8 == 0 && a16(x) && a16(u) && a16(conv_w) && a16(conv_b)) {
      dim3 grid16((Tn + 31) / 32, (E + 511) / 512);
      if (l2r)
        hipLaunchKernelGGL((conv_silu16_kernel<true>), grid16, dim3(256), 0, st, Tn, E, x, ld_x, conv_w, conv_b, u,
                           cu, nseq);
      else
        hipLaunchKernelGGL((conv_silu16_kernel<false>), grid16, dim3(256), 0, st, Tn, E, x, ld_x, conv_w, conv_b, u,
                           cu, nseq);
      return hipGetLastError();
    }
  }
  dim3 grid((Tn + 31) / 32, E / 64);
  if (l2r)
    hipLaunchKernelGGL((conv_silu_kernel<T, true>), grid, dim3(256), 0, st, Tn, E, x, ld_x, conv_w,
                       conv_b, u, cu, nseq);
  else
    hipLaunchKernelGGL((conv_silu_kernel<T, false>), grid, dim3(256), 0, st, Tn, E, x, ld_x, conv_w,
                       conv_b, u, cu, nseq);
  return hipGetLastError();
}
template hipError_t conv_silu<float>(int, int, const float*, long, const float*, const float*,
                                     float*, const int32_t*, int, bool, hipStream_t);
template hipError_t conv_silu<bf16>(int, int, const bf16*, long, const bf16*, const bf16*, bf16*,
                                    const int32_t*, int, bool, hipStream_t);

// ---------------------------------------------------------------------------
// Fused conv + SiLU + x_proj, bf16 on MFMA.
//
// A block covers 32 tokens and all P = R+2N x_proj outputs.  Its 4 waves
// split the E channels in quarters (split-K inside the block).  Each lane
// computes exactly its own MFMA A-fragment: token (lane & 31) and the 8
// channels at offset 8*(lane >> 5) of the current 16-channel k-step, i.e.
// the conv + SiLU happens in registers and u never touches LDS or HBM (it is
// stored only when the caller asks for u).  The x_proj rows come straight
// from global memory (the whole matrix is ~1.3 MB and stays in L2).  The 4
// partial [32 x P] results are summed through LDS in a fixed order (no
// atomics, so results are deterministic).
// ---------------------------------------------------------------------------
// gridDim.y = KS > 1 splits the channels over blocks: block (tile, ks)
// covers channels [ks E/KS, (ks+1) E/KS) and writes its partial sum to slab
// ks of xdbl ([KS][T][P]); sum_slabs adds the slabs.
template <int NCS, bool L2R>
__global__ __launch_bounds__(256) void conv_xproj_kernel(int Tn, int E, int P,
                                                         const bf16* __restrict__ x, long ld_x,
                                                         const bf16* __restrict__ cw,
                                                         const bf16* __restrict__ cb,
                                                         const bf16* __restrict__ Wx,
                                                         bf16* __restrict__ u_out,
                                                         float* __restrict__ xdbl,
                                                         const int32_t* __restrict__ cu, int nseq,
                                                         int R, int RP, bf16* __restrict__ dsplit) {
  constexpr int NC = NCS * 32;
  __shared__ float red[4][32 * NC];
  const int lane = lane_id(), w = wave_id();
  const int tr = lane & 31, kh = lane >> 5;
  const int t0 = blockIdx.x * 32;
  const int t = t0 + tr;
  const bool tv = t < Tn;
  // the sequence end (R2L) or start (L2R) bounds the conv window
  const int sb = tv ? (L2R ? seq_start_of(cu, nseq, t) : seq_end_of(cu, nseq, t, Tn)) : 0;
  const int Eb = E / gridDim.y;                 // channels of this block
  const int Ew = Eb / 4;
  const int cbeg = blockIdx.y * Eb + w * Ew;
  xdbl += (long)blockIdx.y * Tn * P;

  f32x16 acc[NCS];
#pragma unroll
  for (int c = 0; c < NCS; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;

  const bf16x8 zero8 = {};
  // Operands of one 16-channel k-step, loaded PF steps ahead: a wave of a
  // small input has only a few steps (4 at 16 channel splits of 4096), and
  // with every step's loads in flight together it waits for one memory
  // latency instead of one per step.
  constexpr int PF = 4;
  struct Step {
    bf16x8 wv[4], bv, xv[KC], wx[NCS];
  };
  // Loads are unconditional, from clamped (valid) rows; masks are applied
  // when the values are used.  (A per-lane branch around a load makes both
  // paths write the same registers and forces an immediate wait.)
  const int tt = min(t, Tn - 1);
  // the last (R2L) or first (L2R) row this lane may read
  const int xlim = L2R ? (tv ? sb : tt) : (tv ? sb : tt + 1) - 1;
  bool xok[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) xok[j] = tv && (L2R ? t - j >= sb : t + j < sb);
  auto load_step = [&](Step& s, int k0) {
    const int c0 = k0 + kh * 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) s.wv[q] = *(const bf16x8*)(cw + (long)c0 * KC + 8 * q);
    s.bv = *(const bf16x8*)(cb + c0);
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const int row = L2R ? max(tt - j, xlim) : min(tt + j, xlim);   // x[t -+ j]
      s.xv[j] = *(const bf16x8*)(x + (long)row * ld_x + c0);
    }
#pragma unroll
    for (int c = 0; c < NCS; ++c) {
      const int row = min(c * 32 + tr, P - 1);
      s.wx[c] = *(const bf16x8*)(Wx + (long)row * E + c0);
    }
  };
  auto compute_step = [&](const Step& cur, int k0) {
    const int c0 = k0 + kh * 8;
    float ca[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ca[i] = (float)cur.bv[i];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const bf16x8 xj = xok[j] ? cur.xv[j] : zero8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int el = i * KC + (KC - 1 - j);  // channel i, tap K-1-j
        ca[i] = fmaf((float)cur.wv[el >> 3][el & 7], (float)xj[i], ca[i]);
      }
    }
    bf16x8 af;
#pragma unroll
    for (int i = 0; i < 8; ++i) af[i] = (bf16)silu_fast(ca[i]);
    if (!tv) af = zero8;
    if (u_out != nullptr && tv) *(bf16x8*)(u_out + (long)t * E + c0) = af;
#pragma unroll
    for (int c = 0; c < NCS; ++c) {
      const bf16x8 bfr = (c * 32 + tr < P) ? cur.wx[c] : zero8;
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, acc[c], 0, 0, 0);
    }
  };
  const int nst = Ew / 16;
  Step ring[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i)
    if (i < nst) load_step(ring[i], cbeg + 16 * i);
  for (int g = 0; g < nst; g += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (g + i < nst) {
        compute_step(ring[i], cbeg + 16 * (g + i));
        if (g + i + PF < nst) load_step(ring[i], cbeg + 16 * (g + i + PF));
      }
    }
  }
  // D layout: lane holds output column (lane & 31) of each 32-wide slice and
  // token rows 8*(r/4) + 4*(lane/32) + r%4.  Every wave's partial sums go to
  // LDS; wave w then adds, for its token rows 8 w .. 8 w + 7 (its registers
  // r = 4 w .. 4 w + 3), the four waves' values in the fixed order 0, 1, 2, 3.
  // All the LDS reads come before the (bounds-checked) stores, so their
  // latencies overlap.
#pragma unroll
  for (int c = 0; c < NCS; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * kh + (r & 3);
      red[w][row * NC + c * 32 + tr] = acc[c][r];
    }
  __syncthreads();
  float vs[NCS][4];
#pragma unroll
  for (int c = 0; c < NCS; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = (8 * w + 4 * kh + q) * NC + c * 32 + tr;
      vs[c][q] = ((red[0][idx] + red[1][idx]) + red[2][idx]) + red[3][idx];
    }
#pragma unroll
  for (int c = 0; c < NCS; ++c) {
    const int col = c * 32 + tr;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 8 * w + 4 * kh + q;
      if (col < P && t0 + row < Tn) {
        xdbl[(long)(t0 + row) * P + col] = vs[c][q];
        if (dsplit != nullptr) split_store<1>(dsplit, t0 + row, col, R, RP, &vs[c][q]);
      }
    }
  }
}

// out[i] = sum over k < ks of slab[k][i] (slab stride n), in order of k.
// A thread owns 4 consecutive elements and loads all of its slabs (up to
// 32) before adding, so the loads are in flight together.
// dsplit (optional): also the delta split of the sum (out is [n / P, P]).
__global__ __launch_bounds__(256) void sum_slabs_kernel(long n, int ks, const float* __restrict__ slab,
                                                        float* __restrict__ out, int P, int R, int RP,
                                                        bf16* __restrict__ dsplit) {
  const long i = (blockIdx.x * 256L + threadIdx.x) * 4;
  if (i >= n) return;
  if (i + 4 <= n && (n & 3) == 0) {
    f32x4 v[32];
#pragma unroll
    for (int k = 0; k < 32; ++k)
      if (k < ks) v[k] = *(const f32x4*)(slab + k * n + i);
    f32x4 acc = v[0];
#pragma unroll
    for (int k = 1; k < 32; ++k)
      if (k < ks) acc += v[k];
    *(f32x4*)(out + i) = acc;
    if (dsplit != nullptr)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = acc[e];
        split_store<1>(dsplit, (i + e) / P, (int)((i + e) % P), R, RP, &a);
      }
  } else {
    for (long j = i; j < i + 4 && j < n; ++j) {
      float v = 0.0f;
      for (int k = 0; k < ks; ++k) v += slab[k * n + j];
      out[j] = v;
      if (dsplit != nullptr) split_store<1>(dsplit, j / P, (int)(j % P), R, RP, &v);
    }
  }
}

hipError_t conv_xproj_bf16(int Tn, int E, int P, const bf16* x, long ld_x, const bf16* conv_w,
                           const bf16* conv_b, const bf16* x_proj_w, bf16* u_out, float* xdbl,
                           const int32_t* cu, int nseq, bool l2r, hipStream_t st, float* ws,
                           size_t ws_bytes, int ncu, int R, bf16* dsplit) {
  if (Tn <= 0) return hipSuccess;
  const int ncs = (P + 31) / 32;
  const int ntiles = (Tn + 31) / 32;
  const int RP = dsplit != nullptr ? delta_split_width(R) : 0;
  if (RP == 0) dsplit = nullptr;
  // Few token tiles for the GPU: split the channels over KS blocks per tile
  // (each wave keeps at least one 16-channel step), partial sums in ws.
  int ks = 1;
  if (ws != nullptr && u_out == nullptr && ncu > 0) {
    while (ks < 32 && ntiles * ks * 2 <= ncu && (E / (ks * 2)) % 64 == 0 &&
           (size_t)(ks * 2) * Tn * P * sizeof(float) <= ws_bytes)
      ks *= 2;
  }
  float* dst = ks > 1 ? ws : xdbl;
  dim3 grid(ntiles, ks), block(256);
#define R2L_CX(n)                                                                                 \
  case n:                                                                                         \
    if (l2r)                                                                                      \
      hipLaunchKernelGGL((conv_xproj_kernel<n, true>), grid, block, 0, st, Tn, E, P, x, ld_x,     \
                         conv_w, conv_b, x_proj_w, u_out, dst, cu, nseq, R, RP,                   \
                         ks > 1 ? nullptr : dsplit);                                              \
    else                                                                                          \
      hipLaunchKernelGGL((conv_xproj_kernel<n, false>), grid, block, 0, st, Tn, E, P, x, ld_x,    \
                         conv_w, conv_b, x_proj_w, u_out, dst, cu, nseq, R, RP,                   \
                         ks > 1 ? nullptr : dsplit);                                              \
    break;
  switch (ncs) {
    R2L_CX(1) R2L_CX(2) R2L_CX(3) R2L_CX(4) R2L_CX(5) R2L_CX(6) R2L_CX(7) R2L_CX(8)
    default: return hipErrorInvalidValue;
  }
#undef R2L_CX
  if (ks > 1) {   // (ks <= 32, as sum_slabs_kernel needs)
    const long n = (long)Tn * P;
    hipLaunchKernelGGL(sum_slabs_kernel, dim3((unsigned)((n / 4 + 255) / 256 + 1)), dim3(256), 0, st, n, ks,
                       (const float*)ws, xdbl, P, R, RP, dsplit);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused conv + SiLU + x_proj for large inputs, split along K ("stream-K").
//
// Work is the grid of (128-token tile, 32-channel step) pairs, walked tile
// by tile; block b of G takes the contiguous range [b W / G, (b+1) W / G) of
// the W = tiles * E/32 steps, so every block does the same amount of work
// whatever the token count (a plain split into 128-token tiles would leave
// e.g. 258 tiles for 256 CUs, i.e. two rounds).  With tiles >= G / 2 every
// block holds at least half a tile's steps, so a tile is covered by at most
// three blocks: the piece holding its step 0 writes its partial sum to part0,
// the next to part1, a third to part2.  The summing kernel counts each
// tile's pieces from the same step ranges and adds (part0 + part1) + part2,
// in that order and only the parts that exist, so results are deterministic
// and no part is ever cleared.  (Two blocks run per CU when the ring fits
// twice in LDS; a third piece can only occur then.)
//
// The 4 waves of a block own 32 tokens each and walk the same steps, so one
// copy of each W_x slice (and the conv taps) per block serves 128 tokens.
// Every operand of a step is copied global -> LDS by buffer_load ... lds
// into a ring of RS stages (rows past the token count read as zero through
// the buffer descriptor's range).  A step reads its own stage only, so the
// barrier of step q waits for step q's copies alone: each copy has RS - 1
// steps to land.  x and W_x stage rows are 64 bytes with the
// 16-byte chunk index XOR-ed by (row >> 2) & 3 against bank conflicts.
// Lanes compute their own MFMA A-fragments (token lane & 31, 8 channels) as
// in conv_xproj_kernel.
// ---------------------------------------------------------------------------
namespace {

constexpr int kSkTok = 128, kSkK = 32;

template <int NCS>
struct SkGeo {
  // A step's operands travel as 1 KB copies (64 lanes x 16 bytes): W_x rows
  // (16 rows of 64 bytes per copy), the tile's x rows with the conv halo (131), the conv taps and
  // the conv bias.  Copy i of a step is wave (i % 4)'s copy i / 4; the last
  // few slots are padding that reads nothing (zeros land in LDS), so every
  // wave issues the same number of copies per step.
  static constexpr int NW = (NCS * 32 * 4 + 63) / 64;          // W_x rows
  static constexpr int NX = ((kSkTok + 3) * 4 + 63) / 64;      // x rows of the tile and its halo
  static constexpr int PER_WAVE = (NW + NX + 2 + 3) / 4;       // + taps, bias
  static constexpr int NI = 4 * PER_WAVE;
  static constexpr int SBYTES = NI * 1024;
  static constexpr int OFF_X = NW * 1024, OFF_CW = (NW + NX) * 1024, OFF_CB = OFF_CW + 1024;
  // two blocks per CU with a 3-stage ring when it fits, else one with 5 (or 4)
  static constexpr int BPC = 2 * 3 * SBYTES <= 160 * 1024 ? 2 : 1;
  static constexpr int RS = BPC == 2 ? 3 : (5 * SBYTES <= 160 * 1024 ? 5 : 4);
};

constexpr int sk_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

R2L_DEV void sk_dma16(__amdgpu_buffer_rsrc_t r, void* lds, unsigned voff, unsigned soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
R2L_DEV int sk_swz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

}  // namespace

template <int NCS, bool L2R>
__global__ __launch_bounds__(256, SkGeo<NCS>::BPC) void conv_xproj_sk_kernel(int Tn, int E, int P,
                                                               const bf16* __restrict__ x, long ld_x,
                                                               const bf16* __restrict__ cw,
                                                               const bf16* __restrict__ cb,
                                                               const bf16* __restrict__ Wx,
                                                               float* __restrict__ part0,
                                                               float* __restrict__ part1,
                                                               long part_stride,   // part2 = part1 + part_stride
                                                               const int32_t* __restrict__ cu, int nseq) {
  using Geo = SkGeo<NCS>;
  constexpr int RS = Geo::RS, PW = Geo::PER_WAVE;
  __shared__ __attribute__((aligned(1024))) char s0[Geo::SBYTES];
  __shared__ __attribute__((aligned(1024))) char s1[Geo::SBYTES];
  __shared__ __attribute__((aligned(1024))) char s2[Geo::SBYTES];
  __shared__ __attribute__((aligned(1024))) char s3[Geo::RS > 3 ? Geo::SBYTES : 16];
  __shared__ __attribute__((aligned(1024))) char s4[Geo::RS > 4 ? Geo::SBYTES : 16];
  auto stage = [&](int s) -> char* { return s == 0 ? s0 : s == 1 ? s1 : s == 2 ? s2 : s == 3 ? s3 : s4; };

  const int lane = lane_id(), w = wave_id();
  const int tr = lane & 31, kh = lane >> 5;
  const int S = E / kSkK;                        // steps per tile
  const int ntiles = (Tn + kSkTok - 1) / kSkTok;
  const long W = (long)ntiles * S;
  const int lo = (int)(W * blockIdx.x / gridDim.x), hi = (int)(W * (blockIdx.x + 1) / gridDim.x);
  if (lo >= hi) return;
  const int n = hi - lo;

  // constant descriptors (W_x, conv taps, conv bias) and this lane's offsets
  const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc((void*)Wx, 0, (int)((long)P * E * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rCW = __builtin_amdgcn_make_buffer_rsrc((void*)cw, 0, (int)((long)E * 8), 0x00020000);
  const __amdgpu_buffer_rsrc_t rCB = __builtin_amdgcn_make_buffer_rsrc((void*)cb, 0, (int)((long)E * 2), 0x00020000);
  // copy m of this wave is copy i = 4 m + w of the step; its kind depends
  // on i, so it is uniform over the wave
  unsigned voff[PW];
#pragma unroll
  for (int m = 0; m < PW; ++m) {
    const int i = 4 * m + w;
    // W_x rows (rows past P lie past the descriptor's range and read as zero)
    const int pw = i * 64 + lane, roww = pw >> 2;
    const unsigned vw = (unsigned)(((long)roww * E + sk_swz(roww, pw & 3) * 8) * 2);
    // x rows
    const int px = (i - Geo::NW) * 64 + lane, rowx = px >> 2;
    const unsigned vx = (unsigned)(((long)rowx * ld_x + sk_swz(rowx, px & 3) * 8) * 2);
    // taps of channels c0 + 2 lane, +1; bias of channels c0 + 8 lane .. +7;
    // padding slots read past every range
    const unsigned vt = lane < 16 ? lane * 16 : 0, vb = lane < 4 ? lane * 16 : 0;
    voff[m] = i < Geo::NW ? vw : i < Geo::NW + Geo::NX ? vx : i == Geo::NW + Geo::NX ? vt
            : i == Geo::NW + Geo::NX + 1 ? vb : 0x80000000u;
  }
  // Copy position: the step RS-1 ahead of the one being computed, as
  // (tile, channel offset); it stops advancing at the block's last step
  // (later copies reload that step into stages that are never read).
  int it_tile = lo / S, it_c0 = (lo % S) * kSkK, it_left = n;
  auto issue = [&](int s) {
    // stage rows: tokens t0 .. t0+130 (R2L) or t0-3 .. t0+127 (L2R); the
    // descriptor starts at a real row, and rows before it (L2R, first tile)
    // get a negative offset that wraps past the range and reads as zero
    const long t0 = (long)it_tile * kSkTok;
    const long r0 = L2R ? (t0 >= 3 ? t0 - 3 : 0) : t0;
    const unsigned xshift = L2R ? (unsigned)((t0 - 3 - r0) * ld_x * 2) : 0u;
    const long xbytes = (long)(Tn - r0) * ld_x * 2;
    const __amdgpu_buffer_rsrc_t rX = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + r0 * ld_x), 0, (int)(xbytes < (1L << 30) ? xbytes : (1L << 30)), 0x00020000);
    char* base = stage(s);
#pragma unroll
    for (int m = 0; m < PW; ++m) {
      // (wave-uniform choices of descriptor and offset)
      const int i = 4 * m + w;
      const bool tap = i == Geo::NW + Geo::NX;
      const bool xcopy = i >= Geo::NW && i < Geo::NW + Geo::NX;
      const __amdgpu_buffer_rsrc_t r = i < Geo::NW ? rW : xcopy ? rX : tap ? rCW : rCB;
      // lane l lands at base + 1024 i + 16 l
      sk_dma16(r, base + i * 1024, voff[m] + (xcopy ? xshift : 0u), (unsigned)(it_c0 * (tap ? 8 : 2)));
    }
    if (--it_left > 0) {
      it_c0 += kSkK;
      if (it_c0 == E) { it_c0 = 0; ++it_tile; }
    }
  };

  // Look up this lane's sequence end in the block's first and last tile now,
  // before any copy is in flight (a lookup inside the loop waits for all of
  // them); tiles in between, when the range spans more than two, are looked
  // up when they start.
  const int tileA = lo / S, tileB = (hi - 1) / S;
  const int tA = tileA * kSkTok + w * 32 + tr, tB = tileB * kSkTok + w * 32 + tr;
  // the sequence end (R2L) or start (L2R) bounds each lane's conv window
  auto bound_of = [&](int t) __attribute__((always_inline)) {
    return L2R ? seq_start_of(cu, nseq, t) : seq_end_of(cu, nseq, t, Tn);
  };
  const int seA = tA < Tn ? bound_of(tA) : 0;
  const int seB = tB < Tn ? bound_of(tB) : 0;

  f32x16 acc[NCS];
  int c_tile = lo / S, c_ks = lo % S;   // step being computed
  // index of the piece within its tile (0: holds step 0); only a block's
  // first piece can start inside a tile, after one or two earlier pieces
  const int lo_prev = blockIdx.x > 0 ? (int)(W * (blockIdx.x - 1) / gridDim.x) : 0;
  const int first_pidx = c_ks == 0 ? 0 : (blockIdx.x > 0 && lo_prev > c_tile * S ? 2 : 1);
  int pidx = first_pidx;
  bool tv = false, ok1 = false, ok2 = false, ok3 = false, masked = false;
  auto start_piece = [&]() {
#pragma unroll
    for (int c = 0; c < NCS; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    const int t = c_tile * kSkTok + w * 32 + tr;
    tv = t < Tn;
    const int se = c_tile == tileA ? seA : c_tile == tileB ? seB : (tv ? bound_of(t) : 0);
    ok1 = L2R ? t - 1 >= se : t + 1 < se;
    ok2 = L2R ? t - 2 >= se : t + 2 < se;
    ok3 = L2R ? t - 3 >= se : t + 3 < se;
    // taps past a sequence end are zeroed only in waves that have such a lane
    masked = __any(tv && !(ok1 && ok2 && ok3));
  };
  auto end_piece = [&]() {
    // (part1 + stride selects part1 / part2: a three-way pointer choice here
    // keeps the compiler from holding the block's state in registers)
    float* dst = (pidx == 0 ? part0 : part1 + (pidx - 1) * part_stride) + ((long)c_tile * kSkTok + w * 32) * P;
    const int rows = min(32, Tn - (c_tile * kSkTok + w * 32));
#pragma unroll
    for (int c = 0; c < NCS; ++c) {
      const int col = c * 32 + tr;
      if (col >= P) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * kh + (r & 3);
        if (row < rows) {
          dst[row * P + col] = acc[c][r];
        }
      }
    }
  };
  const bf16x8 zero8 = {};
  auto compute = [&](const char* base) {
    if (c_tile * S + c_ks == lo || c_ks == 0) {
      pidx = c_ks == 0 ? 0 : first_pidx;
      start_piece();
    }
    const char* wx_s = base;
    const char* x_s = base + Geo::OFF_X;
    const char* cw_s = base + Geo::OFF_CW;
    const char* cb_s = base + Geo::OFF_CB;
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const int kc = ss * 2 + kh;            // 16-byte chunk of the 64-byte row
      const int cc = ss * 16 + kh * 8;       // first of this lane's 8 channels in the step
      i32x4 xr[KC], wt[4];
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const int row = w * 32 + tr + (L2R ? 3 - j : j);   // x[t -+ j]
        xr[j] = *(const i32x4*)(x_s + row * 64 + sk_swz(row, kc) * 16);
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) wt[q4] = *(const i32x4*)(cw_s + cc * 8 + 16 * q4);
      const i32x4 bv = *(const i32x4*)(cb_s + cc * 2);
      bf16x8 wf[NCS];
#pragma unroll
      for (int c = 0; c < NCS; ++c) {
        const int row = c * 32 + tr;
        wf[c] = *(const bf16x8*)(wx_s + row * 64 + sk_swz(row, kc) * 16);
      }
      if (masked) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          xr[1][d] = ok1 ? xr[1][d] : 0;
          xr[2][d] = ok2 ? xr[2][d] : 0;
          xr[3][d] = ok3 ? xr[3][d] : 0;
        }
      }
      // channel 2d (+1) of the lane's 8: dword d of each x row holds the
      // pair; taps (w0, w1) and (w2, w3) of channel i are dwords 2i, 2i+1.
      // c_i = b_i + w3 x(t) + w2 x(t+1) + w1 x(t+2) + w0 x(t+3)
      float ca[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const unsigned b = (unsigned)bv[d];
        const unsigned x0 = xr[0][d], x1 = xr[1][d], x2 = xr[2][d], x3 = xr[3][d];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int i = 2 * d + hh;
          const unsigned sel = hh ? 0x07060302u : 0x05040100u;   // high / low bf16 of each row
          const unsigned x10 = __builtin_amdgcn_perm(x0, x1, sel);   // (x(t+1), x(t))
          const unsigned x32 = __builtin_amdgcn_perm(x2, x3, sel);   // (x(t+3), x(t+2))
          const unsigned w01 = (unsigned)wt[i >> 1][2 * (i & 1)], w23 = (unsigned)wt[i >> 1][2 * (i & 1) + 1];
          float c = __builtin_bit_cast(float, hh ? (b & 0xffff0000u) : (b << 16));
          c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w23), __builtin_bit_cast(bf16x2, x10), c, false);
          c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w01), __builtin_bit_cast(bf16x2, x32), c, false);
          ca[i] = c;
        }
      }
      // rows of tokens past the end get garbage here and are never stored
      bf16x8 af;
#pragma unroll
      for (int i = 0; i < 8; ++i) af[i] = (bf16)silu_fast(ca[i]);
#pragma unroll
      for (int c = 0; c < NCS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wf[c], acc[c], 0, 0, 0);
    }
    const bool last = c_tile * S + c_ks == hi - 1;
    if (last || c_ks == S - 1) end_piece();
    if (++c_ks == S) { c_ks = 0; ++c_tile; }
  };

#pragma unroll
  for (int s = 0; s + 1 < RS; ++s) issue(s);
  __builtin_amdgcn_s_waitcnt(sk_vmcnt((RS - 2) * PW));
  asm volatile("s_barrier" ::: "memory");
  for (int i0 = 0; i0 < n; i0 += RS) {
#pragma unroll
    for (int s = 0; s < RS; ++s) {
      // own copies of step q done (those of steps q+1 .. q+RS-2 may fly: the
      // copies complete in order, and partial-sum stores issued between them
      // can only make this wait longer); after the barrier everyone's are,
      // and every wave is done with the stage of step q-1, which receives
      // the copies of step q+RS-1
      __builtin_amdgcn_s_waitcnt(sk_vmcnt((RS - 2) * PW));
      asm volatile("s_barrier" ::: "memory");
      issue((s + RS - 1) % RS);
      if (i0 + s < n) compute(stage(s));
    }
  }
  __builtin_amdgcn_s_waitcnt(sk_vmcnt(0));
}

// Sum of the split conv's partial x_proj outputs: row t of xdbl lies in
// tile t / 128, whose pieces are counted from the block step ranges
// [floor(W b / G), floor(W (b+1) / G)) exactly as the conv kernel cut them.
// One thread per 4 consecutive floats of a row (P % 4 == 0) or per float.
R2L_DEV int sk_pieces(long tile, long S, long W, long G) {
  // #{b in 1 .. G-1 : floor(W b / G) < X} for X >= 1
  auto below = [&](long X) { const long k = (X * G + W - 1) / W - 1; return k < 0 ? 0L : (k > G - 1 ? G - 1 : k); };
  const long lo = tile * S;
  return (int)(1 + below(lo + S) - below(lo + 1));
}

template <int V>
__global__ __launch_bounds__(256) void sk_sum_kernel(long rows, int P, int S, long W, int G,
                                                     float* __restrict__ a, const float* __restrict__ b,
                                                     const float* __restrict__ c, int R, int RP,
                                                     bf16* __restrict__ dsplit) {
  const long per_row = P / V;
  const long n = rows * per_row;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const long row = i / per_row;
    const int pieces = sk_pieces(row / kSkTok, S, W, G);
    float* pa = a + row * P + (i % per_row) * V;
    const long off = pa - a;
    if constexpr (V == 4) {
      f32x4 v = *(f32x4*)pa;
      if (pieces > 1) v = v + *(const f32x4*)(b + off);
      if (pieces > 2) v = v + *(const f32x4*)(c + off);
      *(f32x4*)pa = v;
      if (dsplit != nullptr) {
        const float vv[4] = {v[0], v[1], v[2], v[3]};
        split_store<4>(dsplit, row, (int)(i % per_row) * 4, R, RP, vv);
      }
    } else {
      float v = *pa;
      if (pieces > 1) v = v + b[off];
      if (pieces > 2) v = v + c[off];
      *pa = v;
      if (dsplit != nullptr) split_store<1>(dsplit, row, (int)(i % per_row), R, RP, &v);
    }
  }
}

template <int NCS>
static int sk_blocks(int ncu) { return ncu * SkGeo<NCS>::BPC; }

static int sk_grid(int P, int ncu) {
  switch ((P + 31) / 32) {
    case 1: return sk_blocks<1>(ncu);
    case 2: return sk_blocks<2>(ncu);
    case 3: return sk_blocks<3>(ncu);
    case 4: return sk_blocks<4>(ncu);
    case 5: return sk_blocks<5>(ncu);
    case 6: return sk_blocks<6>(ncu);
    case 7: return sk_blocks<7>(ncu);
    default: return sk_blocks<8>(ncu);
  }
}

hipError_t conv_sk_sum(int Tn, int E, int P, float* part0, const float* part1, const float* part2, int ncu,
                       hipStream_t st, int R, bf16* dsplit) {
  if (Tn <= 0) return hipSuccess;
  const int RP = dsplit != nullptr ? delta_split_width(R) : 0;
  if (RP == 0) dsplit = nullptr;
  const int S = E / kSkK;
  const long W = (long)((Tn + kSkTok - 1) / kSkTok) * S;
  const int G = sk_grid(P, ncu);
  const long n = (long)Tn * (P % 4 == 0 ? P / 4 : P);
  const long want = (n + 255) / 256;
  const dim3 grid((unsigned)(want < 1 ? 1 : (want < 4096 ? want : 4096)));
  if (P % 4 == 0)
    hipLaunchKernelGGL(sk_sum_kernel<4>, grid, dim3(256), 0, st, (long)Tn, P, S, W, G, part0, part1, part2, R, RP,
                       dsplit);
  else
    hipLaunchKernelGGL(sk_sum_kernel<1>, grid, dim3(256), 0, st, (long)Tn, P, S, W, G, part0, part1, part2, R, RP,
                       dsplit);
  return hipGetLastError();
}

hipError_t conv_xproj_bf16_sk(int Tn, int E, int P, const bf16* x, long ld_x, const bf16* conv_w,
                              const bf16* conv_b, const bf16* x_proj_w, float* part0, float* part1,
                              float* part2, const int32_t* cu, int nseq, int ncu, bool l2r, hipStream_t st) {
  if (Tn <= 0) return hipSuccess;
  const int ncs = (P + 31) / 32;
  dim3 block(256);
#define R2L_SK(n)                                                                                 \
  case n:                                                                                         \
    if (l2r)                                                                                      \
      hipLaunchKernelGGL((conv_xproj_sk_kernel<n, true>), dim3(sk_blocks<n>(ncu)), block, 0, st,  \
                         Tn, E, P, x, ld_x, conv_w, conv_b, x_proj_w, part0, part1,               \
                         part2 - part1, cu, nseq);                                                \
    else                                                                                          \
      hipLaunchKernelGGL((conv_xproj_sk_kernel<n, false>), dim3(sk_blocks<n>(ncu)), block, 0, st, \
                         Tn, E, P, x, ld_x, conv_w, conv_b, x_proj_w, part0, part1,               \
                         part2 - part1, cu, nseq);                                                \
    break;
  switch (ncs) {
    R2L_SK(1) R2L_SK(2) R2L_SK(3) R2L_SK(4) R2L_SK(5) R2L_SK(6) R2L_SK(7) R2L_SK(8)
    default: return hipErrorInvalidValue;
  }
#undef R2L_SK
  return hipGetLastError();
}

}  // namespace r2l
