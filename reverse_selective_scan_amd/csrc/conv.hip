// Anti-causal depthwise conv1d + bias + SiLU, optionally fused with x_proj
// ("Bifocal Diffusion Language Models", §3.4 steps 1-2: the Mamba-1 block's
// causal conv run over the flipped sequence is, in the original order, a
// conv that looks at a token and the K-1 tokens to its right):
//   u[t,e] = SiLU(b[e] + sum_{j=0}^{K-1} w[e,K-1-j] * x[t+j,e]),
// with x past the end of t's sequence taken as 0.
#include "kernels.h"

namespace r2l {

constexpr int KC = 4;  // d_conv (§4.1)

// ---------------------------------------------------------------------------
// Standalone conv: block = 64 channels x 32 tokens; wave w handles 8 tokens,
// lane = channel, so every load/store instruction touches 64 consecutive
// channels of one token row.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void conv_silu_kernel(int Tn, int E, const T* __restrict__ x,
                                                        long ld_x, const T* __restrict__ cw,
                                                        const T* __restrict__ cb, T* __restrict__ u,
                                                        const int32_t* __restrict__ cu, int nseq) {
  const int lane = lane_id(), w = wave_id();
  const int e = blockIdx.y * 64 + lane;
  const int tb = blockIdx.x * 32 + w * 8;
  float wt[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) wt[k] = to_f32(cw[(long)e * KC + k]);
  const float b = to_f32(cb[e]);
  for (int i = 0; i < 8; ++i) {
    const int t = tb + i;
    if (t >= Tn) break;
    const int se = seq_end_of(cu, nseq, t, Tn);
    float c = b;
#pragma unroll
    for (int j = 0; j < KC; ++j)
      if (t + j < se) c = fmaf(wt[KC - 1 - j], to_f32(x[(long)(t + j) * ld_x + e]), c);
    u[(long)t * E + e] = from_f32<T>(silu_fast(c));
  }
}

template <typename T>
hipError_t conv_silu(int Tn, int E, const T* x, long ld_x, const T* conv_w, const T* conv_b, T* u,
                     const int32_t* cu, int nseq, hipStream_t st) {
  if (Tn <= 0) return hipSuccess;
  dim3 grid((Tn + 31) / 32, E / 64);
  hipLaunchKernelGGL((conv_silu_kernel<T>), grid, dim3(256), 0, st, Tn, E, x, ld_x, conv_w, conv_b,
                     u, cu, nseq);
  return hipGetLastError();
}
template hipError_t conv_silu<float>(int, int, const float*, long, const float*, const float*,
                                     float*, const int32_t*, int, hipStream_t);
template hipError_t conv_silu<bf16>(int, int, const bf16*, long, const bf16*, const bf16*, bf16*,
                                    const int32_t*, int, hipStream_t);

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
template <int NCS>
__global__ __launch_bounds__(256) void conv_xproj_kernel(int Tn, int E, int P,
                                                         const bf16* __restrict__ x, long ld_x,
                                                         const bf16* __restrict__ cw,
                                                         const bf16* __restrict__ cb,
                                                         const bf16* __restrict__ Wx,
                                                         bf16* __restrict__ u_out,
                                                         float* __restrict__ xdbl,
                                                         const int32_t* __restrict__ cu, int nseq) {
  constexpr int NC = NCS * 32;
  __shared__ float red[3][32 * NC];
  const int lane = lane_id(), w = wave_id();
  const int tr = lane & 31, kh = lane >> 5;
  const int t0 = blockIdx.x * 32;
  const int t = t0 + tr;
  const bool tv = t < Tn;
  const int se = tv ? seq_end_of(cu, nseq, t, Tn) : 0;
  const int Ew = E / 4;
  const int cbeg = w * Ew;

  f32x16 acc[NCS];
#pragma unroll
  for (int c = 0; c < NCS; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;

  const bf16x8 zero8 = {};
  // Operands of one 16-channel k-step; the next step's are loaded while the
  // current one is computed (the loads would otherwise stall every step).
  struct Step {
    bf16x8 wv[4], bv, xv[KC], wx[NCS];
  };
  // Loads are unconditional, from clamped (valid) rows; masks are applied
  // when the values are used.  (A per-lane branch around a load makes both
  // paths write the same registers and forces an immediate wait.)
  const int tt = min(t, Tn - 1);
  const int xlast = (tv ? se : tt + 1) - 1;   // last row this lane may read
  bool xok[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) xok[j] = tv && t + j < se;
  auto load_step = [&](Step& s, int k0) {
    const int c0 = k0 + kh * 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) s.wv[q] = *(const bf16x8*)(cw + (long)c0 * KC + 8 * q);
    s.bv = *(const bf16x8*)(cb + c0);
#pragma unroll
    for (int j = 0; j < KC; ++j) s.xv[j] = *(const bf16x8*)(x + (long)min(tt + j, xlast) * ld_x + c0);
#pragma unroll
    for (int c = 0; c < NCS; ++c) {
      const int row = min(c * 32 + tr, P - 1);
      s.wx[c] = *(const bf16x8*)(Wx + (long)row * E + c0);
    }
  };
  Step cur, nxt;
  load_step(cur, cbeg);
  for (int k0 = cbeg; k0 < cbeg + Ew; k0 += 16) {
    if (k0 + 16 < cbeg + Ew) load_step(nxt, k0 + 16);
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
    cur = nxt;
  }
  // D layout: lane holds output column (lane & 31) of each 32-wide slice and
  // token rows 8*(r/4) + 4*(lane/32) + r%4.
  if (w > 0) {
#pragma unroll
    for (int c = 0; c < NCS; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * kh + (r & 3);
        red[w - 1][row * NC + c * 32 + tr] = acc[c][r];
      }
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int c = 0; c < NCS; ++c) {
      const int col = c * 32 + tr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * kh + (r & 3);
        const int idx = row * NC + col;
        const float v = acc[c][r] + red[0][idx] + red[1][idx] + red[2][idx];
        if (col < P && t0 + row < Tn) xdbl[(long)(t0 + row) * P + col] = v;
      }
    }
  }
}

hipError_t conv_xproj_bf16(int Tn, int E, int P, const bf16* x, long ld_x, const bf16* conv_w,
                           const bf16* conv_b, const bf16* x_proj_w, bf16* u_out, float* xdbl,
                           const int32_t* cu, int nseq, hipStream_t st) {
  if (Tn <= 0) return hipSuccess;
  const int ncs = (P + 31) / 32;
  dim3 grid((Tn + 31) / 32), block(256);
#define R2L_CX(n)                                                                               \
  case n:                                                                                       \
    hipLaunchKernelGGL((conv_xproj_kernel<n>), grid, block, 0, st, Tn, E, P, x, ld_x, conv_w,   \
                       conv_b, x_proj_w, u_out, xdbl, cu, nseq);                                \
    break;
  switch (ncs) {
    R2L_CX(1) R2L_CX(2) R2L_CX(3) R2L_CX(4) R2L_CX(5) R2L_CX(6) R2L_CX(7) R2L_CX(8)
    default: return hipErrorInvalidValue;
  }
#undef R2L_CX
  return hipGetLastError();
}

}  // namespace r2l
