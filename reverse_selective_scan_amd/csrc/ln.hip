// Stream-local LayerNorm and tanh(s)-gated residual ("Bifocal Diffusion
// Language Models", §3.4 steps 3-4):
//   r = gamma (.) (o - mean) / sqrt(var + eps) + beta      (per token, over D)
//   h_out = h_in + tanh(s) r
// The unflip of step 3 is implicit: every kernel of the library already works
// in the original token order.  When tanh(s) == 0 the output is h_in copied
// bit for bit (§3.5: a zero gate leaves the causal baseline unchanged), which
// also keeps -0.0 inputs and non-finite branch values from leaking through.
//
// One wave per token row; the row (D <= 64 * VPL floats) stays in registers
// between the two reductions (mean, then centred second moment).  o, the
// out_proj output, is read as fp32 (also for bf16 activations).
#include "kernels.h"

namespace r2l {

// Lane layout: chunk i of the row (i = 0 .. D/512 - 1) gives lane l the 8
// consecutive elements [512 i + 8 l, +8): 16-byte loads of h and stores of h+
// (bf16), 2 x 16-byte loads of the fp32 branch input.
R2L_DEV void ld8(const float* p, float v[8]) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}
R2L_DEV void ld8(const bf16* p, float v[8]) {
  const bf16x8 q = *(const bf16x8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)q[i];
}
R2L_DEV void st8(float* p, const float v[8]) {
  *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
  *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
R2L_DEV void st8(bf16* p, const float v[8]) {
  bf16x8 q;
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = (bf16)v[i];
  *(bf16x8*)p = q;
}
template <typename T> struct Raw8h;
template <> struct Raw8h<bf16> { bf16x8 v; };
template <> struct Raw8h<float> { f32x4 a, b; };

template <typename T, typename O, int NCH>
__global__ __launch_bounds__(256) void ln_gate_kernel(int Tn, int D, const O* __restrict__ o,
                                                      const T* h_in, T* h_out,  // may alias
                                                      const float* __restrict__ gamma,
                                                      const float* __restrict__ beta,
                                                      const float* __restrict__ s,
                                                      float* __restrict__ branch, int no_ln,
                                                      float eps) {
  const int lane = lane_id();
  const int row = blockIdx.x * 4 + wave_id();
  if (row >= Tn) return;
  const int nch = D / 512;  // D % 512 == 0 here (other widths use the generic kernel)
  const O* orow = o + (long)row * D;
  const long rb = (long)row * D;
  float v[NCH][8];
  // every load of the row is issued first (o, h, gamma, beta), so that h's,
  // gamma's and beta's latencies hide behind the two reductions; h is read
  // before any store, so h_out may alias h_in
  Raw8h<T> hraw[NCH];
  float gm[NCH][8], bt[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c < nch) {
      ld8(orow + 512 * c + 8 * lane, v[c]);
      const long off = rb + 512 * c + 8 * lane;
      if constexpr (sizeof(T) == 2) {
        hraw[c].v = *(const bf16x8*)(h_in + off);
      } else {
        hraw[c].a = *(const f32x4*)(h_in + off);
        hraw[c].b = *(const f32x4*)(h_in + off + 4);
      }
      if (!no_ln) {
        ld8(gamma + 512 * c + 8 * lane, gm[c]);
        ld8(beta + 512 * c + 8 * lane, bt[c]);
      }
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    if (c < nch)
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += v[c][i];
  const float invD = 1.0f / (float)D;
  if (!no_ln) {
    const float mu = wave_sum(sum) * invD;
    float sq = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (c < nch)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[c][i] -= mu;
          sq = fmaf(v[c][i], v[c][i], sq);
        }
    const float rstd = 1.0f / sqrtf(wave_sum(sq) * invD + eps);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (c < nch)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[c][i] = fmaf(gm[c][i], v[c][i] * rstd, bt[c][i]);
  }
  const float g = tanhf(s[0]);
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    if (c < nch) {
      const long off = rb + 512 * c + 8 * lane;
      if (branch != nullptr) st8(branch + off, v[c]);
      if (g == 0.0f) {
        // a zero gate copies h bit for bit (no arithmetic on it at all)
        if constexpr (sizeof(T) == 2) {
          *(bf16x8*)(h_out + off) = hraw[c].v;
        } else {
          *(f32x4*)(h_out + off) = hraw[c].a;
          *(f32x4*)(h_out + off + 4) = hraw[c].b;
        }
      } else {
        float hv[8];
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int i = 0; i < 8; ++i) hv[i] = (float)hraw[c].v[i];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) { hv[i] = hraw[c].a[i]; hv[4 + i] = hraw[c].b[i]; }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = fmaf(g, v[c][i], hv[i]);
        st8(h_out + off, hv);
      }
    }
}

// Generic widths (D a multiple of 64): lane l holds elements 64 i + l.
template <typename T, typename O, int VPL>
__global__ __launch_bounds__(256) void ln_gate_generic_kernel(int Tn, int D, const O* __restrict__ o,
                                                              const T* h_in, T* h_out,  // may alias
                                                              const float* __restrict__ gamma,
                                                              const float* __restrict__ beta,
                                                              const float* __restrict__ s,
                                                              float* __restrict__ branch, int no_ln,
                                                              float eps) {
  const int lane = lane_id();
  const int row = blockIdx.x * 4 + wave_id();
  if (row >= Tn) return;
  const int cnt = D / 64;
  const O* orow = o + (long)row * D;
  float v[VPL];
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    v[i] = (i < cnt) ? to_f32(orow[i * 64 + lane]) : 0.0f;
    sum += v[i];
  }
  const float invD = 1.0f / (float)D;
  if (!no_ln) {
    const float mu = wave_sum(sum) * invD;
    float sq = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const float dv = (i < cnt) ? v[i] - mu : 0.0f;
      v[i] = dv;
      sq = fmaf(dv, dv, sq);
    }
    const float rstd = 1.0f / sqrtf(wave_sum(sq) * invD + eps);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (i < cnt) {
        const int dd = i * 64 + lane;
        v[i] = fmaf(gamma[dd], v[i] * rstd, beta[dd]);
      }
  }
  const float g = tanhf(s[0]);
  const T* hrow = h_in + (long)row * D;
  T* outrow = h_out + (long)row * D;
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (i < cnt) {
      const int dd = i * 64 + lane;
      if (branch != nullptr) branch[(long)row * D + dd] = v[i];
      const T hv = hrow[dd];
      outrow[dd] = (g == 0.0f) ? hv : from_f32<T>(fmaf(g, v[i], to_f32(hv)));
    }
}

// The same step on the K-split parts of o (a small input's out_proj): o is
// the sum over s, in order, of the partial tiles part[(t splits + s) 128 128]
// (tile t of the row-major grid of 128 x 128 output tiles, row-major inside),
// the order the GEMM's own sum uses, so o has the same values.  One block per
// token row; thread tid holds columns 8 (tid + 256 c) .. +7, and the row's two
// reductions run across the block (wave sums, then the four waves' totals in
// a fixed order).  Every load of the row is issued before the first wait.
template <typename T, int NCH, int S>
__global__ __launch_bounds__(256) void ln_gate_parts_kernel(int Tn, int D, const float* __restrict__ part,
                                                            const T* h_in, T* h_out,  // may alias
                                                            const float* __restrict__ gamma,
                                                            const float* __restrict__ beta,
                                                            const float* __restrict__ s,
                                                            float* __restrict__ branch,
                                                            float* __restrict__ o_save, int no_ln, float eps) {
  __shared__ float red[2][4];
  const int row = blockIdx.x;
  if (row >= Tn) return;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const long tile_row = (long)(row / 128) * (D / 128);
  const int rr = row % 128;
  const long rb = (long)row * D;
  f32x4 pa[NCH][S][2];
  Raw8h<T> hraw[NCH];
  float gm[NCH][8], bt[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int col = 8 * (tid + 256 * c);
    const float* p = part + ((tile_row + col / 128) * S) * (128 * 128) + rr * 128 + (col % 128);
#pragma unroll
    for (int sp = 0; sp < S; ++sp) {
      pa[c][sp][0] = *(const f32x4*)(p + (long)sp * (128 * 128));
      pa[c][sp][1] = *(const f32x4*)(p + (long)sp * (128 * 128) + 4);
    }
    const long off = rb + col;
    if constexpr (sizeof(T) == 2) {
      hraw[c].v = *(const bf16x8*)(h_in + off);
    } else {
      hraw[c].a = *(const f32x4*)(h_in + off);
      hraw[c].b = *(const f32x4*)(h_in + off + 4);
    }
    if (!no_ln) {
      ld8(gamma + col, gm[c]);
      ld8(beta + col, bt[c]);
    }
  }
  float v[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    f32x4 a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sp = 0; sp < S; ++sp) {
      a0 = a0 + pa[c][sp][0];
      a1 = a1 + pa[c][sp][1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[c][i] = a0[i]; v[c][4 + i] = a1[i]; }
    if (o_save != nullptr) st8(o_save + rb + 8 * (tid + 256 * c), v[c]);
  }
  auto block_sum = [&](float x, int k) {
    x = wave_sum(x);
    if (lane == 0) red[k][w] = x;
    __syncthreads();
    return ((red[k][0] + red[k][1]) + red[k][2]) + red[k][3];
  };
  const float invD = 1.0f / (float)D;
  if (!no_ln) {
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += v[c][i];
    const float mu = block_sum(sum, 0) * invD;
    float sq = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[c][i] -= mu;
        sq = fmaf(v[c][i], v[c][i], sq);
      }
    const float rstd = 1.0f / sqrtf(block_sum(sq, 1) * invD + eps);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) v[c][i] = fmaf(gm[c][i], v[c][i] * rstd, bt[c][i]);
  }
  const float g = tanhf(s[0]);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const long off = rb + 8 * (tid + 256 * c);
    if (branch != nullptr) st8(branch + off, v[c]);
    if (g == 0.0f) {
      // a zero gate copies h bit for bit (no arithmetic on it at all)
      if constexpr (sizeof(T) == 2) {
        *(bf16x8*)(h_out + off) = hraw[c].v;
      } else {
        *(f32x4*)(h_out + off) = hraw[c].a;
        *(f32x4*)(h_out + off + 4) = hraw[c].b;
      }
    } else {
      float hv[8];
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = (float)hraw[c].v[i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) { hv[i] = hraw[c].a[i]; hv[4 + i] = hraw[c].b[i]; }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) hv[i] = fmaf(g, v[c][i], hv[i]);
      st8(h_out + off, hv);
    }
  }
}

bool ln_gate_parts_fits(int D, int splits) {
  return (D == 2048 || D == 4096 || D == 8192) && (splits == 2 || splits == 4 || splits == 8);
}

template <typename T>
hipError_t ln_gate_parts(int Tn, int D, int splits, const float* part, const T* h_in, T* h_out,
                         const float* gamma, const float* beta, const float* s, float* branch, float* o_save,
                         bool no_ln, float eps, hipStream_t st) {
  if (!ln_gate_parts_fits(D, splits)) return hipErrorInvalidValue;
  if (Tn <= 0) return hipSuccess;
  const int nl = no_ln ? 1 : 0;
#define R2L_LNP(C, S)                                                                                      \
  hipLaunchKernelGGL((ln_gate_parts_kernel<T, C, S>), dim3(Tn), dim3(256), 0, st, Tn, D, part, h_in, h_out, \
                     gamma, beta, s, branch, o_save, nl, eps)
#define R2L_LNP_S(C)              \
  if (splits == 2) R2L_LNP(C, 2); \
  else if (splits == 4) R2L_LNP(C, 4); \
  else R2L_LNP(C, 8);
  if (D == 2048) { R2L_LNP_S(1) }
  else if (D == 4096) { R2L_LNP_S(2) }
  else { R2L_LNP_S(4) }
#undef R2L_LNP_S
#undef R2L_LNP
  return hipGetLastError();
}
template hipError_t ln_gate_parts<bf16>(int, int, int, const float*, const bf16*, bf16*, const float*, const float*,
                                        const float*, float*, float*, bool, float, hipStream_t);
template hipError_t ln_gate_parts<float>(int, int, int, const float*, const float*, float*, const float*,
                                         const float*, const float*, float*, float*, bool, float, hipStream_t);

template <typename T, typename O>
hipError_t ln_gate(int Tn, int D, const O* o, const T* h_in, T* h_out, const float* gamma,
                   const float* beta, const float* s, float* branch, bool no_ln, float eps,
                   hipStream_t st) {
  if (Tn <= 0) return hipSuccess;
  dim3 grid((Tn + 3) / 4), block(256);
  const int nl = no_ln ? 1 : 0;
  if (D % 512 == 0 && D <= 8192) {
#define R2L_LNV(C) \
  hipLaunchKernelGGL((ln_gate_kernel<T, O, C>), grid, block, 0, st, Tn, D, o, h_in, h_out, gamma, beta, s, branch, nl, eps)
    if (D <= 1024) R2L_LNV(2);
    else if (D <= 2048) R2L_LNV(4);
    else if (D <= 4096) R2L_LNV(8);
    else R2L_LNV(16);
#undef R2L_LNV
    return hipGetLastError();
  }
  const int cnt = D / 64;
#define R2L_LN(V)                                                                                      \
  hipLaunchKernelGGL((ln_gate_generic_kernel<T, O, V>), grid, block, 0, st, Tn, D, o, h_in, h_out, gamma, \
                     beta, s, branch, nl, eps)
  if (cnt <= 4) R2L_LN(4);
  else if (cnt <= 16) R2L_LN(16);
  else if (cnt <= 32) R2L_LN(32);
  else if (cnt <= 64) R2L_LN(64);
  else R2L_LN(128);
#undef R2L_LN
  return hipGetLastError();
}
template hipError_t ln_gate<float, float>(int, int, const float*, const float*, float*, const float*,
                                          const float*, const float*, float*, bool, float, hipStream_t);
template hipError_t ln_gate<bf16, float>(int, int, const float*, const bf16*, bf16*, const float*,
                                         const float*, const float*, float*, bool, float, hipStream_t);

}  // namespace r2l
