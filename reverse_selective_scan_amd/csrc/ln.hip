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
// between the two reductions (mean, then centred second moment).
#include "kernels.h"

namespace r2l {

template <typename T, int VPL>
__global__ __launch_bounds__(256) void ln_gate_kernel(int Tn, int D, const float* __restrict__ o,
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
  const float* orow = o + (long)row * D;
  float v[VPL];
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    v[i] = (i < cnt) ? orow[i * 64 + lane] : 0.0f;
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

template <typename T>
hipError_t ln_gate(int Tn, int D, const float* o, const T* h_in, T* h_out, const float* gamma,
                   const float* beta, const float* s, float* branch, bool no_ln, float eps,
                   hipStream_t st) {
  if (Tn <= 0) return hipSuccess;
  dim3 grid((Tn + 3) / 4), block(256);
  const int cnt = D / 64;
#define R2L_LN(V)                                                                              \
  hipLaunchKernelGGL((ln_gate_kernel<T, V>), grid, block, 0, st, Tn, D, o, h_in, h_out, gamma, \
                     beta, s, branch, no_ln ? 1 : 0, eps)
  if (cnt <= 4) R2L_LN(4);
  else if (cnt <= 16) R2L_LN(16);
  else if (cnt <= 32) R2L_LN(32);
  else if (cnt <= 64) R2L_LN(64);
  else R2L_LN(128);
#undef R2L_LN
  return hipGetLastError();
}
template hipError_t ln_gate<float>(int, int, const float*, const float*, float*, const float*,
                                   const float*, const float*, float*, bool, float, hipStream_t);
template hipError_t ln_gate<bf16>(int, int, const float*, const bf16*, bf16*, const float*,
                                  const float*, const float*, float*, bool, float, hipStream_t);

}  // namespace r2l
