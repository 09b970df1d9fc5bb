// Kernels of the layer's backward pass other than the scan's and the GEMMs
// (the gradient of one ReverseMambaLayer hook, "Bifocal Diffusion Language
// Models", §3.4 steps 1-4, for training the sidecar: §3.5, plug-in mode).
// Each is a plain, memory-bound pass; every sum over tokens is taken in a
// fixed order (per-block partial sums, then a second pass over the blocks).
#include "kernels.h"

namespace r2l {

constexpr int KC_ = 4;   // d_conv

// ---------------------------------------------------------------------------
// out [cols, rows_pad] (act) = in [rows, cols]^T (row stride ld_in), with
// zeros in columns rows .. rows_pad - 1 of out.  64 x 64 tiles through LDS.
// ---------------------------------------------------------------------------
template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void transpose_kernel(int rows, int cols, int rows_pad, const Tin* __restrict__ in,
                                                        long ld_in, Tout* __restrict__ out) {
  __shared__ float tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? to_f32(in[(long)r * ld_in + c]) : 0.0f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows_pad) out[(long)c * rows_pad + r] = from_f32<Tout>(tile[tx][i]);
  }
}

template <typename Tin, typename Tout>
hipError_t transpose(int rows, int cols, int rows_pad, const Tin* in, long ld_in, Tout* out, hipStream_t st) {
  if (cols <= 0 || rows_pad <= 0) return hipSuccess;
  dim3 grid((cols + 63) / 64, (rows_pad + 63) / 64);
  hipLaunchKernelGGL((transpose_kernel<Tin, Tout>), grid, dim3(256), 0, st, rows, cols, rows_pad, in, ld_in, out);
  return hipGetLastError();
}
template hipError_t transpose<float, bf16>(int, int, int, const float*, long, bf16*, hipStream_t);
template hipError_t transpose<bf16, bf16>(int, int, int, const bf16*, long, bf16*, hipStream_t);
template hipError_t transpose<float, float>(int, int, int, const float*, long, float*, hipStream_t);

// ---------------------------------------------------------------------------
// Elementwise passes over [rows, cols] (row strides given).
// ---------------------------------------------------------------------------
// kConvert:      out = in
// kSoftplusBias: out = softplus(in + vec[col])              (dt from dt_proj's product)
// kDtPre:        out = in (1 - exp(-aux))                   (ddt through softplus: sigmoid(pre) = 1 - e^-dt)
// kAddTo:        out = in + aux                             (dh = g + the branch's gradient)
template <int OP, typename Tin, typename Tout>
__global__ __launch_bounds__(256) void elementwise_kernel(int rows, int cols, const Tin* __restrict__ in, long ld_in,
                                                          const float* __restrict__ aux, long ld_aux,
                                                          const float* __restrict__ vec, Tout* __restrict__ out,
                                                          long ld_out) {
  const long n = (long)rows * cols;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const long r = i / cols;
    const int c = (int)(i % cols);
    const float v = to_f32(in[r * ld_in + c]);
    float o;
    if (OP == kConvert) o = v;
    else if (OP == kSoftplusBias) o = softplus_f(v + vec[c]);
    else if (OP == kDtPre) o = v * (1.0f - expf(-aux[r * ld_aux + c]));
    else o = v + aux[r * ld_aux + c];
    out[r * ld_out + c] = from_f32<Tout>(o);
  }
}

template <int OP, typename Tin, typename Tout>
hipError_t elementwise(int rows, int cols, const Tin* in, long ld_in, const float* aux, long ld_aux,
                       const float* vec, Tout* out, long ld_out, hipStream_t st) {
  const long n = (long)rows * cols;
  if (n <= 0) return hipSuccess;
  const long want = (n + 255) / 256;
  hipLaunchKernelGGL((elementwise_kernel<OP, Tin, Tout>), dim3((unsigned)(want < 8192 ? want : 8192)), dim3(256), 0,
                     st, rows, cols, in, ld_in, aux, ld_aux, vec, out, ld_out);
  return hipGetLastError();
}
#define R2L_EW(OP, TI, TO)                                                                                \
  template hipError_t elementwise<OP, TI, TO>(int, int, const TI*, long, const float*, long, const float*, \
                                              TO*, long, hipStream_t);
R2L_EW(kConvert, float, bf16) R2L_EW(kConvert, float, float) R2L_EW(kConvert, bf16, bf16)
R2L_EW(kSoftplusBias, float, float) R2L_EW(kDtPre, float, float)
R2L_EW(kAddTo, bf16, bf16) R2L_EW(kAddTo, float, float)
#undef R2L_EW

// ---------------------------------------------------------------------------
// Column sums of f32 [rows, cols]: pass 1, block b sums rows
// [b rows/nb, (b+1) rows/nb) of 256 columns; pass 2 sums the nb partials in
// order and scales.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void colsum_part_kernel(int rows, int cols, const float* __restrict__ in, long ld,
                                                          float* __restrict__ part) {
  const int nb = gridDim.y, b = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  const long r0 = (long)rows * b / nb, r1 = (long)rows * (b + 1) / nb;
  float s = 0.0f;
  for (long r = r0; r < r1; ++r) s += in[r * ld + c];
  part[(long)b * cols + c] = s;
}
__global__ __launch_bounds__(256) void colsum_final_kernel(int cols, int nb, const float* __restrict__ part,
                                                           float scale, float* __restrict__ out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  float s = 0.0f;
  for (int b = 0; b < nb; ++b) s += part[(long)b * cols + c];
  out[c] = s * scale;
}
// part: at least colsum_parts(rows) * cols floats
int colsum_parts(int rows) { return rows < 64 ? 1 : (rows / 64 < 256 ? rows / 64 : 256); }
hipError_t colsum(int rows, int cols, const float* in, long ld, float* part, float scale, float* out, hipStream_t st) {
  if (cols <= 0) return hipSuccess;
  const int nb = colsum_parts(rows);
  hipLaunchKernelGGL(colsum_part_kernel, dim3((cols + 255) / 256, nb), dim3(256), 0, st, rows, cols, in, ld, part);
  hipLaunchKernelGGL(colsum_final_kernel, dim3((cols + 255) / 256), dim3(256), 0, st, cols, nb, (const float*)part,
                     scale, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LayerNorm + gate backward, one wave per token row (D a multiple of 64).
//   h+ = h + th r, r = gamma xhat + beta, xhat = (o - mu) / sigma, th = tanh(s):
//   do = th / sigma (gamma g - mean(gamma g) - xhat mean(gamma g xhat));
//   gx[t] = th [g xhat | g] (f32 [T, 2D]: summed over t, d gamma and d beta);
//   gr[t] = (1 - th^2) sum_d g r (summed over t, d s).
// Without the LayerNorm r = o: do = th g.
// ---------------------------------------------------------------------------
template <typename T, int VPL>
__global__ __launch_bounds__(256) void ln_gate_bwd_kernel(int Tn, int D, const T* __restrict__ g, const float* __restrict__ o,
                                                          const float* __restrict__ gamma, const float* __restrict__ beta,
                                                          const float* __restrict__ s, int no_ln, float eps,
                                                          float* __restrict__ dout, float* __restrict__ gx,
                                                          float* __restrict__ gr) {
  const int lane = lane_id();
  const int row = blockIdx.x * 4 + wave_id();
  if (row >= Tn) return;
  const int cnt = D / 64;
  const float th = tanhf(s[0]);
  float x[VPL], gg[VPL];
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int dd = i * 64 + lane;
    x[i] = i < cnt ? o[(long)row * D + dd] : 0.0f;
    gg[i] = i < cnt ? to_f32(g[(long)row * D + dd]) : 0.0f;
    sum += x[i];
  }
  const float invD = 1.0f / (float)D;
  if (no_ln) {
    float p = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (i < cnt) {
        const int dd = i * 64 + lane;
        dout[(long)row * D + dd] = th * gg[i];
        p = fmaf(gg[i], x[i], p);
      }
    p = wave_sum(p);
    if (lane == 0) gr[row] = (1.0f - th * th) * p;
    return;
  }
  const float mu = wave_sum(sum) * invD;
  float sq = 0.0f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    x[i] = i < cnt ? x[i] - mu : 0.0f;
    sq = fmaf(x[i], x[i], sq);
  }
  const float rstd = 1.0f / sqrtf(wave_sum(sq) * invD + eps);
  float m1 = 0.0f, m2 = 0.0f, p = 0.0f;
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (i < cnt) {
      const int dd = i * 64 + lane;
      x[i] *= rstd;                                    // xhat
      const float gg_gamma = gg[i] * gamma[dd];
      m1 += gg_gamma;
      m2 = fmaf(gg_gamma, x[i], m2);
      p = fmaf(gg[i], fmaf(gamma[dd], x[i], beta[dd]), p);
      gx[(long)row * 2 * D + dd] = th * gg[i] * x[i];
      gx[(long)row * 2 * D + D + dd] = th * gg[i];
    }
  m1 = wave_sum(m1) * invD;
  m2 = wave_sum(m2) * invD;
  p = wave_sum(p);
  if (lane == 0) gr[row] = (1.0f - th * th) * p;
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (i < cnt) {
      const int dd = i * 64 + lane;
      dout[(long)row * D + dd] = th * rstd * (gg[i] * gamma[dd] - m1 - x[i] * m2);
    }
}

template <typename T>
hipError_t ln_gate_bwd(int Tn, int D, const T* g, const float* o, const float* gamma, const float* beta,
                       const float* s, bool no_ln, float eps, float* dout, float* gx, float* gr, hipStream_t st) {
  if (Tn <= 0) return hipSuccess;
  dim3 grid((Tn + 3) / 4), block(256);
  const int cnt = D / 64, nl = no_ln ? 1 : 0;
#define R2L_LNB(V) \
  hipLaunchKernelGGL((ln_gate_bwd_kernel<T, V>), grid, block, 0, st, Tn, D, g, o, gamma, beta, s, nl, eps, dout, gx, gr)
  if (cnt <= 4) R2L_LNB(4);
  else if (cnt <= 16) R2L_LNB(16);
  else if (cnt <= 32) R2L_LNB(32);
  else if (cnt <= 64) R2L_LNB(64);
  else R2L_LNB(128);
#undef R2L_LNB
  return hipGetLastError();
}
template hipError_t ln_gate_bwd<float>(int, int, const float*, const float*, const float*, const float*, const float*,
                                       bool, float, float*, float*, float*, hipStream_t);
template hipError_t ln_gate_bwd<bf16>(int, int, const bf16*, const float*, const float*, const float*, const float*,
                                      bool, float, float*, float*, float*, hipStream_t);

// ---------------------------------------------------------------------------
// Anti-causal conv + SiLU backward (K = 4).  Forward:
//   c_t = b + sum_j w[K-1-j] x_{t+j} (x past t's sequence end = 0), u = SiLU(c).
// dc_t = du_t SiLU'(c_t) (c recomputed from x);  dx_s = sum_j w[K-1-j] dc_{s-j}
// over s-j at or after s's sequence start;  dw[K-1-j] = sum_t dc_t x_{t+j},
// db = sum_t dc_t, as per-(row block) partials [nb][E][K+1].
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void conv_dc_kernel(int Tn, int E, const T* __restrict__ x, long ld_x,
                                                      const T* __restrict__ cw, const T* __restrict__ cb,
                                                      const float* __restrict__ du, const float* __restrict__ du2,
                                                      float* __restrict__ dc, const int32_t* __restrict__ cu, int nseq) {
  const long n = (long)Tn * E;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const int t = (int)(i / E), e = (int)(i % E);
    const int se = seq_end_of(cu, nseq, t, Tn);
    float c = to_f32(cb[e]);
    for (int j = 0; j < KC_; ++j)
      if (t + j < se) c = fmaf(to_f32(cw[(long)e * KC_ + KC_ - 1 - j]), to_f32(x[(long)(t + j) * ld_x + e]), c);
    const float sg = 1.0f / (1.0f + expf(-c));
    const float g = du[i] + (du2 ? du2[i] : 0.0f);
    dc[i] = g * sg * (1.0f + c * (1.0f - sg));
  }
}

template <typename T>
__global__ __launch_bounds__(256) void conv_dx_kernel(int Tn, int E, const T* __restrict__ x, long ld_x,
                                                      const T* __restrict__ cw, const float* __restrict__ dc,
                                                      float* __restrict__ dx, float* __restrict__ part,
                                                      const int32_t* __restrict__ cu, int nseq) {
  // block: 64 channels x a contiguous range of rows; thread = (channel, row phase)
  const int nb = gridDim.y, b = blockIdx.y;
  const int e = blockIdx.x * 64 + (threadIdx.x & 63), ph = threadIdx.x >> 6;
  __shared__ float red[4][64][KC_ + 1];
  float acc[KC_ + 1] = {};
  const long r0 = (long)Tn * b / nb, r1 = (long)Tn * (b + 1) / nb;
  float w[KC_];
  for (int k = 0; k < KC_; ++k) w[k] = to_f32(cw[(long)e * KC_ + k]);
  for (long s = r0 + ph; s < r1; s += 4) {
    const int t = (int)s;
    const int sl = seq_start_of(cu, nseq, t), se = seq_end_of(cu, nseq, t, Tn);
    float v = 0.0f;
    for (int j = 0; j < KC_; ++j)
      if (t - j >= sl) v = fmaf(w[KC_ - 1 - j], dc[(long)(t - j) * E + e], v);
    dx[(long)t * E + e] = v;
    const float d = dc[(long)t * E + e];
    for (int j = 0; j < KC_; ++j)
      if (t + j < se) acc[KC_ - 1 - j] = fmaf(d, to_f32(x[(long)(t + j) * ld_x + e]), acc[KC_ - 1 - j]);
    acc[KC_] += d;
  }
  for (int k = 0; k <= KC_; ++k) red[ph][threadIdx.x & 63][k] = acc[k];
  __syncthreads();
  if (ph == 0)
    for (int k = 0; k <= KC_; ++k)
      part[((long)b * E + e) * (KC_ + 1) + k] =
          ((red[0][threadIdx.x][k] + red[1][threadIdx.x][k]) + red[2][threadIdx.x][k]) + red[3][threadIdx.x][k];
}

__global__ __launch_bounds__(256) void conv_wsum_kernel(int E, int nb, const float* __restrict__ part,
                                                        float* __restrict__ dw, float* __restrict__ db) {
  const long i = blockIdx.x * 256L + threadIdx.x;
  if (i >= (long)E * (KC_ + 1)) return;
  float s = 0.0f;
  for (int b = 0; b < nb; ++b) s += part[(long)b * E * (KC_ + 1) + i];
  const long e = i / (KC_ + 1);
  const int k = (int)(i % (KC_ + 1));
  if (k < KC_) dw[e * KC_ + k] = s;
  else db[e] = s;
}

int conv_bwd_parts(int Tn) { return Tn < 256 ? 1 : (Tn / 256 < 128 ? Tn / 256 : 128); }

template <typename T>
hipError_t conv_bwd(int Tn, int E, const T* x, long ld_x, const T* cw, const T* cb, const float* du, const float* du2,
                    float* dc, float* dx, float* part, float* dw, float* db, const int32_t* cu, int nseq,
                    hipStream_t st) {
  if (Tn <= 0) return hipSuccess;
  const long n = (long)Tn * E;
  const long want = (n + 255) / 256;
  hipLaunchKernelGGL((conv_dc_kernel<T>), dim3((unsigned)(want < 8192 ? want : 8192)), dim3(256), 0, st, Tn, E, x,
                     ld_x, cw, cb, du, du2, dc, cu, nseq);
  const int nb = conv_bwd_parts(Tn);
  hipLaunchKernelGGL((conv_dx_kernel<T>), dim3(E / 64, nb), dim3(256), 0, st, Tn, E, x, ld_x, cw, (const float*)dc,
                     dx, part, cu, nseq);
  hipLaunchKernelGGL(conv_wsum_kernel, dim3((E * (KC_ + 1) + 255) / 256), dim3(256), 0, st, E, nb,
                     (const float*)part, dw, db);
  return hipGetLastError();
}
template hipError_t conv_bwd<float>(int, int, const float*, long, const float*, const float*, const float*,
                                    const float*, float*, float*, float*, float*, float*, const int32_t*, int,
                                    hipStream_t);
template hipError_t conv_bwd<bf16>(int, int, const bf16*, long, const bf16*, const bf16*, const float*, const float*,
                                   float*, float*, float*, float*, float*, const int32_t*, int, hipStream_t);

// out[t] (act, ld_out) = [a (f32 [T, na]) | b (f32 [T, nb]) | c (f32 [T, nc])]
template <typename Tout>
__global__ __launch_bounds__(256) void concat3_kernel(int Tn, int na, int nb, int nc, const float* __restrict__ a,
                                                      const float* __restrict__ b, const float* __restrict__ c,
                                                      Tout* __restrict__ out, long ld_out) {
  const int w = na + nb + nc;
  const long n = (long)Tn * w;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const long t = i / w;
    const int k = (int)(i % w);
    const float v = k < na ? a[t * na + k] : (k < na + nb ? b[t * nb + k - na] : c[t * nc + k - na - nb]);
    out[t * ld_out + k] = from_f32<Tout>(v);
  }
}
template <typename Tout>
hipError_t concat3(int Tn, int na, int nb, int nc, const float* a, const float* b, const float* c, Tout* out,
                   long ld_out, hipStream_t st) {
  const long n = (long)Tn * (na + nb + nc);
  if (n <= 0) return hipSuccess;
  const long want = (n + 255) / 256;
  hipLaunchKernelGGL((concat3_kernel<Tout>), dim3((unsigned)(want < 8192 ? want : 8192)), dim3(256), 0, st, Tn, na,
                     nb, nc, a, b, c, out, ld_out);
  return hipGetLastError();
}
template hipError_t concat3<bf16>(int, int, int, int, const float*, const float*, const float*, bf16*, long,
                                  hipStream_t);
template hipError_t concat3<float>(int, int, int, int, const float*, const float*, const float*, float*, long,
                                   hipStream_t);

}  // namespace r2l
