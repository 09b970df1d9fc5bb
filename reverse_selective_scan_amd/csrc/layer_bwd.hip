// Kernels of the layer's backward pass other than the scan's and the GEMMs
// (the gradient of one ReverseMambaLayer hook, "Bifocal Diffusion Language
// Models", §3.4 steps 1-4, for training the sidecar: §3.5, plug-in mode).
// Each is a plain, memory-bound pass; every sum over tokens is taken in a
// fixed order (per-block partial sums, then a second pass over the blocks).
#include <type_traits>

#include "kernels.h"

namespace r2l {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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

// The same for bf16 with 16-byte rows (cols, ld_in and rows_pad multiples of
// 8, both pointers 16-byte aligned): each lane moves an 8 x 8 block, eight
// 16-byte row loads, the 16-bit transpose in registers (one byte permute per
// output dword) and eight 16-byte row stores; a wave covers 64 x 64, so
// eight lanes share each 128-byte row segment on both sides.  Block = four
// waves side by side along the columns.
__global__ __launch_bounds__(256) void transpose16_kernel(int rows, int cols, int rows_pad, const bf16* __restrict__ in,
                                                          long ld_in, bf16* __restrict__ out) {
  const int lane = lane_id(), w = wave_id();
  const int c = (blockIdx.x * 4 + w) * 64 + 8 * (lane >> 3);   // the lane's first input column
  const int r = blockIdx.y * 64 + 8 * (lane & 7);              // its first input row
  if (c >= cols || r >= rows_pad) return;
  u32x4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    v[j] = r + j < rows ? *(const u32x4*)(in + (long)(r + j) * ld_in + c) : u32x4{0u, 0u, 0u, 0u};
  // output row c + i, dword d = (element i of input row 2d, of row 2d + 1)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const unsigned sel = (i & 1) ? 0x07060302u : 0x05040100u;   // high / low bf16 of each input dword
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] = __builtin_amdgcn_perm(v[2 * d + 1][i >> 1], v[2 * d][i >> 1], sel);
    *(u32x4*)(out + (long)(c + i) * rows_pad + r) = o;
  }
}

template <typename Tin, typename Tout>
hipError_t transpose(int rows, int cols, int rows_pad, const Tin* in, long ld_in, Tout* out, hipStream_t st) {
  if (cols <= 0 || rows_pad <= 0) return hipSuccess;
  if constexpr (std::is_same<Tin, bf16>::value && std::is_same<Tout, bf16>::value) {
    if (cols % 8 == 0 && ld_in % 8 == 0 && rows_pad % 8 == 0 && ((uintptr_t)in & 15) == 0 &&
        ((uintptr_t)out & 15) == 0) {
      dim3 grid((cols + 255) / 256, (rows_pad + 63) / 64);
      hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, st, rows, cols, rows_pad, in, ld_in, out);
      return hipGetLastError();
    }
  }
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
template <int OP>
R2L_DEV float ew_op(float v, const float* aux, long ai, const float* vec, int c) {
  if (OP == kConvert) return v;
  if (OP == kSoftplusBias) return softplus_f(v + vec[c]);
  if (OP == kDtPre) return v * (1.0f - expf(-aux[ai]));
  return v + aux[ai];
}

// grid (column blocks of 256, row groups); each block walks its rows
template <int OP, typename Tin, typename Tout>
__global__ __launch_bounds__(256) void elementwise_kernel(int rows, int cols, const Tin* __restrict__ in, long ld_in,
                                                          const float* __restrict__ aux, long ld_aux,
                                                          const float* __restrict__ vec, Tout* __restrict__ out,
                                                          long ld_out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  for (int r = blockIdx.y; r < rows; r += gridDim.y) {
    const float v = to_f32(in[(long)r * ld_in + c]);
    out[(long)r * ld_out + c] = from_f32<Tout>(ew_op<OP>(v, aux, (long)r * ld_aux + c, vec, c));
  }
}

// The same for f32 -> f32 four columns per thread (16-byte accesses), the
// same arithmetic per element.
template <int OP>
__global__ __launch_bounds__(256) void elementwise4_kernel(int rows, int cols, const float* __restrict__ in,
                                                           long ld_in, const float* __restrict__ aux, long ld_aux,
                                                           const float* __restrict__ vec, float* __restrict__ out,
                                                           long ld_out) {
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= cols) return;
  f32x4 vv = {};
  if (OP == kSoftplusBias) vv = *(const f32x4*)(vec + c);
  for (int r = blockIdx.y; r < rows; r += gridDim.y) {
    const f32x4 x = *(const f32x4*)(in + (long)r * ld_in + c);
    f32x4 a = {};
    if (OP == kDtPre || OP == kAddTo) a = *(const f32x4*)(aux + (long)r * ld_aux + c);
    f32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float v = x[k];
      if (OP == kConvert) o[k] = v;
      else if (OP == kSoftplusBias) o[k] = softplus_f(v + vv[k]);
      else if (OP == kDtPre) o[k] = v * (1.0f - expf(-a[k]));
      else o[k] = v + a[k];
    }
    *(f32x4*)(out + (long)r * ld_out + c) = o;
  }
}

template <int OP, typename Tin, typename Tout>
hipError_t elementwise(int rows, int cols, const Tin* in, long ld_in, const float* aux, long ld_aux,
                       const float* vec, Tout* out, long ld_out, hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if constexpr (std::is_same<Tin, float>::value && std::is_same<Tout, float>::value) {
    auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    const bool aux_ok = !(OP == kDtPre || OP == kAddTo) || (ld_aux % 4 == 0 && a16(aux));
    if (cols % 4 == 0 && ld_in % 4 == 0 && ld_out % 4 == 0 && a16(in) && a16(out) && aux_ok &&
        (OP != kSoftplusBias || a16(vec))) {
      const int cb4 = (cols / 4 + 255) / 256;
      const int rg4 = rows < 65535 ? rows : 65535;
      const int ry4 = cb4 * rg4 > 16384 ? (16384 + cb4 - 1) / cb4 : rg4;
      hipLaunchKernelGGL((elementwise4_kernel<OP>), dim3(cb4, ry4 > 0 ? ry4 : 1), dim3(256), 0, st, rows, cols, in,
                         ld_in, aux, ld_aux, vec, out, ld_out);
      return hipGetLastError();
    }
  }
  const int cb = (cols + 255) / 256;
  const int rg = rows < 65535 ? rows : 65535;
  const int ry = cb * rg > 16384 ? (16384 + cb - 1) / cb : rg;   // about 16K blocks
  hipLaunchKernelGGL((elementwise_kernel<OP, Tin, Tout>), dim3(cb, ry > 0 ? ry : 1), dim3(256), 0, st, rows, cols,
                     in, ld_in, aux, ld_aux, vec, out, ld_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// One pass over 64 x 64 tiles of [rows, cols]: v = op(in, aux); optional
// row-major copy out_rm (row stride ld_rm), transposed copy out_t
// [cols, rows_pad] (zeros past rows) and per-tile-row column sums
// colpart [ceil(rows / 64)][cols] (each the sum of 64 rows, four row phases
// added in order).
// ---------------------------------------------------------------------------
template <int OP, typename Tin, typename Tout>
__global__ __launch_bounds__(256) void fused_t_kernel(int rows, int cols, int rows_pad, const Tin* __restrict__ in,
                                                      long ld_in, const float* __restrict__ aux, long ld_aux,
                                                      Tout* __restrict__ out_rm, long ld_rm, Tout* __restrict__ out_t,
                                                      float* __restrict__ colpart) {
  __shared__ float tile[64][65];
  __shared__ float cs[4][64];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int c = c0 + tx;
  float sum = 0.0f;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i;
    float v = 0.0f;
    if (r < rows && c < cols) {
      v = ew_op<OP>(to_f32(in[(long)r * ld_in + c]), aux, (long)r * ld_aux + c, nullptr, c);
      if (out_rm) out_rm[(long)r * ld_rm + c] = from_f32<Tout>(v);
    }
    tile[i][tx] = v;
    sum += v;
  }
  cs[ty][tx] = sum;
  __syncthreads();
  if (colpart && ty == 0 && c < cols && r0 < rows)
    colpart[(long)blockIdx.y * cols + c] = ((cs[0][tx] + cs[1][tx]) + cs[2][tx]) + cs[3][tx];
  if (out_t) {
    for (int i = ty; i < 64; i += 4) {
      const int cc = c0 + i, r = r0 + tx;
      if (cc < cols && r < rows_pad) out_t[(long)cc * rows_pad + r] = from_f32<Tout>(tile[tx][i]);
    }
  }
}

// The same pass for f32 -> bf16 with 16-byte rows (cols, ld_rm and rows_pad
// multiples of 8, ld_in and ld_aux of 4, pointers 16-byte aligned): each lane
// takes an 8 x 8 block as transpose16_kernel does (32-byte f32 row loads,
// 16-byte bf16 row stores, the transposed copy by byte permutes in
// registers).  Column sums: each lane adds its 8 rows in order, then the 8
// lanes of a 64-row tile combine by a fixed butterfly.
template <int OP>
__global__ __launch_bounds__(256) void fused_t16_kernel(int rows, int cols, int rows_pad, const float* __restrict__ in,
                                                        long ld_in, const float* __restrict__ aux, long ld_aux,
                                                        bf16* __restrict__ out_rm, long ld_rm,
                                                        bf16* __restrict__ out_t, float* __restrict__ colpart) {
  const int lane = lane_id(), w = wave_id();
  const int c = (blockIdx.x * 4 + w) * 64 + 8 * (lane >> 3);   // the lane's first column
  const int r0 = blockIdx.y * 64, r = r0 + 8 * (lane & 7);     // the tile's and the lane's first row
  if (c >= cols) return;                                       // (whole 8-lane groups: no lane of a butterfly leaves)
  u32x4 pk[8];
  float sum[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) sum[k] = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float v[8];
    if (r + j < rows) {
      const f32x4 a0 = *(const f32x4*)(in + (long)(r + j) * ld_in + c);
      const f32x4 a1 = *(const f32x4*)(in + (long)(r + j) * ld_in + c + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) { v[k] = a0[k]; v[4 + k] = a1[k]; }
      if (OP == kDtPre) {
        const f32x4 b0 = *(const f32x4*)(aux + (long)(r + j) * ld_aux + c);
        const f32x4 b1 = *(const f32x4*)(aux + (long)(r + j) * ld_aux + c + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[k] = v[k] * (1.0f - expf(-b0[k]));
          v[4 + k] = v[4 + k] * (1.0f - expf(-b1[k]));
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) sum[k] += v[k];
    const bf16x8 b = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3], (bf16)v[4], (bf16)v[5], (bf16)v[6], (bf16)v[7]};
    pk[j] = __builtin_bit_cast(u32x4, b);
    if (out_rm && r + j < rows) *(u32x4*)(out_rm + (long)(r + j) * ld_rm + c) = pk[j];
  }
  if (colpart && r0 < rows) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sum[k] += __shfl_xor(sum[k], 1, 64);
      sum[k] += __shfl_xor(sum[k], 2, 64);
      sum[k] += __shfl_xor(sum[k], 4, 64);
    }
    if ((lane & 7) == 0) {
      float* dst = colpart + (long)blockIdx.y * cols + c;
      *(f32x4*)dst = f32x4{sum[0], sum[1], sum[2], sum[3]};
      *(f32x4*)(dst + 4) = f32x4{sum[4], sum[5], sum[6], sum[7]};
    }
  }
  if (out_t && r < rows_pad) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned sel = (i & 1) ? 0x07060302u : 0x05040100u;
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) o[d] = __builtin_amdgcn_perm(pk[2 * d + 1][i >> 1], pk[2 * d][i >> 1], sel);
      *(u32x4*)(out_t + (long)(c + i) * rows_pad + r) = o;
    }
  }
}

template <int OP, typename Tin, typename Tout>
hipError_t fused_t(int rows, int cols, int rows_pad, const Tin* in, long ld_in, const float* aux, long ld_aux,
                   Tout* out_rm, long ld_rm, Tout* out_t, float* colpart, hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if constexpr (std::is_same<Tin, float>::value && std::is_same<Tout, bf16>::value) {
    auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    if (cols % 8 == 0 && rows_pad % 8 == 0 && ld_in % 4 == 0 && a16(in) && (OP != kDtPre || (ld_aux % 4 == 0 && a16(aux))) &&
        (!out_rm || (ld_rm % 8 == 0 && a16(out_rm))) && (!out_t || a16(out_t)) && (!colpart || a16(colpart))) {
      const int ry16 = ((out_t ? rows_pad : rows) + 63) / 64;
      hipLaunchKernelGGL((fused_t16_kernel<OP>), dim3((cols + 255) / 256, ry16), dim3(256), 0, st, rows, cols, rows_pad,
                         in, ld_in, aux, ld_aux, out_rm, ld_rm, out_t, colpart);
      return hipGetLastError();
    }
  }
  const int ry = ((out_t ? rows_pad : rows) + 63) / 64;
  hipLaunchKernelGGL((fused_t_kernel<OP, Tin, Tout>), dim3((cols + 63) / 64, ry), dim3(256), 0, st, rows, cols,
                     rows_pad, in, ld_in, aux, ld_aux, out_rm, ld_rm, out_t, colpart);
  return hipGetLastError();
}
#define R2L_FT(OP, TI, TO)                                                                                     \
  template hipError_t fused_t<OP, TI, TO>(int, int, int, const TI*, long, const float*, long, TO*, long, TO*, \
                                          float*, hipStream_t);
R2L_FT(kConvert, float, bf16) R2L_FT(kConvert, float, float) R2L_FT(kDtPre, float, bf16) R2L_FT(kDtPre, float, float)
#undef R2L_FT

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
// LayerNorm + gate backward (D a multiple of 64).
//   h+ = h + th r, r = gamma xhat + beta, xhat = (o - mu) / sigma, th = tanh(s):
//   do = th / sigma (gamma g - mean(gamma g) - xhat mean(gamma g xhat));
//   part[block] = sum over the block's rows of th [g xhat | g] (f32 [2D]; the
//   partials, summed over blocks in order, are d gamma and d beta);
//   gr[t] = (1 - th^2) sum_d g r (summed over t, d s).
// Without the LayerNorm r = o: do = th g, and part is not written.
// A block walks kLnRowsPerBlock rows; each of its waves owns a quarter of
// the columns (lane: columns q + 64 i + lane), so the per-column sums stay in
// a few registers.  The row statistics are summed over the lanes, then over
// the four waves through LDS in a fixed order (three rounds per row).
// ---------------------------------------------------------------------------
constexpr int kLnRowsPerBlock = 16;

template <typename T, int VPL>
__global__ __launch_bounds__(256) void ln_gate_bwd_kernel(int Tn, int D, const T* __restrict__ g, const float* __restrict__ o,
                                                          const float* __restrict__ gamma, const float* __restrict__ beta,
                                                          const float* __restrict__ s, int no_ln, float eps,
                                                          float* __restrict__ dout, float* __restrict__ part,
                                                          float* __restrict__ gr) {
  __shared__ float red[3][4][4];
  const int lane = lane_id(), w = wave_id();
  const int cw = D / 4;                       // columns per wave (a multiple of 16)
  const int q0 = w * cw;                      // this wave's first column
  const int row0 = blockIdx.x * kLnRowsPerBlock;
  const float th = tanhf(s[0]);
  const float invD = 1.0f / (float)D;
  float gm[VPL], bt[VPL], ax[VPL], ag[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int dd = q0 + i * 64 + lane;
    const bool ok = !no_ln && i * 64 + lane < cw;
    gm[i] = ok ? gamma[dd] : 0.0f;
    bt[i] = ok ? beta[dd] : 0.0f;
    ax[i] = ag[i] = 0.0f;
  }
  // the four waves' partial sums of one statistic, added in wave order
  auto block_sum = [&](int slot, int k, float v) __attribute__((always_inline)) {
    v = wave_sum(v);
    if (lane == 0) red[slot][w][k] = v;
    __syncthreads();
    return ((red[slot][0][k] + red[slot][1][k]) + red[slot][2][k]) + red[slot][3][k];
  };
  const int nrows = min(kLnRowsPerBlock, Tn - row0);
  for (int k = 0; k < nrows; ++k) {
    const int row = row0 + k;
    float x[VPL], gg[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int dd = q0 + i * 64 + lane;
      const bool ok = i * 64 + lane < cw;
      x[i] = ok ? o[(long)row * D + dd] : 0.0f;
      gg[i] = ok ? to_f32(g[(long)row * D + dd]) : 0.0f;
    }
    if (no_ln) {
      float p = 0.0f;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (i * 64 + lane < cw) {
          dout[(long)row * D + q0 + i * 64 + lane] = th * gg[i];
          p = fmaf(gg[i], x[i], p);
        }
      p = block_sum(0, 0, p);
      if (threadIdx.x == 0) gr[row] = (1.0f - th * th) * p;
      __syncthreads();   // red is rewritten by the next row
      continue;
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) sum += x[i];
    const float mu = block_sum(0, 0, sum) * invD;
    float sq = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      x[i] = i * 64 + lane < cw ? x[i] - mu : 0.0f;
      sq = fmaf(x[i], x[i], sq);
    }
    const float rstd = 1.0f / sqrtf(block_sum(1, 0, sq) * invD + eps);
    float m1 = 0.0f, m2 = 0.0f, p = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      x[i] *= rstd;                                    // xhat
      const float gg_gamma = gg[i] * gm[i];
      m1 += gg_gamma;
      m2 = fmaf(gg_gamma, x[i], m2);
      p = fmaf(gg[i], fmaf(gm[i], x[i], bt[i]), p);
      ax[i] = fmaf(th * gg[i], x[i], ax[i]);
      ag[i] = fmaf(th, gg[i], ag[i]);
    }
    // three statistics in one round: slot 2, entries 0..2
    m1 = wave_sum(m1);
    m2 = wave_sum(m2);
    p = wave_sum(p);
    if (lane == 0) { red[2][w][0] = m1; red[2][w][1] = m2; red[2][w][2] = p; }
    __syncthreads();
    m1 = (((red[2][0][0] + red[2][1][0]) + red[2][2][0]) + red[2][3][0]) * invD;
    m2 = (((red[2][0][1] + red[2][1][1]) + red[2][2][1]) + red[2][3][1]) * invD;
    p = ((red[2][0][2] + red[2][1][2]) + red[2][2][2]) + red[2][3][2];
    if (threadIdx.x == 0) gr[row] = (1.0f - th * th) * p;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (i * 64 + lane < cw) dout[(long)row * D + q0 + i * 64 + lane] = th * rstd * (gg[i] * gm[i] - m1 - x[i] * m2);
    // (slot 0 is rewritten by the next row only after every wave has passed
    // that row's first round, i.e. after all reads of this row's slot 2)
  }
  if (!no_ln && nrows > 0) {
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (i * 64 + lane < cw) {
        const int dd = q0 + i * 64 + lane;
        part[(long)blockIdx.x * 2 * D + dd] = ax[i];
        part[(long)blockIdx.x * 2 * D + D + dd] = ag[i];
      }
  }
}

int ln_bwd_parts(int Tn) { return (Tn + kLnRowsPerBlock - 1) / kLnRowsPerBlock; }

// The same for bf16 g and D a multiple of 512 (16-byte aligned rows): a block
// is one wave and walks the same kLnRowsPerBlock rows; lane l owns columns
// 512 c + 8 l .. +7 of every 512-column chunk c, read and written in 16-byte
// (g) and 32-byte (o, dout) pieces.  Row statistics are wave sums (no block
// barriers); the per-column sums stay in the lane's registers and leave as
// the block's partial row, as above.
template <int NC>
__global__ __launch_bounds__(64) void ln_gate_bwd16_kernel(int Tn, int D, const bf16* __restrict__ g,
                                                           const float* __restrict__ o,
                                                           const float* __restrict__ gamma,
                                                           const float* __restrict__ beta,
                                                           const float* __restrict__ s, int no_ln, float eps,
                                                           float* __restrict__ dout, float* __restrict__ part,
                                                           float* __restrict__ gr) {
  constexpr int V = 8 * NC;   // columns per lane
  const int lane = lane_id();
  const int row0 = blockIdx.x * kLnRowsPerBlock;
  const float th = tanhf(s[0]);
  const float invD = 1.0f / (float)D;
  auto col = [&](int c) { return 512 * c + 8 * lane; };
  float gm[V], bt[V], ax[V], ag[V];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 a = no_ln ? f32x4{} : *(const f32x4*)(gamma + col(c) + 4 * h);
      const f32x4 b = no_ln ? f32x4{} : *(const f32x4*)(beta + col(c) + 4 * h);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        gm[8 * c + 4 * h + k] = a[k];
        bt[8 * c + 4 * h + k] = b[k];
        ax[8 * c + 4 * h + k] = ag[8 * c + 4 * h + k] = 0.0f;
      }
    }
  const int nrows = min(kLnRowsPerBlock, Tn - row0);
  for (int k = 0; k < nrows; ++k) {
    const long row = row0 + k;
    float x[V], gg[V];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const f32x4 a0 = *(const f32x4*)(o + row * D + col(c));
      const f32x4 a1 = *(const f32x4*)(o + row * D + col(c) + 4);
      const bf16x8 gv = *(const bf16x8*)(g + row * D + col(c));
#pragma unroll
      for (int i = 0; i < 4; ++i) { x[8 * c + i] = a0[i]; x[8 * c + 4 + i] = a1[i]; }
#pragma unroll
      for (int i = 0; i < 8; ++i) gg[8 * c + i] = (float)gv[i];
    }
    float dv[V];
    if (no_ln) {
      float p = 0.0f;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        dv[i] = th * gg[i];
        p = fmaf(gg[i], x[i], p);
      }
      p = wave_sum(p);
      if (lane == 0) gr[row] = (1.0f - th * th) * p;
    } else {
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < V; ++i) sum += x[i];
      const float mu = wave_sum(sum) * invD;
      float sq = 0.0f;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        x[i] -= mu;
        sq = fmaf(x[i], x[i], sq);
      }
      const float rstd = 1.0f / sqrtf(wave_sum(sq) * invD + eps);
      float m1 = 0.0f, m2 = 0.0f, p = 0.0f;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        x[i] *= rstd;                                  // xhat
        const float gg_gamma = gg[i] * gm[i];
        m1 += gg_gamma;
        m2 = fmaf(gg_gamma, x[i], m2);
        p = fmaf(gg[i], fmaf(gm[i], x[i], bt[i]), p);
        ax[i] = fmaf(th * gg[i], x[i], ax[i]);
        ag[i] = fmaf(th, gg[i], ag[i]);
      }
      m1 = wave_sum(m1) * invD;
      m2 = wave_sum(m2) * invD;
      p = wave_sum(p);
      if (lane == 0) gr[row] = (1.0f - th * th) * p;
#pragma unroll
      for (int i = 0; i < V; ++i) dv[i] = th * rstd * (gg[i] * gm[i] - m1 - x[i] * m2);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      *(f32x4*)(dout + row * D + col(c)) = f32x4{dv[8 * c], dv[8 * c + 1], dv[8 * c + 2], dv[8 * c + 3]};
      *(f32x4*)(dout + row * D + col(c) + 4) = f32x4{dv[8 * c + 4], dv[8 * c + 5], dv[8 * c + 6], dv[8 * c + 7]};
    }
  }
  if (!no_ln && nrows > 0) {
    float* pa = part + (long)blockIdx.x * 2 * D;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i0 = 8 * c + 4 * h;
        *(f32x4*)(pa + col(c) + 4 * h) = f32x4{ax[i0], ax[i0 + 1], ax[i0 + 2], ax[i0 + 3]};
        *(f32x4*)(pa + D + col(c) + 4 * h) = f32x4{ag[i0], ag[i0 + 1], ag[i0 + 2], ag[i0 + 3]};
      }
  }
}

template <typename T>
hipError_t ln_gate_bwd(int Tn, int D, const T* g, const float* o, const float* gamma, const float* beta,
                       const float* s, bool no_ln, float eps, float* dout, float* part, float* gr, hipStream_t st) {
  if (Tn <= 0) return hipSuccess;
  dim3 grid(ln_bwd_parts(Tn)), block(256);
  const int cnt = (D / 4 + 63) / 64, nl = no_ln ? 1 : 0;   // columns per lane
  if constexpr (std::is_same<T, bf16>::value) {
    auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    const int nc = D / 512;
    if (D % 512 == 0 && nc <= 4 && a16(g) && a16(o) && a16(dout) && a16(part) &&
        (no_ln || (a16(gamma) && a16(beta)))) {
#define R2L_LNB16(C)                                                                                             \
  hipLaunchKernelGGL((ln_gate_bwd16_kernel<C>), grid, dim3(64), 0, st, Tn, D, g, o, gamma, beta, s, nl, eps, dout, \
                     part, gr)
      if (nc == 1) R2L_LNB16(1);
      else if (nc == 2) R2L_LNB16(2);
      else if (nc == 3) R2L_LNB16(3);
      else R2L_LNB16(4);
#undef R2L_LNB16
      return hipGetLastError();
    }
  }
#define R2L_LNB(V) \
  hipLaunchKernelGGL((ln_gate_bwd_kernel<T, V>), grid, block, 0, st, Tn, D, g, o, gamma, beta, s, nl, eps, dout, part, gr)
  if (cnt <= 1) R2L_LNB(1);
  else if (cnt <= 4) R2L_LNB(4);
  else if (cnt <= 8) R2L_LNB(8);
  else if (cnt <= 16) R2L_LNB(16);
  else R2L_LNB(32);
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
// db = sum_t dc_t.
//
// A block owns 64 channels (lane = channel) of a contiguous range of rows,
// split into four consecutive runs, one per wave.  Each wave walks its run
// top to bottom with the conv window (x_t .. x_{t+3}) and the last three dc
// values in registers: dx_t needs dc_t .. dc_{t-3}, so dc is never stored.
// The three dc values before the run are recomputed.  The current sequence's
// bounds advance with the walk (offsets are sanitised: non-decreasing, from 0
// to the token count).  The tap and bias gradients are summed per lane, then
// over the four waves in a fixed order, into per-block partials [nb][E][K+1]
// that a second kernel adds in block order.
// ---------------------------------------------------------------------------
template <typename T, typename TO>
__global__ __launch_bounds__(256) void conv_bwd_kernel(int Tn, int E, const T* __restrict__ x, long ld_x,
                                                       const T* __restrict__ cw, const T* __restrict__ cb,
                                                       const float* __restrict__ du, const float* __restrict__ du2,
                                                       TO* __restrict__ dx, long ld_dx, float* __restrict__ part,
                                                       const int32_t* __restrict__ cu, int nseq) {
  const int nb = gridDim.y, b = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const long r0 = (long)Tn * b / nb, r1 = (long)Tn * (b + 1) / nb;
  const int ra = (int)(r0 + (r1 - r0) * wv / 4), rz = (int)(r0 + (r1 - r0) * (wv + 1) / 4);
  float w[KC_];
#pragma unroll
  for (int k = 0; k < KC_; ++k) w[k] = to_f32(cw[(long)e * KC_ + k]);
  const float bias = to_f32(cb[e]);
  auto xat = [&](int t) __attribute__((always_inline)) {
    return t < Tn ? to_f32(x[(long)t * ld_x + e]) : 0.0f;
  };
  auto gat = [&](int t) __attribute__((always_inline)) {
    const long i = (long)t * E + e;
    return du2 ? du[i] + du2[i] : du[i];
  };
  // dc_t from the window x_t .. x_{t+3}, n = rows of it inside the sequence (>= 1)
  auto dc_of = [&](float g, float x0, float x1, float x2, float x3, int n) __attribute__((always_inline)) {
    float c = fmaf(w[KC_ - 1], x0, bias);
    c = fmaf(w[KC_ - 2], n > 1 ? x1 : 0.0f, c);
    c = fmaf(w[KC_ - 3], n > 2 ? x2 : 0.0f, c);
    c = fmaf(w[KC_ - 4], n > 3 ? x3 : 0.0f, c);
    const float sg = sigmoid_fast(c);
    return g * sg * fmaf(c, 1.0f - sg, 1.0f);
  };
  float acc[KC_ + 1] = {};
  if (ra < rz) {
    int q = 0;
    {
      int lo = 0, hi = nseq;   // the last q with cu[q] <= ra
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= ra) lo = mid; else hi = mid;
      }
      q = lo;
    }
    int sl = cu[q], se = max(cu[q + 1], ra + 1);
    // dc of the three rows before the run, when they are in the same sequence
    float d1 = 0.0f, d2 = 0.0f, d3 = 0.0f;
    {
      float xs[6];
#pragma unroll
      for (int i = 0; i < 6; ++i) xs[i] = ra - 3 + i >= sl ? xat(ra - 3 + i) : 0.0f;
      if (ra - 1 >= sl) d1 = dc_of(gat(ra - 1), xs[2], xs[3], xs[4], xs[5], se - (ra - 1));
      if (ra - 2 >= sl) d2 = dc_of(gat(ra - 2), xs[1], xs[2], xs[3], xs[4], se - (ra - 2));
      if (ra - 3 >= sl) d3 = dc_of(gat(ra - 3), xs[0], xs[1], xs[2], xs[3], se - (ra - 3));
    }
    float x0 = xat(ra), x1 = xat(ra + 1), x2 = xat(ra + 2);
    auto step = [&](int t, float g, float x3) __attribute__((always_inline)) {
      const int n = se - t;
      const float d = dc_of(g, x0, x1, x2, x3, n);
      const float v = fmaf(w[KC_ - 1], d, fmaf(w[KC_ - 2], d1, fmaf(w[KC_ - 3], d2, w[KC_ - 4] * d3)));
      dx[(long)t * ld_dx + e] = from_f32<TO>(v);
      acc[KC_ - 1] = fmaf(d, x0, acc[KC_ - 1]);
      acc[KC_ - 2] = fmaf(d, n > 1 ? x1 : 0.0f, acc[KC_ - 2]);
      acc[KC_ - 3] = fmaf(d, n > 2 ? x2 : 0.0f, acc[KC_ - 3]);
      acc[KC_ - 4] = fmaf(d, n > 3 ? x3 : 0.0f, acc[KC_ - 4]);
      acc[KC_] += d;
      d3 = d2; d2 = d1; d1 = d;
      x0 = x1; x1 = x2; x2 = x3;
    };
    int t = ra;
    while (t < rz) {
      if (t >= se) {   // next non-empty sequence; the dc history starts over
        while (q + 1 < nseq && cu[q + 1] <= t) ++q;
        sl = cu[q];
        // (rows past the last offset, which valid offsets never leave, are
        // taken one at a time)
        se = max(cu[q + 1], t + 1);
        d1 = d2 = d3 = 0.0f;
      }
      if (t + 4 <= rz && t + 4 <= se) {
        // four rows of one sequence: every load first
        float xn[4], gn[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) { xn[i] = xat(t + 3 + i); gn[i] = gat(t + i); }
#pragma unroll
        for (int i = 0; i < 4; ++i) step(t + i, gn[i], xn[i]);
        t += 4;
      } else {
        step(t, gat(t), xat(t + 3));
        t += 1;
      }
    }
  }
  __shared__ float red[4][KC_ + 1][64];
#pragma unroll
  for (int k = 0; k <= KC_; ++k) red[wv][k][lane] = acc[k];
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int k = 0; k <= KC_; ++k)
      part[((long)b * E + e) * (KC_ + 1) + k] = ((red[0][k][lane] + red[1][k][lane]) + red[2][k][lane]) + red[3][k][lane];
  }
}

// The same walk for bf16 with 8 channels per lane (E a multiple of 512;
// x, dx, du, du2 and the taps 16-byte aligned, ld_x and ld_dx multiples of
// 8): a wave covers 512 channels of its run of rows, every access a 16- or
// 32-byte piece of a token row.  The control flow (rows, sequence bounds) is
// the wave's as above; per channel the arithmetic is the same, in the same
// order, so dx and the partial sums are the same bits.
__global__ __launch_bounds__(256) void conv_bwd16_kernel(int Tn, int E, const bf16* __restrict__ x, long ld_x,
                                                         const bf16* __restrict__ cw, const bf16* __restrict__ cb,
                                                         const float* __restrict__ du, const float* __restrict__ du2,
                                                         bf16* __restrict__ dx, long ld_dx, float* __restrict__ part,
                                                         const int32_t* __restrict__ cu, int nseq) {
  constexpr int C = 8;
  const int nb = gridDim.y, b = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = (blockIdx.x * 64 + lane) * C;   // the lane's first channel
  const long r0 = (long)Tn * b / nb, r1 = (long)Tn * (b + 1) / nb;
  const int ra = (int)(r0 + (r1 - r0) * wv / 4), rz = (int)(r0 + (r1 - r0) * (wv + 1) / 4);
  float w[C][KC_], bias[C];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x8 tv = *(const bf16x8*)(cw + (long)e * KC_ + 8 * q);   // taps of channels e + 2q, e + 2q + 1
#pragma unroll
    for (int k = 0; k < 8; ++k) w[2 * q + k / KC_][k % KC_] = (float)tv[k];
  }
  {
    const bf16x8 bv = *(const bf16x8*)(cb + e);
#pragma unroll
    for (int c = 0; c < C; ++c) bias[c] = (float)bv[c];
  }
  typedef float fv8 __attribute__((ext_vector_type(8)));
  auto xat = [&](int t) __attribute__((always_inline)) {
    fv8 v = {};
    if (t < Tn) {
      const bf16x8 q = *(const bf16x8*)(x + (long)t * ld_x + e);
#pragma unroll
      for (int c = 0; c < C; ++c) v[c] = (float)q[c];
    }
    return v;
  };
  auto gat = [&](int t) __attribute__((always_inline)) {
    const long i = (long)t * E + e;
    const f32x4 a0 = *(const f32x4*)(du + i), a1 = *(const f32x4*)(du + i + 4);
    fv8 v = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    if (du2) {
      const f32x4 b0 = *(const f32x4*)(du2 + i), b1 = *(const f32x4*)(du2 + i + 4);
      const fv8 u = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int c = 0; c < C; ++c) v[c] = v[c] + u[c];
    }
    return v;
  };
  // dc of channel c at t from the window x_t .. x_{t+3}, n = rows of it inside the sequence (>= 1)
  auto dc_of = [&](int c, float g, float x0, float x1, float x2, float x3, int n) __attribute__((always_inline)) {
    float cc = fmaf(w[c][KC_ - 1], x0, bias[c]);
    cc = fmaf(w[c][KC_ - 2], n > 1 ? x1 : 0.0f, cc);
    cc = fmaf(w[c][KC_ - 3], n > 2 ? x2 : 0.0f, cc);
    cc = fmaf(w[c][KC_ - 4], n > 3 ? x3 : 0.0f, cc);
    const float sg = sigmoid_fast(cc);
    return g * sg * fmaf(cc, 1.0f - sg, 1.0f);
  };
  float acc[C][KC_ + 1];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int k = 0; k <= KC_; ++k) acc[c][k] = 0.0f;
  if (ra < rz) {
    int q = 0;
    {
      int lo = 0, hi = nseq;   // the last q with cu[q] <= ra
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= ra) lo = mid; else hi = mid;
      }
      q = lo;
    }
    int sl = cu[q], se = max(cu[q + 1], ra + 1);
    fv8 d1 = {}, d2 = {}, d3 = {};
    {
      fv8 xs[6];
#pragma unroll
      for (int i = 0; i < 6; ++i) xs[i] = ra - 3 + i >= sl ? xat(ra - 3 + i) : fv8{};
      if (ra - 1 >= sl) {
        const fv8 g = gat(ra - 1);
#pragma unroll
        for (int c = 0; c < C; ++c) d1[c] = dc_of(c, g[c], xs[2][c], xs[3][c], xs[4][c], xs[5][c], se - (ra - 1));
      }
      if (ra - 2 >= sl) {
        const fv8 g = gat(ra - 2);
#pragma unroll
        for (int c = 0; c < C; ++c) d2[c] = dc_of(c, g[c], xs[1][c], xs[2][c], xs[3][c], xs[4][c], se - (ra - 2));
      }
      if (ra - 3 >= sl) {
        const fv8 g = gat(ra - 3);
#pragma unroll
        for (int c = 0; c < C; ++c) d3[c] = dc_of(c, g[c], xs[0][c], xs[1][c], xs[2][c], xs[3][c], se - (ra - 3));
      }
    }
    fv8 x0 = xat(ra), x1 = xat(ra + 1), x2 = xat(ra + 2);
    auto step = [&](int t, const fv8& g, const fv8& x3) __attribute__((always_inline)) {
      const int n = se - t;
      bf16x8 o;
      fv8 d;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        d[c] = dc_of(c, g[c], x0[c], x1[c], x2[c], x3[c], n);
        const float v = fmaf(w[c][KC_ - 1], d[c], fmaf(w[c][KC_ - 2], d1[c], fmaf(w[c][KC_ - 3], d2[c], w[c][KC_ - 4] * d3[c])));
        o[c] = from_f32<bf16>(v);
        acc[c][KC_ - 1] = fmaf(d[c], x0[c], acc[c][KC_ - 1]);
        acc[c][KC_ - 2] = fmaf(d[c], n > 1 ? x1[c] : 0.0f, acc[c][KC_ - 2]);
        acc[c][KC_ - 3] = fmaf(d[c], n > 2 ? x2[c] : 0.0f, acc[c][KC_ - 3]);
        acc[c][KC_ - 4] = fmaf(d[c], n > 3 ? x3[c] : 0.0f, acc[c][KC_ - 4]);
        acc[c][KC_] += d[c];
      }
      *(bf16x8*)(dx + (long)t * ld_dx + e) = o;
      d3 = d2; d2 = d1; d1 = d;
      x0 = x1; x1 = x2; x2 = x3;
    };
    int t = ra;
    while (t < rz) {
      if (t >= se) {   // next non-empty sequence; the dc history starts over
        while (q + 1 < nseq && cu[q + 1] <= t) ++q;
        sl = cu[q];
        se = max(cu[q + 1], t + 1);
        d1 = d2 = d3 = fv8{};
      }
      if (t + 2 <= rz && t + 2 <= se) {
        // two rows of one sequence: every load first
        const fv8 xa = xat(t + 3), xb = xat(t + 4), ga = gat(t), gb = gat(t + 1);
        step(t, ga, xa);
        step(t + 1, gb, xb);
        t += 2;
      } else {
        step(t, gat(t), xat(t + 3));
        t += 1;
      }
    }
  }
  __shared__ float red[4][KC_ + 1][64 * C];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int k = 0; k <= KC_; ++k) red[wv][k][lane * C + c] = acc[c][k];
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int k = 0; k <= KC_; ++k)
        part[((long)b * E + e + c) * (KC_ + 1) + k] =
            ((red[0][k][lane * C + c] + red[1][k][lane * C + c]) + red[2][k][lane * C + c]) + red[3][k][lane * C + c];
  }
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

// row blocks: about 64 rows per wave, at most 1024 blocks of rows
int conv_bwd_parts(int Tn) { return Tn < 256 ? 1 : (Tn / 256 < 1024 ? Tn / 256 : 1024); }

template <typename T>
hipError_t conv_bwd(int Tn, int E, const T* x, long ld_x, const T* cw, const T* cb, const float* du, const float* du2,
                    T* dx, long ld_dx, float* part, float* dw, float* db, const int32_t* cu, int nseq,
                    hipStream_t st) {
  if (Tn <= 0) return hipSuccess;
  const int nb = conv_bwd_parts(Tn);
  bool wide = false;
  if constexpr (std::is_same<T, bf16>::value) {
    auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    wide = E % 512 == 0 && ld_x % 8 == 0 && ld_dx % 8 == 0 && a16(x) && a16(dx) && a16(du) && (!du2 || a16(du2)) &&
           a16(cw) && a16(cb);
    if (wide)
      hipLaunchKernelGGL(conv_bwd16_kernel, dim3(E / 512, nb), dim3(256), 0, st, Tn, E, x, ld_x, cw, cb, du, du2, dx,
                         ld_dx, part, cu, nseq);
  }
  if (!wide)
    hipLaunchKernelGGL((conv_bwd_kernel<T, T>), dim3(E / 64, nb), dim3(256), 0, st, Tn, E, x, ld_x, cw, cb, du, du2,
                       dx, ld_dx, part, cu, nseq);
  hipLaunchKernelGGL(conv_wsum_kernel, dim3((E * (KC_ + 1) + 255) / 256), dim3(256), 0, st, E, nb,
                     (const float*)part, dw, db);
  return hipGetLastError();
}
template hipError_t conv_bwd<float>(int, int, const float*, long, const float*, const float*, const float*,
                                    const float*, float*, long, float*, float*, float*, const int32_t*, int,
                                    hipStream_t);
template hipError_t conv_bwd<bf16>(int, int, const bf16*, long, const bf16*, const bf16*, const float*, const float*,
                                   bf16*, long, float*, float*, float*, const int32_t*, int, hipStream_t);

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

namespace r2l {

// ---------------------------------------------------------------------------
// Per-sequence row reversal: row t of sequence [s, e) <-> row s + e - 1 - t.
// The backward of the left-to-right layer is the default layer's backward
// on every sequence reversed, reversed back (the layer seen in the other
// direction).  Sequence lookups are clamped (seq_start_of / seq_end_of), so
// malformed offsets stay in bounds.  in_place: out == in, each pair swapped
// once by the row of the pair that comes first.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void flip_rows_kernel(int Tn, int cols, const T* in, long ld_in, T* out,
                                                        long ld_out, const int32_t* __restrict__ cu, int nseq,
                                                        int in_place) {
  for (int t = blockIdx.x; t < Tn; t += gridDim.x) {
    const int s = seq_start_of(cu, nseq, t), e = seq_end_of(cu, nseq, t, Tn);
    const int m = s + e - 1 - t;
    if (m < 0 || m >= Tn) continue;
    if (in_place) {
      if (t >= m) continue;
      for (int c = threadIdx.x; c < cols; c += 256) {
        const T a = out[(long)t * ld_out + c], b = out[(long)m * ld_out + c];
        out[(long)t * ld_out + c] = b;
        out[(long)m * ld_out + c] = a;
      }
    } else {
      for (int c = threadIdx.x; c < cols; c += 256) out[(long)t * ld_out + c] = in[(long)m * ld_in + c];
    }
  }
}

template <typename T>
hipError_t flip_rows(int Tn, int cols, const T* in, long ld_in, T* out, long ld_out, const int32_t* cu, int nseq,
                     hipStream_t st) {
  if (Tn <= 0 || cols <= 0) return hipSuccess;
  const int blocks = Tn < 16384 ? Tn : 16384;
  hipLaunchKernelGGL((flip_rows_kernel<T>), dim3(blocks), dim3(256), 0, st, Tn, cols, in, ld_in, out, ld_out, cu,
                     nseq, in == out ? 1 : 0);
  return hipGetLastError();
}
template hipError_t flip_rows<float>(int, int, const float*, long, float*, long, const int32_t*, int, hipStream_t);
template hipError_t flip_rows<bf16>(int, int, const bf16*, long, bf16*, long, const int32_t*, int, hipStream_t);

}  // namespace r2l
