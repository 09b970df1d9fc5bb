// Dense projections C = A . B^T (in_proj and out_proj of the Mamba-1 block,
// "Bifocal Diffusion Language Models", §3.4 step 2).
//
// bf16: MFMA v_mfma_f32_32x32x16_bf16 on gfx950.  A block of 256 threads
// (4 waves, 2 x 2) computes a BM x BN tile; each wave owns a (BM/2) x (BN/2)
// sub-tile made of 32 x 32 MFMA tiles.  Both operands are K-contiguous, so a
// lane's MFMA fragment (8 consecutive k of one row) is one 16-byte LDS read.
// K is walked in BK = 64 steps through a double-buffered LDS tile; the next
// step's global loads are issued into registers before the current step's
// MFMAs.  Rows of the LDS tiles are padded by 16 bytes so that the 32 rows a
// fragment read touches spread over the banks.  Block indices are remapped so
// that each XCD works on a contiguous, group-M-ordered range of tiles.
#include "kernels.h"

namespace r2l {

template <int BM, int BN, bool OUT_F32>
__global__ __launch_bounds__(256, 1) void gemm_bf16_nt_kernel(int M, int N, int K,
                                                              const bf16* __restrict__ A, long lda,
                                                              const bf16* __restrict__ B, long ldb,
                                                              void* __restrict__ Cv, long ldc) {
  constexpr int BK = 64;
  constexpr int LS = BK + 8;                 // LDS row stride (bf16 elements)
  constexpr int WM = BM / 2, WN = BN / 2;    // wave tile
  constexpr int SM = WM / 32, SN = WN / 32;  // 32x32 MFMA tiles per wave
  constexpr int CPR = BK / 8;                // 16-byte chunks per tile row
  constexpr int AC = BM * CPR / 256, BC = BN * CPR / 256;
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * LS];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * LS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
  const int nTm = (M + BM - 1) / BM, nTn = (N + BN - 1) / BN;
  const int lid = xcd_remap(blockIdx.x, nTm * nTn);
  constexpr int G = 8;
  const int per_group = G * nTn;
  const int first_m = (lid / per_group) * G;
  const int gsz = min(nTm - first_m, G);
  const int tm = first_m + (lid % per_group) % gsz;
  const int tn = (lid % per_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  i32x4 ra[AC], rb[BC];
  const i32x4 zero4 = {0, 0, 0, 0};

#define R2L_GLOAD(k0)                                                              \
  _Pragma("unroll") for (int i = 0; i < AC; ++i) {                                 \
    const int c = tid + 256 * i, row = c / CPR, col = (c % CPR) * 8;               \
    const int gm = m0 + row, gk = (k0) + col;                                      \
    ra[i] = (gm < M && gk < K) ? *(const i32x4*)(A + (long)gm * lda + gk) : zero4; \
  }                                                                                \
  _Pragma("unroll") for (int i = 0; i < BC; ++i) {                                 \
    const int c = tid + 256 * i, row = c / CPR, col = (c % CPR) * 8;               \
    const int gn = n0 + row, gk = (k0) + col;                                      \
    rb[i] = (gn < N && gk < K) ? *(const i32x4*)(B + (long)gn * ldb + gk) : zero4; \
  }
#define R2L_SSTORE(buf)                                                 \
  _Pragma("unroll") for (int i = 0; i < AC; ++i) {                      \
    const int c = tid + 256 * i, row = c / CPR, col = (c % CPR) * 8;    \
    *(i32x4*)(&As[buf][row * LS + col]) = ra[i];                        \
  }                                                                     \
  _Pragma("unroll") for (int i = 0; i < BC; ++i) {                      \
    const int c = tid + 256 * i, row = c / CPR, col = (c % CPR) * 8;    \
    *(i32x4*)(&Bs[buf][row * LS + col]) = rb[i];                        \
  }

  f32x16 acc[SM][SN];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Pipeline: on entry to iteration kt, LDS buffer kt%2 holds tile kt and the
  // registers hold tile kt+1.  The registers go to the other LDS buffer first
  // (that buffer's last readers finished before the previous barrier), then
  // the loads of tile kt+2 are issued, then tile kt's MFMAs run.
  const int nk = (K + BK - 1) / BK;
  R2L_GLOAD(0);
  R2L_SSTORE(0);
  if (nk > 1) { R2L_GLOAD(BK); }
  __syncthreads();
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) { R2L_SSTORE(cur ^ 1); }
    if (kt + 2 < nk) { R2L_GLOAD((kt + 2) * BK); }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[SM], bfr[SN];
#pragma unroll
      for (int i = 0; i < SM; ++i)
        af[i] = *(const bf16x8*)(&As[cur][(wm + 32 * i + fr) * LS + ks * 16 + fk]);
#pragma unroll
      for (int j = 0; j < SN; ++j)
        bfr[j] = *(const bf16x8*)(&Bs[cur][(wn + 32 * j + fr) * LS + ks * 16 + fk]);
#pragma unroll
      for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#undef R2L_GLOAD
#undef R2L_SSTORE

  // D tile layout: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4.
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int n = n0 + wn + 32 * j + fr;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M) {
          if (OUT_F32) ((float*)Cv)[(long)m * ldc + n] = acc[i][j][r];
          else ((bf16*)Cv)[(long)m * ldc + n] = (bf16)acc[i][j][r];
        }
      }
    }
}

template <int BM, int BN>
static void launch_gemm(int M, int N, int K, const bf16* A, long lda, const bf16* B, long ldb,
                        void* C, long ldc, bool out_f32, hipStream_t st) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (out_f32)
    hipLaunchKernelGGL((gemm_bf16_nt_kernel<BM, BN, true>), dim3(tiles), dim3(256), 0, st, M, N, K,
                       A, lda, B, ldb, C, ldc);
  else
    hipLaunchKernelGGL((gemm_bf16_nt_kernel<BM, BN, false>), dim3(tiles), dim3(256), 0, st, M, N,
                       K, A, lda, B, ldb, C, ldc);
}

hipError_t gemm_bf16_nt(int M, int N, int K, const bf16* A, long lda, const bf16* B, long ldb,
                        void* C, long ldc, bool out_f32, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  // 128 x 128 tiles (4 waves of 64 x 64, two blocks per CU) measured fastest
  // on the layer's projection shapes; 256 x 256 (one block per CU) exposes
  // more latency than it saves in LDS traffic.
  launch_gemm<128, 128>(M, N, K, A, lda, B, ldb, C, ldc, out_f32, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 path: a plain LDS-tiled VALU GEMM (64 x 64 tile, 4 x 4 per thread).
// Used for the fp32 configuration only, where exact fp32 products matter
// more than speed.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_f32_nt_kernel(int M, int N, int K,
                                                          const float* __restrict__ A, long lda,
                                                          const float* __restrict__ B, long ldb,
                                                          float* __restrict__ C, long ldc) {
  __shared__ float As[16][64 + 4], Bs[16][64 + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i, r = idx >> 4, kk = idx & 15;
      const int gk = k0 + kk, gm = m0 + r, gn = n0 + r;
      As[kk][r] = (gm < M && gk < K) ? A[(long)gm * lda + gk] : 0.0f;
      Bs[kk][r] = (gn < N && gk < K) ? B[(long)gn * ldb + gk] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        b[i] = Bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < M && n < N) C[(long)m * ldc + n] = acc[i][j];
    }
}

hipError_t gemm_f32_nt(int M, int N, int K, const float* A, long lda, const float* B, long ldb,
                       float* C, long ldc, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL(gemm_f32_nt_kernel, grid, dim3(256), 0, st, M, N, K, A, lda, B, ldb, C, ldc);
  return hipGetLastError();
}

}  // namespace r2l
