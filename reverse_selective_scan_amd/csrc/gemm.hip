// Dense projections C = A . B^T (in_proj and out_proj of the Mamba-1 block,
// "Bifocal Diffusion Language Models", §3.4 step 2).
//
// bf16 kernels on the MFMA matrix cores (v_mfma_f32_32x32x16_bf16):
//
//  * gemm_bf16_big_kernel -- the large-problem kernel.  One block of 256
//    threads (one wave per SIMD) owns a 256 x 256 tile; each wave owns a
//    128 x 128 quarter (16 accumulator tiles, 256 AGPRs), so every 16-byte
//    LDS fragment read feeds four MFMAs.  K is walked in 32-wide steps
//    through four LDS stages filled directly from global memory by
//    buffer_load ... lds (no VGPR round trip; rows past M or N read as zero
//    through the buffer descriptor's range).  The block barrier of step kt
//    waits for step kt+1's data, so each wave can read the first fragments
//    of the next step before finishing the current one, and loads run two
//    steps ahead.  Stage rows are 64 bytes with a 16-byte-chunk XOR swizzle
//    so that fragment reads are bank-conflict free.  The MFMA operands are
//    swapped (B-tile rows as the "A" operand) so that each lane ends up with
//    4 consecutive output columns of one row: 8- or 16-byte stores.
//  * gemm_bf16_pers_kernel -- the big kernel made persistent for bf16
//    outputs (in_proj): one block per CU walks its tiles with the K-step
//    pipeline running on across tile boundaries, and writes each finished
//    tile (through LDS, a quarter at a time) while it computes the next one.
//  * gemm_bf16_mid_kernel -- the big kernel's pipeline on 128 x 128 tiles
//    (16 KB stages, two blocks per CU) for small problems and last tile rows.
//  * gemm_bf16_nt_kernel -- the general kernel (any shape with K a multiple
//    of 8): 128 x 128 tiles, 2 x 2 waves of 64 x 64, register-staged
//    double-buffered LDS tiles.
//
// Block indices are remapped so that each XCD works on a contiguous,
// group-M-ordered range of tiles (tiles that share operands share an L2).
#include <type_traits>

#include "kernels.h"

namespace r2l {

// splits == 0: block b computes a whole output tile into C.  splits > 0:
// block u computes K range [s kchunk, (s+1) kchunk) (s = u % splits) of tile
// u / splits (row-major tile order) as an fp32 partial sum into
// part[u][BM][BN]; gemm_small_reduce_kernel adds the partials.
template <int BM, int BN, bool OUT_F32>
__global__ __launch_bounds__(256, 1) void gemm_bf16_nt_kernel(int M, int N, int K,
                                                              const bf16* __restrict__ A, long lda,
                                                              const bf16* __restrict__ B, long ldb,
                                                              void* __restrict__ Cv, long ldc,
                                                              int splits, int kchunk,
                                                              float* __restrict__ part) {
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
  int tm, tn, kbeg = 0, kend = K;
  if (splits) {
    const int tile = blockIdx.x / splits, sp = blockIdx.x % splits;
    tm = tile / nTn;
    tn = tile % nTn;
    kbeg = sp * kchunk;
    kend = min(K, kbeg + kchunk);
  } else {
    const int lid = xcd_remap(blockIdx.x, nTm * nTn);
    constexpr int G = 8;
    const int per_group = G * nTn;
    const int first_m = (lid / per_group) * G;
    const int gsz = min(nTm - first_m, G);
    tm = first_m + (lid % per_group) % gsz;
    tn = (lid % per_group) / gsz;
  }
  const int m0 = tm * BM, n0 = tn * BN;

  i32x4 ra[AC], rb[BC];
  const i32x4 zero4 = {0, 0, 0, 0};

#define R2L_GLOAD(k0)                                                              \
  _Pragma("unroll") for (int i = 0; i < AC; ++i) {                                 \
    const int c = tid + 256 * i, row = c / CPR, col = (c % CPR) * 8;               \
    const int gm = m0 + row, gk = kbeg + (k0) + col;                               \
    ra[i] = (gm < M && gk < kend) ? *(const i32x4*)(A + (long)gm * lda + gk) : zero4; \
  }                                                                                \
  _Pragma("unroll") for (int i = 0; i < BC; ++i) {                                 \
    const int c = tid + 256 * i, row = c / CPR, col = (c % CPR) * 8;               \
    const int gn = n0 + row, gk = kbeg + (k0) + col;                               \
    rb[i] = (gn < N && gk < kend) ? *(const i32x4*)(B + (long)gn * ldb + gk) : zero4; \
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
  const int nk = (kend - kbeg + BK - 1) / BK;
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
  if (splits) {
    float* pt = part + (long)blockIdx.x * (BM * BN);
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pt[(wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * BN + wn + 32 * j + fr] = acc[i][j][r];
    return;
  }
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


// ---------------------------------------------------------------------------
// Large-problem kernel (see the file header).
// ---------------------------------------------------------------------------
namespace {

constexpr int kBigBM = 256, kBigBN = 256, kBigBK = 32, kBigST = 4;
constexpr int kBigCPR = kBigBK / 8;            // 16-byte chunks per stage row
constexpr int kBigLPT = 2 * kBigCPR;           // global->LDS loads per thread per stage
constexpr int kBigSROW = kBigBK * 2;           // stage row bytes
constexpr int kBigSBYTES = (kBigBM + kBigBN) * kBigSROW;
constexpr int kBigSH = 2;                      // swizzle: chunk ^= (row >> 2) & 3

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt immediate that waits for vmcnt <= n and leaves the other counters alone
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// 16-byte per lane global -> LDS copy; lane l writes lds + 16 l.
R2L_DEV void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, unsigned voff, unsigned soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

R2L_DEV int big_swz(int row, int chunk) { return chunk ^ ((row >> kBigSH) & (kBigCPR - 1)); }

// Linear tile index -> (row tile, column tile): group-M raster, G row tiles
// sweep all column tiles; narrow outputs (few column tiles) use taller groups
// (measured best: 8 for <= 8 column tiles).
template <int G>
R2L_DEV void big_tile(int lid, int nTm, int nTn, int& tm, int& tn) {
  const int per_group = G * nTn;
  const int first_m = (lid / per_group) * G;
  const int gsz = min(nTm - first_m, G);
  tm = first_m + (lid % per_group) % gsz;
  tn = (lid % per_group) / gsz;
}

}  // namespace

// n_dp = number of whole tiles of the main launch.  !TAIL: block b
// computes tile xcd_remap(b) of those, over all of K, into C.  TAIL (the
// tail launch, splits > 0): block u computes K-steps [s ksteps, (s+1) ksteps) with
// s = u % splits of tile n_dp + u / splits, as an fp32 partial sum into
// part[u][256][256].
template <bool OUT_F32, int G, bool TAIL>
__global__ __launch_bounds__(256, 1) void gemm_bf16_big_kernel(int M, int N, int K,
                                                               const bf16* __restrict__ A, long lda,
                                                               const bf16* __restrict__ B, long ldb,
                                                               void* __restrict__ Cv, long ldc,
                                                               int n_dp, int splits, int ksteps,
                                                               float* __restrict__ part) {
  constexpr int BM = kBigBM, BN = kBigBN, BK = kBigBK, ST = kBigST, LPT = kBigLPT, SROW = kBigSROW;
  // one LDS object per stage: the compiler then knows that reading one stage
  // does not have to wait for the loads still in flight into another
  __shared__ __attribute__((aligned(1024))) char s0[kBigSBYTES];
  __shared__ __attribute__((aligned(1024))) char s1[kBigSBYTES];
  __shared__ __attribute__((aligned(1024))) char s2[kBigSBYTES];
  __shared__ __attribute__((aligned(1024))) char s3[kBigSBYTES];
  auto stage = [&](int s) -> char* { return s == 0 ? s0 : s == 1 ? s1 : s == 2 ? s2 : s3; };

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  const int nTm = (M + BM - 1) / BM, nTn = (N + BN - 1) / BN;
  const int lid = TAIL ? n_dp + (int)blockIdx.x / splits : xcd_remap(blockIdx.x, n_dp);
  const int kbeg = TAIL ? ((int)blockIdx.x % splits) * ksteps : 0;
  int tm, tn;
  big_tile<G>(lid, nTm, nTn, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Buffer descriptors over this tile's rows: reads past row M (N) return 0.
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + (long)m0 * lda), 0, (int)((long)min(BM, M - m0) * lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(B + (long)n0 * ldb), 0, (int)((long)min(BN, N - n0) * ldb * 2), 0x00020000);
  // Stage layout: rows [0, BM) hold A rows, rows [BM, BM+BN) hold B rows; load
  // i of this thread fills 16-byte slot i*256 + tid, i.e. row (i*256+tid)/4,
  // physical chunk tid%4, which holds logical k-chunk big_swz(row, tid%4).
  unsigned voff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int p = i * 256 + tid, row = p / kBigCPR;
    const int kc = big_swz(row, p % kBigCPR);
    voff[i] = i < LPT / 2 ? (unsigned)(((long)row * lda + kc * 8) * 2)
                          : (unsigned)(((long)(row - BM) * ldb + kc * 8) * 2);
  }
  const int nk = TAIL ? ksteps : K / BK;
  auto issue = [&](int s, int kt) {  // k-step kt -> stage s (past the end: reload the last step)
    char* base = stage(s);
    const unsigned kb = (unsigned)((kbeg + min(kt, nk - 1)) * BK * 2);
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      lds_dma16(i < LPT / 2 ? rA : rB, base + (i * 256 + wave * 64) * 16, voff[i], kb);
  };

  // fragment byte offsets inside a stage: k-chunk fh (first 16 of the step) and 2 + fh
  const int fr = lane & 31, fh = lane >> 5;
  int offA0[4], offB0[4], offA1[4], offB1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm + 32 * i + fr, rb = BM + wn + 32 * i + fr;
    offA0[i] = ra * SROW + big_swz(ra, fh) * 16;
    offB0[i] = rb * SROW + big_swz(rb, fh) * 16;
    offA1[i] = ra * SROW + big_swz(ra, 2 + fh) * 16;
    offB1[i] = rb * SROW + big_swz(rb, 2 + fh) * 16;
  }
  bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
  auto rd0 = [&](const char* base) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa0[i] = *(const bf16x8*)(base + offA0[i]);
      fb0[i] = *(const bf16x8*)(base + offB0[i]);
    }
  };
  auto rd1 = [&](const char* base) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa1[i] = *(const bf16x8*)(base + offA1[i]);
      fb1[i] = *(const bf16x8*)(base + offB1[i]);
    }
  };
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  // acc[i][j] = (B rows wn+32j..) x (A rows wm+32i..)^T = C^T sub-tile
  auto mm0 = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb0[j], fa0[i], acc[i][j], 0, 0, 0);
  };
  auto mm1 = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb1[j], fa1[i], acc[i][j], 0, 0, 0);
  };

  // Prologue: steps 0..2 in flight, step 0 visible to all waves, its first
  // fragments in registers.  A bare s_barrier (no fence) is used so that the
  // loads still in flight into other stages are not drained; the explicit
  // vmcnt wait before it makes this wave's own loads of the awaited step
  // complete, and the barrier then makes every wave's loads complete.
  issue(0, 0);
  issue(1, 1);
  issue(2, 2);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPT));
  asm volatile("s_barrier" ::: "memory");
  rd0(s0);
  for (int kt0 = 0; kt0 < nk; kt0 += ST) {
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      const int kt = kt0 + s;
      // this wave's loads of step kt+1 are done (step kt+2 may still fly);
      // after the barrier every wave's are, and every wave has finished
      // reading the stage of step kt-1, which is refilled with step kt+3
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPT));
      asm volatile("s_barrier" ::: "memory");
      issue((s + ST - 1) % ST, kt + ST - 1);
      rd1(stage(s));
      mm0();
#pragma unroll
      for (int q = 0; q < LPT; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global->LDS load
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      rd0(stage((s + 1) % ST));  // step kt+1: visible since this step's barrier
      mm1();
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // acc[i][j] register 4q+e holds C[m][n] with m = m0+wm+32i+(lane&31) and
  // n = n0+wn+32j+8q+4*(lane>>5)+e: four consecutive columns per store.
  if constexpr (TAIL) {
    float* pt = part + (long)blockIdx.x * (BM * BN);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wm + 32 * i + fr, c = wn + 32 * j + 8 * q + 4 * fh;
          *(f32x4*)(pt + r * BN + c) = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        }
    return;
  }
  // Direct epilogue through LDS: the four stages (free now) hold the tile in
  // row-major order, each 16-byte chunk of a row at chunk ^ (row & 31)
  // against bank conflicts; then every store instruction writes whole rows
  // (64 lanes x 16 bytes).  bf16: 64 rows of 512 bytes per stage, one pass;
  // f32: 32 rows of 1 KB per stage, two passes.  (Scattered 8-byte stores
  // straight from the MFMA layout took several times longer.)
  constexpr int ES = OUT_F32 ? 4 : 2;
  constexpr int RB = BN * ES;                  // row bytes
  constexpr int RPS = kBigSBYTES / RB;         // rows per stage
  constexpr int RPP = 4 * RPS;                 // rows per pass
  constexpr int LPR = RB / 16;                 // lanes per row in the store phase
  asm volatile("s_barrier" ::: "memory");      // every wave is done reading the stages
#pragma unroll
  for (int pass = 0; pass < BM / RPP; ++pass) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm + 32 * i + fr;
      if (r / RPP != pass) continue;           // uniform per (wave, i)
      const int rl = r - pass * RPP, rr = rl % RPS;
      char* sb = stage(rl / RPS) + rr * RB;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cb = (wn + 32 * j + 8 * q + 4 * fh) * ES;
          char* dst = sb + (((cb >> 4) ^ (rr & 31)) << 4) + (cb & 15);
          const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          if (OUT_F32) *(f32x4*)dst = v;
          else *(bf16x4*)dst = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
        }
    }
    __syncthreads();
    for (int rl = wave * (64 / LPR) + lane / LPR; rl < RPP; rl += 4 * (64 / LPR)) {
      const int rr = rl % RPS, ch = lane % LPR;
      const int m = m0 + pass * RPP + rl, n = n0 + ch * (16 / ES);
      const i32x4 v = *(const i32x4*)(stage(rl / RPS) + rr * RB + ((ch ^ (rr & 31)) << 4));
      if (m < M) {
        char* g = (char*)Cv + ((long)m * ldc + n) * ES;
        if (n + 16 / ES <= N) *(i32x4*)g = v;
        else if (!OUT_F32 && n + 4 <= N) *(int2*)g = int2{v[0], v[1]};   // N % 4 == 0 (bf16: 8-column chunks)
      }
    }
    if (pass + 1 < BM / RPP) __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// out_proj with the stream LayerNorm and the tanh(s)-gated residual in its
// epilogue ("Bifocal Diffusion Language Models", §3.4 steps 3-4):
//   o = y W_out^T,  r = gamma (.) (o - mean) / sqrt(var + eps) + beta,
//   h_out = h_in + tanh(s) r   (h_in copied bit for bit when tanh(s) == 0),
// mean and var over each token's d_model outputs.  o never leaves the
// registers: a token row spans the NT = d_model / 256 column tiles of its
// 256-row block, so the NT tiles of a row block run at the same time on NT
// blocks of one XCD and exchange per-row partial statistics.
//
// Persistent grid of G = 8 x NT x c blocks (at most one per CU, all resident
// together): block b on XCD b % 8 owns column tile (b / 8) % NT of row block
// (round x G / NT) + (b % 8) (G / 8 / NT) + (b / 8) / NT in every round.
// Each tile runs the big kernel's K loop (256 x 256 tile, four 32-deep LDS
// stages filled by buffer_load ... lds), then:
//  1. per row, the tile's mean and centred sum of squares (M2) over its 256
//     columns, from the accumulators (lane pairs by a shuffle, wave pairs
//     through LDS, always in the same order);
//  2. publishes them with agent-scope atomic stores, waits for those stores,
//     and adds 1 to the row block's counter (an agent-scope atomic, zeroed by
//     the layer's first kernel); one thread polls the counter until all NT
//     tiles have published, with a bounded number of sleeps (past it the
//     tile writes NaN, so a scheduling failure can never hang the GPU or go
//     unnoticed);
//  3. combines the NT partials of its rows in tile order (Chan's pairwise
//     mean/M2 update: the same result on every tile, whatever the timing);
//  4. stages its h tile in LDS with whole-row loads, normalises the
//     accumulators, adds the gated branch, and writes h_out with whole-row
//     stores (and the branch r, when asked for, from the registers).
// NO_LN: r = o, no statistics or exchange.
// ---------------------------------------------------------------------------
struct OutLnArgs {
  int K;                         // d_inner (a multiple of 32)
  const bf16* A; long lda;       // y [M, K]
  const bf16* B; long ldb;       // W_out [N, K], N = NT x 256
  const bf16* h; bf16* out; long ldh;   // h_in, h_out [M, N] (may alias)
  const float* gamma; const float* beta; const float* s;
  float* branch;                 // optional fp32 [M, ldh]
  float* o_save;                 // optional fp32 [M, ldh]: the out_proj output itself (training)
  float eps;
  unsigned long long* stats;     // [row blocks][NT][256]: (mean, M2) per tile row as two fp32
  int* cnt;                      // [row blocks], zero on entry
  int nt, rounds;
};
constexpr int kOutLnSpins = 1 << 24;

// EXTRA: also the optional fp32 outputs (branch, o_save); the plain forward
// runs the instance without them, which keeps its registers for the K loop.
template <bool NO_LN, bool EXTRA>
__global__ __launch_bounds__(256, 1) void gemm_out_ln_kernel(OutLnArgs a) {
  constexpr int BM = kBigBM, BN = kBigBN, BK = kBigBK, ST = kBigST, LPT = kBigLPT, SROW = kBigSROW;
  __shared__ __attribute__((aligned(1024))) char s0[kBigSBYTES];
  __shared__ __attribute__((aligned(1024))) char s1[kBigSBYTES];
  __shared__ __attribute__((aligned(1024))) char s2[kBigSBYTES];
  __shared__ __attribute__((aligned(1024))) char s3[kBigSBYTES];
  __shared__ float red[4][4][32];      // [wave][i][row]: per-wave row sums
  __shared__ float2 rstat[BM];         // (mean, 1 / std) of the tile's rows
  __shared__ __attribute__((aligned(16))) float gb_s[2][BN];   // gamma, beta of this block's columns
  __shared__ int okflag;
  auto stage = [&](int s) -> char* { return s == 0 ? s0 : s == 1 ? s1 : s == 2 ? s2 : s3; };

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm0 = (wave >> 1) * 128, wn0 = (wave & 1) * 128;
  const int fr0 = lane & 31, fh0 = lane >> 5;
  const int NT = a.nt, G = gridDim.x, per_xcd = G >> 3;
  const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
  const int rb0 = xcd * (per_xcd / NT) + pos / NT, ct = pos % NT;
  const int n0 = ct * BN;
  const float tg = tanhf(a.s[0]);
  if constexpr (!NO_LN) {   // the block's column tile is the same in every round
    gb_s[0][tid] = a.gamma[n0 + tid];
    gb_s[1][tid] = a.beta[n0 + tid];
  }
  // the row statistics of all blocks, read with the agent-coherent cache
  // policy (as the atomic stores that wrote them) but as plain loads, so
  // that a thread's NT loads are in flight together
  const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.stats, 0, 0x7fffffff, 0x00020000);

  unsigned voff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int p = i * 256 + tid, row = p / kBigCPR;
    const int kc = big_swz(row, p % kBigCPR);
    voff[i] = i < LPT / 2 ? (unsigned)(((long)row * a.lda + kc * 8) * 2)
                          : (unsigned)(((long)(row - BM) * a.ldb + kc * 8) * 2);
  }
  const int nk = a.K / BK;
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.B + (long)n0 * a.ldb), 0, (int)((long)BN * a.ldb * 2), 0x00020000);
  int offA0[4], offB0[4], offA1[4], offB1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm0 + 32 * i + fr0, rbr = BM + wn0 + 32 * i + fr0;
    offA0[i] = ra * SROW + big_swz(ra, fh0) * 16;
    offB0[i] = rbr * SROW + big_swz(rbr, fh0) * 16;
    offA1[i] = ra * SROW + big_swz(ra, 2 + fh0) * 16;
    offB1[i] = rbr * SROW + big_swz(rbr, 2 + fh0) * 16;
  }

  for (int rd = 0; rd < a.rounds; ++rd) {
    const int rbk = rd * (G / NT) + rb0;
    const long m0 = (long)rbk * BM;
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.A + m0 * a.lda), 0, (int)((long)BM * a.lda * 2), 0x00020000);
    auto issue = [&](int s, int kt) {  // k-step kt -> stage s (past the end: reload the last step)
      char* base = stage(s);
      const unsigned kb = (unsigned)(min(kt, nk - 1) * BK * 2);
#pragma unroll
      for (int i = 0; i < LPT; ++i)
        lds_dma16(i < LPT / 2 ? rA : rB, base + (i * 256 + wave * 64) * 16, voff[i], kb);
    };
    bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
    auto rd0 = [&](const char* base) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa0[i] = *(const bf16x8*)(base + offA0[i]);
        fb0[i] = *(const bf16x8*)(base + offB0[i]);
      }
    };
    auto rd1 = [&](const char* base) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa1[i] = *(const bf16x8*)(base + offA1[i]);
        fb1[i] = *(const bf16x8*)(base + offB1[i]);
      }
    };
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    // ---------------- the K loop (as gemm_bf16_big_kernel) ----------------
    issue(0, 0);
    issue(1, 1);
    issue(2, 2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPT));
    asm volatile("s_barrier" ::: "memory");
    rd0(s0);
    for (int kt0 = 0; kt0 < nk; kt0 += ST) {
#pragma unroll
      for (int s = 0; s < ST; ++s) {
        const int kt = kt0 + s;
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPT));
        asm volatile("s_barrier" ::: "memory");
        issue((s + ST - 1) % ST, kt + ST - 1);
        rd1(stage(s));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb0[j], fa0[i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int q = 0; q < LPT; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        rd0(stage((s + 1) % ST));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb1[j], fa1[i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    asm volatile("s_barrier" ::: "memory");   // every wave is done with the stages
    __builtin_amdgcn_sched_barrier(0);
    // acc[i][j] register 4q+e: row wm+32i+fr, column wn+32j+8q+4fh+e of the tile.
    // The epilogue forms its addresses from opaque copies of the lane
    // coordinates, so that none of them is hoisted out of the round loop
    // (they would stay live across the K loop and push it into spilling).
    int fr = fr0, fh = fh0, wm = wm0, wn = wn0;
    asm volatile("" : "+v"(fr), "+v"(fh), "+v"(wm), "+v"(wn));

    // ---------------- 1-3: row statistics over all NT tiles ----------------
    if constexpr (!NO_LN) {
      float mean[4], part[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sm = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) sm += acc[i][j][r];
        part[i] = sm + __shfl_xor(sm, 32, 64);
      }
      if (lane < 32)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][i][lane] = part[i];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) mean[i] = (red[wave & 2][i][fr] + red[(wave & 2) | 1][i][fr]) * (1.0f / BN);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sq = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float d = acc[i][j][r] - mean[i];
            sq = fmaf(d, d, sq);
          }
        part[i] = sq + __shfl_xor(sq, 32, 64);
      }
      if (lane < 32)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][i][lane] = part[i];
      __syncthreads();
      unsigned long long* my = a.stats + ((size_t)rbk * NT + ct) * BM;
      if ((wave & 1) == 0 && lane < 32)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float m2 = red[wave][i][lane] + red[wave | 1][i][lane];
          const unsigned long long v = (unsigned long long)__builtin_bit_cast(unsigned, mean[i]) |
                                       ((unsigned long long)__builtin_bit_cast(unsigned, m2) << 32);
          __hip_atomic_store(my + wm + 32 * i + lane, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      __builtin_amdgcn_s_waitcnt(0);   // this thread's statistics have reached memory
      __syncthreads();
      if (tid == 0) {
        __hip_atomic_fetch_add(a.cnt + rbk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int spins = 0;
        while (__hip_atomic_load(a.cnt + rbk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < NT &&
               ++spins < kOutLnSpins)
          __builtin_amdgcn_s_sleep(2);
        okflag = spins < kOutLnSpins;
      }
      __syncthreads();
      {
        // thread t combines the NT partials of tile row t in tile order
        const unsigned base = (unsigned)((size_t)rbk * NT * BM + tid) * 8u;
        float mu = 0.0f, m2 = 0.0f, n = 0.0f;
        for (int k0 = 0; k0 < NT; k0 += 8) {
          unsigned long long v[8];
#pragma unroll
          for (int k = 0; k < 8; ++k)
            v[k] = k0 + k < NT ? __builtin_bit_cast(unsigned long long, __builtin_amdgcn_raw_buffer_load_b64(
                                     rS, base + (unsigned)((k0 + k) * BM * 8), 0, 16))
                               : 0ull;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            if (k0 + k >= NT) break;
            const float mk = __builtin_bit_cast(float, (unsigned)v[k]);
            const float qk = __builtin_bit_cast(float, (unsigned)(v[k] >> 32));
            if (k0 + k == 0) {
              mu = mk;
              m2 = qk;
            } else {
              // Chan's update for two sets of n and BN values
              const float d = mk - mu, f = (float)BN / (n + BN);
              mu = fmaf(d, f, mu);
              m2 = m2 + qk + d * d * n * f;
            }
            n += BN;
          }
        }
        const float rstd = 1.0f / sqrtf(m2 / n + a.eps);
        rstat[tid] = okflag ? make_float2(mu, rstd) : make_float2(__builtin_nanf(""), __builtin_nanf(""));
      }
    }
    // ---------------- 4: h tile in LDS (row rr at stage rr / 64, 16-byte chunk c at c ^ (rr & 31)) --------
    const __amdgpu_buffer_rsrc_t rH = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.h + m0 * a.ldh + n0), 0, (int)((long)BM * a.ldh * 2), 0x00020000);
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int rr = 64 * wave + 2 * k + fh;
      const unsigned c = (unsigned)(fr ^ (rr & 31));
      lds_dma16(rH, stage(wave) + (2 * k) * 512, (unsigned)(rr * a.ldh * 2) + c * 16u, 0);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    // r from the accumulators; h_out = h + tanh(s) r back into the h tile
    // (a zero gate leaves the tile as loaded); the branch, when asked for,
    // straight from the registers
    auto branch_at = [&](int i, int j, int q) -> f32x4 {
      const int cl = wn + 32 * j + 8 * q + 4 * fh, row = wm + 32 * i + fr;
      f32x4 rv;
      if constexpr (NO_LN) {
#pragma unroll
        for (int e = 0; e < 4; ++e) rv[e] = acc[i][j][4 * q + e];
      } else {
        const float2 st = rstat[row];
        const f32x4 gm = *(const f32x4*)&gb_s[0][cl], bt = *(const f32x4*)&gb_s[1][cl];
#pragma unroll
        for (int e = 0; e < 4; ++e) rv[e] = fmaf(gm[e], (acc[i][j][4 * q + e] - st.x) * st.y, bt[e]);
      }
      return rv;
    };
    auto h_at = [&](int i, int j, int q) -> char* {
      const int cl = wn + 32 * j + 8 * q + 4 * fh, row = wm + 32 * i + fr;
      return stage(row >> 6) + (row & 63) * 512 + (((cl >> 3) ^ (row & 31)) << 4) + (fh << 3);
    };
    if (tg != 0.0f) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 rv = branch_at(i, j, q);
            char* p = h_at(i, j, q);
            const bf16x4 hv = *(const bf16x4*)p;
            bf16x4 ov;
#pragma unroll
            for (int e = 0; e < 4; ++e) ov[e] = (bf16)fmaf(tg, rv[e], (float)hv[e]);
            *(bf16x4*)p = ov;
          }
    }
    if (EXTRA && a.branch != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int cl = wn + 32 * j + 8 * q + 4 * fh, row = wm + 32 * i + fr;
            *(f32x4*)(a.branch + (m0 + row) * a.ldh + n0 + cl) = branch_at(i, j, q);
          }
    }
    if (EXTRA && a.o_save != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int cl = wn + 32 * j + 8 * q + 4 * fh, row = wm + 32 * i + fr;
            *(f32x4*)(a.o_save + (m0 + row) * a.ldh + n0 + cl) =
                f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          }
    }
    __syncthreads();
    // h_out rows from LDS, whole rows per store
    const __amdgpu_buffer_rsrc_t rO = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.out + m0 * a.ldh + n0), 0, (int)((long)BM * a.ldh * 2), 0x00020000);
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int rr = 64 * wave + 2 * k + fh;
      const unsigned c = (unsigned)(fr ^ (rr & 31));
      const u32x4 v = *(const u32x4*)(stage(wave) + (2 * k) * 512 + lane * 16);
      __builtin_amdgcn_raw_buffer_store_b128(v, rO, (unsigned)(rr * a.ldh * 2) + c * 16u, 0, 0);
    }
    __syncthreads();   // the stages are refilled by the next tile
  }
}

// Persistent form of the big kernel for bf16 outputs whose width is a
// multiple of 256 (in_proj).  The grid is a multiple of 8 blocks, at most one
// per CU; block b computes tiles xcd_remap(b + w * grid, n_dp), w = 0, 1, ...,
// which is the order in which a one-tile-per-block launch would hand tiles
// to that CU's XCD.  Two things differ from one launch per tile:
//  * the K-step pipeline runs on across tile boundaries: the next tile's
//    first three steps are loaded while this one finishes, so no tile but
//    the first waits for a prologue;
//  * a finished tile is written during the next tile's first 16 steps, a
//    quarter at a time through a fifth LDS buffer, with whole-row stores
//    (details at the write-out below).  With one launch per tile every CU
//    writes its 128 KB tile at the same moment at the end of each round and
//    its next loads wait behind those writes (one in-order vmcnt counter
//    covers both); spread over the next tile, the writes overlap the MFMAs.
// The last tile of each block is written out after the loop.
template <int G>
__global__ __launch_bounds__(256, 1) void gemm_bf16_pers_kernel(int M, int N, int K,
                                                                const bf16* __restrict__ A, long lda,
                                                                const bf16* __restrict__ B, long ldb,
                                                                bf16* __restrict__ C, long ldc, int n_dp) {
  constexpr int BM = kBigBM, BN = kBigBN, BK = kBigBK, ST = kBigST, LPT = kBigLPT, SROW = kBigSROW;
  __shared__ __attribute__((aligned(1024))) char s0[kBigSBYTES];
  __shared__ __attribute__((aligned(1024))) char s1[kBigSBYTES];
  __shared__ __attribute__((aligned(1024))) char s2[kBigSBYTES];
  __shared__ __attribute__((aligned(1024))) char s3[kBigSBYTES];
  __shared__ __attribute__((aligned(1024))) char sE[64 * 512];   // a quarter of a finished tile
  auto stage = [&](int s) -> char* { return s == 0 ? s0 : s == 1 ? s1 : s == 2 ? s2 : s3; };

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  const int nTm = (M + BM - 1) / BM, nTn = (N + BN - 1) / BN;
  const int grid = gridDim.x, b = blockIdx.x;
  const int ntile = (n_dp - b + grid - 1) / grid;  // >= 1: the grid is at most n_dp
  auto tile_of = [&](int w, int& m0, int& n0) {
    int tm, tn;
    big_tile<G>(xcd_remap(b + w * grid, n_dp), nTm, nTn, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
  };
  // buffer descriptors over a tile's operand rows (reads past row M or N return 0)
  auto rsrc_a = [&](int m0) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(A + (long)m0 * lda), 0, (int)((long)min(BM, M - m0) * lda * 2), 0x00020000);
  };
  auto rsrc_b = [&](int n0) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(B + (long)n0 * ldb), 0, (int)((long)min(BN, N - n0) * ldb * 2), 0x00020000);
  };
  int m0, n0, m1, n1;
  tile_of(0, m0, n0);
  m1 = m0;
  n1 = n0;
  if (ntile > 1) tile_of(1, m1, n1);
  __amdgpu_buffer_rsrc_t rA = rsrc_a(m0), rB = rsrc_b(n0), rAn = rsrc_a(m1), rBn = rsrc_b(n1);

  unsigned voff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int p = i * 256 + tid, row = p / kBigCPR;
    const int kc = big_swz(row, p % kBigCPR);
    voff[i] = i < LPT / 2 ? (unsigned)(((long)row * lda + kc * 8) * 2)
                          : (unsigned)(((long)(row - BM) * ldb + kc * 8) * 2);
  }
  const int nk = K / BK;
  // k-step kt of the current tile (nx: of the next tile; past the block's
  // last tile that is the current tile again, loaded but never read) -> stage s
  auto issue = [&](int s, int kt, bool nx) {
    char* base = stage(s);
    const __amdgpu_buffer_rsrc_t ra = nx ? rAn : rA, rb = nx ? rBn : rB;
    const unsigned kb = (unsigned)(kt * BK * 2);
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      lds_dma16(i < LPT / 2 ? ra : rb, base + (i * 256 + wave * 64) * 16, voff[i], kb);
  };

  const int fr = lane & 31, fh = lane >> 5;
  // fragment rows wm + 32 i + fr (A) and BM + wn + 32 i + fr (B): the
  // swizzle depends on them only through (fr >> 2) & 3, so fragment i sits
  // 32 rows (2 KB) after fragment 0
  const int offA0 = (wm + fr) * SROW + big_swz(fr, fh) * 16, offA1 = (wm + fr) * SROW + big_swz(fr, 2 + fh) * 16;
  const int offB0 = (BM + wn + fr) * SROW + big_swz(fr, fh) * 16, offB1 = (BM + wn + fr) * SROW + big_swz(fr, 2 + fh) * 16;
  bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
  auto rd0 = [&](const char* base) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa0[i] = *(const bf16x8*)(base + offA0 + 32 * SROW * i);
      fb0[i] = *(const bf16x8*)(base + offB0 + 32 * SROW * i);
    }
  };
  auto rd1 = [&](const char* base) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa1[i] = *(const bf16x8*)(base + offA1 + 32 * SROW * i);
      fb1[i] = *(const bf16x8*)(base + offB1 + 32 * SROW * i);
    }
  };
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  auto mm0 = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb0[j], fa0[i], acc[i][j], 0, 0, 0);
  };
  auto mm0_first = [&]() {  // a tile's first MFMAs start from zero
    const f32x16 z = {};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb0[j], fa0[i], z, 0, 0, 0);
  };
  auto mm1 = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb1[j], fa1[i], acc[i][j], 0, 0, 0);
  };
  auto sched_main = [&]() {
#pragma unroll
    for (int q = 0; q < LPT; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global->LDS load
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };
  auto sched_tail = [&]() {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };

  // Write-out of a finished tile, a quarter at a time: quarter k is row
  // block i = k of every wave (tile rows 32k + [0, 32) and 128 + 32k +
  // [0, 32), all 256 columns, 32 KB in bf16).  At the tile boundary quarter
  // 0 goes to sE and quarters 1..3 wait in pend (bf16, MFMA layout:
  // pend[16 (k - 1) + 4 j + q] holds columns n0+wn+32j+8q+4*(lane>>5) .. +3
  // of row m0+wm+32k+(lane&31)).  During the next tile's first 16 steps,
  // quarter k is read back from sE a row per instruction at steps
  // 4k+1..4k+3 and written with whole-row stores (64 lanes x 8 bytes);
  // quarter k+1 is copied from pend to sE at step 4k+4.  sE holds 64 rows of
  // 512 bytes; 8-byte slot c of local row r sits at slot c ^ (r & 31), so
  // that neither the column writes (32 rows, one slot) nor the row reads
  // meet a bank twice.
  bf16x4 pend[48];
#pragma unroll
  for (int p = 0; p < 48; ++p) pend[p] = bf16x4{};  // (written out, into an empty range, by the first tile)
  __amdgpu_buffer_rsrc_t rC = __builtin_amdgcn_make_buffer_rsrc((void*)C, 0, 0, 0x00020000);
  // quarter -> sE: this lane's local row is (wm ? 32 : 0) + (lane & 31); its
  // slot for (j, q) is wn / 4 + 8 j + 2 q + (lane >> 5)
  const int lrw = (wm ? 32 : 0) + fr;
  auto quarter_to_lds = [&](const bf16x4* v) {  // v[4 j + q]
    // opaque copies: the 16 addresses are formed here, not hoisted out of
    // the tile loop as 16 more VGPRs
    int row = lrw * 512, sl = fh ^ fr;
    asm volatile("" : "+v"(row), "+v"(sl));
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(bf16x4*)(sE + row + ((wn / 4 + ((8 * j + 2 * q) ^ sl)) << 3)) = v[4 * j + q];
  };
  // sE -> C: wave w writes local rows 16 w + rr, rr = 0..15; local rows
  // 0..31 are tile rows 32k + r, 32..63 are 128 + 32k + r - 32
  const unsigned voffE = (unsigned)(lane * 8);
  auto drain_rows = [&](int k, int r0, int r1) {
    // opaque copies of the wave's first row and the row stride: the row
    // addresses are formed here, not hoisted out of the tile loop as more
    // registers
    int w16 = 16 * wave, rb = (int)(ldc * 2);
    asm volatile("" : "+v"(w16), "+v"(rb));
    const int lr0 = __builtin_amdgcn_readfirstlane(w16), rbs = __builtin_amdgcn_readfirstlane(rb);
    const int x8 = (lane ^ (lr0 & 31)) << 3;   // (lr0 & 31) is 0 or 16, rr < 16: the XOR of rr goes in separately
    const int row0 = (wave < 2 ? 0 : 96) + 32 * k + lr0;   // tile row of rr = 0
#pragma unroll
    for (int rr = r0; rr < r1; ++rr) {
      const u32x2 v = *(const u32x2*)(sE + (lr0 + rr) * 512 + (x8 ^ (rr << 3)));
      __builtin_amdgcn_raw_buffer_store_b64(v, rC, voffE, (row0 + rr) * rbs, 0);
    }
  };



  // one K step: barrier, refill the stage of step kt-1 with step kt+3 (of the
  // next tile when nx), the second half of step kt and the first half of
  // step kt+1 from LDS.  t in [0, 16): also this step's part of the
  // previous tile's write-out.
  auto step = [&](int s, int kt, bool nx, bool first, int t) {
    const bool wr = t >= 4 && t % 4 == 0;      // pend quarter t / 4 -> sE
    const bool rd = t >= 0 && t % 4 != 0;      // sE quarter t / 4 -> C: rows 6 (t % 4 - 1) ..
    const int k = t / 4, c0 = rd ? 6 * (t % 4 - 1) : 0, c1 = rd ? min(c0 + 6, 16) : 0;
    if (t >= 0 && t % 4 == 1) __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's sE writes landed
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPT));
    asm volatile("s_barrier" ::: "memory");
    issue((s + ST - 1) % ST, nx ? kt + ST - 1 - nk : kt + ST - 1, nx);
    rd1(stage(s));
    if (first) mm0_first();
    else mm0();
    sched_main();
    rd0(stage((s + 1) % ST));
    if (wr) quarter_to_lds(pend + 16 * (k - 1));
    if (rd) drain_rows(k, c0, c1);
    mm1();
    sched_tail();
  };

  issue(0, 0, false);
  issue(1, 1, false);
  issue(2, 2, false);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPT));
  asm volatile("s_barrier" ::: "memory");
  rd0(s0);
  for (int w = 0; w < ntile; ++w) {
    // the first 16 steps also write out the previous tile (for the first
    // tile rC has an empty range and the stores are dropped)
#pragma unroll
    for (int t = 0; t < 16; ++t) step(t % ST, t, false, t == 0, t);
    for (int kt0 = 16; kt0 < nk - ST; kt0 += ST) {
#pragma unroll
      for (int s = 0; s < ST; ++s) step(s, kt0 + s, false, false, -1);
    }
    // last group: steps 1..3 load the next tile's first steps
#pragma unroll
    for (int s = 0; s < ST; ++s) step(s, nk - ST + s, s > 0, false, -1);
    __builtin_amdgcn_sched_barrier(0);  // keep the rounding out of the last step's MFMA schedule
    // rows past M are dropped by the descriptor's range; N % 256 == 0
    rC = __builtin_amdgcn_make_buffer_rsrc((void*)(C + (long)m0 * ldc + n0), 0,
                                           (int)((long)min(BM, M - m0) * ldc * 2), 0x00020000);
    bf16x4 q0[16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x4 v = {(bf16)acc[i][j][4 * q], (bf16)acc[i][j][4 * q + 1], (bf16)acc[i][j][4 * q + 2],
                            (bf16)acc[i][j][4 * q + 3]};
          if (i == 0) q0[4 * j + q] = v;
          else pend[16 * (i - 1) + 4 * j + q] = v;
        }
    quarter_to_lds(q0);
    __builtin_amdgcn_sched_barrier(0);
    m0 = m1;
    n0 = n1;
    rA = rAn;
    rB = rBn;
    if (w + 2 < ntile) {
      tile_of(w + 2, m1, n1);
      rAn = rsrc_a(m1);
      rBn = rsrc_b(n1);
    }
  }
  // the last tile: quarter 0 is in sE, quarters 1..3 in pend
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k > 0) {
      __syncthreads();  // every wave has read quarter k - 1
      quarter_to_lds(pend + 16 * (k - 1));
    }
    __syncthreads();
    drain_rows(k, 0, 16);
  }
}

// Mid-size kernel (the tiles of small problems and of the last tile row of
// large ones): the big kernel's pipeline on 128 x BN tiles, BN = 128 or 256.
// ST LDS stages of 32-wide K steps ((128 + BN) rows of 64 bytes: 16 KB, or
// 24 KB for 256-wide tiles) filled by buffer_load ... lds ST - 1 steps
// ahead, the same swizzle and the same barrier / vmcnt discipline; each wave
// owns a 64 x BN/2 part (2 x BN/64 MFMA tiles).  ST = 4 fits two 128 x 128
// blocks in a CU; ST = 8 (128 KB) is for launches of at most one block per
// CU, where a block's own copies in flight set the pace.  The last ST steps
// issue nothing new and wait for exactly the copies they read.
// splits == 0: block b computes tile b (row-major) into C.  splits > 0:
// block u computes K steps [s ksteps, (s+1) ksteps), s = u % splits, of tile
// u / splits as an fp32 partial sum into part[u][128][128], added by
// gemm_small_reduce4_kernel.  The K steps per block are a multiple of ST.
constexpr int kMidB = 128, kMidSBYTES = 2 * kMidB * kBigSROW;

// s_waitcnt until at most n stages of LPT copies each are outstanding (n is
// a constant once the calling loop is unrolled)
template <int LPT>
R2L_DEV void wait_stages(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPT)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPT)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * LPT)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * LPT)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5 * LPT)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6 * LPT)); break;
  }
}

template <bool OUT_F32, int ST, bool PLAN, int BN = kMidB>
__global__ __launch_bounds__(256, ST == 4 && BN == kMidB ? 2 : 1) void gemm_bf16_mid_kernel(
    int M, int N, int K, const bf16* __restrict__ A, long lda, const bf16* __restrict__ B, long ldb,
    void* __restrict__ Cv, long ldc, int splits, int ksteps, float* __restrict__ part, PlanArgs plan) {
  static_assert(ST == 4 || ST == 8, "four or eight stages");
  static_assert(BN == kMidB || BN == 2 * kMidB, "128- or 256-wide tiles");
  // BN = 256: twice the MFMAs per barrier and per fragment read; no K split
  // (the partial tiles are 128 x 128)
  constexpr int BM = kMidB, NJ = BN / 64, STAGE = (BM + BN) * kBigSROW;
  constexpr int BK = kBigBK, SROW = kBigSROW, LPT = (BM + BN) / 64;
  constexpr int XB = ST == 8 ? STAGE : 16;
  // one object per stage: the compiler orders LDS copies against reads per object
  __shared__ __attribute__((aligned(1024))) char s0[STAGE];
  __shared__ __attribute__((aligned(1024))) char s1[STAGE];
  __shared__ __attribute__((aligned(1024))) char s2[STAGE];
  __shared__ __attribute__((aligned(1024))) char s3[STAGE];
  __shared__ __attribute__((aligned(1024))) char s4[XB];
  __shared__ __attribute__((aligned(1024))) char s5[XB];
  __shared__ __attribute__((aligned(1024))) char s6[XB];
  __shared__ __attribute__((aligned(1024))) char s7[XB];
  if constexpr (PLAN) {
    // PLAN: one extra block at the end of the grid runs the scan's chunk
    // planning (dispatched last, it takes the first CU a tile block frees)
    if (blockIdx.x == gridDim.x - 1) {
      plan_chunks_block(plan, (int*)s0);
      return;
    }
  }
  auto stage = [&](int s) -> char* {
    switch (s) {
      case 0: return s0;
      case 1: return s1;
      case 2: return s2;
      case 3: return s3;
      case 4: return s4;
      case 5: return s5;
      case 6: return s6;
      default: return s7;
    }
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * (BN / 2), fr = lane & 31, fh = lane >> 5;
  const int nTn = (N + BN - 1) / BN;
  const int u = blockIdx.x;
  const int tile = splits ? u / splits : u;
  const int kbeg = splits ? (u % splits) * ksteps : 0;
  const int nk = splits ? ksteps : K / BK;
  const int m0 = (tile / nTn) * BM, n0 = (tile % nTn) * BN;
  // rows past M or N read as 0 through the descriptors' ranges
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + (long)m0 * lda), 0, (int)((long)min(BM, M - m0) * lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(B + (long)n0 * ldb), 0, (int)((long)min(BN, N - n0) * ldb * 2), 0x00020000);
  // load i fills stage slot 256 i + tid: stage row 64 i + tid / 4 (A rows for
  // i < 2, then B rows), physical chunk tid % 4
  unsigned voff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int row = 64 * i + tid / 4;
    const int kc = big_swz(row, tid % 4);
    voff[i] = i < 2 ? (unsigned)(((long)row * lda + kc * 8) * 2)
                    : (unsigned)(((long)(row - BM) * ldb + kc * 8) * 2);
  }
  auto issue = [&](int s, int kt) {
    char* base = stage(s);
    const unsigned kb = (unsigned)((kbeg + kt) * BK * 2);
#pragma unroll
    for (int i = 0; i < LPT; ++i) lds_dma16(i < 2 ? rA : rB, base + (i * 256 + wave * 64) * 16, voff[i], kb);
  };
  int offA0[2], offA1[2], offB0[NJ], offB1[NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ra = wm + 32 * i + fr;
    offA0[i] = ra * SROW + big_swz(ra, fh) * 16;
    offA1[i] = ra * SROW + big_swz(ra, 2 + fh) * 16;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int rb = BM + wn + 32 * j + fr;
    offB0[j] = rb * SROW + big_swz(rb, fh) * 16;
    offB1[j] = rb * SROW + big_swz(rb, 2 + fh) * 16;
  }
  bf16x8 fa0[2], fa1[2], fb0[NJ], fb1[NJ];
  auto rd0 = [&](const char* base) {
#pragma unroll
    for (int i = 0; i < 2; ++i) fa0[i] = *(const bf16x8*)(base + offA0[i]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb0[j] = *(const bf16x8*)(base + offB0[j]);
  };
  auto rd1 = [&](const char* base) {
#pragma unroll
    for (int i = 0; i < 2; ++i) fa1[i] = *(const bf16x8*)(base + offA1[i]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb1[j] = *(const bf16x8*)(base + offB1[j]);
  };
  f32x16 acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // nk is a positive multiple of ST.  Step kt reads the second half of stage
  // kt and the first half of stage kt + 1, so its wait leaves outstanding only
  // the stages issued after kt + 1; stage kt + ST - 1 goes into the slot that
  // step kt - 1 finished reading (the barrier orders it after those reads).
#pragma unroll
  for (int s = 0; s < ST - 1; ++s) issue(s, s);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((ST - 2) * LPT));
  asm volatile("s_barrier" ::: "memory");
  rd0(s0);
  // the waits are constants once the loops are unrolled: a branch on "last
  // group" inside the loop would make the compiler assume the fewer copies of
  // either path and add waits of its own
  auto step = [&](int s, int wait, bool iss, int kt, bool next) {
    wait_stages<LPT>(wait);
    asm volatile("s_barrier" ::: "memory");
    if (iss) issue((s + ST - 1) % ST, kt + ST - 1);
    rd1(stage(s));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb0[j], fa0[i], acc[i][j], 0, 0, 0);
    if (next) rd0(stage((s + 1) % ST));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb1[j], fa1[i], acc[i][j], 0, 0, 0);
  };
  for (int kt0 = 0; kt0 < nk - ST; kt0 += ST) {
#pragma unroll
    for (int s = 0; s < ST; ++s) step(s, ST - 3, true, kt0 + s, true);
  }
  // the last ST steps: only the first issues (stage nk - 1)
#pragma unroll
  for (int s = 0; s < ST; ++s)
    step(s, s == 0 ? ST - 3 : (s >= ST - 2 ? 0 : ST - 2 - s), s == 0, nk - ST + s, s < ST - 1);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // acc[i][j] register 4q+e holds row wm+32i+(lane&31), column
  // wn+32j+8q+4*(lane>>5)+e of the tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = wm + 32 * i + fr, c = wn + 32 * j + 8 * q + 4 * fh;
        const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        if (BN == kMidB && splits) {
          *(f32x4*)(part + (long)u * (kMidB * kMidB) + r * kMidB + c) = v;
        } else if (m0 + r < M && n0 + c < N) {   // N % 4 == 0: all four columns or none
          const long off = (long)(m0 + r) * ldc + n0 + c;
          if (OUT_F32) *(f32x4*)((float*)Cv + off) = v;
          else *(bf16x4*)((bf16*)Cv + off) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
        }
      }
}

// C tile n_dp + t = sum over s of part[t * splits + s], in order of s.
// Block: 4 rows of 256 columns of one tail tile; thread: 4 consecutive columns.
template <bool OUT_F32, int G>
__global__ __launch_bounds__(256) void gemm_tail_reduce_kernel(int M, int N, int n_dp, int splits,
                                                               const float* __restrict__ part,
                                                               void* __restrict__ Cv, long ldc) {
  const int nTm = (M + kBigBM - 1) / kBigBM, nTn = (N + kBigBN - 1) / kBigBN;
  const int t = blockIdx.x / (kBigBM / 4), r = (blockIdx.x % (kBigBM / 4)) * 4 + (threadIdx.x >> 6);
  const int c = (threadIdx.x & 63) * 4;
  int tm, tn;
  big_tile<G>(n_dp + t, nTm, nTn, tm, tn);
  const int m = tm * kBigBM + r, n = tn * kBigBN + c;
  if (m >= M || n >= N) return;
  f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < splits; ++s) v = v + *(const f32x4*)(part + ((long)t * splits + s) * (kBigBM * kBigBN) + r * kBigBN + c);
  if (OUT_F32) *(f32x4*)((float*)Cv + (long)m * ldc + n) = v;
  else *(bf16x4*)((bf16*)Cv + (long)m * ldc + n) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// C = sum over s of the 128 x 128 partial tiles part[tile * splits + s], in
// order of s (row-major tiles); one thread per output element.
template <int BM, int BN, bool OUT_F32>
__global__ __launch_bounds__(256) void gemm_small_reduce_kernel(int M, int N, int splits,
                                                                const float* __restrict__ part,
                                                                void* __restrict__ Cv, long ldc) {
  const int nTn = (N + BN - 1) / BN;
  const long e = blockIdx.x * 256L + threadIdx.x;
  const int m = (int)(e / N), n = (int)(e % N);
  if (m >= M) return;
  const int tile = (m / BM) * nTn + n / BN, r = m % BM, c = n % BN;
  float v = 0.0f;
  for (int s = 0; s < splits; ++s) v += part[((long)tile * splits + s) * (BM * BN) + r * BN + c];
  if (OUT_F32) ((float*)Cv)[(long)m * ldc + n] = v;
  else ((bf16*)Cv)[(long)m * ldc + n] = (bf16)v;
}

// The same sum four columns at a time (N % 4 == 0): one 16-byte load per
// partial and one 16- or 8-byte store per thread, partials added in order of s.
// PLAN: one extra block at the end of the grid runs the scan's chunk planning
// (this kernel takes no LDS, so that block starts at once, beside the sum).
template <int BM, int BN, bool OUT_F32, bool PLAN = false>
__global__ __launch_bounds__(256) void gemm_small_reduce4_kernel(int M, int N, int splits,
                                                                 const float* __restrict__ part,
                                                                 void* __restrict__ Cv, long ldc,
                                                                 PlanArgs plan = PlanArgs{}) {
  if constexpr (PLAN) {
    __shared__ int s_v[256];
    if (blockIdx.x == gridDim.x - 1) {
      plan_chunks_block(plan, s_v);
      return;
    }
  }
  const int nTn = (N + BN - 1) / BN, nq = N / 4;
  const long e = blockIdx.x * 256L + threadIdx.x;
  const int m = (int)(e / nq), n = (int)(e % nq) * 4;
  if (m >= M) return;
  const int tile = (m / BM) * nTn + n / BN, r = m % BM, c = n % BN;
  f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < splits; ++s) v = v + *(const f32x4*)(part + ((long)tile * splits + s) * (BM * BN) + r * BN + c);
  if (OUT_F32) *(f32x4*)((float*)Cv + (long)m * ldc + n) = v;
  else *(bf16x4*)((bf16*)Cv + (long)m * ldc + n) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// Enough 256 x 256 tiles for the large-problem kernel: a whole round over
// the CUs, or at least half of one with a long K (a weight gradient summed
// over tokens), which that kernel splits along K.  With fewer tiles and a
// short K, the mid-size kernel's smaller tiles fill the GPU instead
// (measured at 1024 x 8192 x 2048: 43-48 us against 50-57).
static bool big_enough(long big_tiles, int K) { return big_tiles >= 256 || (big_tiles >= 128 && K > 4096); }

// The mid-size kernel takes whole 128-wide K chunks and 16-byte operand rows
// whose 128-row byte ranges fit the 32-bit buffer descriptor.
static bool mid_fits(int K, const bf16* A, long lda, const bf16* B, long ldb) {
  return K % (kBigBK * kBigST) == 0 && lda % 8 == 0 && ldb % 8 == 0 && ((uintptr_t)A & 15) == 0 &&
         ((uintptr_t)B & 15) == 0 && (long)kMidB * lda * 2 < (1L << 31) && (long)kMidB * ldb * 2 < (1L << 31);
}

// Its K split: while the tiles do not fill the GPU, doubled as long as every
// split keeps whole 128-wide chunks of at least 8 steps and the fp32 partial
// tiles fit the workspace.
static int mid_split(int tiles, int nk, const float* ws, size_t ws_bytes, int ncu) {
  int splits = 1;
  if (ws != nullptr && ((uintptr_t)ws & 15) == 0 && ncu > 0 && tiles * 2 <= ncu) {
    while (tiles * splits * 2 <= ncu && nk % (splits * 2 * kBigST) == 0 && nk / (splits * 2) >= 8 &&
           (size_t)tiles * splits * 2 * kMidB * kMidB * sizeof(float) <= ws_bytes)
      splits *= 2;
  }
  return splits;
}

// One launch of the mid-size kernel: whole tiles into C (splits == 1), or
// the fp32 partial tiles of a K split into part.  Eight LDS stages when every
// block has a CU of its own.  Without a split, 128 x 256 tiles when they
// still give every CU a block (twice the MFMAs per barrier and per fragment
// read: 1,024 x 8,192 x 2,048 in 43 us against 48 on 128 x 128 tiles,
// graph replays).
template <bool OUT_F32>
static void launch_mid(int M, int N, int K, const bf16* A, long lda, const bf16* B, long ldb, void* C, long ldc,
                       int tiles, int splits, float* part, hipStream_t st, int ncu, PlanArgs* plan = nullptr) {
  const int nk = K / kBigBK;
  const int wide_tiles = ((M + kMidB - 1) / kMidB) * ((N + 2 * kMidB - 1) / (2 * kMidB));
  const bool wide = splits <= 1 && ncu > 0 && wide_tiles >= ncu;
  const int blocks = wide ? wide_tiles : splits > 1 ? tiles * splits : tiles;
  const bool deep = !wide && ncu > 0 && blocks <= ncu && (nk / splits) % 8 == 0;
  const int sp = splits > 1 ? splits : 0;
  const PlanArgs pa = plan ? *plan : PlanArgs{};
#define R2L_MID(S, P, W)                                                                                      \
  hipLaunchKernelGGL((gemm_bf16_mid_kernel<OUT_F32, S, P, W>), dim3(blocks + (P ? 1 : 0)), dim3(256), 0, st, M, \
                     N, K, A, lda, B, ldb, C, ldc, sp, sp ? nk / sp : 0, part, pa)
  if (plan) {
    if (wide) R2L_MID(4, true, 2 * kMidB);
    else if (deep) R2L_MID(8, true, kMidB);
    else R2L_MID(4, true, kMidB);
    plan->hosted = 1;
  } else {
    if (wide) R2L_MID(4, false, 2 * kMidB);
    else if (deep) R2L_MID(8, false, kMidB);
    else R2L_MID(4, false, kMidB);
  }
#undef R2L_MID
}

template <int BM, int BN>
static void launch_gemm(int M, int N, int K, const bf16* A, long lda, const bf16* B, long ldb,
                        void* C, long ldc, bool out_f32, hipStream_t st, float* ws, size_t ws_bytes,
                        int ncu, PlanArgs* plan) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  // The mid-size kernel, with 4-column output groups; the K split, when the
  // tiles do not fill the GPU, keeps whole 128-wide chunks per split.
  static_assert(BM == kMidB && BN == kMidB, "the mid-size kernel has 128 x 128 tiles");
  if (mid_fits(K, A, lda, B, ldb) && N % 4 == 0 && ldc % 4 == 0 && ((uintptr_t)C & (out_f32 ? 15 : 7)) == 0) {
    const int splits = mid_split(tiles, K / kBigBK, ws, ws_bytes, ncu);
    if (splits > 1) {
      // the chunk planning (when asked for) rides on the sum: a block of the
      // split GEMM would wait for a whole CU's LDS to come free
      launch_mid<true>(M, N, K, A, lda, B, ldb, C, ldc, tiles, splits, ws, st, ncu);
      const long n4 = (long)M * (N / 4);
      const unsigned g4 = (unsigned)((n4 + 255) / 256);
      if (plan) {
        if (out_f32)
          hipLaunchKernelGGL((gemm_small_reduce4_kernel<BM, BN, true, true>), dim3(g4 + 1), dim3(256), 0, st,
                             M, N, splits, (const float*)ws, C, ldc, *plan);
        else
          hipLaunchKernelGGL((gemm_small_reduce4_kernel<BM, BN, false, true>), dim3(g4 + 1), dim3(256), 0, st,
                             M, N, splits, (const float*)ws, C, ldc, *plan);
        plan->hosted = 1;
      } else if (out_f32) {
        hipLaunchKernelGGL((gemm_small_reduce4_kernel<BM, BN, true>), dim3(g4), dim3(256), 0, st,
                           M, N, splits, (const float*)ws, C, ldc, PlanArgs{});
      } else {
        hipLaunchKernelGGL((gemm_small_reduce4_kernel<BM, BN, false>), dim3(g4), dim3(256), 0,
                           st, M, N, splits, (const float*)ws, C, ldc, PlanArgs{});
      }
    } else if (out_f32) {
      launch_mid<true>(M, N, K, A, lda, B, ldb, C, ldc, tiles, 1, nullptr, st, ncu, plan);
    } else {
      launch_mid<false>(M, N, K, A, lda, B, ldb, C, ldc, tiles, 1, nullptr, st, ncu, plan);
    }
    return;
  }
  // Few tiles for the GPU: split K over several blocks per tile (each split
  // at least 4 of the kernel's 64-wide K steps), fp32 partials in ws.
  int splits = 1;
  if (ws != nullptr && ncu > 0 && tiles * 2 <= ncu) {
    while (tiles * splits * 2 <= ncu && K / (splits * 2) >= 256 &&
           (size_t)tiles * splits * 2 * BM * BN * sizeof(float) <= ws_bytes)
      splits *= 2;
  }
  if (splits > 1) {
    const int kchunk = ((K + splits - 1) / splits + 63) / 64 * 64;
    hipLaunchKernelGGL((gemm_bf16_nt_kernel<BM, BN, true>), dim3(tiles * splits), dim3(256), 0, st, M,
                       N, K, A, lda, B, ldb, C, ldc, splits, kchunk, ws);
    const long n = (long)M * N;
    if (out_f32)
      hipLaunchKernelGGL((gemm_small_reduce_kernel<BM, BN, true>), dim3((n + 255) / 256), dim3(256), 0, st,
                         M, N, splits, (const float*)ws, C, ldc);
    else
      hipLaunchKernelGGL((gemm_small_reduce_kernel<BM, BN, false>), dim3((n + 255) / 256), dim3(256), 0,
                         st, M, N, splits, (const float*)ws, C, ldc);
    return;
  }
  if (out_f32)
    hipLaunchKernelGGL((gemm_bf16_nt_kernel<BM, BN, true>), dim3(tiles), dim3(256), 0, st, M, N, K,
                       A, lda, B, ldb, C, ldc, 0, 0, (float*)nullptr);
  else
    hipLaunchKernelGGL((gemm_bf16_nt_kernel<BM, BN, false>), dim3(tiles), dim3(256), 0, st, M, N,
                       K, A, lda, B, ldb, C, ldc, 0, 0, (float*)nullptr);
}

template <int G>
static void launch_big(int M, int N, int K, const bf16* A, long lda, const bf16* B, long ldb, void* C,
                       long ldc, bool out_f32, int n_dp, int rem, int splits, int nk, float* ws,
                       hipStream_t st, int ncu) {
  // the persistent form: bf16 output a whole number of tiles wide, at least
  // 20 K steps per tile (16 write out the previous tile, the last 3 load the
  // next one), and at least two tiles per CU
  const int pgrid = ncu & ~7;
  const bool pers = !out_f32 && N % kBigBN == 0 && nk >= 20 && pgrid > 0 && n_dp >= 2 * pgrid &&
                    (long)kBigBM * ldc * 2 < (1L << 31);
  if (pers)
    hipLaunchKernelGGL((gemm_bf16_pers_kernel<G>), dim3(pgrid), dim3(256), 0, st, M, N, K, A, lda, B, ldb,
                       (bf16*)C, ldc, n_dp);
  else if (n_dp > 0 && out_f32)
    hipLaunchKernelGGL((gemm_bf16_big_kernel<true, G, false>), dim3(n_dp), dim3(256), 0, st, M, N, K, A, lda,
                       B, ldb, C, ldc, n_dp, 0, 0, (float*)nullptr);
  else if (n_dp > 0)
    hipLaunchKernelGGL((gemm_bf16_big_kernel<false, G, false>), dim3(n_dp), dim3(256), 0, st, M, N, K, A, lda,
                       B, ldb, C, ldc, n_dp, 0, 0, (float*)nullptr);
  if (splits) {
    const int ksteps = nk / splits;
    // (the kernel's OUT_F32 only shapes the direct epilogue; partials are fp32)
    hipLaunchKernelGGL((gemm_bf16_big_kernel<true, G, true>), dim3(rem * splits), dim3(256), 0, st, M, N, K,
                       A, lda, B, ldb, C, ldc, n_dp, splits, ksteps, ws);
    if (out_f32)
      hipLaunchKernelGGL((gemm_tail_reduce_kernel<true, G>), dim3(rem * (kBigBM / 4)), dim3(256), 0, st, M,
                         N, n_dp, splits, (const float*)ws, C, ldc);
    else
      hipLaunchKernelGGL((gemm_tail_reduce_kernel<false, G>), dim3(rem * (kBigBM / 4)), dim3(256), 0, st, M,
                         N, n_dp, splits, (const float*)ws, C, ldc);
  }
}

int gemm_bf16_nt_parts_split(int M, int N, int K, const bf16* A, long lda, const bf16* B, long ldb,
                             const float* ws, size_t ws_bytes, int ncu) {
  if (M <= 0 || N <= 0 || N % 4 != 0) return 0;
  const long big_tiles = (long)((M + kBigBM - 1) / kBigBM) * ((N + kBigBN - 1) / kBigBN);
  if (big_enough(big_tiles, K) || !mid_fits(K, A, lda, B, ldb)) return 0;   // not the mid-size kernel's problem
  const int tiles = ((M + kMidB - 1) / kMidB) * ((N + kMidB - 1) / kMidB);
  const int splits = mid_split(tiles, K / kBigBK, ws, ws_bytes, ncu);
  return splits > 1 ? splits : 0;
}

hipError_t gemm_bf16_nt_parts(int M, int N, int K, const bf16* A, long lda, const bf16* B, long ldb, int splits,
                              hipStream_t st, float* ws, int ncu) {
  const int tiles = ((M + kMidB - 1) / kMidB) * ((N + kMidB - 1) / kMidB);
  launch_mid<true>(M, N, K, A, lda, B, ldb, nullptr, N, tiles, splits, ws, st, ncu);
  return hipGetLastError();
}

OutLnPlan plan_out_ln(int T, int D, int K, int ncu) {
  OutLnPlan p{};
  // (the K loop walks whole groups of four 32-deep stages, as the big
  // kernel's does: a K of 64 modulo 128 runs the unfused path)
  if (D % kBigBN || K % (kBigBK * kBigST) || ncu <= 0) return p;
  const int nt = D / kBigBN;
  const int grid = 8 * nt * (ncu / (8 * nt));   // whole row blocks on every XCD, at most one block per CU
  if (grid <= 0) return p;
  const int rb_round = grid / nt;
  const int rounds = (T / kBigBM) / rb_round;
  if (rounds < 1 || (long)kBigBM * K * 2 >= (1L << 31) || (long)kBigBM * D * 2 >= (1L << 31)) return p;
  p.nt = nt;
  p.grid = grid;
  p.rounds = rounds;
  p.rows = rounds * rb_round * kBigBM;
  p.row_blocks = rounds * rb_round;
  return p;
}

hipError_t gemm_out_ln(const OutLnPlan& p, int K, const bf16* y, long ldy, const bf16* W, long ldw, const bf16* h,
                       bf16* out, long ldh, const float* gamma, const float* beta, const float* s, float* branch,
                       float* o_save, bool no_ln, float eps, unsigned long long* stats, int* cnt, hipStream_t st) {
  if (p.rows <= 0) return hipSuccess;
  OutLnArgs a{};
  a.K = K;
  a.A = y; a.lda = ldy;
  a.B = W; a.ldb = ldw;
  a.h = h; a.out = out; a.ldh = ldh;
  a.gamma = gamma; a.beta = beta; a.s = s; a.branch = branch; a.o_save = o_save; a.eps = eps;
  a.stats = stats; a.cnt = cnt;
  a.nt = p.nt;
  a.rounds = p.rounds;
  const bool extra = branch != nullptr || o_save != nullptr;
  if (no_ln && extra)
    hipLaunchKernelGGL((gemm_out_ln_kernel<true, true>), dim3(p.grid), dim3(256), 0, st, a);
  else if (no_ln)
    hipLaunchKernelGGL((gemm_out_ln_kernel<true, false>), dim3(p.grid), dim3(256), 0, st, a);
  else if (extra)
    hipLaunchKernelGGL((gemm_out_ln_kernel<false, true>), dim3(p.grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_out_ln_kernel<false, false>), dim3(p.grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t gemm_bf16_nt(int M, int N, int K, const bf16* A, long lda, const bf16* B, long ldb,
                        void* C, long ldc, bool out_f32, hipStream_t st, float* ws, size_t ws_bytes,
                        int ncu, PlanArgs* plan) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const long big_tiles = (long)((M + kBigBM - 1) / kBigBM) * ((N + kBigBN - 1) / kBigBN);
  const unsigned long align = out_f32 ? 16 : 8;
  // The large-problem kernel needs whole 128-wide K chunks (four stages of
  // 32), 4-column output groups, 16-byte operand rows, per-tile byte ranges
  // that fit the 32-bit buffer descriptor, and enough tiles to fill the GPU.
  const bool big = K % (kBigBK * kBigST) == 0 && N % 4 == 0 && ldc % 4 == 0 &&
                   lda % 8 == 0 && ldb % 8 == 0 && ((uintptr_t)A & 15) == 0 &&
                   ((uintptr_t)B & 15) == 0 && ((uintptr_t)C & (align - 1)) == 0 &&
                   (long)kBigBM * lda * 2 < (1L << 31) && (long)kBigBN * ldb * 2 < (1L << 31) &&
                   big_enough(big_tiles, K);
  if (big) {
    // Tiles beyond the last whole round (tiles mod #CUs) would take a round of
    // their own; with a workspace they are split along K over up to all CUs
    // instead, and their fp32 partial sums added in a fixed order.  The split
    // costs two launches and the partials' traffic, so it is used only for a
    // small leftover (measured: a gain at 1/32 of a round, a loss at 1/8).
    // Fewer tiles than CUs (a long K over a small output, e.g. a weight
    // gradient summed over tokens): every tile is split along K the same way.
    const int nk = K / kBigBK;
    const int rem = ncu > 0 ? (int)(big_tiles % ncu) : 0;
    int splits = 0;
    if (ws != nullptr && rem > 0 && (rem * 16 <= ncu || big_tiles * 2 <= ncu)) {
      for (int s = 64; s >= 2; s /= 2)
        if ((long)rem * s <= ncu && nk % (s * kBigST) == 0 &&
            (size_t)rem * s * kBigBM * kBigBN * sizeof(float) <= ws_bytes && ((uintptr_t)ws & 15) == 0) {
          splits = s;
          break;
        }
    }
    // groups of G tile rows walk the tile columns: 8 rows for narrow
    // outputs (<= 8 tile columns), else 4
    const int nTn = (N + kBigBN - 1) / kBigBN, nTm = (M + kBigBM - 1) / kBigBM;
    const int G = nTn <= 8 ? 8 : 4;
    // A leftover that is exactly the last row of tiles (the last group holds
    // one tile row, and the leftover is that row): those rows go to the
    // 128 x 128 kernel instead, after the whole rounds, where they fill the
    // chip rather than a fraction of it (measured faster than the split
    // tail for both projections of the serving shape).
    if (ws != nullptr && big_tiles > ncu && rem == nTn && nTm % G == 1) {
      const int m_tail = (nTm - 1) * kBigBM;
      if (G == 8) launch_big<8>(m_tail, N, K, A, lda, B, ldb, C, ldc, out_f32, (int)big_tiles - rem, 0, 0, nk, ws, st, ncu);
      else launch_big<4>(m_tail, N, K, A, lda, B, ldb, C, ldc, out_f32, (int)big_tiles - rem, 0, 0, nk, ws, st, ncu);
      const long ce = out_f32 ? 4 : 2;
      launch_gemm<128, 128>(M - m_tail, N, K, A + (long)m_tail * lda, lda, B, ldb,
                            (char*)C + (long)m_tail * ldc * ce, ldc, out_f32, st, ws, ws_bytes, ncu, plan);
      return hipGetLastError();
    }
    const int n_dp = (int)big_tiles - (splits ? rem : 0);
    if (G == 8) launch_big<8>(M, N, K, A, lda, B, ldb, C, ldc, out_f32, n_dp, rem, splits, nk, ws, st, ncu);
    else launch_big<4>(M, N, K, A, lda, B, ldb, C, ldc, out_f32, n_dp, rem, splits, nk, ws, st, ncu);
    return hipGetLastError();
  }
  // 128 x 128 tiles (4 waves of 64 x 64, two blocks per CU).
  launch_gemm<128, 128>(M, N, K, A, lda, B, ldb, C, ldc, out_f32, st, ws, ws_bytes, ncu, plan);
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
