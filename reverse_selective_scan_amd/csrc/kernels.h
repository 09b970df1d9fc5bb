// Launchers of the device kernels (internal to libr2l.so).  Each launcher
// enqueues its kernel(s) on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "plan.h"

namespace r2l {

// C[M,N] = A[M,K] . B[N,K]^T.  bf16 inputs on MFMA; output bf16 or f32.
// ws (optional, 16-byte aligned, ws_bytes long; may be NULL): scratch for the
// K-split partial sums of the tiles past the last whole round over ncu CUs.
// plan (optional): when the problem (or its last tile row) runs on the
// mid-size kernel, one of its launches (the GEMM, or the sum of a K split)
// also runs the scan's chunk planning as one extra block and sets
// plan->hosted; otherwise plan is left as it is.
hipError_t gemm_bf16_nt(int M, int N, int K, const bf16* A, long lda, const bf16* B, long ldb,
                        void* C, long ldc, bool out_f32, hipStream_t st, float* ws = nullptr,
                        size_t ws_bytes = 0, int ncu = 0, PlanArgs* plan = nullptr);
// The K-split part alone.  gemm_bf16_nt_parts_split: the split count with
// which gemm_bf16_nt would run this problem on its mid-size kernel split
// along K (few 128 x 128 tiles for the GPU), else 0.  gemm_bf16_nt_parts:
// that kernel alone with that count, its fp32 partial tiles left in ws (tile
// t of the row-major tile grid, split s at ws + (t * splits + s) * 128 * 128,
// row-major inside the tile).
int gemm_bf16_nt_parts_split(int M, int N, int K, const bf16* A, long lda, const bf16* B, long ldb,
                             const float* ws, size_t ws_bytes, int ncu);
hipError_t gemm_bf16_nt_parts(int M, int N, int K, const bf16* A, long lda, const bf16* B, long ldb, int splits,
                              hipStream_t st, float* ws, int ncu);
// out_proj fused with the stream LayerNorm and the gated residual (bf16):
// h_out = h + tanh(s) LN(y W^T) for the first `rows` token rows, which the
// plan makes whole rounds of 256-row blocks over a persistent grid (rows = 0:
// the shape does not fit and the caller runs out_proj and ln_gate instead).
// stats: row_blocks * nt * 256 * 8 bytes; cnt: row_blocks ints, zero on entry.
// o_save (optional, fp32 [rows, ldh]): the out_proj output itself (training).
struct OutLnPlan {
  int nt, grid, rounds, rows, row_blocks;
};
OutLnPlan plan_out_ln(int T, int D, int K, int ncu);
hipError_t gemm_out_ln(const OutLnPlan& p, int K, const bf16* y, long ldy, const bf16* W, long ldw, const bf16* h,
                       bf16* out, long ldh, const float* gamma, const float* beta, const float* s, float* branch,
                       float* o_save, bool no_ln, float eps, unsigned long long* stats, int* cnt, hipStream_t st);
// fp32 inputs on the VALU; output f32.
hipError_t gemm_f32_nt(int M, int N, int K, const float* A, long lda, const float* B, long ldb,
                       float* C, long ldc, hipStream_t st);

// Direction of the conv and the scan: l2r = false runs the block over the
// flipped sequence (anti-causal conv, right-to-left scan: the layer of the
// pages), l2r = true in the original order (causal conv, left-to-right
// scan: the L2R control of the pages' ablation).

// Depthwise conv + bias + SiLU -> u (act, contiguous [T,E]).
template <typename T>
hipError_t conv_silu(int T_, int E, const T* x, long ld_x, const T* conv_w, const T* conv_b,
                     T* u, const int32_t* cu, int nseq, bool l2r, hipStream_t st);
// delta split for the scan's dt_proj on MFMA: the first R columns of each
// x_proj output row (delta), as a bf16 pair per value: row t of dsplit
// [T, 2 RP] holds hi = bf16(delta) in columns [0, RP) and lo =
// bf16(delta - hi) in [RP, 2 RP), zeros in columns R .. RP-1.  RP is the
// dt_rank padded to the scan's MFMA k-steps (0: the scan computes dt on the
// VALU from xdbl and needs no split).
int delta_split_width(int R);

// Fused conv + SiLU + x_proj (bf16, MFMA): xdbl f32 [T, P] with P = R+2N;
// u_out optional.  Requires E % 64 == 0 and P <= 256.
// ws (optional, ws_bytes): scratch for splitting the channels over several
// blocks per 32-token tile when there are few tiles (not with u_out).
// dsplit (optional): also written, see delta_split_width.
hipError_t conv_xproj_bf16(int T_, int E, int P, const bf16* x, long ld_x, const bf16* conv_w,
                           const bf16* conv_b, const bf16* x_proj_w, bf16* u_out, float* xdbl,
                           const int32_t* cu, int nseq, bool l2r, hipStream_t st, float* ws = nullptr,
                           size_t ws_bytes = 0, int ncu = 0, int R = 0, bf16* dsplit = nullptr);

// The same for large inputs, split along K over one or two blocks per CU
// (`ncu` CUs) into up to three partial sums; conv_sk_sum (same T, E, P, ncu)
// then leaves xdbl in part0 (and, when dsplit is given, the delta split of
// its first R columns).  Parts [T, P] fp32, 16-byte aligned.  Requires
// E % 64 == 0, P <= 256 and ceil(T / 128) >= ncu.
hipError_t conv_xproj_bf16_sk(int T_, int E, int P, const bf16* x, long ld_x, const bf16* conv_w,
                              const bf16* conv_b, const bf16* x_proj_w, float* part0, float* part1,
                              float* part2, const int32_t* cu, int nseq, int ncu, bool l2r, hipStream_t st);
hipError_t conv_sk_sum(int T_, int E, int P, float* part0, const float* part1, const float* part2, int ncu,
                       hipStream_t st, int R = 0, bf16* dsplit = nullptr);
// The delta split of an x_proj output computed elsewhere (xdbl f32 [T, P]).
hipError_t split_delta(int T_, int P, int R, const float* xdbl, bf16* dsplit, hipStream_t st);

// Chunk planning for the scan: sanitised cu_seqlens and the chunk table
// (chunks cut from the end the scan starts at).
// zero (optional): n_zero ints cleared on the way (counters of later kernels).
hipError_t plan_chunks(const int32_t* cu, int nseq, int T_, int Lc, int max_chunks, bool l2r,
                       int32_t* cu_clean, ChunkDesc* chunks, int32_t* n_chunks, hipStream_t st,
                       int* zero = nullptr, int n_zero = 0);
// The same planning as the arguments of one extra block of another launch
// (gemm_bf16_nt's plan argument; PlanArgs in plan.h).
PlanArgs plan_args(const int32_t* cu, int nseq, int T_, int Lc, int max_chunks, bool l2r, int32_t* cu_clean,
                   ChunkDesc* chunks, int32_t* n_chunks, int* zero = nullptr, int n_zero = 0);

struct ScanArgs {
  int T, E, R, ldp;            // ldp: row stride of xdbl (fused) in floats
  // fused mode: x (in xz), z, xdbl (delta|B|C), conv and dt_proj weights
  const void* x; long ld_x;
  const void* z; long ld_z;
  const float* xdbl;
  const bf16* dsplit;          // delta split (fused bf16 with dt_proj on MFMA), [T, 2 RP]
  const void* conv_w; const void* conv_b;
  const void* dt_w; const float* dt_b;
  // standalone mode: u, dt, B, C
  const void* u; long ld_u;
  const float* dt; long ld_dt;
  const float* Bm; const float* Cm; long ld_bc;
  // both
  const float* A_log; const float* Dskip;
  void* y;
  const ChunkDesc* chunks; const int32_t* n_chunks; int max_chunks;
  float* sumS; float* sumP;    // [max_chunks][16][E] each
  bool l2r;                    // scan direction (see above)
  // backward, first sweep: the gradient of the scan's output, dz (f32
  // [T, E]) and the state entering every 16-token sub-block from the right
  // (f32 [slots][16][E], slot ChunkDesc::slot0 + q for sub-block q counted
  // from the chunk's right end)
  const void* dy; long ld_dy;
  float* dz; float* hc;
};

// Pass 1 (only when some sequence spans several chunks): per-chunk decay
// product and local state.  Pass 2: outputs, with the carry-in of each chunk
// combined from the summaries of the chunks before it in scan order.
template <typename T>
hipError_t scan_summary(const ScanArgs& a, bool fused, hipStream_t st);
template <typename T>
hipError_t scan_main(const ScanArgs& a, bool fused, hipStream_t st);
// Backward of the standalone scan (right to left, one chunk per sequence):
// sweep 1 recomputes the states (kept every 16 tokens in a.hc) and writes dz;
// the adjoint sweep and the reductions live in scan_bwd.hip.
template <typename T>
hipError_t scan_bwd_states(const ScanArgs& a, hipStream_t st);
struct ScanBwdArgs {
  int T, E;
  const void* u; long ld_u;
  const float* dt; long ld_dt;
  const float* Bm; const float* Cm; long ld_bc;
  const float* A_log; const float* Dskip;
  const void* z; long ld_z;
  const void* dy; long ld_dy;
  const ChunkDesc* chunks; const int32_t* n_chunks;
  const float* hc;          // [slots][16][E] from the first sweep
  float* du; float* ddt;    // [T, E]
  float* dbc;               // [E/64][T][32]: dB | dC partial sums of each channel block
  float* dA;                // [max_chunks][E][16] (d/dA_log)
  float* dD;                // [max_chunks][E]
  // time chunks: the adjoint's zero-carry chunk summaries [max_chunks][16][E]
  // (carry out M, decay Q), or null when every sequence is one chunk
  float* adjM; float* adjQ;
};
// The adjoint sweep and the reductions into dA_log [E,16], dB, dC [T,16]
// and dDskip [E] (may be null); with a.adjM set, the chunk summaries first.
template <typename T>
hipError_t scan_bwd_adjoint(const ScanBwdArgs& a, int max_chunks, float* dA_log, float* dB, float* dC,
                            float* dDskip, hipStream_t st);

// ---- backward of the layer (layer_bwd.hip) ----
// out [cols, rows_pad] = in [rows, cols]^T, zero columns past rows.
template <typename Tin, typename Tout>
hipError_t transpose(int rows, int cols, int rows_pad, const Tin* in, long ld_in, Tout* out, hipStream_t st);
enum EwOp { kConvert = 0, kSoftplusBias = 1, kDtPre = 2, kAddTo = 3 };
template <int OP, typename Tin, typename Tout>
hipError_t elementwise(int rows, int cols, const Tin* in, long ld_in, const float* aux, long ld_aux,
                       const float* vec, Tout* out, long ld_out, hipStream_t st);
// out[t] = in[s + e - 1 - t] for t in sequence [s, e) (per-sequence row
// reversal); out == in reverses in place.
template <typename T>
hipError_t flip_rows(int T_, int cols, const T* in, long ld_in, T* out, long ld_out, const int32_t* cu, int nseq,
                     hipStream_t st);
// One pass of v = op(in, aux) over [rows, cols] (kConvert or kDtPre): the
// row-major copy out_rm, the transposed copy out_t [cols, rows_pad] (zeros
// past rows) and column sums of each 64-row band colpart
// [ceil(rows/64)][cols], each optional (null).
template <int OP, typename Tin, typename Tout>
hipError_t fused_t(int rows, int cols, int rows_pad, const Tin* in, long ld_in, const float* aux, long ld_aux,
                   Tout* out_rm, long ld_rm, Tout* out_t, float* colpart, hipStream_t st);
// out[c] = scale * sum_r in[r][c]; part: colsum_parts(rows) * cols floats.
int colsum_parts(int rows);
hipError_t colsum(int rows, int cols, const float* in, long ld, float* part, float scale, float* out, hipStream_t st);
// part: ln_bwd_parts(T) * 2D floats (per-wave sums of th [g xhat | g]).
int ln_bwd_parts(int T_);
template <typename T>
hipError_t ln_gate_bwd(int T_, int D, const T* g, const float* o, const float* gamma, const float* beta,
                       const float* s, bool no_ln, float eps, float* dout, float* part, float* gr, hipStream_t st);
// dx (act, row stride ld_dx) from du (+ du2); dw, db summed over tokens.
// cu: sanitised offsets.  part: conv_bwd_parts(T) * E * 5 floats.
int conv_bwd_parts(int T_);
template <typename T>
hipError_t conv_bwd(int T_, int E, const T* x, long ld_x, const T* cw, const T* cb, const float* du, const float* du2,
                    T* dx, long ld_dx, float* part, float* dw, float* db, const int32_t* cu, int nseq,
                    hipStream_t st);
template <typename Tout>
hipError_t concat3(int T_, int na, int nb, int nc, const float* a, const float* b, const float* c, Tout* out,
                   long ld_out, hipStream_t st);

template <typename T, typename O>
hipError_t ln_gate(int T_, int D, const O* o, const T* h_in, T* h_out, const float* gamma,
                   const float* beta, const float* s, float* branch, bool no_ln, float eps,
                   hipStream_t st);
// ln_gate on the split-K parts of o that gemm_bf16_nt_parts left: o is
// their sum in the order of the split index (the values the GEMM's own sum
// would store), saved to o_save (optional, f32 [T_, D]) for training.
// Returns hipErrorInvalidValue, launching nothing, for widths or split
// counts it does not take (D of 2048, 4096 or 8192; 2, 4 or 8 splits).
bool ln_gate_parts_fits(int D, int splits);
template <typename T>
hipError_t ln_gate_parts(int T_, int D, int splits, const float* part, const T* h_in, T* h_out,
                         const float* gamma, const float* beta, const float* s, float* branch, float* o_save,
                         bool no_ln, float eps, hipStream_t st);

}  // namespace r2l
