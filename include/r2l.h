/*
 * r2l.h -- C ABI of libr2l.so, an MI355X (gfx950) implementation of the
 * R2LM ReverseMambaLayer forward.
 *
 * Source of the operation: "Bifocal Diffusion Language Models: Asymmetric
 * Bidirectional Context for Parallel Generation" (arXiv 2606.27732),
 * §3.4 "R2LM Architecture" (the four steps of the R2L stream: flip, Mamba-1
 * selective-scan block, unflip + stream-local LayerNorm, tanh(s)-gated
 * residual) and §4.1 "Experimental Setup" (d_state 16, d_conv 4, expand 2,
 * one hook after every 4th decoder layer).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Sequences are packed back to back: token t of the packed array belongs
 *    to sequence q when cu_seqlens[q] <= t < cu_seqlens[q+1].  A dense
 *    [B, L] batch is cu_seqlens = {0, L, 2L, ..., BL}.  Zero-length
 *    sequences are allowed.  The "flip" of the pages is never materialised:
 *    every kernel works in the original token order with anti-causal
 *    indexing (a token sees itself and the tokens to its right, up to its
 *    sequence's end).
 *  - All pointers except the r2l_dims / r2l_weights structs themselves and
 *    the optional host copy in r2l_check_cu_seqlens are DEVICE pointers on
 *    the current HIP device.  Matrices are row-major; weights use the
 *    nn.Linear [out_features, in_features] layout.
 *  - Activation tensors and the weights listed as "act" use the activation
 *    dtype (R2L_F32 or R2L_BF16).  Scan state, dt, B, C and all
 *    accumulations are fp32 in both cases.
 *  - Alignment: r2l_layer_fwd needs every tensor pointer it takes to be
 *    16-byte aligned (torch and hipMalloc allocations are).
 *  - Ownership: the caller allocates and owns every buffer (weights,
 *    activations, cu_seqlens, workspace).  The library allocates no device
 *    memory and keeps no pointer after a call returns.
 *  - Execution: work is enqueued on `stream` (a hipStream_t; NULL = the
 *    null stream) without any host synchronisation.  A fault during
 *    execution surfaces at the caller's next synchronisation.
 *  - Errors: every entry point validates its arguments before launching
 *    anything and returns one of the R2L_* status codes; nothing is
 *    launched on error.  cu_seqlens lives on the device and is not read by
 *    the host: the kernels clamp every offset into [0, n_tokens] and treat a
 *    decreasing entry as an empty sequence, so a malformed cu_seqlens gives
 *    wrong numbers but never an out-of-bounds access.  Callers that hold a
 *    host copy can validate it with r2l_check_cu_seqlens first.
 *  - Threading: calls are reentrant; concurrent calls must use distinct
 *    workspaces and outputs.  (The opt-in per-kernel timing below is the
 *    one process-wide state.)
 *  - Co-residency: with bf16 activations and d_model a multiple of 256,
 *    r2l_layer_fwd's out_proj kernel (with the LayerNorm and the residual
 *    in its epilogue) runs at most one block per compute unit, and the
 *    blocks sharing a 256-row block exchange row statistics while they run.
 *    Work on other streams of the same GPU can delay some of them; a block
 *    waits a bounded number of polls (many seconds) and past that writes
 *    NaN for its rows rather than wait longer, so it never hangs the GPU.
 *  - Supported shapes: d_state == 16, d_conv == 4, d_model and d_inner
 *    multiples of 64 with d_model <= 8192, 1 <= dt_rank <= 1024,
 *    nseq >= 1, n_tokens >= 0 (all int32-indexable).
 */
#ifndef R2L_H
#define R2L_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define R2L_VERSION 100

/* Status codes. */
enum {
  R2L_OK = 0,
  R2L_ERR_INVALID_ARG = -1,  /* null pointer, bad size, malformed host cu_seqlens */
  R2L_ERR_UNSUPPORTED = -2,  /* shape or dtype outside the supported set */
  R2L_ERR_WORKSPACE = -3,    /* workspace missing or smaller than the query */
  R2L_ERR_HIP = -4           /* a HIP launch or runtime call failed */
};

/* Flags for r2l_layer_fwd (all three), r2l_conv_fwd and r2l_scan_fwd (R2L_FLAG_L2R). */
#define R2L_FLAG_NO_LN 0x1u  /* skip the stream LayerNorm: r = unflipped Mamba output */
/* Run the conv and the scan left to right instead (a causal conv and a forward
 * scan over each sequence, no flips): the "L2R Mamba" control of the pages'
 * ablation (§4.4, Table 4), the same block in the original direction.  Every
 * other step is unchanged; results are those of the default direction on
 * each sequence reversed, reversed back. */
#define R2L_FLAG_L2R 0x2u
/* r2l_layer_fwd only: keep the activations r2l_layer_bwd reads (the in_proj
 * output, the x_proj output, the gated scan output and the out_proj output)
 * in the workspace, each in a region of its own, so that the backward need
 * not recompute the forward.  The workspace is then
 * r2l_layer_train_workspace_bytes(...) bytes; the results are the same. */
#define R2L_FLAG_TRAIN 0x4u

/* LayerNorm epsilon used by r2l_layer_fwd (biased variance over d_model). */
#define R2L_LN_EPS 1e-5f

/* Activation dtypes, the values of an r2l_dtype argument.  r2l_dtype is a
 * plain 32-bit integer (the size of an enum in this ABI) so that every
 * value a caller passes can be checked: any other value is rejected. */
enum { R2L_F32 = 0, R2L_BF16 = 1 };
typedef int32_t r2l_dtype;

/* Layer dimensions: D = d_model, E = d_inner (expand * D), N = d_state,
 * R = dt_rank, K = d_conv. */
typedef struct {
  int32_t d_model, d_inner, d_state, dt_rank, d_conv;
} r2l_dims;

/* One hook's parameters (device pointers).  "act" = activation dtype. */
typedef struct {
  const void* in_proj_w;   /* act  [2E, D]: rows [0,E) give x, rows [E,2E) give z */
  const void* conv_w;      /* act  [E, K]: depthwise taps in causal order of the flipped sequence */
  const void* conv_b;      /* act  [E] */
  const void* x_proj_w;    /* act  [R+2N, E]: rows [0,R) delta, [R,R+N) B, [R+N,R+2N) C */
  const void* dt_proj_w;   /* act  [E, R] */
  const void* out_proj_w;  /* act  [D, E] */
  const float* dt_proj_b;  /* f32  [E]   (added before softplus) */
  const float* A_log;      /* f32  [E, N] (A = -exp(A_log)) */
  const float* Dskip;      /* f32  [E] */
  const float* ln_w;       /* f32  [D]   LayerNorm gamma */
  const float* ln_b;       /* f32  [D]   LayerNorm beta */
  const float* s;          /* f32  [1]   scalar gate s (device) */
} r2l_weights;

/* Gradients of one hook's parameters (device pointers, f32, same shapes as
 * r2l_weights; written, not accumulated).  ln_w and ln_b may be NULL under
 * R2L_FLAG_NO_LN. */
typedef struct {
  float* in_proj_w;   /* [2E, D] */
  float* conv_w;      /* [E, K] */
  float* conv_b;      /* [E] */
  float* x_proj_w;    /* [R+2N, E] */
  float* dt_proj_w;   /* [E, R] */
  float* out_proj_w;  /* [D, E] */
  float* dt_proj_b;   /* [E] */
  float* A_log;       /* [E, N] */
  float* Dskip;       /* [E] */
  float* ln_w;        /* [D] */
  float* ln_b;        /* [D] */
  float* s;           /* [1] */
} r2l_grads;

/* ------------------------------------------------------------------------
 * r2l_layer_fwd -- one ReverseMambaLayer hook (§3.4 steps 1-4):
 *   h_out = h_in + tanh(s) * LN(flip(Mamba1(flip(h_in))))   per sequence.
 * h_in, h_out: act [n_tokens, D]; h_out may equal h_in (in place).
 * When tanh(s) == 0 the output is a bit-exact copy of h_in (§3.5: a zero
 * gate leaves the causal baseline unchanged).
 * branch_out: optional f32 [n_tokens, D] receiving the branch r (the LN
 * output, or the raw Mamba output under R2L_FLAG_NO_LN); NULL to skip.
 * max_seqlen: an upper bound on the longest sequence (used to plan the
 * scan's time chunks; correctness does not depend on it).
 * workspace: device buffer of at least r2l_layer_workspace_bytes(...)
 * bytes, 256-byte aligned; its contents on entry are ignored.
 * ---------------------------------------------------------------------- */
size_t r2l_layer_workspace_bytes(const r2l_dims* dims, r2l_dtype act, int64_t n_tokens,
                                 int32_t nseq, int32_t max_seqlen);
/* The workspace of r2l_layer_fwd with R2L_FLAG_TRAIN (the "saved" buffer of
 * r2l_layer_bwd). */
size_t r2l_layer_train_workspace_bytes(const r2l_dims* dims, r2l_dtype act, int64_t n_tokens,
                                       int32_t nseq, int32_t max_seqlen);

int r2l_layer_fwd(const r2l_dims* dims, r2l_dtype act, uint32_t flags, const r2l_weights* w,
                  const void* h_in, void* h_out, const int32_t* cu_seqlens, int32_t nseq,
                  int64_t n_tokens, int32_t max_seqlen, void* workspace, size_t workspace_bytes,
                  float* branch_out, void* stream);

/* ------------------------------------------------------------------------
 * r2l_layer_fwd_noalloc -- r2l_layer_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments and results as
 * r2l_layer_fwd minus the workspace: the library's own static device array
 * of R2L_NOALLOC_SCRATCH_BYTES (128 MiB) serves as the workspace.  Each GPU
 * the library runs on holds one copy of it until the process ends; its
 * address is resolved (hipGetSymbolAddress) on the first call on a device,
 * with that device current.  The call allocates nothing.
 *  - Returns R2L_ERR_WORKSPACE when r2l_layer_workspace_bytes(...) for the
 *    call exceeds R2L_NOALLOC_SCRATCH_BYTES (at d_model 2048, d_inner 4096,
 *    dt_rank 128: up to about 2,000 tokens, e.g. a denoise step of 8 blocks
 *    of 128), R2L_ERR_UNSUPPORTED with R2L_FLAG_TRAIN (its saved activations
 *    would be overwritten by the next call), R2L_ERR_INVALID_ARG for shapes
 *    the query rejects, R2L_ERR_HIP if the array cannot be resolved.
 *  - Every call on a GPU shares that GPU's array and leaves its contents
 *    behind; calls do not depend on them.  Calls that overlap in time on one
 *    GPU (concurrent streams or host threads) race on the array: the caller
 *    must order them, e.g. on one stream.
 * ---------------------------------------------------------------------- */
#define R2L_NOALLOC_SCRATCH_BYTES (128ull << 20)
int r2l_layer_fwd_noalloc(const r2l_dims* dims, r2l_dtype act, uint32_t flags, const r2l_weights* w,
                          const void* h_in, void* h_out, const int32_t* cu_seqlens, int32_t nseq,
                          int64_t n_tokens, int32_t max_seqlen, float* branch_out, void* stream);

/* ------------------------------------------------------------------------
 * r2l_layer_bwd -- the gradient of r2l_layer_fwd for training the sidecar
 * (§3.5, plug-in mode: the backbone is frozen, the Mamba block, the stream
 * LayerNorm and the gate s are trained).  Given g_out = dL/dh+ for the
 * output of r2l_layer_fwd on h_in, it writes dh = dL/dh_in (act [n_tokens,
 * D]; may equal g_out) and every parameter gradient (r2l_grads, f32).
 * With saved == NULL the forward is recomputed inside (activation
 * checkpointing): in_proj, the conv + SiLU + x_proj, dt, the scan and
 * out_proj.  saved (read only): the workspace of an r2l_layer_fwd call with
 * R2L_FLAG_TRAIN on the same h_in, Mamba-block weights, direction,
 * offsets and sizes, untouched since; then only the conv + SiLU output and
 * dt are recomputed (the forward keeps neither).  Then, in reverse: the
 * LayerNorm + gate, out_proj, the scan (r2l_scan_bwd's two sweeps), dt_proj
 * and softplus, x_proj, the conv + SiLU and in_proj.  Products go through
 * the same GEMM as the forward (bf16 operands on MFMA, fp32 accumulation
 * and fp32 results for bf16 activations; the fp32 kernel for fp32), with
 * the transposed operands materialised.  Sums over tokens run in a fixed
 * order: results are deterministic.
 * flags: 0, R2L_FLAG_NO_LN and/or R2L_FLAG_L2R (the left-to-right layer:
 * computed as the default layer's gradient of every sequence reversed, with
 * dh reversed back; with saved != NULL it returns R2L_ERR_UNSUPPORTED).
 * bf16 activations need dt_rank a multiple of 8.  Other arguments as in
 * r2l_layer_fwd.  workspace: r2l_layer_bwd_workspace_bytes(...) bytes,
 * 256-byte aligned (several times the forward's: every recomputed
 * activation and its transpose is kept).
 * ---------------------------------------------------------------------- */
size_t r2l_layer_bwd_workspace_bytes(const r2l_dims* dims, r2l_dtype act, int64_t n_tokens, int32_t nseq,
                                     int32_t max_seqlen);

int r2l_layer_bwd(const r2l_dims* dims, r2l_dtype act, uint32_t flags, const r2l_weights* w,
                  const void* h_in, const void* g_out, void* dh, const r2l_grads* grads,
                  const int32_t* cu_seqlens, int32_t nseq, int64_t n_tokens, int32_t max_seqlen,
                  const void* saved, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * r2l_conv_fwd -- the anti-causal depthwise conv1d + bias + SiLU of the
 * flipped Mamba block (§3.4 steps 1-2), optionally followed by x_proj:
 *   u[t,e]  = SiLU(conv_b[e] + sum_{j=0}^{K-1} conv_w[e,K-1-j] * x[t+j,e]),
 *             x past the end of t's sequence taken as 0;
 *   xdbl[t] = x_proj_w @ u[t]            (only when x_proj_w != NULL).
 * x: act [n_tokens, E] with row stride ld_x elements (ld_x >= E; e.g. the
 * x half of an in_proj output has ld_x = 2E).  u_out: act [n_tokens, E]
 * (contiguous) or NULL when only xdbl is wanted; xdbl_out: f32
 * [n_tokens, R+2N] (contiguous), required iff x_proj_w != NULL.  At least
 * one output must be requested.  Needs no workspace.  flags: 0 or
 * R2L_FLAG_L2R (causal taps x[t-j], x before the sequence start taken as 0);
 * other bits return R2L_ERR_INVALID_ARG.
 * ---------------------------------------------------------------------- */
int r2l_conv_fwd(const r2l_dims* dims, r2l_dtype act, uint32_t flags, const void* x, int64_t ld_x,
                 const void* conv_w, const void* conv_b, const void* x_proj_w, void* u_out,
                 float* xdbl_out, const int32_t* cu_seqlens, int32_t nseq, int64_t n_tokens,
                 int32_t max_seqlen, void* stream);

/* ------------------------------------------------------------------------
 * r2l_scan_fwd -- the selective scan run right to left per sequence (the
 * scan of §3.4 step 2 seen from the original token order), with the skip
 * term and the SiLU(z) gate:
 *   h_t = exp(dt_t * A) (.) h_{t+1} + (dt_t * u_t) (x) B_t,  h = 0 past the
 *   sequence end, A = -exp(A_log);
 *   y_t = (h_t . C_t + Dskip (.) u_t) * SiLU(z_t).
 * u: act [n_tokens, E] (row stride ld_u); dt: f32 [n_tokens, E] (row
 * stride ld_dt), already softplus-ed; B, C: f32 [n_tokens, N] (row stride
 * ld_bc each); Dskip: f32 [E] or NULL (no skip term); z: act (row stride
 * ld_z) or NULL (no gate); y_out: act [n_tokens, E] contiguous.
 * u, dt, z and y_out must be 16-byte aligned, with ld_u and ld_z multiples
 * of 8 (bf16) or 4 (f32) elements and ld_dt a multiple of 4; B and C have
 * no alignment requirement.  A row stride whose 64 rows exceed 2^31 - 1
 * bytes returns R2L_ERR_UNSUPPORTED (rows are addressed with 32-bit offsets
 * inside windows of a few dozen rows).
 * flags: 0 or R2L_FLAG_L2R (the recurrence run left to right,
 * h_t = exp(dt_t A) h_{t-1} + ..., h = 0 before the sequence start); other
 * bits return R2L_ERR_INVALID_ARG.
 * workspace: r2l_scan_workspace_bytes(...) bytes, 256-byte aligned.
 * ---------------------------------------------------------------------- */
size_t r2l_scan_workspace_bytes(const r2l_dims* dims, int64_t n_tokens, int32_t nseq,
                                int32_t max_seqlen);

int r2l_scan_fwd(const r2l_dims* dims, r2l_dtype act, uint32_t flags, const void* u, int64_t ld_u,
                 const float* dt, int64_t ld_dt, const float* A_log, const float* B,
                 const float* C, int64_t ld_bc, const float* Dskip, const void* z, int64_t ld_z,
                 void* y_out, const int32_t* cu_seqlens, int32_t nseq, int64_t n_tokens,
                 int32_t max_seqlen, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * r2l_scan_bwd -- the gradient of r2l_scan_fwd (the backward of the
 * reverse selective scan, for training the sidecar: §3.5, plug-in mode).
 * Given dy, the gradient of a loss with respect to y_out of r2l_scan_fwd on
 * the same inputs, it writes the gradients with respect to every input:
 *   du, ddt: f32 [n_tokens, E] contiguous;  dA_log: f32 [E, N] (w.r.t.
 *   A_log, summed over tokens);  dB, dC: f32 [n_tokens, N] contiguous;
 *   dDskip: f32 [E] (required iff Dskip != NULL);  dz: f32 [n_tokens, E]
 *   contiguous (required iff z != NULL).
 * Inputs as in r2l_scan_fwd; dy: act [n_tokens, E] (row stride ld_dy, the
 * same alignment rules as u).  flags: 0 (R2L_FLAG_L2R returns
 * R2L_ERR_UNSUPPORTED: the backward runs the default direction only).
 * Method: a first sweep recomputes the states right to left and keeps the
 * state entering every 16-token sub-block; a second sweep runs the adjoint
 * recurrence left to right, recomputing each sub-block's states; sums over
 * channels, chunks and sequences are taken in a fixed order
 * (deterministic).  When the sequences give fewer than 512 blocks of 64
 * channels, both sweeps also cut the sequences into time chunks, carried
 * across through chunk summaries.
 * workspace: r2l_scan_bwd_workspace_bytes(...) bytes, 256-byte aligned.
 * ---------------------------------------------------------------------- */
size_t r2l_scan_bwd_workspace_bytes(const r2l_dims* dims, int64_t n_tokens, int32_t nseq);

int r2l_scan_bwd(const r2l_dims* dims, r2l_dtype act, uint32_t flags, const void* u, int64_t ld_u,
                 const float* dt, int64_t ld_dt, const float* A_log, const float* B, const float* C,
                 int64_t ld_bc, const float* Dskip, const void* z, int64_t ld_z, const void* dy,
                 int64_t ld_dy, float* du, float* ddt, float* dA_log, float* dB, float* dC,
                 float* dDskip, float* dz, const int32_t* cu_seqlens, int32_t nseq, int64_t n_tokens,
                 void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * r2l_gemm_nt -- the dense projection used by the layer (in_proj, out_proj):
 *   C[m, n] = sum_k A[m, k] * B[n, k]      (C = A @ B^T, fp32 accumulate).
 * A: act [M, K] (row stride lda); B: act [N, K] (row stride ldb);
 * C: [M, N] (row stride ldc) in the activation dtype (out_f32 == 0) or in
 * f32 (out_f32 != 0).  bf16 runs on the MFMA matrix cores.  K must be a
 * multiple of 8 and lda/ldb multiples of 8 for bf16.
 * workspace (optional; NULL with workspace_bytes 0 is valid): device
 * scratch, 16-byte aligned.  With it, large bf16 problems split the output
 * tiles left over after the last whole round over the GPU's compute units
 * along K (fp32 partial sums, added in a fixed order, so results are
 * deterministic); up to 256 KiB per compute unit is used.
 * ---------------------------------------------------------------------- */
int r2l_gemm_nt(r2l_dtype act, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                const void* B, int64_t ldb, void* C, int64_t ldc, int out_f32, void* workspace,
                size_t workspace_bytes, void* stream);

/* Host-side validation of a host copy of cu_seqlens: cu[0] == 0,
 * non-decreasing, cu[nseq] == n_tokens, every length <= max_seqlen.
 * Returns R2L_OK or R2L_ERR_INVALID_ARG.  Touches no device. */
int r2l_check_cu_seqlens(const int32_t* cu_seqlens_host, int32_t nseq, int64_t n_tokens,
                         int32_t max_seqlen);

/* ------------------------------------------------------------------------
 * Per-kernel timing, for benchmarking.  Off by default; its state is
 * process-wide (one registry shared by all threads and devices) and it is
 * the one part of the library that holds state between calls.
 * r2l_timing_enable(1) creates a pool of 4096 HIP events on the current
 * device (R2L_ERR_HIP if that fails); no other call creates events.  While
 * enabled, each kernel the library launches is bracketed by a pair of pool
 * events recorded on its stream, except when that stream is being captured
 * into a HIP graph (captured launches are never timed, so graphs hold no
 * event records) or when the pool is exhausted (up to 2048 launches between
 * reads are timed; later ones are not).  r2l_timing_read synchronises on
 * the recorded events, adds each kernel's elapsed time to a per-kernel-name
 * total, returns the events to the pool and clears the list; it returns the
 * number of distinct kernel names (at most max_names are written).
 * names[i] point to static strings.  r2l_timing_reset waits for and drops
 * the recorded events and the totals.
 * ---------------------------------------------------------------------- */
int r2l_timing_enable(int enable);
int r2l_timing_read(const char** names, double* total_ms, int64_t* counts, int max_names);
int r2l_timing_reset(void);

const char* r2l_status_string(int status);
int r2l_version(void);

#ifdef __cplusplus
}
#endif

#endif /* R2L_H */
