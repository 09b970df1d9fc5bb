// C ABI of libr2l.so: argument validation, workspace layout, the launch
// sequence of one ReverseMambaLayer hook, and optional per-kernel timing.
// The operations are those of "Bifocal Diffusion Language Models", §3.4
// (R2L stream steps 1-4); shapes per §4.1.
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/r2l.h"
#include "kernels.h"

using namespace r2l;

namespace {

// ---------------------------------------------------------------------------
// per-kernel timing (process-wide, opt-in): r2l_timing_enable creates a pool
// of events once; a launch is timed only while the pool has two free events
// and its stream is not being captured into a graph, so the launch path
// itself never creates an event and a captured graph holds no event record.
// ---------------------------------------------------------------------------
constexpr size_t kEventPool = 4096;
struct TimingRec {
  const char* name;
  hipEvent_t a, b;
};
struct TimingState {
  std::mutex mu;
  bool enabled = false;
  std::vector<TimingRec> recs;
  std::vector<hipEvent_t> pool;
  std::vector<const char*> names;
  std::vector<double> totals;
  std::vector<int64_t> counts;
};
TimingState& timing() {
  static TimingState* t = new TimingState();  // never destroyed: safe at process exit
  return *t;
}

template <typename F>
int run_kernel(const char* name, hipStream_t st, F&& launch) {
  TimingState& t = timing();
  hipEvent_t ea = nullptr, eb = nullptr;
  bool en;
  {
    std::lock_guard<std::mutex> g(t.mu);
    en = t.enabled && t.pool.size() >= 2;
    if (en) {
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) en = false;
    }
    if (en) {
      ea = t.pool.back();
      t.pool.pop_back();
      eb = t.pool.back();
      t.pool.pop_back();
    }
  }
  if (en && hipEventRecord(ea, st) != hipSuccess) en = false;
  hipError_t err = launch();
  if (en) {
    const bool ok = hipEventRecord(eb, st) == hipSuccess;
    std::lock_guard<std::mutex> g(t.mu);
    if (ok) {
      t.recs.push_back({name, ea, eb});
    } else {
      t.pool.push_back(ea);
      t.pool.push_back(eb);
    }
  } else if (ea || eb) {
    std::lock_guard<std::mutex> g(t.mu);
    if (ea) t.pool.push_back(ea);
    if (eb) t.pool.push_back(eb);
  }
  return err == hipSuccess ? R2L_OK : R2L_ERR_HIP;
}

#define R2L_RUN(name, st, expr)                                 \
  do {                                                          \
    int _rc = run_kernel(name, st, [&]() { return (expr); });   \
    if (_rc != R2L_OK) return _rc;                              \
  } while (0)

// ---------------------------------------------------------------------------
// validation helpers
// ---------------------------------------------------------------------------
constexpr int kTB = 32;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_dims(const r2l_dims* d) {
  if (!d) return R2L_ERR_INVALID_ARG;
  if (d->d_model <= 0 || d->d_inner <= 0 || d->d_state <= 0 || d->dt_rank <= 0 || d->d_conv <= 0)
    return R2L_ERR_INVALID_ARG;
  if (d->d_state != 16 || d->d_conv != 4) return R2L_ERR_UNSUPPORTED;
  if (d->d_model % 64 || d->d_inner % 64 || d->d_model > 8192 || d->d_inner > (1 << 20))
    return R2L_ERR_UNSUPPORTED;
  if (d->dt_rank > 1024) return R2L_ERR_UNSUPPORTED;
  return R2L_OK;
}

int check_tokens(r2l_dtype act, int64_t n_tokens, int32_t nseq, int32_t max_seqlen) {
  if (act != R2L_F32 && act != R2L_BF16) return R2L_ERR_UNSUPPORTED;
  if (n_tokens < 0 || nseq < 1 || max_seqlen < 0) return R2L_ERR_INVALID_ARG;
  if (n_tokens > INT32_MAX / 2 || nseq > (1 << 24)) return R2L_ERR_UNSUPPORTED;
  return R2L_OK;
}

// ---------------------------------------------------------------------------
// scan planning: time-chunk length so that enough blocks exist
// ---------------------------------------------------------------------------
struct ScanPlan {
  int Lc, max_chunks;
  bool summary;
  size_t off_cu, off_chunks, off_n, off_sumS, off_sumP, total;
};

// Compute units of the current device (cached per device; a race between
// threads only stores the same value twice).
int num_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

ScanPlan plan_scan(int E, int64_t T, int32_t nseq, int32_t max_seqlen, size_t base) {
  ScanPlan p{};
  const int64_t NB = E / 64;
  const int64_t target = 512;  // scan blocks resident at once: 2 per CU (LDS-bound)
  int64_t ms = max_seqlen < 1 ? 1 : max_seqlen;
  if (T > 0 && ms > T) ms = T;
  int64_t Lc = ms;
  if ((int64_t)nseq * NB < target && T > 0) {
    int64_t want = (T * NB + target - 1) / target;
    want = ((want + kTB - 1) / kTB) * kTB;
    if (want < 4 * kTB) want = 4 * kTB;
    if (want < Lc) Lc = want;
  }
  if (Lc >= ms) {
    // No chunking wanted: every sequence is one chunk whatever its length
    // (a max_seqlen below the true longest length then costs parallelism,
    // never correctness), and no summary pass is needed.
    Lc = T > 0 ? T : 1;
    p.summary = false;
  } else {
    p.summary = true;  // some sequence may span several chunks
  }
  p.Lc = (int)Lc;
  // every chunk but a sequence's leftmost is full, so there are at most
  // nseq + T / Lc chunks whatever the true sequence lengths are
  p.max_chunks = (int)(nseq + (T + Lc - 1) / Lc);
  if (p.max_chunks < 1) p.max_chunks = 1;
  size_t off = base;
  p.off_cu = off;      off = align_up(off + sizeof(int32_t) * ((size_t)nseq + 1));
  p.off_chunks = off;  off = align_up(off + sizeof(ChunkDesc) * (size_t)p.max_chunks);
  p.off_n = off;       off = align_up(off + sizeof(int32_t));
  const size_t sums = p.summary ? sizeof(float) * 16 * (size_t)E * (size_t)p.max_chunks : 0;
  p.off_sumS = off;    off = align_up(off + sums);
  p.off_sumP = off;    off = align_up(off + sums);
  p.total = off;
  return p;
}

// Workspace of the scan backward: one chunk per sequence (no carries), the
// state entering every 16-token sub-block, the per-channel-block dB | dC
// partials and the per-sequence dA_log / dDskip partials.
// Time chunks as the forward scan cuts them when the sequences alone would
// leave the GPU idle (fewer than 512 blocks of 64 channels): chunks of Lc
// tokens (a multiple of 32) cut from each sequence's end.  Both sweeps then
// carry across chunks through chunk summaries: the state sweep the forward's
// (S, P), the adjoint its own (M, Q).
struct ScanBwdPlan {
  int max_chunks, Lc;
  bool chunked;
  size_t off_cu, off_chunks, off_n, off_hc, off_dbc, off_dA, off_dD, off_sumS, off_sumP, off_adjM, off_adjQ, total;
};

ScanBwdPlan plan_scan_bwd(int E, int64_t T, int32_t nseq) {
  ScanBwdPlan p{};
  const int64_t NB = E / 64, target = 512;
  int64_t Lc = T > 0 ? T : 1;
  if ((int64_t)nseq * NB < target && T > 0) {
    int64_t want = (T * NB + target - 1) / target;
    want = ((want + kTB - 1) / kTB) * kTB;
    if (want < 4 * kTB) want = 4 * kTB;
    if (want < Lc) Lc = want;
  }
  p.chunked = Lc < T;
  p.Lc = (int)Lc;
  p.max_chunks = (int)(nseq + (p.chunked ? (T + Lc - 1) / Lc : 0));
  if (p.max_chunks < 1) p.max_chunks = 1;
  // 16-token state slots: every chunk but a sequence's leftmost is a multiple of 32 long
  const size_t slots = (size_t)(T / 16) + (size_t)p.max_chunks + 1;
  const size_t sumsz = p.chunked ? sizeof(float) * 16 * (size_t)E * (size_t)p.max_chunks : 0;
  size_t off = 0;
  p.off_cu = off;     off = align_up(off + sizeof(int32_t) * ((size_t)nseq + 1));
  p.off_chunks = off; off = align_up(off + sizeof(ChunkDesc) * (size_t)p.max_chunks);
  p.off_n = off;      off = align_up(off + sizeof(int32_t));
  p.off_hc = off;     off = align_up(off + sizeof(float) * 16 * (size_t)E * slots);
  p.off_dbc = off;    off = align_up(off + sizeof(float) * 32 * (size_t)(E / 64) * (size_t)T);
  p.off_dA = off;     off = align_up(off + sizeof(float) * 16 * (size_t)E * (size_t)p.max_chunks);
  p.off_dD = off;     off = align_up(off + sizeof(float) * (size_t)E * (size_t)p.max_chunks);
  p.off_sumS = off;   off = align_up(off + sumsz);
  p.off_sumP = off;   off = align_up(off + sumsz);
  p.off_adjM = off;   off = align_up(off + sumsz);
  p.off_adjQ = off;   off = align_up(off + sumsz);
  p.total = off;
  return p;
}

// Scratch for K-split partial sums (GEMM tiles, conv channel splits): up to
// one 256 x 256 fp32 tile per compute unit of a 256-CU device.
constexpr size_t kSplitScratch = 256ull * 256 * 256 * sizeof(float);

struct LayerPlan {
  size_t off_xz, off_xdbl, off_xdbl2, off_xdbl3, off_dsplit, off_u, off_y, off_scratch, off_o, off_lnst, off_lncnt;
  bool need_u, fuse_ln;   // fuse_ln: out_proj may run fused with the LayerNorm and the gated residual
  ScanPlan scan;
  size_t total;
};

// train: out_proj's output gets a region of its own (the backward reads both
// it and the in_proj output); otherwise it reuses the in_proj output's.
LayerPlan plan_layer(const r2l_dims* d, r2l_dtype act, int64_t T, int32_t nseq, int32_t max_seqlen,
                     bool train = false) {
  LayerPlan p{};
  const size_t sa = act == R2L_BF16 ? 2 : 4;
  const size_t D = d->d_model, E = d->d_inner, P = d->dt_rank + 2 * d->d_state;
  const size_t Tz = (size_t)T;
  size_t off = 0;
  size_t xz = Tz * 2 * E * sa, o = Tz * D * 4;
  p.off_xz = off;   off = align_up(off + (train ? xz : (xz > o ? xz : o)));
  p.off_o = train ? off : p.off_xz;
  if (train) off = align_up(off + o);
  p.off_xdbl = off; off = align_up(off + Tz * P * 4);
  // second and third partial x_proj sums of the split-K conv kernel (bf16, large T)
  p.off_xdbl2 = off; off = align_up(off + (act == R2L_BF16 ? Tz * P * 4 : 0));
  p.off_xdbl3 = off; off = align_up(off + (act == R2L_BF16 ? Tz * P * 4 : 0));
  // delta split for the scan's dt_proj on MFMA (bf16): [T, 2 RP] bf16
  p.off_dsplit = off; off = align_up(off + (act == R2L_BF16 ? Tz * 4 * (size_t)delta_split_width(d->dt_rank) : 0));
  p.need_u = act == R2L_F32 || P > 256;
  p.off_u = off;    off = align_up(off + (p.need_u ? Tz * E * sa : 0));
  p.off_y = off;    off = align_up(off + Tz * E * sa);
  p.off_scratch = off; off = align_up(off + (act == R2L_BF16 ? kSplitScratch : 0));
  // the fused out_proj + LayerNorm (bf16; in training mode it also stores
  // out_proj's output for the backward): per-row partial statistics of
  // every row block's column tiles, and one counter per row block (sized
  // for every whole row block, whatever the device; the launch plan is made
  // per call from the device's compute units)
  p.fuse_ln = act == R2L_BF16 && D % 256 == 0;
  const size_t rbmax = p.fuse_ln ? Tz / 256 : 0;
  p.off_lnst = off;  off = align_up(off + rbmax * D * 8);
  p.off_lncnt = off; off = align_up(off + rbmax * sizeof(int));
  p.scan = plan_scan((int)E, T, nseq, max_seqlen, off);
  p.total = p.scan.total;
  return p;
}

template <typename Tp>
Tp* at(void* ws, size_t off) {
  return (Tp*)((char*)ws + off);
}

template <typename T>
int run_scan(const ScanArgs& a, const ScanPlan& sp, bool fused, const int32_t* cu, int nseq,
             int64_t Tn, int32_t* cu_clean, ChunkDesc* chunks, int32_t* nch, hipStream_t st) {
  R2L_RUN("plan_chunks", st, plan_chunks(cu, nseq, (int)Tn, sp.Lc, sp.max_chunks, a.l2r, cu_clean, chunks, nch, st));
  if (sp.summary) R2L_RUN("scan_summary", st, scan_summary<T>(a, fused, st));
  R2L_RUN("scan_main", st, scan_main<T>(a, fused, st));
  return R2L_OK;
}

// Both sweeps of the scan backward and its reductions; ws laid out by
// plan_scan_bwd(E, T, nseq).
int run_scan_bwd(r2l_dtype act, int E, int R, int T, int nseq, const void* u, int64_t ld_u, const float* dt,
                 int64_t ld_dt, const float* A_log, const float* B, const float* C, int64_t ld_bc,
                 const float* Dskip, const void* z, int64_t ld_z, const void* dy, int64_t ld_dy, float* du,
                 float* ddt, float* dA_log, float* dB, float* dC, float* dDskip, float* dz,
                 const int32_t* cu_seqlens, void* workspace, hipStream_t st) {
  const ScanBwdPlan bp = plan_scan_bwd(E, T, nseq);
  int32_t* cu_clean = at<int32_t>(workspace, bp.off_cu);
  ChunkDesc* chunks = at<ChunkDesc>(workspace, bp.off_chunks);
  int32_t* nch = at<int32_t>(workspace, bp.off_n);
  float* hc = at<float>(workspace, bp.off_hc);
  // time chunks when the sequences alone would leave the GPU idle
  R2L_RUN("plan_chunks", st, plan_chunks(cu_seqlens, nseq, T, bp.Lc, bp.max_chunks, false, cu_clean, chunks, nch, st));
  // sweep 1: states every 16 tokens, and dz
  ScanArgs a{};
  a.T = T; a.E = E; a.R = R; a.ldp = 0;
  a.u = u; a.ld_u = ld_u; a.dt = dt; a.ld_dt = ld_dt;
  a.Bm = B; a.Cm = C; a.ld_bc = ld_bc;
  a.z = z; a.ld_z = ld_z;
  a.A_log = A_log; a.Dskip = Dskip;
  a.chunks = chunks; a.n_chunks = nch; a.max_chunks = bp.max_chunks;
  a.l2r = false;
  a.dy = dy; a.ld_dy = ld_dy; a.dz = dz; a.hc = hc;
  if (bp.chunked) {
    a.sumS = at<float>(workspace, bp.off_sumS);
    a.sumP = at<float>(workspace, bp.off_sumP);
  }
  // sweep 2: the adjoint, then the sums over channel blocks and sequences
  ScanBwdArgs b{};
  b.T = T; b.E = E;
  b.u = u; b.ld_u = ld_u; b.dt = dt; b.ld_dt = ld_dt;
  b.Bm = B; b.Cm = C; b.ld_bc = ld_bc;
  b.A_log = A_log; b.Dskip = Dskip;
  b.z = z; b.ld_z = ld_z; b.dy = dy; b.ld_dy = ld_dy;
  b.chunks = chunks; b.n_chunks = nch;
  b.hc = hc; b.du = du; b.ddt = ddt;
  b.dbc = at<float>(workspace, bp.off_dbc);
  b.dA = at<float>(workspace, bp.off_dA);
  b.dD = at<float>(workspace, bp.off_dD);
  if (bp.chunked) {
    b.adjM = at<float>(workspace, bp.off_adjM);
    b.adjQ = at<float>(workspace, bp.off_adjQ);
  }
  if (act == R2L_BF16) {
    if (bp.chunked) R2L_RUN("scan_bwd_summary", st, scan_summary<bf16>(a, false, st));
    R2L_RUN("scan_bwd_states", st, scan_bwd_states<bf16>(a, st));
    R2L_RUN("scan_bwd_adjoint", st, scan_bwd_adjoint<bf16>(b, bp.max_chunks, dA_log, dB, dC, dDskip, st));
  } else {
    if (bp.chunked) R2L_RUN("scan_bwd_summary", st, scan_summary<float>(a, false, st));
    R2L_RUN("scan_bwd_states", st, scan_bwd_states<float>(a, st));
    R2L_RUN("scan_bwd_adjoint", st, scan_bwd_adjoint<float>(b, bp.max_chunks, dA_log, dB, dC, dDskip, st));
  }
  return R2L_OK;
}

// Workspace of the layer backward: every recomputed activation, the
// gradient buffers and the transposed GEMM operands (tokens padded to Tp, a
// multiple of 128 or 1,024, in the transposes), the forward scan's and the scan
// backward's own regions, and the GEMM split scratch.
struct LayerBwdPlan {
  size_t xz, u, xdbl, xdbl2, xdbl3, delta, dt, yg, o, scanf, dout, gx, gr, do_a, doT, ygT, wT, dyg, du, ddt, dz, dB,
      dC, scanb, ddt_a, ddtT, deltaT, ddelta, dxdbl_a, dxdblT, uT, dux, convp, dxz_a, dxzT, hT, dhb, colp, dtpart,
      hflip, gflip, scratch;
  ScanPlan sp;
  int Tp;
  size_t total;
};

LayerBwdPlan plan_layer_bwd(const r2l_dims* d, r2l_dtype act, int64_t T, int32_t nseq, int32_t max_seqlen) {
  LayerBwdPlan p{};
  const size_t sa = act == R2L_BF16 ? 2 : 4, f = 4;
  const size_t D = d->d_model, E = d->d_inner, N = d->d_state, R = d->dt_rank, P = R + 2 * N;
  const size_t Tz = (size_t)T;
  // Tp is the K of the weight-gradient GEMMs (sums over tokens).  A multiple
  // of 1,024 (when that pads by at most 1/32 of T) lets them split K over
  // the CUs their few output tiles leave idle: the splits keep whole 128-deep
  // chunks, so e.g. 33,024 tokens as 33,152 (1,036 steps of 32) allow none,
  // as 33,792 (1,056 steps) two to eight.  The padded tokens are zeros.
  p.Tp = (int)(((T + 1023) / 1024) * 1024);
  if (p.Tp - T > T / 32) p.Tp = (int)(((T + 127) / 128) * 128);
  const size_t Tp = (size_t)p.Tp;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  p.xz = take(Tz * 2 * E * sa);
  p.u = take(Tz * E * sa);
  p.xdbl = take(Tz * P * f);
  p.xdbl2 = take(act == R2L_BF16 ? Tz * P * f : 0);
  p.xdbl3 = take(act == R2L_BF16 ? Tz * P * f : 0);
  p.delta = take(Tz * R * sa);
  p.dt = take(Tz * E * f);
  p.yg = take(Tz * E * sa);
  p.o = take(Tz * D * f);
  p.sp = plan_scan((int)E, T, nseq, max_seqlen, 0);
  p.scanf = take(p.sp.total);
  p.dout = take(Tz * D * f);
  p.gx = take((size_t)ln_bwd_parts((int)T) * 2 * D * f);
  p.gr = take(Tz * f);
  p.do_a = take(Tz * D * sa);
  p.doT = take(D * Tp * sa);
  p.ygT = take(E * Tp * sa);
  // W_out^T [E, D], W_dt^T [R, E], W_x^T [E, P], W_in^T [D, 2E] share one
  // region, sized for the largest of the four (P = R + 2N exceeds 2D when
  // the model is narrow and dt_rank large)
  size_t wt = 2 * E * D;
  if (R * E > wt) wt = R * E;
  if (E * P > wt) wt = E * P;
  p.wT = take(wt * sa);
  p.dyg = take(Tz * E * sa);
  p.du = take(Tz * E * f);
  p.ddt = take(Tz * E * f);
  p.dz = take(Tz * E * f);
  p.dB = take(Tz * N * f);
  p.dC = take(Tz * N * f);
  p.scanb = take(plan_scan_bwd((int)E, T, nseq).total);
  p.ddt_a = take(Tz * E * sa);
  p.ddtT = take(E * Tp * sa);
  p.deltaT = take(R * Tp * sa);
  p.ddelta = take(Tz * R * f);
  p.dxdbl_a = take(Tz * P * sa);
  p.dxdblT = take(P * Tp * sa);
  p.uT = take(E * Tp * sa);
  p.dux = take(Tz * E * f);
  p.convp = take((size_t)conv_bwd_parts((int)T) * E * 5 * f);
  p.dxz_a = take(Tz * 2 * E * sa);
  p.dxzT = take(2 * E * Tp * sa);
  p.hT = take(D * Tp * sa);
  p.dhb = take(Tz * D * f);
  p.colp = take((size_t)colsum_parts((int)T) * (E > D ? E : D) * f);
  p.dtpart = take((size_t)((T + 63) / 64) * E * f);
  // h and g reversed per sequence (the left-to-right direction)
  p.hflip = take(Tz * D * sa);
  p.gflip = take(Tz * D * sa);
  p.scratch = take(act == R2L_BF16 ? kSplitScratch : 0);
  p.total = off;
  return p;
}

// l2r: the left-to-right layer's gradient is the default layer's gradient
// of every sequence reversed (h and g), with dh reversed back; the
// parameter gradients are the same.
template <typename A>
int run_layer_bwd(const r2l_dims* d, r2l_dtype act, bool no_ln, bool l2r, const r2l_weights* w, const A* h,
                  const A* g, A* dh, const r2l_grads* gr, const int32_t* cu_seqlens, int nseq, int T,
                  int32_t max_seqlen, const void* saved, void* ws, hipStream_t st) {
  const LayerBwdPlan p = plan_layer_bwd(d, act, T, nseq, max_seqlen);
  if (l2r) {
    A* hf = at<A>(ws, p.hflip);
    A* gf = at<A>(ws, p.gflip);
    R2L_RUN("bwd_flip", st, flip_rows<A>(T, d->d_model, h, d->d_model, hf, d->d_model, cu_seqlens, nseq, st));
    R2L_RUN("bwd_flip", st, flip_rows<A>(T, d->d_model, g, d->d_model, gf, d->d_model, cu_seqlens, nseq, st));
    h = hf;
    g = gf;
  }
  const int D = d->d_model, E = d->d_inner, N = d->d_state, R = d->dt_rank, P = R + 2 * N, Tp = p.Tp;
  const bool bf = act == R2L_BF16;
  const int ncu = bf ? num_cus() : 0;
  float* scratch = at<float>(ws, p.scratch);
  // C = A B^T: bf16 operands on MFMA (act-typed or f32 result), or the fp32 kernel
  auto gemm = [&](int M, int Nn, int K, const A* a, long lda, const A* b, long ldb, void* c, long ldc,
                  bool out_f32) -> hipError_t {
    if constexpr (std::is_same<A, bf16>::value)
      return gemm_bf16_nt(M, Nn, K, a, lda, b, ldb, c, ldc, out_f32, st, scratch, kSplitScratch, ncu);
    else
      return gemm_f32_nt(M, Nn, K, a, lda, b, ldb, (float*)c, ldc, st);
  };
  A* xz = at<A>(ws, p.xz);
  A* u = at<A>(ws, p.u);
  float* xdbl = at<float>(ws, p.xdbl);
  A* delta = at<A>(ws, p.delta);
  float* dt = at<float>(ws, p.dt);
  A* yg = at<A>(ws, p.yg);
  float* o = at<float>(ws, p.o);
  A* wT = at<A>(ws, p.wT);
  const A* Win = (const A*)w->in_proj_w;
  const A* Wx = (const A*)w->x_proj_w;
  const A* Wdt = (const A*)w->dt_proj_w;
  const A* Wout = (const A*)w->out_proj_w;
  const A* cw = (const A*)w->conv_w;
  const A* cb = (const A*)w->conv_b;
  if (saved) {
    // the forward's activations, laid out by its training plan (read only)
    const LayerPlan fp = plan_layer(d, act, T, nseq, max_seqlen, true);
    void* sv = const_cast<void*>(saved);
    xz = at<A>(sv, fp.off_xz);
    xdbl = at<float>(sv, fp.off_xdbl);
    yg = at<A>(sv, fp.off_y);
    o = at<float>(sv, fp.off_o);
  }

  // ---------------- forward recompute (u and dt only, with saved activations) ----------------
  void* sfw = at<char>(ws, p.scanf);
  int32_t* cu_clean = at<int32_t>(sfw, p.sp.off_cu);
  ChunkDesc* chunks = at<ChunkDesc>(sfw, p.sp.off_chunks);
  int32_t* nch = at<int32_t>(sfw, p.sp.off_n);
  R2L_RUN("plan_chunks", st, plan_chunks(cu_seqlens, nseq, T, p.sp.Lc, p.sp.max_chunks, false, cu_clean, chunks, nch, st));
  if (!saved) R2L_RUN("bwd_in_proj", st, gemm(T, 2 * E, D, h, D, Win, D, xz, 2L * E, false));
  if constexpr (std::is_same<A, bf16>::value) {
    if (P <= 256) {
      // xdbl as the forward computes it (the split-K kernel for large inputs), u on its own
      R2L_RUN("bwd_u", st, conv_silu<bf16>(T, E, xz, 2L * E, cw, cb, u, cu_clean, nseq, false, st));
      const bool sk = (T + 127) / 128 >= ncu && (long)((T + 127) / 128) * (E / 32) < (1L << 31);
      if (!saved && sk) {
        float* xdbl2 = at<float>(ws, p.xdbl2);
        float* xdbl3 = at<float>(ws, p.xdbl3);
        R2L_RUN("bwd_conv", st, conv_xproj_bf16_sk(T, E, P, xz, 2L * E, cw, cb, Wx, xdbl, xdbl2, xdbl3, cu_clean,
                                                   nseq, ncu, false, st));
        R2L_RUN("bwd_conv_sum", st, conv_sk_sum(T, E, P, xdbl, xdbl2, xdbl3, ncu, st));
      } else if (!saved) {
        R2L_RUN("bwd_conv", st, conv_xproj_bf16(T, E, P, xz, 2L * E, cw, cb, Wx, nullptr, xdbl, cu_clean, nseq, false,
                                                st, scratch, kSplitScratch, ncu));
      }
    } else {
      R2L_RUN("bwd_conv", st, conv_silu<bf16>(T, E, xz, 2L * E, cw, cb, u, cu_clean, nseq, false, st));
      if (!saved) R2L_RUN("bwd_x_proj", st, gemm(T, P, E, u, E, Wx, E, xdbl, P, true));
    }
  } else {
    R2L_RUN("bwd_conv", st, conv_silu<float>(T, E, xz, 2L * E, cw, cb, u, cu_clean, nseq, false, st));
    if (!saved) R2L_RUN("bwd_x_proj", st, gemm(T, P, E, u, E, Wx, E, xdbl, P, true));
  }
  R2L_RUN("bwd_delta", st, (elementwise<kConvert, float, A>(T, R, xdbl, P, nullptr, 0, nullptr, delta, R, st)));
  R2L_RUN("bwd_dt_proj", st, gemm(T, E, R, delta, R, Wdt, R, dt, E, true));
  R2L_RUN("bwd_softplus", st, (elementwise<kSoftplusBias, float, float>(T, E, dt, E, nullptr, 0, w->dt_proj_b, dt, E, st)));
  if (!saved) {
    ScanArgs a{};
    a.T = T; a.E = E; a.R = R; a.ldp = 0;
    a.u = u; a.ld_u = E; a.dt = dt; a.ld_dt = E;
    a.Bm = xdbl + R; a.Cm = xdbl + R + N; a.ld_bc = P;
    a.z = xz + E; a.ld_z = 2L * E;
    a.A_log = w->A_log; a.Dskip = w->Dskip; a.y = yg;
    a.chunks = chunks; a.n_chunks = nch; a.max_chunks = p.sp.max_chunks;
    a.sumS = at<float>(sfw, p.sp.off_sumS); a.sumP = at<float>(sfw, p.sp.off_sumP);
    a.l2r = false;
    if (p.sp.summary) R2L_RUN("bwd_scan_summary", st, scan_summary<A>(a, false, st));
    R2L_RUN("bwd_scan", st, scan_main<A>(a, false, st));
    R2L_RUN("bwd_out_proj", st, gemm(T, D, E, yg, E, Wout, E, o, D, true));
  }

  // ---------------- backward ----------------
  float* dout = at<float>(ws, p.dout);
  float* gx = at<float>(ws, p.gx);
  float* grr = at<float>(ws, p.gr);
  float* colp = at<float>(ws, p.colp);
  R2L_RUN("bwd_ln_gate", st, ln_gate_bwd<A>(T, D, g, o, w->ln_w, w->ln_b, w->s, no_ln, R2L_LN_EPS, dout, gx, grr, st));
  if (!no_ln) {
    const int np = ln_bwd_parts(T);
    R2L_RUN("bwd_ln_w", st, colsum(np, D, gx, 2L * D, colp, 1.0f, gr->ln_w, st));
    R2L_RUN("bwd_ln_b", st, colsum(np, D, gx + D, 2L * D, colp, 1.0f, gr->ln_b, st));
  }
  R2L_RUN("bwd_s", st, colsum(T, 1, grr, 1, colp, 1.0f, gr->s, st));
  // out_proj: dyg = do W_out, dW_out = do^T yg
  A* do_a = at<A>(ws, p.do_a);
  A* dyg = at<A>(ws, p.dyg);
  A* doT = at<A>(ws, p.doT);
  A* ygT = at<A>(ws, p.ygT);
  R2L_RUN("bwd_do", st, (fused_t<kConvert, float, A>(T, D, Tp, dout, D, nullptr, 0, do_a, D, doT, nullptr, st)));
  R2L_RUN("bwd_WoutT", st, (transpose<A, A>(D, E, D, Wout, E, wT, st)));
  R2L_RUN("bwd_dyg", st, gemm(T, E, D, do_a, D, wT, D, dyg, E, !bf));
  R2L_RUN("bwd_ygT", st, (transpose<A, A>(T, E, Tp, yg, E, ygT, st)));
  R2L_RUN("bwd_dWout", st, gemm(D, E, Tp, doT, Tp, ygT, Tp, gr->out_proj_w, E, true));
  // the scan
  float* du = at<float>(ws, p.du);
  float* ddt = at<float>(ws, p.ddt);
  float* dz = at<float>(ws, p.dz);
  float* dB = at<float>(ws, p.dB);
  float* dC = at<float>(ws, p.dC);
  {
    const int rc = run_scan_bwd(act, E, R, T, nseq, u, E, dt, E, w->A_log, xdbl + R, xdbl + R + N, P, w->Dskip,
                                xz + E, 2L * E, dyg, E, du, ddt, gr->A_log, dB, dC, gr->Dskip, dz, cu_seqlens,
                                at<char>(ws, p.scanb), st);
    if (rc != R2L_OK) return rc;
  }
  // dt_proj + softplus: ddt_pre = ddt sigmoid(pre); d b_dt = sum ddt_pre; d delta = ddt_pre W_dt; dW_dt = ddt_pre^T delta
  // (one pass: ddt_pre, its activation-typed copy, its transpose and column sums)
  A* ddt_a = at<A>(ws, p.ddt_a);
  A* ddtT = at<A>(ws, p.ddtT);
  float* dtpart = at<float>(ws, p.dtpart);
  R2L_RUN("bwd_dt_pre", st, (fused_t<kDtPre, float, A>(T, E, Tp, ddt, E, dt, E, ddt_a, E, ddtT, dtpart, st)));
  R2L_RUN("bwd_dt_b", st, colsum((T + 63) / 64, E, dtpart, E, colp, 1.0f, gr->dt_proj_b, st));
  float* ddelta = at<float>(ws, p.ddelta);
  R2L_RUN("bwd_WdtT", st, (transpose<A, A>(E, R, E, Wdt, R, wT, st)));
  R2L_RUN("bwd_ddelta", st, gemm(T, R, E, ddt_a, E, wT, E, ddelta, R, true));
  A* deltaT = at<A>(ws, p.deltaT);
  R2L_RUN("bwd_deltaT", st, (transpose<A, A>(T, R, Tp, delta, R, deltaT, st)));
  R2L_RUN("bwd_dWdt", st, gemm(E, R, Tp, ddtT, Tp, deltaT, Tp, gr->dt_proj_w, R, true));
  // x_proj: dxdbl = [d delta | dB | dC]; du += dxdbl W_x; dW_x = dxdbl^T u
  A* dxdbl_a = at<A>(ws, p.dxdbl_a);
  float* dux = at<float>(ws, p.dux);
  R2L_RUN("bwd_dxdbl", st, concat3<A>(T, R, N, N, ddelta, dB, dC, dxdbl_a, P, st));
  R2L_RUN("bwd_WxT", st, (transpose<A, A>(P, E, P, Wx, E, wT, st)));
  R2L_RUN("bwd_dux", st, gemm(T, E, P, dxdbl_a, P, wT, P, dux, E, true));
  A* dxdblT = at<A>(ws, p.dxdblT);
  A* uT = at<A>(ws, p.uT);
  R2L_RUN("bwd_dxdblT", st, (transpose<A, A>(T, P, Tp, dxdbl_a, P, dxdblT, st)));
  R2L_RUN("bwd_uT", st, (transpose<A, A>(T, E, Tp, u, E, uT, st)));
  R2L_RUN("bwd_dWx", st, gemm(P, E, Tp, dxdblT, Tp, uT, Tp, gr->x_proj_w, E, true));
  // conv + SiLU: dx goes straight into the x half of dxz = [dx | dz]
  A* dxz_a = at<A>(ws, p.dxz_a);
  R2L_RUN("bwd_conv_bwd", st, conv_bwd<A>(T, E, xz, 2L * E, cw, cb, du, dux, dxz_a, 2L * E, at<float>(ws, p.convp),
                                          gr->conv_w, gr->conv_b, cu_clean, nseq, st));
  // in_proj: dh = g + dxz W_in; dW_in = dxz^T h
  float* dhb = at<float>(ws, p.dhb);
  A* dxzT = at<A>(ws, p.dxzT);
  // dz into the z half of dxz and of its transpose; the x half is transposed from dx
  R2L_RUN("bwd_dz", st, (fused_t<kConvert, float, A>(T, E, Tp, dz, E, nullptr, 0, dxz_a + E, 2L * E,
                                                      dxzT + (size_t)E * Tp, nullptr, st)));
  R2L_RUN("bwd_WinT", st, (transpose<A, A>(2 * E, D, 2 * E, Win, D, wT, st)));
  R2L_RUN("bwd_dh_branch", st, gemm(T, D, 2 * E, dxz_a, 2L * E, wT, 2L * E, dhb, D, true));
  A* hT = at<A>(ws, p.hT);
  R2L_RUN("bwd_dxT", st, (transpose<A, A>(T, E, Tp, dxz_a, 2L * E, dxzT, st)));
  R2L_RUN("bwd_hT", st, (transpose<A, A>(T, D, Tp, h, D, hT, st)));
  R2L_RUN("bwd_dWin", st, gemm(2 * E, D, Tp, dxzT, Tp, hT, Tp, gr->in_proj_w, D, true));
  R2L_RUN("bwd_dh", st, (elementwise<kAddTo, A, A>(T, D, g, D, dhb, D, nullptr, dh, D, st)));
  if (l2r) R2L_RUN("bwd_flip", st, flip_rows<A>(T, D, dh, D, dh, D, cu_seqlens, nseq, st));
  return R2L_OK;
}

}  // namespace

// ===========================================================================
extern "C" {

const char* r2l_status_string(int status) {
  switch (status) {
    case R2L_OK: return "ok";
    case R2L_ERR_INVALID_ARG: return "invalid argument";
    case R2L_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case R2L_ERR_WORKSPACE: return "workspace missing or too small";
    case R2L_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int r2l_version(void) { return R2L_VERSION; }

int r2l_check_cu_seqlens(const int32_t* cu, int32_t nseq, int64_t n_tokens, int32_t max_seqlen) {
  if (!cu || nseq < 1 || n_tokens < 0) return R2L_ERR_INVALID_ARG;
  if (cu[0] != 0 || (int64_t)cu[nseq] != n_tokens) return R2L_ERR_INVALID_ARG;
  for (int32_t q = 0; q < nseq; ++q) {
    const int64_t len = (int64_t)cu[q + 1] - cu[q];
    if (len < 0 || len > max_seqlen) return R2L_ERR_INVALID_ARG;
  }
  return R2L_OK;
}

size_t r2l_layer_workspace_bytes(const r2l_dims* dims, r2l_dtype act, int64_t n_tokens,
                                 int32_t nseq, int32_t max_seqlen) {
  if (check_dims(dims) != R2L_OK || check_tokens(act, n_tokens, nseq, max_seqlen) != R2L_OK)
    return 0;
  return plan_layer(dims, act, n_tokens, nseq, max_seqlen).total;
}

size_t r2l_layer_train_workspace_bytes(const r2l_dims* dims, r2l_dtype act, int64_t n_tokens,
                                       int32_t nseq, int32_t max_seqlen) {
  if (check_dims(dims) != R2L_OK || check_tokens(act, n_tokens, nseq, max_seqlen) != R2L_OK)
    return 0;
  return plan_layer(dims, act, n_tokens, nseq, max_seqlen, true).total;
}

size_t r2l_scan_workspace_bytes(const r2l_dims* dims, int64_t n_tokens, int32_t nseq,
                                int32_t max_seqlen) {
  if (check_dims(dims) != R2L_OK || check_tokens(R2L_F32, n_tokens, nseq, max_seqlen) != R2L_OK)
    return 0;
  return plan_scan(dims->d_inner, n_tokens, nseq, max_seqlen, 0).total;
}

size_t r2l_scan_bwd_workspace_bytes(const r2l_dims* dims, int64_t n_tokens, int32_t nseq) {
  if (check_dims(dims) != R2L_OK || check_tokens(R2L_F32, n_tokens, nseq, 0) != R2L_OK) return 0;
  return plan_scan_bwd(dims->d_inner, n_tokens, nseq).total;
}

int r2l_layer_fwd(const r2l_dims* d, r2l_dtype act, uint32_t flags, const r2l_weights* w,
                  const void* h_in, void* h_out, const int32_t* cu_seqlens, int32_t nseq,
                  int64_t n_tokens, int32_t max_seqlen, void* workspace, size_t workspace_bytes,
                  float* branch_out, void* stream) {
  int rc = check_dims(d);
  if (rc != R2L_OK) return rc;
  if ((rc = check_tokens(act, n_tokens, nseq, max_seqlen)) != R2L_OK) return rc;
  if (flags & ~(R2L_FLAG_NO_LN | R2L_FLAG_L2R | R2L_FLAG_TRAIN)) return R2L_ERR_INVALID_ARG;
  const bool l2r = flags & R2L_FLAG_L2R;
  if (!w || !h_in || !h_out || !cu_seqlens) return R2L_ERR_INVALID_ARG;
  if (!w->in_proj_w || !w->conv_w || !w->conv_b || !w->x_proj_w || !w->dt_proj_w ||
      !w->out_proj_w || !w->dt_proj_b || !w->A_log || !w->Dskip || !w->s)
    return R2L_ERR_INVALID_ARG;
  const bool no_ln = flags & R2L_FLAG_NO_LN;
  if (!no_ln && (!w->ln_w || !w->ln_b)) return R2L_ERR_INVALID_ARG;
  {
    // every tensor is accessed with 16-byte vectors somewhere on the path
    const void* ptrs[] = {h_in, h_out, branch_out, w->in_proj_w, w->conv_w, w->conv_b, w->x_proj_w,
                          w->dt_proj_w, w->out_proj_w, w->ln_w, w->ln_b};
    for (const void* p : ptrs)
      if (p && !aligned16(p)) return R2L_ERR_INVALID_ARG;
  }
  const LayerPlan lp = plan_layer(d, act, n_tokens, nseq, max_seqlen, (flags & R2L_FLAG_TRAIN) != 0);
  if (!workspace || workspace_bytes < lp.total) return R2L_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return R2L_ERR_INVALID_ARG;
  if (n_tokens == 0) return R2L_OK;

  hipStream_t st = (hipStream_t)stream;
  const int T = (int)n_tokens, D = d->d_model, E = d->d_inner, R = d->dt_rank;
  const int P = R + 2 * d->d_state;
  const ScanPlan& sp = lp.scan;
  int32_t* cu_clean = at<int32_t>(workspace, sp.off_cu);
  ChunkDesc* chunks = at<ChunkDesc>(workspace, sp.off_chunks);
  int32_t* nch = at<int32_t>(workspace, sp.off_n);
  float* xdbl = at<float>(workspace, lp.off_xdbl);
  float* o = at<float>(workspace, lp.off_o);  // xz's region unless training: xz is dead by then

  ScanArgs a{};
  a.T = T; a.E = E; a.R = R; a.ldp = P;
  a.ld_x = 2L * E; a.ld_z = 2L * E;
  a.xdbl = xdbl;
  a.conv_w = w->conv_w; a.conv_b = w->conv_b;
  a.dt_w = w->dt_proj_w; a.dt_b = w->dt_proj_b;
  a.A_log = w->A_log; a.Dskip = w->Dskip;
  a.chunks = chunks; a.n_chunks = nch; a.max_chunks = sp.max_chunks;
  a.sumS = at<float>(workspace, sp.off_sumS);
  a.sumP = at<float>(workspace, sp.off_sumP);
  a.l2r = l2r;

  // the chunk table (the conv kernel also reads the sanitised offsets, and
  // the fused out_proj's counters start at zero) before the conv
  const OutLnPlan oln = lp.fuse_ln ? plan_out_ln(T, D, E, num_cus()) : OutLnPlan{};
  int* lncnt = at<int>(workspace, lp.off_lncnt);
  PlanArgs plan = plan_args(cu_seqlens, nseq, T, sp.Lc, sp.max_chunks, l2r, cu_clean, chunks, nch, lncnt,
                            oln.row_blocks);
  if (act != R2L_BF16)
    R2L_RUN("plan_chunks", st, plan_chunks(cu_seqlens, nseq, T, sp.Lc, sp.max_chunks, l2r, cu_clean, chunks, nch, st,
                                           lncnt, oln.row_blocks));

  if (act == R2L_BF16) {
    bf16* xz = at<bf16>(workspace, lp.off_xz);
    bf16* y = at<bf16>(workspace, lp.off_y);
    const int ncu = num_cus();
    float* scratch = at<float>(workspace, lp.off_scratch);
    bf16* dsplit = delta_split_width(R) > 0 ? at<bf16>(workspace, lp.off_dsplit) : nullptr;
    // in_proj; when it runs (or ends) on the mid-size kernel, one of its
    // launches (the GEMM, or its split-K sum) also runs the chunk planning,
    // as one extra block (a launch fewer)
    R2L_RUN("in_proj_gemm", st, gemm_bf16_nt(T, 2 * E, D, (const bf16*)h_in, D, (const bf16*)w->in_proj_w, D, xz, 2L * E, false, st,
                                             scratch, kSplitScratch, ncu, &plan));
    if (!plan.hosted)
      R2L_RUN("plan_chunks", st, plan_chunks(cu_seqlens, nseq, T, sp.Lc, sp.max_chunks, l2r, cu_clean, chunks, nch, st,
                                             lncnt, oln.row_blocks));
    if (!lp.need_u) {
      // (the split kernel counts (tile, step) pairs in 32 bits)
      if ((T + 127) / 128 >= ncu && (long)((T + 127) / 128) * (E / 32) < (1L << 31)) {
        // large input: split-K over one or two blocks per CU, then the parts are summed
        float* xdbl2 = at<float>(workspace, lp.off_xdbl2);
        float* xdbl3 = at<float>(workspace, lp.off_xdbl3);
        R2L_RUN("conv_xproj", st, conv_xproj_bf16_sk(T, E, P, xz, 2L * E, (const bf16*)w->conv_w, (const bf16*)w->conv_b, (const bf16*)w->x_proj_w, xdbl, xdbl2, xdbl3, cu_clean, nseq, ncu, l2r, st));
        R2L_RUN("conv_sum", st, conv_sk_sum(T, E, P, xdbl, xdbl2, xdbl3, ncu, st, R, dsplit));
      } else {
        R2L_RUN("conv_xproj", st, conv_xproj_bf16(T, E, P, xz, 2L * E, (const bf16*)w->conv_w, (const bf16*)w->conv_b, (const bf16*)w->x_proj_w, nullptr, xdbl, cu_clean, nseq, l2r, st,
                                                  scratch, kSplitScratch, ncu, R, dsplit));
      }
    } else {
      bf16* u = at<bf16>(workspace, lp.off_u);
      R2L_RUN("conv_silu", st, conv_silu<bf16>(T, E, xz, 2L * E, (const bf16*)w->conv_w, (const bf16*)w->conv_b, u, cu_clean, nseq, l2r, st));
      // x_proj with a bf16 output would lose precision; run it through the fp32-out MFMA GEMM
      R2L_RUN("x_proj_gemm", st, gemm_bf16_nt(T, P, E, u, E, (const bf16*)w->x_proj_w, E, xdbl, P, true, st));
      if (dsplit) R2L_RUN("split_delta", st, split_delta(T, P, R, xdbl, dsplit, st));
    }
    a.x = xz; a.z = xz + E; a.y = y; a.dsplit = dsplit;
    if (sp.summary) R2L_RUN("scan_summary", st, scan_summary<bf16>(a, true, st));
    R2L_RUN("scan_main", st, scan_main<bf16>(a, true, st));
    // out_proj, the LayerNorm and the gated residual in one kernel over
    // whole rounds of row blocks; o stays in registers (fp32: rounding it to
    // bf16 before the LayerNorm would add up to half a bf16 step of
    // |o| / std(o) to r at the rows' extremes)
    const int Tf = oln.rows;
    if (Tf > 0)
      R2L_RUN("out_proj_ln", st, gemm_out_ln(oln, E, y, E, (const bf16*)w->out_proj_w, E, (const bf16*)h_in,
                                             (bf16*)h_out, D, w->ln_w, w->ln_b, w->s, branch_out,
                                             (flags & R2L_FLAG_TRAIN) ? o : nullptr, no_ln, R2L_LN_EPS,
                                             at<unsigned long long>(workspace, lp.off_lnst), lncnt, st));
    // the remaining rows: out_proj into o (fp32, at its rows: the backward
    // reads all of o in training mode), then the LayerNorm kernel
    if (Tf < T) {
      const long r0 = Tf;
      // few rows (out_proj split along K): the LayerNorm kernel adds the
      // split's partial tiles itself, one launch fewer than summing them
      // into o first
      const int parts = gemm_bf16_nt_parts_split(T - Tf, D, E, y + r0 * E, E, (const bf16*)w->out_proj_w, E,
                                                 scratch, kSplitScratch, ncu);
      if (parts > 0 && ln_gate_parts_fits(D, parts)) {
        R2L_RUN("out_proj_gemm", st, gemm_bf16_nt_parts(T - Tf, D, E, y + r0 * E, E, (const bf16*)w->out_proj_w, E,
                                                        parts, st, scratch, ncu));
        R2L_RUN("ln_gate", st, (ln_gate_parts<bf16>(T - Tf, D, parts, scratch, (const bf16*)h_in + r0 * D,
                                                    (bf16*)h_out + r0 * D, w->ln_w, w->ln_b, w->s,
                                                    branch_out ? branch_out + r0 * D : nullptr,
                                                    (flags & R2L_FLAG_TRAIN) ? o + r0 * D : nullptr, no_ln,
                                                    R2L_LN_EPS, st)));
      } else {
        R2L_RUN("out_proj_gemm", st, gemm_bf16_nt(T - Tf, D, E, y + r0 * E, E, (const bf16*)w->out_proj_w, E,
                                                  o + r0 * D, D, true, st, scratch, kSplitScratch, ncu));
        R2L_RUN("ln_gate", st, (ln_gate<bf16, float>(T - Tf, D, o + r0 * D, (const bf16*)h_in + r0 * D, (bf16*)h_out + r0 * D,
                                                      w->ln_w, w->ln_b, w->s, branch_out ? branch_out + r0 * D : nullptr,
                                                      no_ln, R2L_LN_EPS, st)));
      }
    }
  } else {
    float* xz = at<float>(workspace, lp.off_xz);
    float* u = at<float>(workspace, lp.off_u);
    float* y = at<float>(workspace, lp.off_y);
    R2L_RUN("in_proj_gemm", st, gemm_f32_nt(T, 2 * E, D, (const float*)h_in, D, (const float*)w->in_proj_w, D, xz, 2L * E, st));
    R2L_RUN("conv_silu", st, conv_silu<float>(T, E, xz, 2L * E, (const float*)w->conv_w, (const float*)w->conv_b, u, cu_clean, nseq, l2r, st));
    R2L_RUN("x_proj_gemm", st, gemm_f32_nt(T, P, E, u, E, (const float*)w->x_proj_w, E, xdbl, P, st));
    a.x = xz; a.z = xz + E; a.y = y;
    if (sp.summary) R2L_RUN("scan_summary", st, scan_summary<float>(a, true, st));
    R2L_RUN("scan_main", st, scan_main<float>(a, true, st));
    R2L_RUN("out_proj_gemm", st, gemm_f32_nt(T, D, E, y, E, (const float*)w->out_proj_w, E, o, D, st));
    R2L_RUN("ln_gate", st, (ln_gate<float, float>(T, D, o, (const float*)h_in, (float*)h_out, w->ln_w, w->ln_b, w->s, branch_out, no_ln, R2L_LN_EPS, st)));
  }
  return R2L_OK;
}

int r2l_conv_fwd(const r2l_dims* d, r2l_dtype act, uint32_t flags, const void* x, int64_t ld_x,
                 const void* conv_w, const void* conv_b, const void* x_proj_w, void* u_out,
                 float* xdbl_out, const int32_t* cu_seqlens, int32_t nseq, int64_t n_tokens,
                 int32_t max_seqlen, void* stream) {
  int rc = check_dims(d);
  if (rc != R2L_OK) return rc;
  if (flags & ~R2L_FLAG_L2R) return R2L_ERR_INVALID_ARG;
  const bool l2r = flags & R2L_FLAG_L2R;
  if ((rc = check_tokens(act, n_tokens, nseq, max_seqlen)) != R2L_OK) return rc;
  const int E = d->d_inner, P = d->dt_rank + 2 * d->d_state;
  if (!x || !conv_w || !conv_b || !cu_seqlens || ld_x < E) return R2L_ERR_INVALID_ARG;
  if (!u_out && !x_proj_w) return R2L_ERR_INVALID_ARG;
  if ((x_proj_w != nullptr) != (xdbl_out != nullptr)) return R2L_ERR_INVALID_ARG;
  if (act == R2L_BF16 && (!aligned16(x) || ld_x % 8 || !aligned16(conv_w) || !aligned16(conv_b) ||
                          (x_proj_w && !aligned16(x_proj_w)) || (u_out && !aligned16(u_out))))
    return R2L_ERR_INVALID_ARG;
  const bool fused = act == R2L_BF16 && x_proj_w && P <= 256;
  if (x_proj_w && !fused && !u_out) return R2L_ERR_UNSUPPORTED;  // the unfused path stages u in u_out
  if (n_tokens == 0) return R2L_OK;
  hipStream_t st = (hipStream_t)stream;
  const int T = (int)n_tokens;
  if (act == R2L_BF16) {
    if (fused) {
      R2L_RUN("conv_xproj", st, conv_xproj_bf16(T, E, P, (const bf16*)x, ld_x, (const bf16*)conv_w, (const bf16*)conv_b, (const bf16*)x_proj_w, (bf16*)u_out, xdbl_out, cu_seqlens, nseq, l2r, st));
    } else {
      R2L_RUN("conv_silu", st, conv_silu<bf16>(T, E, (const bf16*)x, ld_x, (const bf16*)conv_w, (const bf16*)conv_b, (bf16*)u_out, cu_seqlens, nseq, l2r, st));
      if (x_proj_w) R2L_RUN("x_proj_gemm", st, gemm_bf16_nt(T, P, E, (const bf16*)u_out, E, (const bf16*)x_proj_w, E, xdbl_out, P, true, st));
    }
  } else {
    R2L_RUN("conv_silu", st, conv_silu<float>(T, E, (const float*)x, ld_x, (const float*)conv_w, (const float*)conv_b, (float*)u_out, cu_seqlens, nseq, l2r, st));
    if (x_proj_w) R2L_RUN("x_proj_gemm", st, gemm_f32_nt(T, P, E, (const float*)u_out, E, (const float*)x_proj_w, E, xdbl_out, P, st));
  }
  return R2L_OK;
}

int r2l_scan_fwd(const r2l_dims* d, r2l_dtype act, uint32_t flags, const void* u, int64_t ld_u,
                 const float* dt, int64_t ld_dt, const float* A_log, const float* B, const float* C,
                 int64_t ld_bc, const float* Dskip, const void* z, int64_t ld_z, void* y_out,
                 const int32_t* cu_seqlens, int32_t nseq, int64_t n_tokens, int32_t max_seqlen,
                 void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims(d);
  if (rc != R2L_OK) return rc;
  if (flags & ~R2L_FLAG_L2R) return R2L_ERR_INVALID_ARG;
  if ((rc = check_tokens(act, n_tokens, nseq, max_seqlen)) != R2L_OK) return rc;
  const int E = d->d_inner;
  if (!u || !dt || !A_log || !B || !C || !y_out || !cu_seqlens) return R2L_ERR_INVALID_ARG;
  if (ld_u < E || ld_dt < E || ld_bc < d->d_state || (z && ld_z < E)) return R2L_ERR_INVALID_ARG;
  // u, z, dt rows and y are accessed with 16-byte vectors
  const int64_t vec = act == R2L_BF16 ? 8 : 4;
  if (!aligned16(u) || !aligned16(dt) || !aligned16(y_out) || (z && !aligned16(z)) || ld_u % vec ||
      ld_dt % 4 || (z && ld_z % vec))
    return R2L_ERR_INVALID_ARG;
  // rows are read through 32-bit buffer windows of a few dozen rows
  const int64_t win = 64 * (act == R2L_BF16 ? 2 : 4);
  if (ld_u > INT32_MAX / win || ld_dt > INT32_MAX / 256 || ld_bc > INT32_MAX / 256 ||
      (z && ld_z > INT32_MAX / win))
    return R2L_ERR_UNSUPPORTED;
  const ScanPlan sp = plan_scan(E, n_tokens, nseq, max_seqlen, 0);
  if (!workspace || workspace_bytes < sp.total) return R2L_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return R2L_ERR_INVALID_ARG;
  if (n_tokens == 0) return R2L_OK;
  hipStream_t st = (hipStream_t)stream;
  ScanArgs a{};
  a.T = (int)n_tokens; a.E = E; a.R = d->dt_rank; a.ldp = 0;
  a.u = u; a.ld_u = ld_u; a.dt = dt; a.ld_dt = ld_dt;
  a.Bm = B; a.Cm = C; a.ld_bc = ld_bc;
  a.z = z; a.ld_z = ld_z;
  a.A_log = A_log; a.Dskip = Dskip; a.y = y_out;
  a.chunks = at<ChunkDesc>(workspace, sp.off_chunks);
  a.n_chunks = at<int32_t>(workspace, sp.off_n);
  a.max_chunks = sp.max_chunks;
  a.sumS = at<float>(workspace, sp.off_sumS);
  a.sumP = at<float>(workspace, sp.off_sumP);
  a.l2r = flags & R2L_FLAG_L2R;
  int32_t* cu_clean = at<int32_t>(workspace, sp.off_cu);
  if (act == R2L_BF16)
    return run_scan<bf16>(a, sp, false, cu_seqlens, nseq, n_tokens, cu_clean, (ChunkDesc*)a.chunks, (int32_t*)a.n_chunks, st);
  return run_scan<float>(a, sp, false, cu_seqlens, nseq, n_tokens, cu_clean, (ChunkDesc*)a.chunks, (int32_t*)a.n_chunks, st);
}

int r2l_scan_bwd(const r2l_dims* d, r2l_dtype act, uint32_t flags, const void* u, int64_t ld_u,
                 const float* dt, int64_t ld_dt, const float* A_log, const float* B, const float* C,
                 int64_t ld_bc, const float* Dskip, const void* z, int64_t ld_z, const void* dy,
                 int64_t ld_dy, float* du, float* ddt, float* dA_log, float* dB, float* dC,
                 float* dDskip, float* dz, const int32_t* cu_seqlens, int32_t nseq, int64_t n_tokens,
                 void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims(d);
  if (rc != R2L_OK) return rc;
  if ((rc = check_tokens(act, n_tokens, nseq, 0)) != R2L_OK) return rc;
  if (flags & R2L_FLAG_L2R) return R2L_ERR_UNSUPPORTED;   // the backward runs the default direction only
  if (flags) return R2L_ERR_INVALID_ARG;
  const int E = d->d_inner;
  if (!u || !dt || !A_log || !B || !C || !dy || !du || !ddt || !dA_log || !dB || !dC || !cu_seqlens)
    return R2L_ERR_INVALID_ARG;
  if ((Dskip != nullptr) != (dDskip != nullptr) || (z != nullptr) != (dz != nullptr)) return R2L_ERR_INVALID_ARG;
  if (ld_u < E || ld_dt < E || ld_bc < d->d_state || ld_dy < E || (z && ld_z < E)) return R2L_ERR_INVALID_ARG;
  // u, z, dy and dt rows are read with 16-byte vectors, the outputs written with them
  const int64_t vec = act == R2L_BF16 ? 8 : 4;
  if (!aligned16(u) || !aligned16(dy) || (z && !aligned16(z)) || !aligned16(dt) || !aligned16(du) ||
      !aligned16(ddt) || (dz && !aligned16(dz)) || ld_u % vec || ld_dy % vec || (z && ld_z % vec) || ld_dt % 4)
    return R2L_ERR_INVALID_ARG;
  const int64_t win = 64 * (act == R2L_BF16 ? 2 : 4);
  if (ld_u > INT32_MAX / win || ld_dy > INT32_MAX / win || ld_dt > INT32_MAX / 256 || ld_bc > INT32_MAX / 256 ||
      (z && ld_z > INT32_MAX / win) || (int64_t)E * 256 > INT32_MAX)
    return R2L_ERR_UNSUPPORTED;
  const ScanBwdPlan bp = plan_scan_bwd(E, n_tokens, nseq);
  if (!workspace || workspace_bytes < bp.total) return R2L_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return R2L_ERR_INVALID_ARG;
  if (n_tokens == 0) return R2L_OK;
  return run_scan_bwd(act, E, d->dt_rank, (int)n_tokens, nseq, u, ld_u, dt, ld_dt, A_log, B, C, ld_bc, Dskip, z,
                      ld_z, dy, ld_dy, du, ddt, dA_log, dB, dC, dDskip, dz, cu_seqlens, workspace,
                      (hipStream_t)stream);
}

size_t r2l_layer_bwd_workspace_bytes(const r2l_dims* dims, r2l_dtype act, int64_t n_tokens, int32_t nseq,
                                     int32_t max_seqlen) {
  if (check_dims(dims) != R2L_OK || check_tokens(act, n_tokens, nseq, max_seqlen) != R2L_OK) return 0;
  return plan_layer_bwd(dims, act, n_tokens, nseq, max_seqlen).total;
}

int r2l_layer_bwd(const r2l_dims* d, r2l_dtype act, uint32_t flags, const r2l_weights* w, const void* h_in,
                  const void* g_out, void* dh, const r2l_grads* gr, const int32_t* cu_seqlens, int32_t nseq,
                  int64_t n_tokens, int32_t max_seqlen, const void* saved, void* workspace,
                  size_t workspace_bytes, void* stream) {
  int rc = check_dims(d);
  if (rc != R2L_OK) return rc;
  if ((rc = check_tokens(act, n_tokens, nseq, max_seqlen)) != R2L_OK) return rc;
  if (flags & ~(R2L_FLAG_NO_LN | R2L_FLAG_L2R)) return R2L_ERR_INVALID_ARG;
  const bool no_ln = flags & R2L_FLAG_NO_LN, l2r = flags & R2L_FLAG_L2R;
  if (l2r && saved) return R2L_ERR_UNSUPPORTED;   // saved activations: the default direction only
  if (!w || !gr || !h_in || !g_out || !dh || !cu_seqlens) return R2L_ERR_INVALID_ARG;
  if (!w->in_proj_w || !w->conv_w || !w->conv_b || !w->x_proj_w || !w->dt_proj_w || !w->out_proj_w ||
      !w->dt_proj_b || !w->A_log || !w->Dskip || !w->s || (!no_ln && (!w->ln_w || !w->ln_b)))
    return R2L_ERR_INVALID_ARG;
  if (!gr->in_proj_w || !gr->conv_w || !gr->conv_b || !gr->x_proj_w || !gr->dt_proj_w || !gr->out_proj_w ||
      !gr->dt_proj_b || !gr->A_log || !gr->Dskip || !gr->s || (!no_ln && (!gr->ln_w || !gr->ln_b)))
    return R2L_ERR_INVALID_ARG;
  {
    const void* ptrs[] = {h_in, g_out, dh, w->in_proj_w, w->conv_w, w->conv_b, w->x_proj_w, w->dt_proj_w,
                          w->out_proj_w};
    for (const void* q : ptrs)
      if (!aligned16(q)) return R2L_ERR_INVALID_ARG;
  }
  if (act == R2L_BF16 && d->dt_rank % 8) return R2L_ERR_UNSUPPORTED;   // bf16 GEMMs over K = R and R + 2N
  const LayerBwdPlan p = plan_layer_bwd(d, act, n_tokens, nseq, max_seqlen);
  if (!workspace || workspace_bytes < p.total) return R2L_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return R2L_ERR_INVALID_ARG;
  if (saved && ((uintptr_t)saved & (kAlign - 1)) != 0) return R2L_ERR_INVALID_ARG;
  if (n_tokens == 0) return R2L_OK;
  hipStream_t st = (hipStream_t)stream;
  if (act == R2L_BF16)
    return run_layer_bwd<bf16>(d, act, no_ln, l2r, w, (const bf16*)h_in, (const bf16*)g_out, (bf16*)dh, gr,
                               cu_seqlens, nseq, (int)n_tokens, max_seqlen, saved, workspace, st);
  return run_layer_bwd<float>(d, act, no_ln, l2r, w, (const float*)h_in, (const float*)g_out, (float*)dh, gr,
                              cu_seqlens, nseq, (int)n_tokens, max_seqlen, saved, workspace, st);
}

int r2l_gemm_nt(r2l_dtype act, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                const void* B, int64_t ldb, void* C, int64_t ldc, int out_f32, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (act != R2L_F32 && act != R2L_BF16) return R2L_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
    return R2L_ERR_INVALID_ARG;
  if (!A || !B || !C || lda < K || ldb < K || ldc < N) return R2L_ERR_INVALID_ARG;
  if ((workspace == nullptr) != (workspace_bytes == 0) || (workspace && !aligned16(workspace)))
    return R2L_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (act == R2L_BF16) {
    if (K % 8 || lda % 8 || ldb % 8 || !aligned16(A) || !aligned16(B)) return R2L_ERR_UNSUPPORTED;
    R2L_RUN("gemm_bf16", st, gemm_bf16_nt((int)M, (int)N, (int)K, (const bf16*)A, lda, (const bf16*)B, ldb, C, ldc, out_f32 != 0, st,
                                          (float*)workspace, workspace_bytes, num_cus()));
  } else {
    R2L_RUN("gemm_f32", st, gemm_f32_nt((int)M, (int)N, (int)K, (const float*)A, lda, (const float*)B, ldb, (float*)C, ldc, st));
  }
  return R2L_OK;
}

int r2l_timing_enable(int enable) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (enable) {
    // the whole pool is created here, once (events in flight count as taken)
    const size_t have = t.pool.size() + 2 * t.recs.size();
    for (size_t i = have; i < kEventPool; ++i) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return R2L_ERR_HIP;
      t.pool.push_back(e);
    }
  }
  t.enabled = enable != 0;
  return R2L_OK;
}

int r2l_timing_reset(void) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  for (auto& r : t.recs) {
    (void)hipEventSynchronize(r.b);
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  t.recs.clear();
  t.names.clear();
  t.totals.clear();
  t.counts.clear();
  return R2L_OK;
}

int r2l_timing_read(const char** names, double* total_ms, int64_t* counts, int max_names) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  int status = R2L_OK;
  for (auto& r : t.recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      status = R2L_ERR_HIP;
    size_t k = 0;
    while (k < t.names.size() && std::strcmp(t.names[k], r.name) != 0) ++k;
    if (k == t.names.size()) {
      t.names.push_back(r.name);
      t.totals.push_back(0.0);
      t.counts.push_back(0);
    }
    t.totals[k] += ms;
    t.counts[k] += 1;
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  t.recs.clear();
  if (status != R2L_OK) return status;
  const int n = (int)t.names.size();
  for (int i = 0; i < n && i < max_names; ++i) {
    if (names) names[i] = t.names[i];
    if (total_ms) total_ms[i] = t.totals[i];
    if (counts) counts[i] = t.counts[i];
  }
  return n;
}

}  // extern "C"
