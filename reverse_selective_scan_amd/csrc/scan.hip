// Reverse selective scan ("Bifocal Diffusion Language Models", §3.4 step 2:
// the Mamba-1 selective scan run over the flipped sequence; in the original
// token order it runs from each sequence's last token to its first):
//   h_t = exp(dt_t A) (.) h_{t+1} + (dt_t u_t) (x) B_t,   h = 0 past the end,
//   y_t = (C_t . h_t + Dskip u_t) * SiLU(z_t),             A = -exp(A_log).
//
// Work decomposition (details at scan_kernel).  A block owns 64 channels of
// one time chunk of one sequence; its 4 waves split the 16 states (wave w keeps
// states 4w..4w+3 of the lane's channel in fp32 registers for the whole chunk)
// and their partial C.h sums meet in LDS.  Time is walked right to left in
// blocks of 32 tokens whose per-(token, channel) inputs are prepared
// cooperatively (conv + SiLU from x, SiLU(z), dt on MFMA) one block at a time,
// with the next block's global loads in flight meanwhile.
// With L2R (the left-to-right control of §4.4, Table 4) everything runs
// mirrored: causal conv, time walked left to right, chunks cut from the
// sequence start.
// Long sequences are cut into chunks so that enough blocks exist to fill the
// GPU.  A first pass computes, per chunk, the state at its left edge from a
// zero carry (S) and the decay across it (P = exp(A * sum dt)); the main pass
// then starts each chunk from the carry combined right to left over the
// summaries of the chunks to its right, H = S_j + P_j H.  Chunks never cross
// a sequence end, and no floating-point atomics are used, so results do not
// depend on scheduling.
#include <type_traits>

#include "kernels.h"

namespace r2l {

constexpr int NS = 16;    // d_state (§4.1)

// ---------------------------------------------------------------------------
// chunk planning (one block; plan.h)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_chunks_kernel(PlanArgs p) {
  __shared__ int s_v[256];
  plan_chunks_block(p, s_v);
}

PlanArgs plan_args(const int32_t* cu, int nseq, int Tn, int Lc, int max_chunks, bool l2r, int32_t* cu_clean,
                   ChunkDesc* chunks, int32_t* n_chunks, int* zero, int n_zero) {
  PlanArgs p{};
  p.cu = cu; p.nseq = nseq; p.Tn = Tn; p.Lc = Lc; p.max_chunks = max_chunks; p.l2r = l2r ? 1 : 0;
  p.cu_clean = cu_clean; p.chunks = chunks; p.n_chunks = n_chunks;
  p.zero = zero; p.n_zero = zero ? n_zero : 0;
  return p;
}

hipError_t plan_chunks(const int32_t* cu, int nseq, int Tn, int Lc, int max_chunks, bool l2r,
                       int32_t* cu_clean, ChunkDesc* chunks, int32_t* n_chunks, hipStream_t st, int* zero,
                       int n_zero) {
  hipLaunchKernelGGL(plan_chunks_kernel, dim3(1), dim3(256), 0, st,
                     plan_args(cu, nseq, Tn, Lc, max_chunks, l2r, cu_clean, chunks, n_chunks, zero, n_zero));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row-window buffer resources.  Every per-token input is read through a
// buffer resource that covers exactly the rows a block may use: reads past
// its end return zeros without touching memory (rows past a sequence end for
// the conv window, rows past the block for the rest) and stores past its end
// are dropped, so no row index is clamped or selected per lane.  Offsets are
// relative to the window's first row and stay far below 2^31 (the host
// limits row pitches accordingly).
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

R2L_DEV Rsrc row_window(const void* base, long row0, long pitch_bytes, int rows) {
  const long bytes = rows > 0 ? rows * pitch_bytes : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)base + row0 * pitch_bytes), 0, (int)bytes,
                                           0x00020000);
}
R2L_DEV u32x4 bload16(Rsrc r, unsigned off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
R2L_DEV u32x2 bload8(Rsrc r, unsigned off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
R2L_DEV float bload4(Rsrc r, unsigned off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
R2L_DEV void bstore16(Rsrc r, unsigned off, u32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0); }
constexpr unsigned kOutside = 0x80000000u;   // an offset past every window

// 8 channels of one row: one 16-byte load (bf16) or two (fp32)
template <typename T> struct Raw8;
template <> struct Raw8<bf16> { u32x4 v; };
template <> struct Raw8<float> { f32x4 a, b; };
R2L_DEV void raw_load(Raw8<bf16>& r, Rsrc s, unsigned off) { r.v = bload16(s, off); }
// (fp32 lanes are reinterpreted as a whole vector: extracting one 32-bit
// element of a 16-byte buffer load and reinterpreting it as a float makes
// this compiler narrow the load to its first dword)
R2L_DEV void raw_load(Raw8<float>& r, Rsrc s, unsigned off) {
  r.a = __builtin_bit_cast(f32x4, bload16(s, off));
  r.b = __builtin_bit_cast(f32x4, bload16(s, off + 16));
}
R2L_DEV float raw_at(const Raw8<bf16>& r, int i) {
  const unsigned w = r.v[i >> 1];
  return __builtin_bit_cast(float, (i & 1) ? (w & 0xffff0000u) : (w << 16));
}
R2L_DEV float raw_at(const Raw8<float>& r, int i) { return i < 4 ? r.a[i] : r.b[i - 4]; }
R2L_DEV void store8(Rsrc s, unsigned off, const float v[8], bf16*) {
  u32x4 q;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 p = {(bf16)v[2 * i], (bf16)v[2 * i + 1]};
    q[i] = __builtin_bit_cast(unsigned, p);
  }
  bstore16(s, off, q);
}
R2L_DEV void store8(Rsrc s, unsigned off, const float v[8], float*) {
  bstore16(s, off, __builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]}));
  bstore16(s, off + 16, __builtin_bit_cast(u32x4, f32x4{v[4], v[5], v[6], v[7]}));
}

// softplus for dt.  bf16 activations: log2(1 + 2^(-|v| log2 e)) ln 2 on the
// transcendental unit (rounding 1 + w costs < 2^-24 / w relative, i.e.
// < 1e-4 at the smallest dt the layer uses, far below the bf16 roundings
// around it); fp32 activations: the series/log form of softplus_f.
template <typename T> R2L_DEV float softplus_dt(float v);
template <> R2L_DEV float softplus_dt<float>(float v) { return softplus_f(v); }
template <> R2L_DEV float softplus_dt<bf16>(float v) {
  const float w = exp2_fast(-fabsf(v) * kLog2e);
  // max(v, 0) as the median of (v, 0, 3e38): fmaxf on an MFMA result would
  // first be canonicalised (one more instruction), and with +inf as the bound
  // the compiler turns the median back into that fmaxf.  Pre-activations
  // above 3e38 (clamped here) give no meaningful dt either way; a NaN still
  // reaches dt through the log term.
  return __builtin_amdgcn_fmed3f(v, 0.0f, 3.0e38f) + __builtin_amdgcn_logf(1.0f + w) * kLn2;
}

// ---------------------------------------------------------------------------
// The scan kernel.  SUMMARY = pass 1 (chunk summaries), otherwise the main
// pass.  KS = number of 32-wide k-steps of dt_proj on MFMA (fused bf16 only;
// 0 = VALU).
//
// A block of 4 waves owns 64 channels of one time chunk; time is walked right
// to left in blocks of TB = 32 tokens:
//   A  thread (r8 = tid / 8, c8 = tid % 8): token row r8, channels 8 c8 .. +7:
//      consumes the registers loaded for this block (conv + SiLU -> u,
//      SiLU(z), Dskip u, delta -> LDS in bf16, B and C -> LDS), then issues
//      the next block's loads;
//   M  wave w: dt = softplus(delta . W_dt^T + b) for channels 16 w .. +15 of
//      all 32 rows on MFMA (16x16x32 bf16); fp32 uses the VALU;
//   B  wave w, lane c: channel c, states 4 w .. 4 w + 3 in registers, the
//      recurrence over the block's tokens.  Per token the decay is applied
//      on the VALU (h <- exp(dt A) h) and the input term dt u B is added by
//      one 4x4x1 fp32 MFMA over 16 blocks, whose accumulator layout is
//      exactly this one: block b = lanes 4b..4b+3, lane 4b+j holds column j
//      in its 4 result registers (rows = states), with A operand B_t[4w + i]
//      in lane 4b+i and B operand dt u of the lane's own channel.  The LDS
//      operands run 4 tokens ahead of the arithmetic;
//   C  same layout as A: y = (sum of the 4 partial C.h + Dskip u) SiLU(z),
//      one 16-byte store per thread.
// ---------------------------------------------------------------------------
//
// BWD (standalone, right to left, no chunk carries): the first sweep of the
// backward pass.  The recurrence runs as above; before each 16-token
// sub-block it stores the state entering it from the right into a.hc, and
// phase C writes dz = dy SiLU'(z) (C.h + Dskip u) instead of y.
// (Two blocks per CU; with dt_rank above 128 the delta rows alone take so
// much LDS that one block per CU is all that fits.)
template <typename T, bool FUSED, bool SUMMARY, int KS, bool L2R, bool BWD = false>
__global__ __launch_bounds__(256, KS > 4 ? 1 : 2) void scan_kernel(ScanArgs a) {
  static_assert(!BWD || (!FUSED && !SUMMARY && !L2R), "the backward sweep is standalone and right to left");
  constexpr int TB = 32;
  constexpr bool MFMA_DT = FUSED && KS > 0;
  constexpr int RP = MFMA_DT ? KS * 32 : 32;   // padded dt_rank for the MFMA k loop
  // delta in LDS as two bf16 parts per value, hi = bf16(delta) in columns
  // [0, RP) and lo = bf16(delta - hi) in [RP, 2 RP): the two MFMAs of a
  // k-step then carry delta to about 16 significant bits (the weights are
  // bf16, so every product is exact in the fp32 accumulator)
  constexpr int DLS = 2 * RP + 8;               // delta row stride in LDS (bf16)
  constexpr int DPT = RP / 8;                   // delta floats per thread per row (4..32)
  constexpr bool BF = std::is_same<T, bf16>::value;
  constexpr unsigned SZ = sizeof(T);
  // Rows of yp_s, pre_s and u_s are padded by 4 words: the accesses that
  // touch several rows at once (16 lanes over rows 4 apart in the dt phase,
  // 8 lanes per row over 2 rows in phases A and C) then fall in distinct banks.
  // (At dt_rank 128 the five arrays take 80 KB: two blocks fill a CU's LDS.)
  constexpr int RW = 64 + 4;
  __shared__ __attribute__((aligned(16))) float yp_s[4][TB][RW];   // partial C.h of each wave
  __shared__ __attribute__((aligned(16))) float2 pre_s[TB][RW];    // (dt, dt*u)
  __shared__ __attribute__((aligned(16))) f32x4 bc_s[TB][8];       // B[0..16) C[0..16)
  __shared__ __attribute__((aligned(16))) float u_s[FUSED ? TB : 1][RW];
  __shared__ __attribute__((aligned(16))) bf16 dl_s[MFMA_DT ? TB * DLS : 8];

  const int E = a.E;
  const int NB = E / 64;
  // Blocks of one chunk are consecutive, so the hardware's round-robin
  // spreads every chunk over all XCDs; the grid is sized by an upper bound on
  // the chunk count, and the surplus blocks (the highest indices) exit here
  // evenly across the XCDs.  (Blocks share no operands worth keeping in one
  // XCD's L2.)
  const int ci = blockIdx.x / NB, cblk = blockIdx.x % NB;
  if (ci >= *a.n_chunks) return;
  const ChunkDesc d = a.chunks[ci];
  if (SUMMARY && d.j == d.n_in_seq - 1) return;  // last chunk in scan order: its summary is never used
  const int tid = threadIdx.x;
  const int lane = lane_id(), w = wave_id();
  const int e0 = cblk * 64;
  const int e = e0 + lane;                 // B channel
  const int r8 = tid >> 3, c8 = tid & 7;   // A/C row and channel group
  const int ea = e0 + 8 * c8;              // A/C first channel

  // Per-channel parameters in 16-byte loads where the pointers allow (a
  // block of a short input runs a single 32-token block, and element loads
  // would be a large part of its time).  The layer's tensors are 16-byte
  // aligned; the standalone scan's A_log and Dskip need not be.
  float A2[4];
  if ((reinterpret_cast<uintptr_t>(a.A_log) & 15) == 0) {
    const f32x4 al = *(const f32x4*)(a.A_log + (long)e * NS + 4 * w);
#pragma unroll
    for (int i = 0; i < 4; ++i) A2[i] = -expf(al[i]) * kLog2e;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) A2[i] = -expf(a.A_log[(long)e * NS + 4 * w + i]) * kLog2e;
  }
  float dsk8[8], cb8[8];
  float cwr[BF ? 1 : 8][4];        // fp32 conv taps
  unsigned w10[8], w32[8];         // bf16 conv taps as pairs (tap for row t | row t+1), (t+2 | t+3)
  if (a.Dskip == nullptr) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dsk8[i] = 0.0f;
  } else if ((reinterpret_cast<uintptr_t>(a.Dskip) & 15) == 0) {
    const f32x4 d0 = *(const f32x4*)(a.Dskip + ea), d1 = *(const f32x4*)(a.Dskip + ea + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { dsk8[i] = d0[i]; dsk8[4 + i] = d1[i]; }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) dsk8[i] = a.Dskip[ea + i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) cb8[i] = 0.0f;
  if constexpr (FUSED) {
    if constexpr (BF) {
      const bf16x8 cb = *(const bf16x8*)((const bf16*)a.conv_b + ea);
#pragma unroll
      for (int i = 0; i < 8; ++i) cb8[i] = (float)cb[i];
      // taps k = 0..3 of channel i as two dwords (k0|k1), (k2|k3); the conv
      // weight for row t + j is tap 3 - j
      const u32x4* cw = (const u32x4*)((const unsigned*)a.conv_w + (long)ea * 2);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 v = cw[q];   // channels ea + 2q, ea + 2q + 1
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int i = 2 * q + hh;
          w10[i] = __builtin_amdgcn_alignbit(v[2 * hh + 1], v[2 * hh + 1], 16);   // (tap 3 | tap 2)
          w32[i] = __builtin_amdgcn_alignbit(v[2 * hh], v[2 * hh], 16);           // (tap 1 | tap 0)
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) cb8[i] = ((const float*)a.conv_b)[ea + i];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) cwr[i][k] = ((const float*)a.conv_w)[(long)(ea + i) * 4 + k];
    }
  }
  // dt_proj fragments (B operand of the 16x16x32 MFMA): channel
  // e0 + 16 w + (lane & 15), k = 32 ks + 8 (lane >> 4) .. +7.
  bf16x8 wdt[MFMA_DT ? KS : 1];
  const int dcol = 16 * w + (lane & 15);
  float dtb_col = 0.0f;
  if constexpr (MFMA_DT) {
    const bf16* W = (const bf16*)a.dt_w;
    const long rowoff = (long)(e0 + dcol) * a.R;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k = ks * 32 + (lane >> 4) * 8;
      if ((a.R & 7) == 0) {
        // whole 16-byte row pieces; those past dt_rank read as zeros
        wdt[ks] = *(const bf16x8*)(W + rowoff + min(k, a.R - 8));
        if (k >= a.R) wdt[ks] = bf16x8{};
      } else {
#pragma unroll
        for (int p = 0; p < 8; ++p) wdt[ks][p] = W[rowoff + min(k + p, a.R - 1)];
#pragma unroll
        for (int p = 0; p < 8; ++p) if (k + p >= a.R) wdt[ks][p] = (bf16)0.0f;
      }
    }
    dtb_col = a.dt_b[e0 + dcol];
  }

  // carry into this chunk from the chunks before it in scan order
  f32x4 h = {0.0f, 0.0f, 0.0f, 0.0f};
  if (!SUMMARY) {
    for (int jj = 0; jj < d.j; ++jj) {
      const long base = (long)(d.first + jj) * NS * E;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long off = base + (long)(4 * w + i) * E + e;
        h[i] = fmaf(a.sumP[off], h[i], a.sumS[off]);
      }
    }
  }
  float sdt = 0.0f;

  // ---------------- per-thread window offsets (constant over blocks) ----------------
  const void* xin = FUSED ? a.x : a.u;
  const long ldx_b = (FUSED ? a.ld_x : a.ld_u) * (long)SZ;     // x or u row pitch, bytes
  const long ldz_b = a.ld_z * (long)SZ;
  const long ldp_b = (long)a.ldp * 4;
  const long lddt_b = a.ld_dt * 4, ldbc_b = a.ld_bc * 4;
  const long ldy_b = (long)E * SZ;
  const void* zin = a.z;
  const bool has_z = FUSED || zin != nullptr;   // the layer always gates
  const unsigned offX = (unsigned)(r8 * ldx_b) + (unsigned)ea * SZ;
  const unsigned offZ = (unsigned)(r8 * ldz_b) + (unsigned)ea * SZ;
  const unsigned offY = (unsigned)(r8 * ldy_b) + (unsigned)ea * SZ;
  const unsigned offS = (unsigned)(r8 * RP * 4) + (unsigned)(c8 * DPT) * 2;         // delta split (fused)
  const unsigned offBC = (unsigned)(r8 * ldp_b) + (unsigned)(a.R + 4 * c8) * 4;   // B then C (fused)
  const unsigned offDT = (unsigned)(r8 * lddt_b) + (unsigned)ea * 4;               // dt (standalone)
  const unsigned offB = c8 < 4 ? (unsigned)(r8 * ldbc_b) + 16u * c8 : kOutside;    // B (standalone)
  const unsigned offC = c8 < 4 ? kOutside : (unsigned)(r8 * ldbc_b) + 16u * (c8 - 4);
  const long lddy_b = a.ld_dy * (long)SZ;
  const unsigned offDY = (unsigned)(r8 * lddy_b) + (unsigned)ea * SZ;               // dy (backward)
  const unsigned offDZ = (unsigned)(r8 * (long)E * 4) + (unsigned)ea * 4;          // dz (backward)

  // ---------------- prefetch registers ----------------
  Raw8<T> px[FUSED ? 4 : 1];   // x rows r8 .. r8+3 (fused) or the u row r8
  Raw8<T> pz;                  // z row r8
  Raw8<T> pdy;                 // dy row r8 (backward)
  u32x4 pd[FUSED ? (MFMA_DT ? DPT / 4 : 1) : 2];   // delta split (fused) or dt (standalone) of row r8
  float pbc[4];                // 4 of the row's 32 B/C floats

  auto issue = [&](int blo, int bhi) {
    const int rows = bhi - blo;
    if constexpr (FUSED) {
      // the conv window reaches 3 rows past the block (R2L) or before it
      // (L2R), never out of the sequence; px[j] = x[t + j] (R2L) or x[t - j]
      // (L2R), rows outside the window reading as zero (a negative L2R
      // offset wraps past the window's end)
      const int wb = L2R ? max(d.seq_lo, blo - 3) : blo;
      const Rsrc rX = row_window(xin, wb, ldx_b, (L2R ? bhi : min(d.seq_end, bhi + 3)) - wb);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        raw_load(px[j], rX, offX + (unsigned)((L2R ? blo - wb - j : j) * ldx_b));
      const Rsrc rD = row_window(a.xdbl, blo, ldp_b, rows);
      if constexpr (MFMA_DT) {
        // this thread's DPT columns of the delta split's hi and lo halves
        const Rsrc rS = row_window(a.dsplit, blo, (long)RP * 4, rows);
        if constexpr (DPT >= 8) {
#pragma unroll
          for (int q = 0; q < DPT / 8; ++q) {
            pd[q] = bload16(rS, offS + 16u * q);
            pd[DPT / 8 + q] = bload16(rS, offS + 2u * RP + 16u * q);
          }
        } else {
          const u32x2 hi = bload8(rS, offS), lo = bload8(rS, offS + 2u * RP);
          pd[0] = u32x4{hi[0], hi[1], lo[0], lo[1]};
        }
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) pbc[p] = bload4(rD, offBC + 4u * p);
    } else {
      raw_load(px[0], row_window(xin, blo, ldx_b, rows), offX);
      const Rsrc rT = row_window(a.dt, blo, lddt_b, rows);
      pd[0] = bload16(rT, offDT);
      pd[1] = bload16(rT, offDT + 16);
      const Rsrc rB = row_window(a.Bm, blo, ldbc_b, rows), rC = row_window(a.Cm, blo, ldbc_b, rows);
#pragma unroll
      for (int p = 0; p < 4; ++p) pbc[p] = bload4(rB, offB + 4u * p) + bload4(rC, offC + 4u * p);
    }
    if constexpr (!SUMMARY) {
      if (has_z) raw_load(pz, row_window(zin, blo, ldz_b, rows), offZ);
    }
    if constexpr (BWD) {
      if (has_z) raw_load(pdy, row_window(a.dy, blo, lddy_b, rows), offDY);
    }
  };

  // SiLU(z) and Dskip*u of this thread's (row, 8 channels): phase A makes
  // them, phase C of the same block uses them.
  float g8[8], du8[8];
  // the chunk's blocks of TB tokens in scan order; only the last is partial
  const int nblk = (d.hi - d.lo + TB - 1) / TB;
  auto blo_of = [&](int k) { return L2R ? d.lo + k * TB : max(d.lo, d.hi - (k + 1) * TB); };
  auto bhi_of = [&](int k) { return L2R ? min(d.hi, d.lo + (k + 1) * TB) : d.hi - k * TB; };
  if (nblk > 0) issue(blo_of(0), bhi_of(0));
  for (int kb = 0; kb < nblk; ++kb) {
    const int blo = blo_of(kb), bhi = bhi_of(kb);
    const int nt = bhi - blo;
    // ---------------- A: consume this block's prefetched inputs ----------------
    // (rows past the block read as zeros, or as the real rows of the conv
    // window; either way their results are never used)
    {
      float uu[8];
      if constexpr (FUSED) {
        if constexpr (BF) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int i = 2 * q + hh;
              const unsigned sel = hh ? 0x07060302u : 0x05040100u;   // high / low bf16 of each row
              const unsigned x10 = __builtin_amdgcn_perm(px[1].v[q], px[0].v[q], sel);   // (row t | row t+1)
              const unsigned x32 = __builtin_amdgcn_perm(px[3].v[q], px[2].v[q], sel);   // (row t+2 | row t+3)
              float c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w10[i]),
                                                        __builtin_bit_cast(bf16x2, x10), cb8[i], false);
              c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w32[i]),
                                                  __builtin_bit_cast(bf16x2, x32), c, false);
              uu[i] = silu_fast(c);
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float c = cb8[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) c = fmaf(cwr[i][3 - j], raw_at(px[j], i), c);
            uu[i] = silu_fast(c);
          }
        }
        if constexpr (MFMA_DT) {
          // the delta split's hi and lo halves; columns at or past dt_rank
          // are set to zero here: the split's writers cover only the x_proj
          // width, so when it is narrower than RP the last columns hold
          // whatever the workspace held, and a NaN there would survive its
          // product with the zeroed weights
          bf16* dst = dl_s + r8 * DLS + c8 * DPT;
          const int R = a.R;
          // a bf16 pair at columns c, c + 1 (column c in the low half)
          auto keep = [R](unsigned v, int c) { return c + 1 < R ? v : (c < R ? (v & 0xffffu) : 0u); };
          if constexpr (DPT >= 8) {
#pragma unroll
            for (int q = 0; q < DPT / 8; ++q) {
              const int c0 = c8 * DPT + 8 * q;
              u32x4 vh = pd[q], vl = pd[DPT / 8 + q];
              if (R < RP) {   // uniform: at a dt_rank that fills RP nothing is masked
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                  vh[d] = keep(vh[d], c0 + 2 * d);
                  vl[d] = keep(vl[d], c0 + 2 * d);
                }
              }
              *(u32x4*)(dst + 8 * q) = vh;
              *(u32x4*)(dst + RP + 8 * q) = vl;
            }
          } else {
            const int c0 = c8 * DPT;
            *(u32x2*)dst = u32x2{keep(pd[0][0], c0), keep(pd[0][1], c0 + 2)};
            *(u32x2*)(dst + RP) = u32x2{keep(pd[0][2], c0), keep(pd[0][3], c0 + 2)};
          }
        }
        *(f32x4*)&u_s[r8][8 * c8] = f32x4{uu[0], uu[1], uu[2], uu[3]};
        *(f32x4*)&u_s[r8][8 * c8 + 4] = f32x4{uu[4], uu[5], uu[6], uu[7]};
      } else {
        const f32x4 d0 = __builtin_bit_cast(f32x4, pd[0]), d1 = __builtin_bit_cast(f32x4, pd[1]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uu[i] = raw_at(px[0], i);
          const float dtv = i < 4 ? d0[i] : d1[i - 4];
          pre_s[r8][8 * c8 + i] = make_float2(dtv, dtv * uu[i]);
        }
      }
      if constexpr (BWD) {
        // g8 = dy SiLU'(z), SiLU'(z) = sig(z) (1 + z (1 - sig(z)))
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float zv = has_z ? raw_at(pz, i) : 0.0f;
          const float sg = sigmoid_fast(zv);
          g8[i] = has_z ? raw_at(pdy, i) * (sg * fmaf(zv, 1.0f - sg, 1.0f)) : 0.0f;
          du8[i] = dsk8[i] * uu[i];
        }
      } else if constexpr (!SUMMARY) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          g8[i] = has_z ? silu_fast(raw_at(pz, i)) : 1.0f;
          du8[i] = dsk8[i] * uu[i];
        }
      }
      bc_s[r8][c8] = f32x4{pbc[0], pbc[1], pbc[2], pbc[3]};
    }
    // the next block's loads go out now and land during this block's compute
    if (kb + 1 < nblk) issue(blo_of(kb + 1), bhi_of(kb + 1));
    __syncthreads();
    // ---------------- M: dt = softplus(delta . W_dt^T + b) ----------------
    if constexpr (FUSED) {
      if constexpr (MFMA_DT) {
        // one accumulator chain per row tile, started at the dt bias, taking
        // the hi and the lo part of delta in turn (an MFMA that only adds to
        // the previous one's accumulator issues back to back with it); the
        // two row tiles' chains alternate
        f32x4 acc[TB / 16];
#pragma unroll
        for (int rt = 0; rt < TB / 16; ++rt) acc[rt] = f32x4{dtb_col, dtb_col, dtb_col, dtb_col};
        const bf16* drow = dl_s + (lane & 15) * DLS + (lane >> 4) * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int part = 0; part < 2; ++part)
#pragma unroll
            for (int rt = 0; rt < TB / 16; ++rt)
              acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  *(const bf16x8*)(drow + rt * 16 * DLS + part * RP + ks * 32), wdt[ks], acc[rt], 0, 0, 0);
#pragma unroll
        for (int rt = 0; rt < TB / 16; ++rt) {
          // D layout: lane holds rows 4 (lane >> 4) + i, column (lane & 15)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = rt * 16 + 4 * (lane >> 4) + i;
            const float dtv = softplus_dt<T>(acc[rt][i]);
            pre_s[rr][dcol] = make_float2(dtv, dtv * u_s[rr][dcol]);
          }
        }
      } else {
        const T* W = (const T*)a.dt_w;
        const float dtb = a.dt_b[e];
        for (int i = 0; i < TB / 4; ++i) {
          const int rr = (TB / 4) * w + i;
          const int t = min(blo + rr, bhi - 1);
          float acc = 0.0f;
          for (int k = 0; k < a.R; ++k)
            acc = fmaf(a.xdbl[(long)t * a.ldp + k], to_f32(W[(long)e * a.R + k]), acc);
          const float dtv = softplus_dt<T>(acc + dtb);
          pre_s[rr][lane] = make_float2(dtv, dtv * u_s[rr][lane]);
        }
      }
      __syncthreads();
    }
    // ---------------- B: the recurrence, in scan order ----------------
    // At raised wave priority: one wave's recurrence is a dependency chain
    // (about 87 cycles per token against 64 of VALU issue), and the other
    // wave on the SIMD, in phases A, M or C of its own block, has the
    // independent work to fill its gaps when the chain gets the issue slot
    // first (measured: scan 0.684 -> 0.629 ms; the reverse order was slower).
    __builtin_amdgcn_s_setprio(2);
    auto compute = [&](int r, float2 p, float bsel, f32x4 Cv) __attribute__((always_inline)) {
      f32x4 hd;
#pragma unroll
      for (int i = 0; i < 4; ++i) hd[i] = exp2_fast(p.x * A2[i]) * h[i];
      h = __builtin_amdgcn_mfma_f32_4x4x1f32(bsel, p.y, hd, 0, 0, 0);
      if constexpr (SUMMARY) {
        sdt += p.x;
      } else {
        yp_s[w][r][lane] = fmaf(Cv[3], h[3], fmaf(Cv[2], h[2], fmaf(Cv[1], h[1], Cv[0] * h[0])));
      }
    };
    const float* bsrc = (const float*)&bc_s[0][w] + (lane & 3);   // B_t[4 w + (lane & 3)] at row 0
    // (backward) the state entering the block's sub-blocks: before its
    // first token and, for a block of more than 16, before its 17th
    auto keep_state = [&](int half) __attribute__((always_inline)) {
      if constexpr (BWD) {
        const long slot = (long)d.slot0 + 2 * kb + half;
#pragma unroll
        for (int i = 0; i < 4; ++i) a.hc[(slot * NS + 4 * w + i) * E + e] = h[i];
      }
    };
    if (nt == TB) {
      // 4-deep ring of LDS operands (indices are constants after unrolling)
      constexpr int LA = 4;
      float2 Pq[LA];
      float Bq[LA];
      f32x4 Cq[LA];
      auto row = [](int k) { return L2R ? k : TB - 1 - k; };   // k-th row in scan order
#pragma unroll
      for (int k = 0; k < LA; ++k) {
        Pq[k] = pre_s[row(k)][lane];
        Bq[k] = bsrc[row(k) * 32];
        Cq[k] = SUMMARY ? f32x4{} : bc_s[row(k)][4 + w];
      }
#pragma unroll
      for (int k = 0; k < TB; ++k) {
        if (k == 0 || k == 16) keep_state(k / 16);
        const int r = row(k), sl = k % LA;
        const float2 p = Pq[sl];
        const float bv = Bq[sl];
        const f32x4 Cv = Cq[sl];
        if (k + LA < TB) {
          const int rn = row(k + LA);
          Pq[sl] = pre_s[rn][lane];
          Bq[sl] = bsrc[rn * 32];
          if constexpr (!SUMMARY) Cq[sl] = bc_s[rn][4 + w];
        }
        compute(r, p, bv, Cv);
      }
    } else {
      for (int k = 0; k < nt; ++k) {
        if (k == 0 || k == 16) keep_state(k / 16);
        const int r = L2R ? k : nt - 1 - k;
        compute(r, pre_s[r][lane], bsrc[r * 32], bc_s[r][4 + w]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    // ---------------- C: combine and store ----------------
    // (rows past the block fall outside the store window and are dropped)
    if constexpr (!SUMMARY) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = du8[i];
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const f32x4 p0 = *(const f32x4*)&yp_s[ww][r8][8 * c8];
        const f32x4 p1 = *(const f32x4*)&yp_s[ww][r8][8 * c8 + 4];
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[i] += p0[i]; v[4 + i] += p1[i]; }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] *= g8[i];
      if constexpr (BWD) {
        if (has_z) store8(row_window(a.dz, blo, (long)E * 4, nt), offDZ, v, (float*)nullptr);
      } else {
        store8(row_window(a.y, blo, ldy_b, nt), offY, v, (T*)nullptr);
      }
      // the next block's phase B rewrites yp_s only after two more barriers
    }
  }
  if constexpr (SUMMARY) {
    const long base = (long)ci * NS * E;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long off = base + (long)(4 * w + i) * E + e;
      a.sumS[off] = h[i];
      a.sumP[off] = exp2_fast(A2[i] * sdt);
    }
  }
}

template <typename T, bool SUMMARY, bool L2R>
static void launch_scan_dir(const ScanArgs& a, bool fused, hipStream_t st) {
  dim3 grid(a.max_chunks * (a.E / 64)), block(256);
  if (!fused) {
    hipLaunchKernelGGL((scan_kernel<T, false, SUMMARY, 0, L2R>), grid, block, 0, st, a);
  } else if constexpr (std::is_same<T, float>::value) {
    hipLaunchKernelGGL((scan_kernel<T, true, SUMMARY, 0, L2R>), grid, block, 0, st, a);
  } else {
    const int ks = (a.R + 31) / 32;
    if (ks > 8) hipLaunchKernelGGL((scan_kernel<T, true, SUMMARY, 0, L2R>), grid, block, 0, st, a);
    else if (ks <= 1) hipLaunchKernelGGL((scan_kernel<T, true, SUMMARY, 1, L2R>), grid, block, 0, st, a);
    else if (ks <= 2) hipLaunchKernelGGL((scan_kernel<T, true, SUMMARY, 2, L2R>), grid, block, 0, st, a);
    else if (ks <= 4) hipLaunchKernelGGL((scan_kernel<T, true, SUMMARY, 4, L2R>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_kernel<T, true, SUMMARY, 8, L2R>), grid, block, 0, st, a);
  }
}

template <typename T, bool SUMMARY>
static hipError_t launch_scan(const ScanArgs& a, bool fused, hipStream_t st) {
  if (a.max_chunks * (a.E / 64) <= 0) return hipSuccess;
  if (a.l2r) launch_scan_dir<T, SUMMARY, true>(a, fused, st);
  else launch_scan_dir<T, SUMMARY, false>(a, fused, st);
  return hipGetLastError();
}

template <typename T>
hipError_t scan_summary(const ScanArgs& a, bool fused, hipStream_t st) {
  return launch_scan<T, true>(a, fused, st);
}
template <typename T>
hipError_t scan_main(const ScanArgs& a, bool fused, hipStream_t st) {
  return launch_scan<T, false>(a, fused, st);
}
template <typename T>
hipError_t scan_bwd_states(const ScanArgs& a, hipStream_t st) {
  if (a.max_chunks * (a.E / 64) <= 0) return hipSuccess;
  hipLaunchKernelGGL((scan_kernel<T, false, false, 0, false, true>), dim3(a.max_chunks * (a.E / 64)), dim3(256),
                     0, st, a);
  return hipGetLastError();
}
template hipError_t scan_bwd_states<float>(const ScanArgs&, hipStream_t);
template hipError_t scan_bwd_states<bf16>(const ScanArgs&, hipStream_t);
template hipError_t scan_summary<float>(const ScanArgs&, bool, hipStream_t);
template hipError_t scan_summary<bf16>(const ScanArgs&, bool, hipStream_t);
template hipError_t scan_main<float>(const ScanArgs&, bool, hipStream_t);
template hipError_t scan_main<bf16>(const ScanArgs&, bool, hipStream_t);

}  // namespace r2l
