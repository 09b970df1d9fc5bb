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
// chunk planning (one block): sanitised cu_seqlens (clamped to [0, T] and
// made non-decreasing) and the chunk table, rightmost chunk of each
// sequence first.
// ---------------------------------------------------------------------------
// Exclusive block-wide scan of one value per thread (256 threads), max or sum,
// Hillis-Steele in LDS: 8 steps.
template <bool MAX>
R2L_DEV int block_exclusive_scan(int v, int* buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
#pragma unroll
  for (int off = 1; off < 256; off <<= 1) {
    const int o = tid >= off ? buf[tid - off] : 0;   // values are >= 0: 0 is neutral for both
    __syncthreads();
    if (tid >= off) buf[tid] = MAX ? max(buf[tid], o) : buf[tid] + o;
    __syncthreads();
  }
  const int excl = tid > 0 ? buf[tid - 1] : 0;
  __syncthreads();
  return excl;
}

__global__ __launch_bounds__(256) void plan_chunks_kernel(const int32_t* __restrict__ cu, int nseq,
                                                          int Tn, int Lc, int max_chunks,
                                                          int32_t* __restrict__ cu_clean,
                                                          ChunkDesc* __restrict__ chunks,
                                                          int32_t* __restrict__ n_chunks) {
  __shared__ int s_v[256];
  const int tid = threadIdx.x;
  const int n1 = nseq + 1;
  const int per = (n1 + 255) / 256;
  const int qa = min(tid * per, n1), qb = min(qa + per, n1);
  auto clampT = [&](int v) { return v < 0 ? 0 : (v > Tn ? Tn : v); };
  // sanitised offsets: clamp into [0, T], then running maximum
  int m = 0;
  for (int q = qa; q < qb; ++q) m = max(m, clampT(cu[q]));
  int run = block_exclusive_scan<true>(m, s_v);
  for (int q = qa; q < qb; ++q) {
    run = max(run, clampT(cu[q]));
    cu_clean[q] = run;
  }
  __syncthreads();
  // chunk counts and each sequence's first table index
  const int ps = (nseq + 255) / 256;
  const int sa = min(tid * ps, nseq), sb = min(sa + ps, nseq);
  int cnt = 0;
  for (int q = sa; q < sb; ++q) {
    const int len = cu_clean[q + 1] - cu_clean[q];
    cnt += (len + Lc - 1) / Lc;
  }
  int base = block_exclusive_scan<false>(cnt, s_v);
  if (tid == 255) *n_chunks = min(base + cnt, max_chunks);
  for (int q = sa; q < sb; ++q) {
    const int slo = cu_clean[q], send = cu_clean[q + 1];
    const int nc = (send - slo + Lc - 1) / Lc;
    for (int j = 0; j < nc; ++j) {
      if (base + j >= max_chunks) break;
      ChunkDesc d;
      d.hi = send - j * Lc;
      d.lo = max(slo, d.hi - Lc);
      d.seq_lo = slo;
      d.seq_end = send;
      d.first = base;
      d.j = j;
      d.n_in_seq = nc;
      d.pad = 0;
      chunks[base + j] = d;
    }
    base += nc;
  }
}

hipError_t plan_chunks(const int32_t* cu, int nseq, int Tn, int Lc, int max_chunks,
                       int32_t* cu_clean, ChunkDesc* chunks, int32_t* n_chunks, hipStream_t st) {
  hipLaunchKernelGGL(plan_chunks_kernel, dim3(1), dim3(256), 0, st, cu, nseq, Tn, Lc, max_chunks,
                     cu_clean, chunks, n_chunks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 8-channel vector helpers (16-byte accesses for bf16, 2 x 16 for fp32)
// ---------------------------------------------------------------------------
template <typename T> struct Raw8;
template <> struct Raw8<bf16> { bf16x8 v; };
template <> struct Raw8<float> { f32x4 a, b; };
R2L_DEV void raw_load(Raw8<bf16>& r, const bf16* p) { r.v = *(const bf16x8*)p; }
R2L_DEV void raw_load(Raw8<float>& r, const float* p) { r.a = *(const f32x4*)p; r.b = *(const f32x4*)(p + 4); }
R2L_DEV float raw_at(const Raw8<bf16>& r, int i) { return (float)r.v[i]; }
R2L_DEV float raw_at(const Raw8<float>& r, int i) { return i < 4 ? r.a[i] : r.b[i - 4]; }
R2L_DEV void store8(bf16* p, const float v[8]) {
  bf16x8 q;
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = (bf16)v[i];
  *(bf16x8*)p = q;
}
R2L_DEV void store8(float* p, const float v[8]) {
  *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
  *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// softplus for dt.  bf16 activations: log2(1 + 2^(-|v| log2 e)) ln 2 on the
// transcendental unit (rounding 1 + w costs < 2^-24 / w relative, i.e.
// < 1e-4 at the smallest dt the layer uses, far below the bf16 roundings
// around it); fp32 activations: the series/log form of softplus_f.
template <typename T> R2L_DEV float softplus_dt(float v);
template <> R2L_DEV float softplus_dt<float>(float v) { return softplus_f(v); }
template <> R2L_DEV float softplus_dt<bf16>(float v) {
  const float w = exp2_fast(-fabsf(v) * kLog2e);
  return fmaxf(v, 0.0f) + __builtin_amdgcn_logf(1.0f + w) * kLn2;
}

// ---------------------------------------------------------------------------
// The scan kernel.  SUMMARY = pass 1 (chunk summaries), otherwise the main
// pass.  KS = number of 32-wide k-steps of dt_proj on MFMA (fused bf16 only;
// 0 = VALU).
//
// A block of 4 waves owns 64 channels of one time chunk; time is walked right
// to left in blocks of TB = 32 tokens:
//   A  thread (r8 = tid / 8, c8 = tid % 8): token row r8, channels 8 c8 .. +7:
//      consumes the registers prefetched for this block (conv + SiLU -> u,
//      SiLU(z), Dskip u, delta -> LDS in bf16, B and C -> LDS), then issues
//      the next block's loads;
//   M  wave w: dt = softplus(delta . W_dt^T + b) for channels 16 w .. +15 of
//      all 32 rows on MFMA (16x16x32 bf16); fp32 uses the VALU;
//   B  wave w, lane c: channel c, states 4 w .. 4 w + 3 in registers, the
//      recurrence over the block's tokens; the LDS operands run 4 tokens ahead
//      of the arithmetic;
//   C  same layout as A: y = (sum of the 4 partial C.h + Dskip u) SiLU(z),
//      one 16-byte store per thread.
// Prefetch loads are unconditional, from clamped rows, with validity applied
// when consumed: a per-lane branch around a load makes both paths write the
// same registers and forces an immediate wait for the load.
// ---------------------------------------------------------------------------
template <typename T, bool FUSED, bool SUMMARY, int KS>
__global__ __launch_bounds__(256, 2) void scan_kernel(ScanArgs a) {
  constexpr int TB = 32;
  constexpr bool MFMA_DT = FUSED && KS > 0;
  constexpr int RP = MFMA_DT ? KS * 32 : 32;   // padded dt_rank for the MFMA k loop
  constexpr int DLS = RP + 8;                   // delta row stride in LDS (bf16)
  constexpr int DPT = RP / 8;                   // delta floats per thread per row (4..32)
  static_assert(TB * DLS * 2 <= 3 * TB * 64 * 4, "delta must fit in yp_s[1..3]");
  // yp_s (partial C.h sums of B/C) also hosts u and delta between A and M
  __shared__ __attribute__((aligned(16))) float yp_s[4][TB][64];
  __shared__ __attribute__((aligned(16))) float2 pre_s[TB][64];   // (dt, dt*u)
  __shared__ __attribute__((aligned(16))) f32x4 bc_s[TB][8];      // B[0..16) C[0..16)
  float (*u_s)[64] = yp_s[0];
  bf16* dl_s = (bf16*)&yp_s[1][0][0];

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
  if (SUMMARY && d.j == d.n_in_seq - 1) return;  // leftmost chunk: its summary is never used
  const int tid = threadIdx.x;
  const int lane = lane_id(), w = wave_id();
  const int e0 = cblk * 64;
  const int e = e0 + lane;                 // B channel
  const int r8 = tid >> 3, c8 = tid & 7;   // A/C row and channel group
  const int ea = e0 + 8 * c8;              // A/C first channel

  float A2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) A2[i] = -expf(a.A_log[(long)e * NS + 4 * w + i]) * kLog2e;
  float cwr[8][4], cb8[8], dsk8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    dsk8[i] = a.Dskip ? a.Dskip[ea + i] : 0.0f;
    cb8[i] = FUSED ? to_f32(((const T*)a.conv_b)[ea + i]) : 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) cwr[i][k] = FUSED ? to_f32(((const T*)a.conv_w)[(long)(ea + i) * 4 + k]) : 0.0f;
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
#pragma unroll
      for (int p = 0; p < 8; ++p) wdt[ks][p] = W[rowoff + min(k + p, a.R - 1)];
#pragma unroll
      for (int p = 0; p < 8; ++p) if (k + p >= a.R) wdt[ks][p] = (bf16)0.0f;
    }
    dtb_col = a.dt_b[e0 + dcol];
  }

  // carry into this chunk from the chunks to its right
  float h[4] = {0.0f, 0.0f, 0.0f, 0.0f};
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

  // ---------------- prefetch registers ----------------
  const T* xin = FUSED ? (const T*)a.x : (const T*)a.u;
  const long ldx = FUSED ? a.ld_x : a.ld_u;
  const T* zin = (const T*)a.z;
  const bool has_z = zin != nullptr;
  Raw8<T> px[FUSED ? 4 : 1];   // x rows r8 .. r8+3 (fused) or the u row r8
  Raw8<T> pz;                  // z row r8
  float pd[FUSED ? DPT : 8];   // delta (fused) or dt (standalone) of row r8
  float pbc[4];                // 4 of the row's 32 B/C floats
  const bool vec_d = FUSED ? ((a.R & 3) == 0 && (a.ldp & 3) == 0) : true;

  auto issue = [&](int blo, int bhi) {
    const int t = min(blo + r8, bhi - 1);        // clamped: always a valid row
    if constexpr (FUSED) {
#pragma unroll
      for (int j = 0; j < 4; ++j) raw_load(px[j], xin + (long)min(t + j, d.seq_end - 1) * ldx + ea);
      if constexpr (MFMA_DT) {
        // c8 * DPT + DPT <= RP <= R + 31 < ldp: always inside row t
        const float* src = a.xdbl + (long)t * a.ldp + c8 * DPT;
        if (vec_d) {
#pragma unroll
          for (int q = 0; q < DPT / 4; ++q) {
            const f32x4 v = *(const f32x4*)(src + 4 * q);
#pragma unroll
            for (int p = 0; p < 4; ++p) pd[4 * q + p] = v[p];
          }
        } else {
#pragma unroll
          for (int p = 0; p < DPT; ++p) pd[p] = src[p];
        }
      }
      const float* bsrc = a.xdbl + (long)t * a.ldp + a.R + 4 * c8;   // B then C, contiguous
      if (vec_d) {
        const f32x4 v = *(const f32x4*)bsrc;
#pragma unroll
        for (int p = 0; p < 4; ++p) pbc[p] = v[p];
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) pbc[p] = bsrc[p];
      }
    } else {
      raw_load(px[0], xin + (long)t * ldx + ea);
      const f32x4 v0 = *(const f32x4*)(a.dt + (long)t * a.ld_dt + ea);
      const f32x4 v1 = *(const f32x4*)(a.dt + (long)t * a.ld_dt + ea + 4);
#pragma unroll
      for (int p = 0; p < 4; ++p) { pd[p] = v0[p]; pd[4 + p] = v1[p]; }
      const float* src = (c8 < 4 ? a.Bm + 4 * c8 : a.Cm + 4 * (c8 - 4)) + (long)t * a.ld_bc;
#pragma unroll
      for (int p = 0; p < 4; ++p) pbc[p] = src[p];
    }
    if constexpr (!SUMMARY) {
      if (has_z) raw_load(pz, zin + (long)t * a.ld_z + ea);
    }
  };

  // SiLU(z) and Dskip*u of this thread's (row, 8 channels): phase A makes
  // them, phase C of the same block uses them.
  float g8[8], du8[8];
  int bhi = d.hi;
  if (bhi > d.lo) issue(max(d.lo, bhi - TB), bhi);
  for (; bhi > d.lo; bhi -= TB) {
    const int blo = max(d.lo, bhi - TB);
    const int nt = bhi - blo;
    const int tr = blo + r8;
    const bool rv = tr < bhi;
    // ---------------- A: consume this block's prefetched inputs ----------------
    {
      float uu[8];
      if constexpr (FUSED) {
        bool xv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[j] = tr + j < d.seq_end;   // zero past the sequence end
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float c = cb8[i];
#pragma unroll
          for (int j = 0; j < 4; ++j) c = fmaf(cwr[i][3 - j], xv[j] ? raw_at(px[j], i) : 0.0f, c);
          uu[i] = silu_fast(c);
        }
        if constexpr (MFMA_DT) {
#pragma unroll
          for (int q = 0; q < DPT / 4; ++q) {
            bf16x4 pk;
#pragma unroll
            for (int p = 0; p < 4; ++p) pk[p] = (rv && c8 * DPT + 4 * q + p < a.R) ? (bf16)pd[4 * q + p] : (bf16)0.0f;
            *(bf16x4*)(dl_s + r8 * DLS + c8 * DPT + 4 * q) = pk;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uu[i] = rv ? raw_at(px[0], i) : 0.0f;
          const float dtv = rv ? pd[i] : 0.0f;
          pre_s[r8][8 * c8 + i] = make_float2(dtv, dtv * uu[i]);
        }
      }
      *(f32x4*)&u_s[r8][8 * c8] = f32x4{uu[0], uu[1], uu[2], uu[3]};
      *(f32x4*)&u_s[r8][8 * c8 + 4] = f32x4{uu[4], uu[5], uu[6], uu[7]};
      if constexpr (!SUMMARY) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          g8[i] = has_z ? silu_fast(rv ? raw_at(pz, i) : 0.0f) : 1.0f;
          du8[i] = dsk8[i] * uu[i];
        }
      }
      bc_s[r8][c8] = rv ? f32x4{pbc[0], pbc[1], pbc[2], pbc[3]} : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // the next block's loads go out now and land during this block's compute
    if (bhi - TB > d.lo) issue(max(d.lo, bhi - 2 * TB), bhi - TB);
    __syncthreads();
    // ---------------- M: dt = softplus(delta . W_dt^T + b) ----------------
    if constexpr (FUSED) {
      if constexpr (MFMA_DT) {
#pragma unroll
        for (int rt = 0; rt < TB / 16; ++rt) {
          f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
          const int row = rt * 16 + (lane & 15);
          bf16x8 af[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) af[ks] = *(const bf16x8*)(dl_s + row * DLS + ks * 32 + (lane >> 4) * 8);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks], wdt[ks], acc, 0, 0, 0);
          // D layout: lane holds rows 4 (lane >> 4) + i, column (lane & 15)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = rt * 16 + 4 * (lane >> 4) + i;
            const float dtv = softplus_dt<T>(acc[i] + dtb_col);
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
    // ---------------- B: the recurrence, right to left ----------------
    auto compute = [&](int r, float2 p, f32x4 Bv, f32x4 Cv) {
      float av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = exp2_fast(p.x * A2[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = fmaf(av[i], h[i], p.y * Bv[i]);
      if constexpr (SUMMARY) {
        sdt += p.x;
      } else {
        yp_s[w][r][lane] = fmaf(Cv[1], h[1], Cv[0] * h[0]) + fmaf(Cv[3], h[3], Cv[2] * h[2]);
      }
    };
    if (nt == TB) {
      // 4-deep ring of LDS operands (indices are constants after unrolling)
      constexpr int LA = 4;
      float2 Pq[LA];
      f32x4 Bq[LA], Cq[LA];
#pragma unroll
      for (int k = 0; k < LA; ++k) {
        Pq[k] = pre_s[TB - 1 - k][lane];
        Bq[k] = bc_s[TB - 1 - k][w];
        Cq[k] = SUMMARY ? Bq[k] : bc_s[TB - 1 - k][4 + w];
      }
#pragma unroll
      for (int k = 0; k < TB; ++k) {
        const int r = TB - 1 - k, sl = k % LA;
        const float2 p = Pq[sl];
        const f32x4 Bv = Bq[sl], Cv = Cq[sl];
        if (k + LA < TB) {
          Pq[sl] = pre_s[r - LA][lane];
          Bq[sl] = bc_s[r - LA][w];
          if constexpr (!SUMMARY) Cq[sl] = bc_s[r - LA][4 + w];
        }
        compute(r, p, Bv, Cv);
      }
    } else {
      for (int r = nt - 1; r >= 0; --r) compute(r, pre_s[r][lane], bc_s[r][w], bc_s[r][4 + w]);
    }
    __syncthreads();
    // ---------------- C: combine and store ----------------
    if constexpr (!SUMMARY) {
      if (rv) {
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
        store8((T*)a.y + (long)tr * E + ea, v);
      }
      __syncthreads();
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

template <typename T, bool SUMMARY>
static hipError_t launch_scan(const ScanArgs& a, bool fused, hipStream_t st) {
  const int nblocks = a.max_chunks * (a.E / 64);
  if (nblocks <= 0) return hipSuccess;
  dim3 grid(nblocks), block(256);
  if (!fused) {
    hipLaunchKernelGGL((scan_kernel<T, false, SUMMARY, 0>), grid, block, 0, st, a);
  } else if constexpr (std::is_same<T, float>::value) {
    hipLaunchKernelGGL((scan_kernel<T, true, SUMMARY, 0>), grid, block, 0, st, a);
  } else {
    const int ks = (a.R + 31) / 32;
    if (ks > 8) hipLaunchKernelGGL((scan_kernel<T, true, SUMMARY, 0>), grid, block, 0, st, a);
    else if (ks <= 1) hipLaunchKernelGGL((scan_kernel<T, true, SUMMARY, 1>), grid, block, 0, st, a);
    else if (ks <= 2) hipLaunchKernelGGL((scan_kernel<T, true, SUMMARY, 2>), grid, block, 0, st, a);
    else if (ks <= 4) hipLaunchKernelGGL((scan_kernel<T, true, SUMMARY, 4>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_kernel<T, true, SUMMARY, 8>), grid, block, 0, st, a);
  }
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
template hipError_t scan_summary<float>(const ScanArgs&, bool, hipStream_t);
template hipError_t scan_summary<bf16>(const ScanArgs&, bool, hipStream_t);
template hipError_t scan_main<float>(const ScanArgs&, bool, hipStream_t);
template hipError_t scan_main<bf16>(const ScanArgs&, bool, hipStream_t);

}  // namespace r2l
