// Reverse selective scan ("Bifocal Diffusion Language Models", §3.4 step 2:
// the Mamba-1 selective scan run over the flipped sequence; in the original
// token order it runs from each sequence's last token to its first):
//   h_t = exp(dt_t A) (.) h_{t+1} + (dt_t u_t) (x) B_t,   h = 0 past the end,
//   y_t = (C_t . h_t + Dskip u_t) * SiLU(z_t),             A = -exp(A_log).
//
// Work decomposition.  A block owns 64 channels of one time chunk of one
// sequence.  Its 4 waves split the 16 states: wave w keeps states
// 4w..4w+3 of the lane's channel in registers (fp32) for the whole chunk, so
// the recurrence needs no communication; the four partial C.h sums meet in
// LDS.  Time is walked right to left in blocks of TB tokens:
//   A1  all lanes prepare the block's per-(token, channel) inputs in LDS:
//       fused mode computes the conv + SiLU from x (x, z are the two halves of
//       in_proj's output), SiLU(z) and Dskip*u; B and C rows are staged too;
//   A2  (fused mode) dt = softplus(delta . W_dt^T + b_dt) for the block on
//       MFMA (16x16x32 bf16; fp32 activations use the VALU);
//   B   the serial recurrence over the block's tokens, 4 states per lane,
//       exp on the transcendental unit (2^x with A pre-scaled by log2 e);
//   C   y = (sum of the 4 partial sums + Dskip u) * SiLU(z), stored.
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

constexpr int TB = 32;    // tokens per time block
constexpr int NS = 16;    // d_state (§4.1)

// ---------------------------------------------------------------------------
// chunk planning (one block): sanitised cu_seqlens (clamped to [0, T] and
// made non-decreasing) and the chunk table, rightmost chunk of each
// sequence first.
// ---------------------------------------------------------------------------
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
  int m = 0;
  for (int q = qa; q < qb; ++q) m = max(m, clampT(cu[q]));
  s_v[tid] = m;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int v = s_v[i];
      s_v[i] = run;  // exclusive prefix max
      run = max(run, v);
    }
  }
  __syncthreads();
  int run = s_v[tid];
  for (int q = qa; q < qb; ++q) {
    run = max(run, clampT(cu[q]));
    cu_clean[q] = run;
  }
  __syncthreads();
  // chunk counts
  const int ps = (nseq + 255) / 256;
  const int sa = min(tid * ps, nseq), sb = min(sa + ps, nseq);
  int cnt = 0;
  for (int q = sa; q < sb; ++q) {
    const int len = cu_clean[q + 1] - cu_clean[q];
    cnt += (len + Lc - 1) / Lc;
  }
  __syncthreads();
  s_v[tid] = cnt;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < 256; ++i) {
      const int v = s_v[i];
      s_v[i] = acc;
      acc += v;
    }
    *n_chunks = min(acc, max_chunks);
  }
  __syncthreads();
  int base = s_v[tid];
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
// 8-channel vector helpers (16-byte loads/stores for bf16, 2 x 16 for fp32)
// ---------------------------------------------------------------------------
R2L_DEV void load8(const bf16* p, float v[8]) {
  const bf16x8 q = *(const bf16x8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)q[i];
}
R2L_DEV void load8(const float* p, float v[8]) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}
R2L_DEV void store8(bf16* p, const float v[8]) {
  bf16x8 q;
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = (bf16)v[i];
  *(bf16x8*)p = q;
}
R2L_DEV void store8(float* p, const float v[8]) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[4 + i]; }
  *(f32x4*)p = a;
  *(f32x4*)(p + 4) = b;
}
template <typename T> struct Raw8;
template <> struct Raw8<bf16> { bf16x8 v; };
template <> struct Raw8<float> { f32x4 a, b; };
R2L_DEV void raw_load(Raw8<bf16>& r, const bf16* p) { r.v = *(const bf16x8*)p; }
R2L_DEV void raw_load(Raw8<float>& r, const float* p) { r.a = *(const f32x4*)p; r.b = *(const f32x4*)(p + 4); }
R2L_DEV void raw_zero(Raw8<bf16>& r) { r.v = bf16x8{}; }
R2L_DEV void raw_zero(Raw8<float>& r) { r.a = f32x4{0, 0, 0, 0}; r.b = r.a; }
R2L_DEV void raw_get(const Raw8<bf16>& r, float v[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)r.v[i];
}
R2L_DEV void raw_get(const Raw8<float>& r, float v[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = r.a[i]; v[4 + i] = r.b[i]; }
}

// ---------------------------------------------------------------------------
// the scan kernel: SUMMARY = pass 1, otherwise the main pass.
// KS = number of 32-wide k-steps of dt_proj on MFMA (fused bf16 only; 0 = VALU).
//
// Thread layouts inside a block of TB = 32 tokens x 64 channels:
//   A, C  thread (r = tid / 8, c8 = tid % 8): token row r, channels 8 c8 .. +7,
//         so every global access is one 16-byte vector per thread;
//   M     wave w: channels 16 w .. +15 of all 32 rows (two 16x16 MFMA tiles);
//   B     wave w, lane c: channel c, states 4 w .. 4 w + 3, tokens in order.
// The next block's global loads are issued before the current block's
// compute, so memory latency overlaps the recurrence.
// ---------------------------------------------------------------------------
template <typename T, bool FUSED, bool SUMMARY, int KS>
__global__ __launch_bounds__(256, 2) void scan_kernel(ScanArgs a) {
  constexpr bool MFMA_DT = FUSED && KS > 0;
  constexpr int RP = MFMA_DT ? KS * 32 : 32;   // padded dt_rank for the MFMA k loop
  constexpr int DLS = RP + 8;                   // delta row stride in LDS (bf16)
  constexpr int DPT = RP / 8;                   // delta floats per thread per row
  static_assert(TB * DLS * 2 + TB * 64 * 4 <= 4 * TB * 64 * 4, "aliases must fit in yp_s");
  // yp_s (partial C.h sums, phase B/C) also hosts u (phases A/M) and delta (A/M)
  __shared__ __attribute__((aligned(16))) float yp_s[4][TB][64];
  __shared__ __attribute__((aligned(16))) float g_s[SUMMARY ? 1 : TB][64];
  __shared__ __attribute__((aligned(16))) float du_s[SUMMARY ? 1 : TB][64];
  __shared__ __attribute__((aligned(16))) float2 pre_s[TB][64];   // (dt, dt*u)
  __shared__ __attribute__((aligned(16))) f32x4 bc_s[TB][8];      // B[0..16) C[0..16)
  float (*u_s)[64] = yp_s[0];
  bf16* dl_s = (bf16*)&yp_s[1][0][0];

  const int E = a.E;
  const int NB = E / 64;
  const int lid = xcd_remap(blockIdx.x, a.max_chunks * NB);
  const int ci = lid / NB, cblk = lid % NB;
  if (ci >= *a.n_chunks) return;
  const ChunkDesc d = a.chunks[ci];
  if (SUMMARY && d.j == d.n_in_seq - 1) return;  // leftmost chunk: its summary is never used
  const int tid = threadIdx.x;
  const int lane = lane_id(), w = wave_id();
  const int e0 = cblk * 64;
  const int e = e0 + lane;                 // phase B channel
  const int r8 = tid >> 3, c8 = tid & 7;   // phase A/C row and channel group
  const int ea = e0 + 8 * c8;              // phase A/C first channel

  float A2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) A2[i] = -expf(a.A_log[(long)e * NS + 4 * w + i]) * kLog2e;

  // phase A constants for channels ea .. ea+7
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
      for (int p = 0; p < 8; ++p) wdt[ks][p] = (k + p < a.R) ? W[rowoff + k + p] : (bf16)0.0f;
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
  Raw8<T> px[FUSED ? 4 : 1];   // x rows r8 .. r8+3 (fused) or u row r8
  Raw8<T> pz;                  // z row r8
  f32x4 pd[FUSED ? DPT / 4 : 2];  // delta (fused) or dt (standalone) of row r8
  f32x4 pbc;                   // 4 of the row's 32 B/C floats
  const bool vec_bc = FUSED ? ((a.R & 3) == 0 && (a.ldp & 3) == 0) : false;

  auto issue = [&](int blo, int bhi) {
    const int t = blo + r8;
    const bool tv = t < bhi;
    if constexpr (FUSED) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (t + j < d.seq_end) raw_load(px[j], xin + (long)(t + j) * ldx + ea);
        else raw_zero(px[j]);
      }
#pragma unroll
      for (int q = 0; q < (MFMA_DT ? DPT / 4 : 0); ++q) {
        const int k = c8 * DPT + 4 * q;
        if (tv && vec_bc && k + 3 < a.R) {
          pd[q] = *(const f32x4*)(a.xdbl + (long)t * a.ldp + k);
        } else {
#pragma unroll
          for (int p = 0; p < 4; ++p) pd[q][p] = (tv && k + p < a.R) ? a.xdbl[(long)t * a.ldp + k + p] : 0.0f;
        }
      }
      if (tv && vec_bc) {
        pbc = *(const f32x4*)(a.xdbl + (long)t * a.ldp + a.R + 4 * c8);
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) pbc[p] = tv ? a.xdbl[(long)t * a.ldp + a.R + 4 * c8 + p] : 0.0f;
      }
    } else {
      if (tv) raw_load(px[0], xin + (long)t * ldx + ea);
      else raw_zero(px[0]);
      if (tv) {
        pd[0] = *(const f32x4*)(a.dt + (long)t * a.ld_dt + ea);
        pd[1] = *(const f32x4*)(a.dt + (long)t * a.ld_dt + ea + 4);
      } else {
        pd[0] = f32x4{0, 0, 0, 0};
        pd[1] = pd[0];
      }
      const float* src = (c8 < 4 ? a.Bm + 4 * c8 : a.Cm + 4 * (c8 - 4)) + (long)t * a.ld_bc;
#pragma unroll
      for (int p = 0; p < 4; ++p) pbc[p] = tv ? src[p] : 0.0f;
    }
    if (!SUMMARY) {
      if (zin != nullptr && tv) raw_load(pz, zin + (long)t * a.ld_z + ea);
      else raw_zero(pz);
    }
  };

  int bhi = d.hi;
  if (bhi > d.lo) issue(max(d.lo, bhi - TB), bhi);
  for (; bhi > d.lo; bhi -= TB) {
    const int blo = max(d.lo, bhi - TB);
    const int nt = bhi - blo;
    // ---------------- A: per-(token, channel) inputs ----------------
    {
      float uu[8];
      if constexpr (FUSED) {
        float xr[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) raw_get(px[j], xr[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float c = cb8[i];
#pragma unroll
          for (int j = 0; j < 4; ++j) c = fmaf(cwr[i][3 - j], xr[j][i], c);
          uu[i] = silu_fast(c);
        }
        if constexpr (MFMA_DT) {
          // delta -> bf16 -> LDS (A operand of the dt MFMA)
#pragma unroll
          for (int q = 0; q < DPT / 4; ++q) {   // DPT is 4, 8, 16 or 32
            bf16x4 pk;
#pragma unroll
            for (int p = 0; p < 4; ++p) pk[p] = (bf16)pd[q][p];
            *(bf16x4*)(dl_s + r8 * DLS + c8 * DPT + 4 * q) = pk;
          }
        }
      } else {
        raw_get(px[0], uu);
        float dtv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) { dtv[i] = pd[0][i]; dtv[4 + i] = pd[1][i]; }
#pragma unroll
        for (int i = 0; i < 8; ++i) pre_s[r8][8 * c8 + i] = make_float2(dtv[i], dtv[i] * uu[i]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) u_s[r8][8 * c8 + i] = uu[i];
      if constexpr (!SUMMARY) {
        float zz[8];
        raw_get(pz, zz);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          g_s[r8][8 * c8 + i] = zin != nullptr ? silu_fast(zz[i]) : 1.0f;
          du_s[r8][8 * c8 + i] = dsk8[i] * uu[i];
        }
      }
      bc_s[r8][c8] = pbc;
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
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 af = *(const bf16x8*)(dl_s + row * DLS + ks * 32 + (lane >> 4) * 8);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, wdt[ks], acc, 0, 0, 0);
          }
          // D layout: lane holds rows 4 (lane >> 4) + i, column (lane & 15)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = rt * 16 + 4 * (lane >> 4) + i;
            const float dtv = softplus_f(acc[i] + dtb_col);
            pre_s[rr][dcol] = make_float2(dtv, dtv * u_s[rr][dcol]);
          }
        }
      } else {
        const T* W = (const T*)a.dt_w;
        const float dtb = a.dt_b[e];
        for (int i = 0; i < TB / 4; ++i) {
          const int rr = (TB / 4) * w + i;
          const int t = blo + rr;
          float acc = 0.0f;
          if (t < bhi)
            for (int k = 0; k < a.R; ++k)
              acc = fmaf(a.xdbl[(long)t * a.ldp + k], to_f32(W[(long)e * a.R + k]), acc);
          const float dtv = softplus_f(acc + dtb);
          pre_s[rr][lane] = make_float2(dtv, dtv * u_s[rr][lane]);
        }
      }
      __syncthreads();
    }
    // ---------------- B: the recurrence, right to left ----------------
    auto step = [&](int r) {
      const float2 p = pre_s[r][lane];
      const f32x4 Bv = bc_s[r][w];
      if constexpr (SUMMARY) {
        sdt += p.x;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = fmaf(exp2_fast(p.x * A2[i]), h[i], p.y * Bv[i]);
      } else {
        const f32x4 Cv = bc_s[r][4 + w];
        float y = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[i] = fmaf(exp2_fast(p.x * A2[i]), h[i], p.y * Bv[i]);
          y = fmaf(Cv[i], h[i], y);
        }
        yp_s[w][r][lane] = y;
      }
    };
    if (nt == TB) {
#pragma unroll
      for (int r = TB - 1; r >= 0; --r) step(r);
    } else {
      for (int r = nt - 1; r >= 0; --r) step(r);
    }
    __syncthreads();
    // ---------------- C: combine and store ----------------
    if constexpr (!SUMMARY) {
      if (r8 < nt) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int cc = 8 * c8 + i;
          v[i] = (yp_s[0][r8][cc] + yp_s[1][r8][cc] + yp_s[2][r8][cc] + yp_s[3][r8][cc] + du_s[r8][cc]) *
                 g_s[r8][cc];
        }
        store8((T*)a.y + (long)(blo + r8) * E + ea, v);
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
