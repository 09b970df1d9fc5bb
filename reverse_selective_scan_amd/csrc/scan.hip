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
// the scan kernel: SUMMARY = pass 1, otherwise the main pass.
// KS = number of 32-wide k-steps of dt_proj on MFMA (fused bf16 only).
// ---------------------------------------------------------------------------
template <typename T, bool FUSED, bool SUMMARY, int KS>
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
  __shared__ float u_s[TB][64];
  __shared__ float dt_s[TB][64];
  __shared__ float g_s[SUMMARY ? 1 : TB][64];
  __shared__ float du_s[SUMMARY ? 1 : TB][64];
  __shared__ f32x4 bc_s[TB][8];
  __shared__ float yp_s[SUMMARY ? 1 : 4][TB][64];

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
  const int e = e0 + lane;

  float A2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) A2[i] = -expf(a.A_log[(long)e * NS + 4 * w + i]) * kLog2e;
  const float Dsk = a.Dskip ? a.Dskip[e] : 0.0f;

  const T* x = (const T*)a.x;
  const T* z = (const T*)a.z;
  const T* uin = (const T*)a.u;
  float cw[4] = {0, 0, 0, 0}, cbias = 0.0f;
  if (FUSED) {
#pragma unroll
    for (int k = 0; k < 4; ++k) cw[k] = to_f32(((const T*)a.conv_w)[(long)e * 4 + k]);
    cbias = to_f32(((const T*)a.conv_b)[e]);
  }
  // dt_proj fragments (B operand of the 16x16x32 MFMA): channel
  // e0 + 16w + (lane & 15), k = 32 ks + 8 (lane >> 4) .. +7.
  constexpr bool MFMA_DT = FUSED && KS > 0;
  bf16x8 wdt[MFMA_DT ? KS : 1];
  const int dcol = 16 * w + (lane & 15);
  float dtb_col = 0.0f;
  if (MFMA_DT) {
    const bf16* W = (const bf16*)a.dt_w;
    const long rowoff = (long)(e0 + dcol) * a.R;
#pragma unroll
    for (int ks = 0; ks < (MFMA_DT ? KS : 1); ++ks) {
      const int k = ks * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int p = 0; p < 8; ++p) wdt[ks][p] = (k + p < a.R) ? W[rowoff + k + p] : (bf16)0.0f;
    }
    dtb_col = a.dt_b[e0 + dcol];
  }
  const float dtb_lane = FUSED ? a.dt_b[e] : 0.0f;

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

  for (int bhi = d.hi; bhi > d.lo; bhi -= TB) {
    const int blo = max(d.lo, bhi - TB);
    const int nt = bhi - blo;
    // ---------------- A1: per-(token, channel) inputs ----------------
    if (FUSED) {
      float xw[8 + 3];
#pragma unroll
      for (int q = 0; q < 11; ++q) {
        const int t = blo + 8 * w + q;
        xw[q] = (t < d.seq_end) ? to_f32(x[(long)t * a.ld_x + e]) : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * w + i;
        const int t = blo + r;
        float c = cbias;
#pragma unroll
        for (int j = 0; j < 4; ++j) c = fmaf(cw[3 - j], xw[i + j], c);
        const float uu = silu_fast(c);
        u_s[r][lane] = uu;
        if (!SUMMARY) {
          const float zz = (z != nullptr && t < bhi) ? to_f32(z[(long)t * a.ld_z + e]) : 0.0f;
          g_s[r][lane] = z != nullptr ? silu_fast(zz) : 1.0f;
          du_s[r][lane] = Dsk * uu;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * w + i;
        const int t = blo + r;
        const bool v = t < bhi;
        const float uu = v ? to_f32(uin[(long)t * a.ld_u + e]) : 0.0f;
        u_s[r][lane] = uu;
        dt_s[r][lane] = v ? a.dt[(long)t * a.ld_dt + e] : 0.0f;
        if (!SUMMARY) {
          const float zz = (z != nullptr && v) ? to_f32(z[(long)t * a.ld_z + e]) : 0.0f;
          g_s[r][lane] = z != nullptr ? silu_fast(zz) : 1.0f;
          du_s[r][lane] = Dsk * uu;
        }
      }
    }
    {
      const int r = tid >> 3, q = tid & 7;
      const int t = blo + r;
      f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
      if (t < bhi) {
        const float* src;
        if (FUSED) src = a.xdbl + (long)t * a.ldp + a.R + 4 * q;  // B then C, contiguous
        else src = (q < 4 ? a.Bm + 4 * q : a.Cm + 4 * (q - 4)) + (long)t * a.ld_bc;
#pragma unroll
        for (int p = 0; p < 4; ++p) v[p] = src[p];
      }
      bc_s[r][q] = v;
    }
    __syncthreads();
    // ---------------- A2: dt = softplus(delta . W_dt^T + b) ----------------
    if (FUSED) {
      if (MFMA_DT) {
#pragma unroll
        for (int rt = 0; rt < TB / 16; ++rt) {
          f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
          const int row = rt * 16 + (lane & 15);
          const int t = blo + row;
#pragma unroll
          for (int ks = 0; ks < (MFMA_DT ? KS : 1); ++ks) {
            const int k = ks * 32 + (lane >> 4) * 8;
            bf16x8 af;
#pragma unroll
            for (int p = 0; p < 8; ++p)
              af[p] = (t < bhi && k + p < a.R) ? (bf16)a.xdbl[(long)t * a.ldp + k + p] : (bf16)0.0f;
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, wdt[ks], acc, 0, 0, 0);
          }
          // D layout: lane holds rows 4*(lane>>4) + i, column (lane & 15)
#pragma unroll
          for (int i = 0; i < 4; ++i) dt_s[rt * 16 + 4 * (lane >> 4) + i][dcol] = softplus_f(acc[i] + dtb_col);
        }
      } else {
        const T* W = (const T*)a.dt_w;
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * w + i;
          const int t = blo + r;
          float acc = 0.0f;
          if (t < bhi)
            for (int k = 0; k < a.R; ++k)
              acc = fmaf(a.xdbl[(long)t * a.ldp + k], to_f32(W[(long)e * a.R + k]), acc);
          dt_s[r][lane] = softplus_f(acc + dtb_lane);
        }
      }
      __syncthreads();
    }
    // ---------------- B: the recurrence, right to left ----------------
    for (int r = nt - 1; r >= 0; --r) {
      const float dtv = dt_s[r][lane];
      const float dtu = dtv * u_s[r][lane];
      const f32x4 Bv = bc_s[r][w];
      if (SUMMARY) sdt += dtv;
      if constexpr (!SUMMARY) {
        const f32x4 Cv = bc_s[r][4 + w];
        float y = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[i] = fmaf(exp2_fast(dtv * A2[i]), h[i], dtu * Bv[i]);
          y = fmaf(Cv[i], h[i], y);
        }
        yp_s[w][r][lane] = y;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = fmaf(exp2_fast(dtv * A2[i]), h[i], dtu * Bv[i]);
      }
    }
    __syncthreads();
    // ---------------- C: combine and store ----------------
    if constexpr (!SUMMARY) {
      T* y = (T*)a.y;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * w + i;
        if (r < nt) {
          float v = yp_s[0][r][lane] + yp_s[1][r][lane] + yp_s[2][r][lane] + yp_s[3][r][lane] +
                    du_s[r][lane];
          v *= g_s[r][lane];
          y[(long)(blo + r) * E + e] = from_f32<T>(v);
        }
      }
      __syncthreads();
    }
  }
  if (SUMMARY) {
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
