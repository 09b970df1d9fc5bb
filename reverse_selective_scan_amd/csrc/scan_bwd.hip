// Backward of the standalone reverse selective scan (the gradient of
// r2l_scan_fwd, for training the sidecar: "Bifocal Diffusion Language
// Models", §3.5, plug-in mode).  Forward, per sequence and channel e, state n:
//   h_t = a_t h_{t+1} + dtu_t B_t[n],  a_t = exp(dt_t A),  dtu_t = dt_t u_t,
//   y_t = (C_t . h_t + D u_t) SiLU(z_t),
// run from the sequence end to its start.  With g_t = dy_t SiLU(z_t) the
// adjoint lambda_t = dL/dh_t runs the other way, left to right:
//   lambda_t = g_t C_t + a_{t-1} lambda_{t-1},
// and the gradients are
//   dC_t[n] = sum_e g_t h_t,        dB_t[n] = sum_e lambda_t dtu_t,
//   du_t = dt_t sum_n lambda_t B_t + D g_t,
//   ddt_t = u_t sum_n lambda_t B_t + sum_n lambda_t h_{t+1} a_t A,
//   dA = sum_t lambda_t h_{t+1} a_t dt_t (dA_log = dA A),  dD = sum_t g_t u_t,
// dz from the first sweep (scan.hip, BWD): dz = dy SiLU'(z) (C.h + D u).
//
// The first sweep stores the state entering every 16-token sub-block from
// the right.  This adjoint sweep walks the sub-blocks left to right: it
// recomputes the sub-block's 16 states right to left into registers (rows
// past a sequence read as zeros, so they are identity steps: dt = 0 gives
// a = 1 and no input), then runs the adjoint over them left to right.  A
// block owns 64 channels of one time chunk (a whole sequence, or a piece of
// one when the sequences alone would leave the GPU idle: the adjoint then
// enters a chunk with the carry of the chunks to its left, from the chunk
// summaries below); its 4 waves split the 16 states as
// in the forward (lane = channel, 4 states per lane, the input term on a
// 4x4x1 fp32 MFMA).  The sums over channels (dB, dC) are reduced across the
// 64 lanes with lane swaps and row rotations, then across channel blocks by
// a second kernel; the sums over states (du, ddt) meet in LDS; the sums over
// time (dA, dD) stay in registers until the sequence ends and are added
// over sequences by the second kernel.  Every sum has a fixed order.
#include "kernels.h"

namespace r2l {

namespace {

constexpr int NS = 16;
constexpr int SB = 16;   // sub-block length

typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

R2L_DEV Rsrc rows_of(const void* base, long row0, long pitch_bytes, int rows) {
  const long bytes = rows > 0 ? rows * pitch_bytes : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)base + row0 * pitch_bytes), 0, (int)bytes,
                                           0x00020000);
}
constexpr unsigned kPast = 0x80000000u;   // an offset past every window

// 4 consecutive channels of one row, as floats
R2L_DEV void load4(float v[4], Rsrc r, unsigned off, bf16*) {
  const u32x2 q = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    v[2 * i] = __builtin_bit_cast(float, q[i] << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, q[i] & 0xffff0000u);
  }
}
// (the 16-byte load is reinterpreted as a whole vector: extracting one
// 32-bit element and reinterpreting it as a float makes this compiler narrow
// the load to its first dword)
R2L_DEV void load4(float v[4], Rsrc r, unsigned off, float*) {
  const f32x4 q = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = q[i];
}
R2L_DEV float ld1(Rsrc r, unsigned off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
R2L_DEV void st4(Rsrc r, unsigned off, const float v[4]) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]}), r, off, 0, 0);
}

// x + the value of the lane `ror` places on within the lane's row of 16
template <int ROR>
R2L_DEV float add_ror(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(unsigned, x),
                                                                     0x120 + ROR, 0xf, 0xf, false));
}
// s = sum of the two halves of a lane swap: (x, y) with the upper 32 lanes
// of x exchanged with the lower 32 of y (16: odd rows of x with even rows
// of y); lanes then hold x summed over lane pairs in the lower half (even
// rows) and y in the upper half (odd rows).
R2L_DEV float swap32_sum(float x, float y) {
  const float2v p = __builtin_bit_cast(float2v, __builtin_amdgcn_permlane32_swap(
      __builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y), false, false));
  return p[0] + p[1];
}
R2L_DEV float swap16_sum(float x, float y) {
  const float2v p = __builtin_bit_cast(float2v, __builtin_amdgcn_permlane16_swap(
      __builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y), false, false));
  return p[0] + p[1];
}

}  // namespace

template <typename T>
__global__ __launch_bounds__(256, 2) void scan_bwd_adj_kernel(ScanBwdArgs a) {
  constexpr unsigned SZ = sizeof(T);
  __shared__ __attribute__((aligned(16))) float2 pre_s[SB][64];     // (dt, dt u)
  __shared__ __attribute__((aligned(16))) float g_s[SB][64];        // dy SiLU(z)
  __shared__ __attribute__((aligned(16))) f32x4 bc_s[SB][8];        // B[0..16) C[0..16)
  __shared__ __attribute__((aligned(16))) float s1_s[4][SB][64];    // per wave: sum_n lambda B
  __shared__ __attribute__((aligned(16))) float s2_s[4][SB][64];    // per wave: sum_n lambda h' a A
  __shared__ __attribute__((aligned(16))) float dbc_s[SB][32];      // dB | dC of the block's channels
  __shared__ __attribute__((aligned(16))) float red_s[SB][64];      // dD over rows

  const int E = a.E;
  const int NB = E / 64;
  const int ci = blockIdx.x / NB, cblk = blockIdx.x % NB;
  if (ci >= *a.n_chunks) return;
  const ChunkDesc d = a.chunks[ci];
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int e0 = cblk * 64, e = e0 + lane;
  const int r16 = tid >> 4, c16 = tid & 15;     // A/C phases: row, 4-channel group
  const int ea = e0 + 4 * c16;

  float A2[4], An[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    An[i] = -expf(a.A_log[(long)e * NS + 4 * w + i]);
    A2[i] = An[i] * kLog2e;
  }
  float dsk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) dsk[j] = a.Dskip ? a.Dskip[ea + j] : 0.0f;
  const bool has_z = a.z != nullptr;

  const long ldu_b = a.ld_u * (long)SZ, lddt_b = a.ld_dt * 4, ldbc_b = a.ld_bc * 4;
  const long ldz_b = a.ld_z * (long)SZ, lddy_b = a.ld_dy * (long)SZ, lde_b = (long)E * 4;
  const unsigned offU = (unsigned)(r16 * ldu_b) + (unsigned)ea * SZ;
  const unsigned offDT = (unsigned)(r16 * lddt_b) + (unsigned)ea * 4;
  const unsigned offZ = (unsigned)(r16 * ldz_b) + (unsigned)ea * SZ;
  const unsigned offDY = (unsigned)(r16 * lddy_b) + (unsigned)ea * SZ;
  const unsigned offE = (unsigned)(r16 * lde_b) + (unsigned)ea * 4;
  // B (c16 < 4) or C (4 <= c16 < 8): 4 of the row's 32 floats
  const unsigned offB = c16 < 4 ? (unsigned)(r16 * ldbc_b) + 16u * c16 : kPast;
  const unsigned offC = (c16 >= 4 && c16 < 8) ? (unsigned)(r16 * ldbc_b) + 16u * (c16 - 4) : kPast;

  // prefetch registers of one sub-block
  float pu[4], pdt[4], pz[4], pdy[4], pbc[4];
  auto issue = [&](int blo, int bhi) __attribute__((always_inline)) {
    const int rows = bhi - blo;
    load4(pu, rows_of(a.u, blo, ldu_b, rows), offU, (T*)nullptr);
    load4(pdt, rows_of(a.dt, blo, lddt_b, rows), offDT, (float*)nullptr);
    load4(pdy, rows_of(a.dy, blo, lddy_b, rows), offDY, (T*)nullptr);
    if (has_z) load4(pz, rows_of(a.z, blo, ldz_b, rows), offZ, (T*)nullptr);
    const Rsrc rB = rows_of(a.Bm, blo, ldbc_b, rows), rC = rows_of(a.Cm, blo, ldbc_b, rows);
#pragma unroll
    for (int p = 0; p < 4; ++p) pbc[p] = ld1(rB, offB + 4u * p) + ld1(rC, offC + 4u * p);
  };

  f32x4 mu = {0.0f, 0.0f, 0.0f, 0.0f};     // a_{t-1} lambda_{t-1}, carried left to right
  if (a.adjM != nullptr) {
    // carry into this chunk from the chunks to its left (scan order: j grows
    // leftward), folded from the leftmost: m = M_j + Q_j m
    for (int jj = d.n_in_seq - 1; jj > d.j; --jj) {
      const long base = (long)(d.first + jj) * NS * E;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long off = base + (long)(4 * w + i) * E + e;
        mu[i] = fmaf(a.adjQ[off], mu[i], a.adjM[off]);
      }
    }
  }
  float dAacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float dDacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int nq = (d.hi - d.lo + SB - 1) / SB;   // sub-blocks, q = 0 at the chunk's right end
  auto blo_of = [&](int q) { return max(d.lo, d.hi - SB * (q + 1)); };
  auto bhi_of = [&](int q) { return d.hi - SB * q; };
  if (nq > 0) issue(blo_of(nq - 1), bhi_of(nq - 1));
  for (int q = nq - 1; q >= 0; --q) {
    const int blo = blo_of(q), bhi = bhi_of(q), nt = bhi - blo;
    // the state entering the sub-block from the right (first sweep)
    f32x4 hcar;
    {
      const float* src = a.hc + ((long)(d.slot0 + q) * NS + 4 * w) * E + e;
#pragma unroll
      for (int i = 0; i < 4; ++i) hcar[i] = src[(long)i * E];
    }
    // ---------------- A: per (token, channel) inputs ----------------
    float gD[4], u4[4], dt4[4];
    {
      float g4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        g4[j] = has_z ? pdy[j] * silu_fast(pz[j]) : pdy[j];   // rows past the sub-block: 0
        u4[j] = pu[j];
        dt4[j] = pdt[j];
        gD[j] = dsk[j] * g4[j];
        dDacc[j] = fmaf(g4[j], pu[j], dDacc[j]);
        pre_s[r16][4 * c16 + j] = make_float2(pdt[j], pdt[j] * pu[j]);
      }
      *(f32x4*)&g_s[r16][4 * c16] = f32x4{g4[0], g4[1], g4[2], g4[3]};
      if (c16 < 8) bc_s[r16][c16] = f32x4{pbc[0], pbc[1], pbc[2], pbc[3]};
    }
    if (q > 0) issue(blo_of(q - 1), bhi_of(q - 1));
    __syncthreads();
    // ---------------- B1: the sub-block's states, right to left ----------------
    // (the two recurrences at raised wave priority: each is one wave's
    // dependency chain, and the other wave on the SIMD, in phase A or C,
    // fills the gaps it leaves; measured 1.5% faster)
    __builtin_amdgcn_s_setprio(2);
    const float* bsrc = (const float*)&bc_s[0][w] + (lane & 3);   // B_t[4 w + (lane & 3)] at row 0
    f32x4 hs[SB];
    {
      f32x4 h = hcar;
#pragma unroll
      for (int r = SB - 1; r >= 0; --r) {
        const float2 p = pre_s[r][lane];
        f32x4 hd;
#pragma unroll
        for (int i = 0; i < 4; ++i) hd[i] = exp2_fast(p.x * A2[i]) * h[i];
        h = __builtin_amdgcn_mfma_f32_4x4x1f32(bsrc[r * 32], p.y, hd, 0, 0, 0);
        hs[r] = h;
      }
    }
    // ---------------- B2: the adjoint, left to right ----------------
#pragma unroll
    for (int r = 0; r < SB; ++r) {
      const float2 p = pre_s[r][lane];
      const float g = g_s[r][lane];
      const f32x4 Bv = bc_s[r][w], Cv = bc_s[r][4 + w];
      const f32x4 hn = r + 1 < SB ? hs[r + 1] : hcar;   // h_{t+1}
      float v[8], s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float at = exp2_fast(p.x * A2[i]);
        const float lam = fmaf(g, Cv[i], mu[i]);
        mu[i] = at * lam;                        // a_t lambda_t, carried to t+1
        const float qa = mu[i] * hn[i];          // lambda h_{t+1} a_t
        v[i] = g * hs[r][i];                     // dC
        v[4 + i] = lam * p.y;                    // dB
        s1 = fmaf(lam, Bv[i], s1);
        s2 = fmaf(qa, An[i], s2);
        dAacc[i] = fmaf(qa, p.x, dAacc[i]);
      }
      s1_s[w][r][lane] = s1;
      s2_s[w][r][lane] = s2;
      // sums over the 64 channels: lanes 0..31 keep dC, 32..63 dB ...
      float x0 = swap32_sum(v[0], v[4]), x1 = swap32_sum(v[1], v[5]);
      float x2 = swap32_sum(v[2], v[6]), x3 = swap32_sum(v[3], v[7]);
      // ... rows 0/2 keep states 0, 1 and rows 1/3 states 2, 3 ...
      float y0 = swap16_sum(x0, x2), y1 = swap16_sum(x1, x3);
      // ... then each row of 16 lanes is summed
      y0 = add_ror<8>(y0); y0 = add_ror<4>(y0); y0 = add_ror<2>(y0); y0 = add_ror<1>(y0);
      y1 = add_ror<8>(y1); y1 = add_ror<4>(y1); y1 = add_ror<2>(y1); y1 = add_ror<1>(y1);
      // row 0: dC[4w], dC[4w+1]; row 1: dC[4w+2], dC[4w+3]; row 2: dB[4w], dB[4w+1]; row 3: dB[4w+2], dB[4w+3]
      if ((lane & 15) == 0) {
        const int row = lane >> 4;
        const int col = (row < 2 ? 16 : 0) + 4 * w + 2 * (row & 1);
        *(float2*)&dbc_s[r][col] = make_float2(y0, y1);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    // ---------------- C: du, ddt; the sub-block's dB | dC ----------------
    {
      float S1[4] = {0.0f, 0.0f, 0.0f, 0.0f}, S2[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const f32x4 p1 = *(const f32x4*)&s1_s[ww][r16][4 * c16];
        const f32x4 p2 = *(const f32x4*)&s2_s[ww][r16][4 * c16];
#pragma unroll
        for (int j = 0; j < 4; ++j) { S1[j] += p1[j]; S2[j] += p2[j]; }
      }
      float du4[4], ddt4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        du4[j] = fmaf(dt4[j], S1[j], gD[j]);
        ddt4[j] = fmaf(u4[j], S1[j], S2[j]);
      }
      // rows past the sub-block fall outside the windows and are dropped
      st4(rows_of(a.du, blo, lde_b, nt), offE, du4);
      st4(rows_of(a.ddt, blo, lde_b, nt), offE, ddt4);
      if (tid < 128) {
        const int row = tid >> 3, col = 4 * (tid & 7);
        const f32x4 v = *(const f32x4*)&dbc_s[row][col];
        const long pitch = 32 * 4;
        st4(rows_of(a.dbc + (long)cblk * a.T * 32, blo, pitch, nt), (unsigned)(row * pitch + col * 4),
            (const float*)&v);
      }
    }
    // (the next sub-block rewrites s1_s, s2_s and dbc_s only after its A -> B barrier)
  }
  // ---------------- per-sequence sums over time ----------------
#pragma unroll
  for (int i = 0; i < 4; ++i) a.dA[((long)ci * E + e) * NS + 4 * w + i] = dAacc[i] * An[i];
  *(f32x4*)&red_s[r16][4 * c16] = f32x4{dDacc[0], dDacc[1], dDacc[2], dDacc[3]};
  __syncthreads();
  if (tid < 64) {
    float s = 0.0f;
    for (int r = 0; r < SB; ++r) s += red_s[r][tid];
    a.dD[(long)ci * E + e0 + tid] = s;
  }
}

// Adjoint chunk summaries.  For a chunk [lo, hi) with nothing coming in from
// its left, walk it left to right: lambda_t = g_t C_t + m, m <- a_t lambda_t,
// Q <- Q a_t; then M = m (the carry leaving the chunk) and Q = the product of
// its a_t, so that a carry m_in entering the chunk leaves as M + Q m_in.
// Layout as the main sweep: a block owns 64 channels of one chunk, the four
// waves split the 16 states; 16-token sub-blocks go through LDS, the next
// one's loads in flight.
template <typename T>
__global__ __launch_bounds__(256) void scan_bwd_adj_summary_kernel(ScanBwdArgs a) {
  constexpr unsigned SZ = sizeof(T);
  __shared__ __attribute__((aligned(16))) float dt_s[SB][64];
  __shared__ __attribute__((aligned(16))) float g_s[SB][64];
  __shared__ __attribute__((aligned(16))) f32x4 c_s[SB][4];     // C[0..16)
  const int E = a.E;
  const int NB = E / 64;
  const int ci = blockIdx.x / NB, cblk = blockIdx.x % NB;
  if (ci >= *a.n_chunks) return;
  const ChunkDesc d = a.chunks[ci];
  if (d.j == 0) return;   // the rightmost chunk of a sequence: no chunk to its right reads it
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int e0 = cblk * 64, e = e0 + lane;
  const int r16 = tid >> 4, c16 = tid & 15;
  const int ea = e0 + 4 * c16;
  float A2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) A2[i] = -expf(a.A_log[(long)e * NS + 4 * w + i]) * kLog2e;
  const bool has_z = a.z != nullptr;
  const long lddt_b = a.ld_dt * 4, ldbc_b = a.ld_bc * 4;
  const long ldz_b = a.ld_z * (long)SZ, lddy_b = a.ld_dy * (long)SZ;
  const unsigned offDT = (unsigned)(r16 * lddt_b) + (unsigned)ea * 4;
  const unsigned offZ = (unsigned)(r16 * ldz_b) + (unsigned)ea * SZ;
  const unsigned offDY = (unsigned)(r16 * lddy_b) + (unsigned)ea * SZ;
  const unsigned offC = c16 < 4 ? (unsigned)(r16 * ldbc_b) + 16u * c16 : kPast;
  float pdt[4], pz[4], pdy[4], pc[4];
  auto issue = [&](int blo, int bhi) __attribute__((always_inline)) {
    const int rows = bhi - blo;
    load4(pdt, rows_of(a.dt, blo, lddt_b, rows), offDT, (float*)nullptr);
    load4(pdy, rows_of(a.dy, blo, lddy_b, rows), offDY, (T*)nullptr);
    if (has_z) load4(pz, rows_of(a.z, blo, ldz_b, rows), offZ, (T*)nullptr);
    const Rsrc rC = rows_of(a.Cm, blo, ldbc_b, rows);
#pragma unroll
    for (int p = 0; p < 4; ++p) pc[p] = ld1(rC, offC + 4u * p);
  };
  float m[4] = {0.0f, 0.0f, 0.0f, 0.0f}, q[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  const int nsb = (d.hi - d.lo + SB - 1) / SB;   // sub-blocks, left to right
  if (nsb > 0) issue(d.lo, min(d.hi, d.lo + SB));
  for (int k = 0; k < nsb; ++k) {
    const int blo = d.lo + SB * k, bhi = min(d.hi, blo + SB), nt = bhi - blo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dt_s[r16][4 * c16 + j] = pdt[j];      // rows past the sub-block: dt = 0, so a = 1 (identity)
      g_s[r16][4 * c16 + j] = has_z ? pdy[j] * silu_fast(pz[j]) : pdy[j];
    }
    if (c16 < 4) c_s[r16][c16] = f32x4{pc[0], pc[1], pc[2], pc[3]};
    if (k + 1 < nsb) issue(blo + SB, min(d.hi, blo + 2 * SB));
    __syncthreads();
    for (int r = 0; r < nt; ++r) {
      const float dtv = dt_s[r][lane], g = g_s[r][lane];
      const f32x4 Cv = c_s[r][w];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float at = exp2_fast(dtv * A2[i]);
        const float lam = fmaf(g, Cv[i], m[i]);
        m[i] = at * lam;
        q[i] *= at;
      }
    }
    __syncthreads();
  }
  const long base = (long)ci * NS * E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const long off = base + (long)(4 * w + i) * E + e;
    a.adjM[off] = m[i];
    a.adjQ[off] = q[i];
  }
}

// dB, dC [T, 16] = sums over channel blocks of the partials, in order.
__global__ __launch_bounds__(256) void scan_bwd_bc_kernel(int T, int NB, const float* __restrict__ part,
                                                          float* __restrict__ dB, float* __restrict__ dC) {
  const long n = (long)T * 32;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    float s = 0.0f;
    for (int b = 0; b < NB; ++b) s += part[(long)b * n + i];
    const long t = i / 32;
    const int c = (int)(i % 32);
    if (c < 16) dB[t * 16 + c] = s;
    else dC[t * 16 + c - 16] = s;
  }
}

// dA_log [E, 16] and dDskip [E] = sums over chunks of the partials, in order.
__global__ __launch_bounds__(256) void scan_bwd_param_kernel(int E, const int32_t* __restrict__ n_chunks,
                                                             const float* __restrict__ dA,
                                                             const float* __restrict__ dD,
                                                             float* __restrict__ dA_log, float* __restrict__ dDskip) {
  const int nc = *n_chunks;
  const long i = blockIdx.x * 256L + threadIdx.x;
  if (i < (long)E * NS) {
    float s = 0.0f;
    for (int c = 0; c < nc; ++c) s += dA[(long)c * E * NS + i];
    dA_log[i] = s;
  }
  if (dDskip != nullptr && i < E) {
    float s = 0.0f;
    for (int c = 0; c < nc; ++c) s += dD[(long)c * E + i];
    dDskip[i] = s;
  }
}

template <typename T>
hipError_t scan_bwd_adjoint(const ScanBwdArgs& a, int max_chunks, float* dA_log, float* dB, float* dC,
                            float* dDskip, hipStream_t st) {
  const int NB = a.E / 64;
  if (max_chunks * NB > 0 && a.adjM != nullptr)
    hipLaunchKernelGGL((scan_bwd_adj_summary_kernel<T>), dim3(max_chunks * NB), dim3(256), 0, st, a);
  if (max_chunks * NB > 0)
    hipLaunchKernelGGL((scan_bwd_adj_kernel<T>), dim3(max_chunks * NB), dim3(256), 0, st, a);
  const long n = (long)a.T * 32;
  const long want = (n + 255) / 256;
  if (n > 0)
    hipLaunchKernelGGL(scan_bwd_bc_kernel, dim3((unsigned)(want < 4096 ? want : 4096)), dim3(256), 0, st, a.T, NB,
                       (const float*)a.dbc, dB, dC);
  hipLaunchKernelGGL(scan_bwd_param_kernel, dim3((a.E * NS + 255) / 256), dim3(256), 0, st, a.E, a.n_chunks,
                     (const float*)a.dA, (const float*)a.dD, dA_log, dDskip);
  return hipGetLastError();
}
template hipError_t scan_bwd_adjoint<float>(const ScanBwdArgs&, int, float*, float*, float*, float*, hipStream_t);
template hipError_t scan_bwd_adjoint<bf16>(const ScanBwdArgs&, int, float*, float*, float*, float*, hipStream_t);

}  // namespace r2l
