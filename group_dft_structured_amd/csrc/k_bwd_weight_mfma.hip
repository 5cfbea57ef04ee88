// Backward with respect to the weight, binary16, on the matrix cores.
//
// In the group Fourier domain (Flash EQ-Linear, "Specializzazione per il
// Gruppo di Rotazione p4": the same length-4 transforms as the forward) the
// weight gradient of every frequency is a reduction over rows,
//     P0 = sum_n G0^T X0          P2 = sum_n G2^T X2
//     Pr = sum_n (Gr^T Xr + Gi^T Xi)    Pi = sum_n (Gi^T Xr - Gr^T Xi)
// with G = DFT_4(dy) and X = DFT_4(x); dW = IDFT_4(P) and dbias = sum_n G0.
//
// Work decomposition: the output (D x C, four planes) is cut into tiles of
// BD x BC channels and the rows into S splits; work-group (split, tile)
// reduces its rows for its tile with fp32 matrix-core accumulators and
// writes one fp32 partial per plane.  A second pass sums the S partials in
// split order (deterministic, no atomics) and applies the inverse butterfly.
// Work-groups of the same split are placed on the same XCD, so the dy and x
// rows that several tiles read come from that XCD's L2.
//
// Data path per 32-row step: dy and x rows arrive through range-checked
// buffer loads (rows past the split read as zeros), each thread owning two
// adjacent columns and four rows; the butterfly gives X0, X2 as exact fp32
// sums (plane 0 also feeds the bias sum) and Xr, Xi by correctly rounded
// binary16 subtraction, and the four planes are written to LDS, double
// buffered, in matrix-core fragment order (the transpose from row-major
// memory to the K-major operand happens in this write).  Loads run two
// steps ahead in a register ring.
#include "eql_device.h"
#include "eql_internal.h"

namespace eql {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_bw(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

}  // namespace

// Fragment (operand block b, plane p): 1 KB; lane (i16, g) of the operand reads
// 16 bytes at (g*16 + i16)*16 = rows 8g..8g+7 of column i16.  Blocks 0..DBLK-1
// hold dy columns, DBLK..DBLK+CBLK-1 hold x columns.
template <int DB, int CB, int NWD, int NWC>
__global__ __launch_bounds__(NWD * NWC * 64) void k_bwd_weight_mfma(
    const _Float16* __restrict__ x, const _Float16* __restrict__ dy, float* __restrict__ part,
    float* __restrict__ part_b, int N, int C, int D, int d_pad, int c_pad, int rows_per_split,
    int n_dt, int n_ct, int S) {
  constexpr int NW = NWD * NWC, NT = NW * 64;
  constexpr int BD = NWD * DB * 16, BC = NWC * CB * 16;
  constexpr int DBLK = BD / 16, CBLK = BC / 16, NBLK = DBLK + CBLK;
  constexpr int FRAG = 512;                        // halves
  constexpr int BUF = 4 * NBLK * FRAG;             // halves per buffer (4 planes)
  constexpr int DUNITS = (BD / 2) * 8;             // (column pair, row quartet) of dy per step
  constexpr int UNITS = (BD / 2 + BC / 2) * 8;
  constexpr int UPT = (UNITS + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) _Float16 lds[2 * BUF];
  __shared__ float bred[8][BD];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar registers)
  const int i16 = lane & 15, g = lane >> 4;
  const int T = n_dt * n_ct;
  const int wgid = blockIdx.x, xcd = wgid & 7, slot = wgid >> 3;
  const int split = (slot / T) * 8 + xcd;
  const int tile = slot % T;
  if (split >= S) return;  // whole work-group: no barrier is skipped
  const int dt = tile / n_ct, ct = tile % n_ct;
  const int d0 = dt * BD, c0 = ct * BC;
  const int r_begin = split * rows_per_split;
  const int r_end = min(N, r_begin + rows_per_split);
  const int nsteps = (r_end - r_begin + 31) / 32;

  const int wd = wave / NWC, wc = wave % NWC;

  // ---- unit loader: unit u -> (operand, column pair, row quartet) --------
  // rows past r_end come back as zeros through the descriptor's range
  auto load_step = [&](half8 (&raw)[UPT][4], int step) {
    const int r0 = r_begin + step * 32;
    const int rows = r0 < r_end ? min(32, r_end - r0) : 0;
    const __amdgpu_buffer_rsrc_t rdy = rsrc_bw(dy + (int64_t)r0 * D * 4, (uint32_t)rows * D * 8);
    const __amdgpu_buffer_rsrc_t rx = rsrc_bw(x + (int64_t)r0 * C * 4, (uint32_t)rows * C * 8);
    static_assert(DUNITS % 64 == 0, "dy and x units split at a wave boundary");
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = k * NT + tid;
      // dy or x is decided per wave (DUNITS is a multiple of 64), so the
      // buffer descriptor is a scalar select, not a per-lane one
      const bool is_dy = __builtin_amdgcn_readfirstlane(k * NT + wave * 64) < DUNITS;
      const int v = is_dy ? u : u - DUNITS;
      const int np = is_dy ? BD / 2 : BC / 2;  // column pairs
      const int cp = v % np, quart = v / np;
      const int col = (is_dy ? d0 : c0) + 2 * cp;
      const int width = is_dy ? D : C;
      const bool ok = (UNITS % NT == 0 || u < UNITS) && col < width;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t off = ok ? (uint32_t)(((quart * 4 + e) * width + col) * 8) : 0x7FFFFFF0u;
        raw[k][e] = __builtin_bit_cast(
            half8, __builtin_amdgcn_raw_buffer_load_b128(is_dy ? rdy : rx, off, 0, 0));
      }
    }
  };
  const f16x2 ones2 = {(_Float16)1.f, (_Float16)1.f};
  const f16x2 pm2 = {(_Float16)1.f, (_Float16)-1.f};
  float bsum[UPT][2];
#pragma unroll
  for (int k = 0; k < UPT; ++k) bsum[k][0] = bsum[k][1] = 0.f;
  // butterfly of a loaded step into LDS buffer `buf` (fragment order)
  auto store_step = [&](const half8 (&raw)[UPT][4], _Float16* buf) {
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = k * NT + tid;
      if (UNITS % NT != 0 && u >= UNITS) break;
      const bool is_dy = __builtin_amdgcn_readfirstlane(k * NT + wave * 64) < DUNITS;
      const int v = is_dy ? u : u - DUNITS;
      const int np = is_dy ? BD / 2 : BC / 2;
      const int cp = v % np, quart = v / np;
      const int lc = 2 * cp;                               // local column
      const int blk = (is_dy ? 0 : DBLK) + (lc >> 4);
      const int gq = quart >> 1, half = quart & 1;         // lane group, which 4 of its 8 rows
      // X0, X2: v_dot2_f32_f16 with +-1 (exact fp32 sums, one rounding);
      // Xr, -Xi: packed binary16 subtraction (correctly rounded)
      f16x4 p0[2], p2[2], pr[2], pi[2];                    // [column][row]
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const half8 w = raw[k][e];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const f16x2 a01 = {w[4 * cc + 0], w[4 * cc + 1]}, a23 = {w[4 * cc + 2], w[4 * cc + 3]};
          const float f0 = __builtin_amdgcn_fdot2(a01, ones2, __builtin_amdgcn_fdot2(a23, ones2, 0.f, false), false);
          const float f2 = __builtin_amdgcn_fdot2(a01, pm2, __builtin_amdgcn_fdot2(a23, pm2, 0.f, false), false);
          const f16x2 dd = a01 - a23;  // (Xr, -Xi)
          if (is_dy) bsum[k][cc] += f0;
          p0[cc][e] = (_Float16)f0;
          p2[cc][e] = (_Float16)f2;
          pr[cc][e] = dd[0];
          pi[cc][e] = -dd[1];
        }
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int i = (lc + cc) & 15;
        _Float16* dst = buf + blk * FRAG + (gq * 16 + i) * 8 + half * 4;
        *reinterpret_cast<f16x4*>(dst + 0 * NBLK * FRAG) = p0[cc];
        *reinterpret_cast<f16x4*>(dst + 1 * NBLK * FRAG) = p2[cc];
        *reinterpret_cast<f16x4*>(dst + 2 * NBLK * FRAG) = pr[cc];
        *reinterpret_cast<f16x4*>(dst + 3 * NBLK * FRAG) = pi[cc];
      }
    }
  };

  f32x4 acc[DB][CB][4];
#pragma unroll
  for (int a = 0; a < DB; ++a)
#pragma unroll
    for (int b = 0; b < CB; ++b)
#pragma unroll
      for (int p = 0; p < 4; ++p) acc[a][b][p] = f32x4{};

  auto compute_step = [&](const _Float16* buf) {
    half8 gf[DB][4];
#pragma unroll
    for (int a = 0; a < DB; ++a)
#pragma unroll
      for (int p = 0; p < 4; ++p)
        gf[a][p] = *reinterpret_cast<const half8*>(buf + p * NBLK * FRAG + (wd * DB + a) * FRAG + lane * 8);
#pragma unroll
    for (int b = 0; b < CB; ++b) {
      const _Float16* xb = buf + (DBLK + wc * CB + b) * FRAG + lane * 8;
      const half8 x0 = *reinterpret_cast<const half8*>(xb + 0 * NBLK * FRAG);
      const half8 x2 = *reinterpret_cast<const half8*>(xb + 1 * NBLK * FRAG);
      const half8 xr = *reinterpret_cast<const half8*>(xb + 2 * NBLK * FRAG);
      const half8 xi = *reinterpret_cast<const half8*>(xb + 3 * NBLK * FRAG);
      const half8 xq = -xi;
#pragma unroll
      for (int a = 0; a < DB; ++a) {
        acc[a][b][0] = mma16(gf[a][0], x0, acc[a][b][0]);
        acc[a][b][2] = mma16(gf[a][2], xr, acc[a][b][2]);
        acc[a][b][1] = mma16(gf[a][1], x2, acc[a][b][1]);
        acc[a][b][3] = mma16(gf[a][3], xr, acc[a][b][3]);
        acc[a][b][2] = mma16(gf[a][3], xi, acc[a][b][2]);
        acc[a][b][3] = mma16(gf[a][2], xq, acc[a][b][3]);
      }
    }
  };

  // ---- software pipeline over 32-row steps (loads two steps ahead) --------
  half8 ra[UPT][4], rb[UPT][4];
  load_step(ra, 0);
  load_step(rb, 1);
  store_step(ra, lds);
  __syncthreads();
  int cur = 0;
  for (int st = 0; st < nsteps;) {
    load_step(ra, st + 2);
    compute_step(lds + cur * BUF);
    store_step(rb, lds + (cur ^ 1) * BUF);
    __syncthreads();
    cur ^= 1;
    if (++st >= nsteps) break;
    load_step(rb, st + 2);
    compute_step(lds + cur * BUF);
    store_step(ra, lds + (cur ^ 1) * BUF);
    __syncthreads();
    cur ^= 1;
    ++st;
  }

  // ---- partial planes: part[split][p][c][d] (d contiguous) ----------------
  const int64_t plane = (int64_t)c_pad * d_pad;
  float* pout = part + (int64_t)split * 4 * plane;
#pragma unroll
  for (int a = 0; a < DB; ++a)
#pragma unroll
    for (int b = 0; b < CB; ++b) {
      const int d = d0 + (wd * DB + a) * 16 + 4 * g;  // rows 4g..4g+3 of the MFMA tile
      const int c = c0 + (wc * CB + b) * 16 + i16;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        *reinterpret_cast<f32x4*>(pout + p * plane + (int64_t)c * d_pad + d) = acc[a][b][p];
    }

  // ---- bias partial: fixed-order sum over the row quartets ----------------
  if (ct == 0) {
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = k * NT + tid;
      if (u < DUNITS) {
        const int cp = u % (BD / 2), quart = u / (BD / 2);
        bred[quart][2 * cp] = bsum[k][0];
        bred[quart][2 * cp + 1] = bsum[k][1];
      }
    }
    __syncthreads();
    for (int j = tid; j < BD; j += NT) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) s += bred[q][j];
      part_b[(int64_t)split * d_pad + d0 + j] = s;
    }
  }
}

// Sum of the S partials, inverse butterfly, dW and dbias.  Work-group =
// 64 consecutive d of one c (lanes) x 4 waves; wave w sums the splits
// s = w, w+4, ... in increasing order, then wave 0 adds the four wave sums in
// wave order: a fixed summation tree, so the result is deterministic.
__global__ __launch_bounds__(256) void k_bwd_weight_finish(const float* __restrict__ part,
                                                           const float* __restrict__ part_b,
                                                           float* __restrict__ dW,
                                                           float* __restrict__ dbias, int C, int D,
                                                           int d_pad, int c_pad, int S) {
  __shared__ float red[4][5][64];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_dchunk = (D + 63) / 64;
  const int c = blockIdx.x / n_dchunk, d = (blockIdx.x % n_dchunk) * 64 + lane;
  const bool bias_block = c == 0 && dbias != nullptr;
  const int64_t plane = (int64_t)c_pad * d_pad;
  float P[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
  if (d < D) {
    const int64_t o = (int64_t)c * d_pad + d;
    // chunks of eight splits per wave: all their loads are in flight before
    // the first add, and the adds keep the split order s = w, w + 4, ...
    constexpr int IT = 8;
    for (int s0 = w; s0 < S; s0 += 4 * IT) {
      float v[IT][5];
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        const int s = s0 + 4 * i;
        if (s < S) {
          const float* ps = part + (int64_t)s * 4 * plane + o;
          v[i][0] = ps[0];
          v[i][1] = ps[plane];
          v[i][2] = ps[2 * plane];
          v[i][3] = ps[3 * plane];
          v[i][4] = bias_block ? part_b[(int64_t)s * d_pad + d] : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        if (s0 + 4 * i < S) {
#pragma unroll
          for (int p = 0; p < 4; ++p) P[p] += v[i][p];
          if (bias_block) P[4] += v[i][4];
        }
      }
    }
  }
#pragma unroll
  for (int p = 0; p < 5; ++p) red[w][p][lane] = P[p];
  __syncthreads();
  if (w == 0 && d < D) {
    float q[5];
#pragma unroll
    for (int p = 0; p < 5; ++p) q[p] = ((red[0][p][lane] + red[1][p][lane]) + red[2][p][lane]) + red[3][p][lane];
    *reinterpret_cast<floatx4*>(dW + ((int64_t)d * C + c) * 4) = idft4(q[0], q[1], q[2], q[3]);
    if (bias_block) dbias[d] = q[4];
  }
}

// ---------------------------------------------------------------------------
static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

struct BwmCfg {
  int db, cb, nwd, nwc;
  int bd() const { return nwd * db * 16; }
  int bc() const { return nwc * cb * 16; }
};

static BwmCfg bwm_cfg(int64_t C) {
  const int sel = env_int("EQL_BWM_CFG", C <= 96 ? 0 : 1);
  switch (sel) {
    case 1: return {1, 3, 4, 1};   // 64 x 48
    case 2: return {1, 3, 2, 2};   // 32 x 96
    case 3: return {1, 3, 8, 1};   // 128 x 48
    case 4: return {1, 1, 1, 6};   // 16 x 96
    case 5: return {1, 1, 2, 6};   // 32 x 96
    case 6: return {1, 2, 1, 3};   // 16 x 96, 3 waves
    default: return {1, 3, 4, 2};  // 64 x 96
  }
}

struct BwmDims {
  BwmCfg cfg;
  int64_t S, R, d_pad, c_pad;
  int n_dt, n_ct;
};

static BwmDims bwm_dims(const eqlinear_plan* p, int64_t N) {
  BwmDims m;
  m.cfg = bwm_cfg(p->C);
  m.n_dt = (int)((p->D + m.cfg.bd() - 1) / m.cfg.bd());
  m.n_ct = (int)((p->C + m.cfg.bc() - 1) / m.cfg.bc());
  m.d_pad = (int64_t)m.n_dt * m.cfg.bd();
  m.c_pad = (int64_t)m.n_ct * m.cfg.bc();
  const int T = m.n_dt * m.n_ct;
  // about one work-group per CU, splits of whole 32-row steps
  int64_t S = env_int("EQL_BWM_S", (int)((256 + T - 1) / T));
  const int64_t steps = (N + 31) / 32;
  if (S > steps) S = steps;
  if (S < 1) S = 1;
  const int64_t steps_per = (steps + S - 1) / S;
  m.R = steps_per * 32;
  m.S = (N + m.R - 1) / m.R;
  if (m.S < 1) m.S = 1;
  return m;
}

size_t bwd_weight_mfma_workspace(const eqlinear_plan* p, int64_t N) {
  if (N <= 0) return 0;
  const BwmDims m = bwm_dims(p, N);
  return (size_t)m.S * (size_t)(4 * m.c_pad * m.d_pad + m.d_pad) * sizeof(float);
}

template <int DB, int CB, int NWD, int NWC>
static hipError_t launch_bwm_t(const BwmDims& m, const eqlinear_plan* p, const void* x,
                               const void* dy, float* part, float* part_b, int64_t N,
                               hipStream_t s) {
  const int T = m.n_dt * m.n_ct;
  const unsigned blocks = (unsigned)(8 * T * ((m.S + 7) / 8));
  hipLaunchKernelGGL((k_bwd_weight_mfma<DB, CB, NWD, NWC>), dim3(blocks), dim3(NWD * NWC * 64), 0, s,
                     (const _Float16*)x, (const _Float16*)dy, part, part_b, (int)N, (int)p->C,
                     (int)p->D, (int)m.d_pad, (int)m.c_pad, (int)m.R, m.n_dt, m.n_ct, (int)m.S);
  return hipGetLastError();
}

hipError_t launch_bwd_weight_mfma(const eqlinear_plan* p, const void* x, const void* dy, float* dW,
                                  float* dbias, int64_t N, void* ws, hipStream_t s) {
  const BwmDims m = bwm_dims(p, N);
  float* part = (float*)ws;
  float* part_b = part + m.S * 4 * m.c_pad * m.d_pad;
  hipError_t e = hipErrorNotSupported;
  const BwmCfg c = m.cfg;
  if (c.db == 1 && c.cb == 3 && c.nwd == 4 && c.nwc == 2)
    e = launch_bwm_t<1, 3, 4, 2>(m, p, x, dy, part, part_b, N, s);
  else if (c.db == 1 && c.cb == 3 && c.nwd == 4 && c.nwc == 1)
    e = launch_bwm_t<1, 3, 4, 1>(m, p, x, dy, part, part_b, N, s);
  else if (c.db == 1 && c.cb == 3 && c.nwd == 2 && c.nwc == 2)
    e = launch_bwm_t<1, 3, 2, 2>(m, p, x, dy, part, part_b, N, s);
  else if (c.db == 1 && c.cb == 3 && c.nwd == 8 && c.nwc == 1)
    e = launch_bwm_t<1, 3, 8, 1>(m, p, x, dy, part, part_b, N, s);
  else if (c.db == 1 && c.cb == 1 && c.nwd == 1 && c.nwc == 6)
    e = launch_bwm_t<1, 1, 1, 6>(m, p, x, dy, part, part_b, N, s);
  else if (c.db == 1 && c.cb == 1 && c.nwd == 2 && c.nwc == 6)
    e = launch_bwm_t<1, 1, 2, 6>(m, p, x, dy, part, part_b, N, s);
  else if (c.db == 1 && c.cb == 2 && c.nwd == 1 && c.nwc == 3)
    e = launch_bwm_t<1, 2, 1, 3>(m, p, x, dy, part, part_b, N, s);
  if (e != hipSuccess) return e;
  return launch_bwd_weight_finish(part, part_b, dW, dbias, p->C, p->D, m.d_pad, m.c_pad, m.S, s);
}

hipError_t launch_bwd_weight_finish(const float* part, const float* part_b, float* dW, float* dbias,
                                    int64_t C, int64_t D, int64_t d_pad, int64_t c_pad, int64_t S,
                                    hipStream_t s) {
  const unsigned fblocks = (unsigned)(C * ((D + 63) / 64));
  hipLaunchKernelGGL(k_bwd_weight_finish, dim3(fblocks), dim3(256), 0, s, part, part_b, dW, dbias,
                     (int)C, (int)D, (int)d_pad, (int)c_pad, (int)S);
  return hipGetLastError();
}

}  // namespace eql
