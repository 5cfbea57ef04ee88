// Backward with respect to the weight, binary16, with producer and consumer
// waves.
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
// writes one fp32 partial per plane; the second pass (the finish kernel of
// the matrix-core path) sums the S partials in split order and applies the
// inverse butterfly.  Consecutive (split, tile) pairs run on one XCD, so the
// x rows that the tiles of a split all read come from that XCD's L2.
//
// Roles inside a work-group, one barrier per 32-row step:
//  * NP producer waves load each step's dy and x rows (range-checked 16-byte
//    buffer loads, three steps ahead in a register ring), apply the length-4
//    butterfly in packed binary16 into the scaled planes (X0/4 and X2/4 as
//    the sum and difference of the rounded quarter pair sums (x0 + x2)/4 and
//    (x1 + x3)/4, Xr/2 = (x0 - x2)/2, Xi/2 = (x3 - x1)/2) and write the four
//    planes to LDS in matrix-core fragment order, transposing rows into the
//    operand's K dimension; dbias is summed from exact fp32 sums of dy over
//    the group;
//  * NWD x NWC consumer waves own DB x CB blocks of 16 x 16 outputs and run
//    v_mfma_f32_16x16x32_f16 on fragments read from LDS (K = 32 rows).
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_bws(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

}  // namespace

// LDS per buffer: plane p, operand block b (dy blocks first, then x blocks):
// one 1 KB fragment at (p*NBLK + b)*520 halves; lane (i16, g) of the operand
// reads the 16 bytes at (g*16 + i16)*16 = rows 8g..8g+7 of column i16.
template <int NWD, int NWC, int DB, int CB, int NP, int KSUB>
__global__ __launch_bounds__((NWD * NWC + NP) * 64) void k_bwd_weight_ws(
    const _Float16* __restrict__ x, const _Float16* __restrict__ dy, float* __restrict__ part,
    float* __restrict__ part_b, int N, int C, int D, int d_pad, int c_pad, int rows_per_split,
    int n_dt, int n_ct, int S, int per_xcd) {
  constexpr int NC = NWD * NWC;
  constexpr int BD = NWD * DB * 16, BC = NWC * CB * 16;
  constexpr int DBLK = BD / 16, CBLK = BC / 16, NBLK = DBLK + CBLK;
  // Fragments are 1 KB; consecutive blocks sit 1040 bytes apart, which moves
  // each block by four LDS banks, so one producer instruction writing two
  // blocks and two row groups hits every bank once.
  constexpr int FRAG = 520;                 // halves between consecutive blocks
  constexpr int PSTR = NBLK * FRAG;         // plane stride (halves)
  constexpr int SUB = 4 * PSTR;             // halves per 32-row sub-step
  constexpr int BUF = KSUB * SUB;           // halves per buffer
  constexpr int SROWS = 32 * KSUB;          // rows per step (one barrier each)
  constexpr int QUARTS = SROWS / 4;         // row quartets per step
  constexpr int DUNITS = (BD / 2) * QUARTS; // (column pair, row quartet) units of dy per step
  constexpr int UNITS = (BD / 2 + BC / 2) * QUARTS;
  constexpr int PT = NP * 64;
  constexpr int UPT = (UNITS + PT - 1) / PT;
  constexpr bool EXACT = UNITS % PT == 0;
  constexpr int DUMMY = EXACT ? 0 : PT * 4;  // halves: one 8-byte slot per producer thread
  static_assert(DUNITS % 64 == 0, "dy and x units split at a wave boundary");
  __shared__ __attribute__((aligned(16))) _Float16 lds[2 * BUF + DUMMY];
  __shared__ float bred[QUARTS][BD];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  // work-group -> (split, tile): XCD x runs pairs [x*per_xcd, (x+1)*per_xcd)
  const int wgid = blockIdx.x, xcd = wgid & 7, slot = wgid >> 3;
  const int T = n_dt * n_ct;
  const int L = xcd * per_xcd + slot;
  if (slot >= per_xcd || L >= S * T) return;  // whole work-group
  const int split = L / T, tile = L % T;
  const int dt = tile / n_ct, ct = tile % n_ct;
  const int d0 = dt * BD, c0 = ct * BC;
  const int r_begin = split * rows_per_split;
  const int r_end = min(N, r_begin + rows_per_split);
  const int nsteps = (r_end - r_begin + SROWS - 1) / SROWS;

  if (wave >= NC) {
    // =========================== producer waves ===========================
    const int pw = wave - NC, ptid = tid - NC * 64;
    const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
    // unit u = k*PT + ptid -> operand (dy for u < DUNITS), column pair, row
    // quartet; the operand is the same for a whole wave
    auto unit_is_dy = [&](int k) { return k * PT + pw * 64 < DUNITS; };
    // per-unit constants (the same every step): global byte offset of the
    // unit's first row within a step (or an out-of-range offset), and the
    // LDS offset of its first fragment word (or the dummy slot)
    uint32_t goff[UPT];
    int loff[UPT];
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = k * PT + ptid;
      const bool is_dy = unit_is_dy(k);
      const int v = is_dy ? u : u - DUNITS;
      const int cp = is_dy ? v % (BD / 2) : v % (BC / 2);
      const int quart = is_dy ? v / (BD / 2) : v / (BC / 2);
      const int col = (is_dy ? d0 : c0) + 2 * cp;
      const int width = is_dy ? D : C;
      const bool ok = (EXACT || u < UNITS) && col < width;
      goff[k] = ok ? (uint32_t)((quart * 4 * width + col) * 8) : 0x7FFFFFF0u;
      const int lc = 2 * cp;
      const int blk = (is_dy ? 0 : DBLK) + (lc >> 4);
      const int sub = quart >> 3, gq = (quart & 7) >> 1, hf = quart & 1;
      loff[k] = (EXACT || u < UNITS) ? sub * SUB + blk * FRAG + (gq * 16 + (lc & 15)) * 8 + hf * 4 : -1;
    }
    auto load_step = [&](half8 (&raw)[UPT][4], int st) {
      const int r0 = r_begin + st * SROWS;
      const int rows = r0 < r_end ? min(SROWS, r_end - r0) : 0;
      const int rb = rows > 0 ? r0 : 0;
      const __amdgpu_buffer_rsrc_t rdy = rsrc_bws(dy + (int64_t)rb * D * 4, (uint32_t)rows * D * 8);
      const __amdgpu_buffer_rsrc_t rx = rsrc_bws(x + (int64_t)rb * C * 4, (uint32_t)rows * C * 8);
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const bool is_dy = unit_is_dy(k);
        const uint32_t rstride = (uint32_t)(is_dy ? D : C) * 8;  // bytes per row
#pragma unroll
        for (int e = 0; e < 4; ++e)
          raw[k][e] = __builtin_bit_cast(
              half8, __builtin_amdgcn_raw_buffer_load_b128(is_dy ? rdy : rx, goff[k] + e * rstride, 0, 0));
      }
    };
    float bsum[UPT][2];
#pragma unroll
    for (int k = 0; k < UPT; ++k) bsum[k][0] = bsum[k][1] = 0.f;
    auto store_step = [&](const half8 (&raw)[UPT][4], _Float16* buf) {
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const bool is_dy = unit_is_dy(k);
        // per row e and column (a: halves 0-3, b: 4-7): pair sums and (Xr, Xi)
        // scaled planes (eql_device.h): the pair sums carry 1/4, so that
        // their sum and difference are X0/4 and X2/4, and the differences
        // 1/2; one packed fused multiply-add each, no overflow for finite
        // inputs
        const f16x2 qq = {(_Float16)SCALE02, (_Float16)SCALE02};
        const f16x2 hh = {(_Float16)SCALE1, (_Float16)SCALE1};
        f16x2 sa[4], sb[4], ra[4], rb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const half8 w = raw[k][e];
          const f16x2 a01 = {w[0], w[1]}, a23 = {w[2], w[3]};
          const f16x2 b01 = {w[4], w[5]}, b23 = {w[6], w[7]};
          sa[e] = __builtin_elementwise_fma(a01, qq, a23 * qq);  // (x0 + x2, x1 + x3)/4
          sb[e] = __builtin_elementwise_fma(b01, qq, b23 * qq);
          const f16x2 a0n1 = {w[0], -w[1]}, na2a3 = {-w[2], w[3]};
          const f16x2 b0n1 = {w[4], -w[5]}, nb2b3 = {-w[6], w[7]};
          ra[e] = __builtin_elementwise_fma(a0n1, hh, na2a3 * hh);  // (x0 - x2, x3 - x1)/2
          rb[e] = __builtin_elementwise_fma(b0n1, hh, nb2b3 * hh);
          if (is_dy) {  // dbias: exact fp32 sum of the group values
            bsum[k][0] = __builtin_amdgcn_fdot2(a01, ones, __builtin_amdgcn_fdot2(a23, ones, bsum[k][0], false), false);
            bsum[k][1] = __builtin_amdgcn_fdot2(b01, ones, __builtin_amdgcn_fdot2(b23, ones, bsum[k][1], false), false);
          }
        }
        f16x4 p0[2], p2[2], pr[2], pi[2];               // [column][row]
#pragma unroll
        for (int h = 0; h < 2; ++h) {                   // row pairs (0,1), (2,3)
          const f16x2 pa = {sa[2 * h][0], sa[2 * h + 1][0]}, qa = {sa[2 * h][1], sa[2 * h + 1][1]};
          const f16x2 pb = {sb[2 * h][0], sb[2 * h + 1][0]}, qb = {sb[2 * h][1], sb[2 * h + 1][1]};
          const f16x2 x0a = pa + qa, x2a = pa - qa, x0b = pb + qb, x2b = pb - qb;
          p0[0][2 * h] = x0a[0]; p0[0][2 * h + 1] = x0a[1];
          p2[0][2 * h] = x2a[0]; p2[0][2 * h + 1] = x2a[1];
          p0[1][2 * h] = x0b[0]; p0[1][2 * h + 1] = x0b[1];
          p2[1][2 * h] = x2b[0]; p2[1][2 * h + 1] = x2b[1];
          pr[0][2 * h] = ra[2 * h][0]; pr[0][2 * h + 1] = ra[2 * h + 1][0];
          pi[0][2 * h] = ra[2 * h][1]; pi[0][2 * h + 1] = ra[2 * h + 1][1];
          pr[1][2 * h] = rb[2 * h][0]; pr[1][2 * h + 1] = rb[2 * h + 1][0];
          pi[1][2 * h] = rb[2 * h][1]; pi[1][2 * h + 1] = rb[2 * h + 1][1];
        }
        const bool real = EXACT || loff[k] >= 0;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          // the pair's second column is the next operand column: 8 halves on
          _Float16* dst = buf + loff[k] + cc * 8;
          _Float16* const dmy = lds + 2 * BUF + ptid * 4;  // units past the step (not EXACT only)
          *reinterpret_cast<f16x4*>(real ? dst + 0 * PSTR : dmy) = p0[cc];
          *reinterpret_cast<f16x4*>(real ? dst + 1 * PSTR : dmy) = p2[cc];
          *reinterpret_cast<f16x4*>(real ? dst + 2 * PSTR : dmy) = pr[cc];
          *reinterpret_cast<f16x4*>(real ? dst + 3 * PSTR : dmy) = pi[cc];
        }
      }
    };
    // Ring: step i sits in slot i % 3 from its load until its transform;
    // between barriers i and i+1 the producers transform step i+1 and load
    // step i+4 into the slot it frees (steps past the split load as zeros).
    half8 ra[UPT][4], rb[UPT][4], rc[UPT][4];
    load_step(ra, 0);
    // every work-group's first step is requested before any later one
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0)
    load_step(rb, 1);
    load_step(rc, 2);
    store_step(ra, lds);
    load_step(ra, 3);
    __syncthreads();  // barrier 0: step 0 is in buffer 0
    __builtin_amdgcn_sched_barrier(0);
    int cur = 1;
    int i = 0;
    for (; i + 3 <= nsteps - 1; i += 3) {
      store_step(rb, lds + cur * BUF);
      __builtin_amdgcn_sched_barrier(0);
      load_step(rb, i + 4);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      cur ^= 1;
      store_step(rc, lds + cur * BUF);
      __builtin_amdgcn_sched_barrier(0);
      load_step(rc, i + 5);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      cur ^= 1;
      store_step(ra, lds + cur * BUF);
      __builtin_amdgcn_sched_barrier(0);
      load_step(ra, i + 6);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      cur ^= 1;
    }
    const int rest = nsteps - 1 - i;
    if (rest > 0) {
      store_step(rb, lds + cur * BUF);
      __syncthreads();
      cur ^= 1;
      if (rest > 1) {
        store_step(rc, lds + cur * BUF);
        __syncthreads();
      }
    }
    // bias partial of this split: per (column, row quartet) sums
    if (ct == 0) {
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const int u = k * PT + ptid;
        if (unit_is_dy(k)) {
          const int cp = u % (BD / 2), quart = u / (BD / 2);
          bred[quart][2 * cp] = bsum[k][0];
          bred[quart][2 * cp + 1] = bsum[k][1];
        }
      }
    }
  } else {
    // =========================== consumer waves ===========================
    const int wd = wave / NWC, wc = wave % NWC;
    // acc[..][3] collects Gi^T Xr and accn the Gr^T Xi it loses (Pi is their
    // difference, taken once at the end): no fragment is ever negated
    f32x4 acc[DB][CB][4], accn[DB][CB];
#pragma unroll
    for (int a = 0; a < DB; ++a)
#pragma unroll
      for (int b = 0; b < CB; ++b) {
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[a][b][p] = f32x4{};
        accn[a][b] = f32x4{};
      }
    auto compute_sub = [&](const _Float16* buf) {
      half8 gf[DB][4];
#pragma unroll
      for (int a = 0; a < DB; ++a)
#pragma unroll
        for (int p = 0; p < 4; ++p)
          gf[a][p] = *reinterpret_cast<const half8*>(buf + p * PSTR + (wd * DB + a) * FRAG + lane * 8);
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        const _Float16* xb = buf + (DBLK + wc * CB + b) * FRAG + lane * 8;
        const half8 x0 = *reinterpret_cast<const half8*>(xb + 0 * PSTR);
        const half8 x2 = *reinterpret_cast<const half8*>(xb + 1 * PSTR);
        const half8 xr = *reinterpret_cast<const half8*>(xb + 2 * PSTR);
        const half8 xi = *reinterpret_cast<const half8*>(xb + 3 * PSTR);
#pragma unroll
        for (int a = 0; a < DB; ++a) {
          acc[a][b][0] = mma16(gf[a][0], x0, acc[a][b][0]);
          acc[a][b][2] = mma16(gf[a][2], xr, acc[a][b][2]);
          acc[a][b][1] = mma16(gf[a][1], x2, acc[a][b][1]);
          acc[a][b][3] = mma16(gf[a][3], xr, acc[a][b][3]);
          acc[a][b][2] = mma16(gf[a][3], xi, acc[a][b][2]);
          accn[a][b] = mma16(gf[a][2], xi, accn[a][b]);
        }
      }
    };
    auto compute_step = [&](const _Float16* buf) {
#pragma unroll
      for (int sb = 0; sb < KSUB; ++sb) compute_sub(buf + sb * SUB);
    };
    __syncthreads();  // barrier 0
    int cur = 0;
    for (int st = 0; st < nsteps; ++st) {
      compute_step(lds + cur * BUF);
      cur ^= 1;
      if (st + 1 < nsteps) __syncthreads();  // barrier st+1
    }
    // partial planes: part[split][p][c][d] (d contiguous); lane (i16, g)
    // holds rows d 4g..4g+3 of column c i16 of each 16 x 16 block
    const int64_t plane = (int64_t)c_pad * d_pad;
    float* pout = part + (int64_t)split * 4 * plane;
    const int i16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int a = 0; a < DB; ++a)
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        const int d = d0 + (wd * DB + a) * 16 + 4 * g;
        const int c = c0 + (wc * CB + b) * 16 + i16;
        acc[a][b][3] -= accn[a][b];
#pragma unroll
        for (int p = 0; p < 4; ++p)
          *reinterpret_cast<f32x4*>(pout + p * plane + (int64_t)c * d_pad + d) = acc[a][b][p];
      }
  }

  // ---- bias partial: fixed-order sum over the row quartets of a step ------
  if (ct == 0) {
    __syncthreads();
    for (int j = tid; j < BD; j += (NC + NP) * 64) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < QUARTS; ++q) s += bred[q][j];
      part_b[(int64_t)split * d_pad + d0 + j] = s;
    }
  }
}

// Sum of the S partials, inverse butterfly, dW and dbias.  Work-group =
// 8 waves over one input channel c and 256 consecutive d (64 lanes x 4 d,
// one 16-byte load per plane and split); wave w sums the splits s = w,
// w + 8, ... in increasing order, then wave 0 adds the eight wave sums in
// wave order: a fixed summation tree, so the result is deterministic.
constexpr int FIN_WAVES = 8;
__global__ __launch_bounds__(64 * FIN_WAVES) void k_bwd_weight_finish(
    const float* __restrict__ part, const float* __restrict__ part_b, float* __restrict__ dW,
    float* __restrict__ dbias, int C, int D, int d_pad, int c_pad, int S) {
  __shared__ f32x4 red[FIN_WAVES][5][64];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_dchunk = (D + 255) / 256;
  const int c = blockIdx.x / n_dchunk, d = (blockIdx.x % n_dchunk) * 256 + 4 * lane;
  const bool bias_block = c == 0 && dbias != nullptr;
  const int64_t plane = (int64_t)c_pad * d_pad;
  f32x4 P[5] = {};
  if (d < D) {  // d_pad is a multiple of 16: d .. d + 3 lie inside the padded planes
    const int64_t o = (int64_t)c * d_pad + d;
    // chunks of four splits per wave: all their loads are in flight before
    // the first add, and the adds keep the split order s = w, w + 8, ...
    constexpr int IT = 4;
    for (int s0 = w; s0 < S; s0 += FIN_WAVES * IT) {
      f32x4 v[IT][5];
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int sp = s0 + FIN_WAVES * it;
        if (sp < S) {
          const float* ps = part + (int64_t)sp * 4 * plane + o;
#pragma unroll
          for (int p = 0; p < 4; ++p) v[it][p] = *reinterpret_cast<const f32x4*>(ps + p * plane);
          v[it][4] = bias_block ? *reinterpret_cast<const f32x4*>(part_b + (int64_t)sp * d_pad + d)
                                : f32x4{};
        }
      }
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        if (s0 + FIN_WAVES * it < S) {
#pragma unroll
          for (int p = 0; p < 5; ++p) P[p] += v[it][p];
        }
      }
    }
  }
#pragma unroll
  for (int p = 0; p < 5; ++p) red[w][p][lane] = P[p];
  __syncthreads();
  if (w == 0 && d < D) {
    f32x4 q[5];
#pragma unroll
    for (int p = 0; p < 5; ++p) {
      q[p] = red[0][p][lane];
#pragma unroll
      for (int ww = 1; ww < FIN_WAVES; ++ww) q[p] += red[ww][p][lane];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (d + j < D) {
        *reinterpret_cast<floatx4*>(dW + ((int64_t)(d + j) * C + c) * 4) =
            idft4(q[0][j], q[1][j], q[2][j], q[3][j]);
        if (bias_block) dbias[d + j] = q[4][j];
      }
    }
  }
}

hipError_t launch_bwd_weight_finish(const float* part, const float* part_b, float* dW, float* dbias,
                                    int64_t C, int64_t D, int64_t d_pad, int64_t c_pad, int64_t S,
                                    hipStream_t s) {
  const unsigned fblocks = (unsigned)(C * ((D + 255) / 256));
  hipLaunchKernelGGL(k_bwd_weight_finish, dim3(fblocks), dim3(64 * FIN_WAVES), 0, s, part, part_b,
                     dW, dbias, (int)C, (int)D, (int)d_pad, (int)c_pad, (int)S);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
struct BwsCfg {
  int nwd, nwc, db, cb, np, ksub;
  int bd() const { return nwd * db * 16; }
  int bc() const { return nwc * cb * 16; }
};

static const BwsCfg kBwsCfgs[] = {
    {2, 2, 1, 3, 8, 1},   // 0: 32 x 96 tiles, 4 consumers + 8 producers, 32-row steps
    {1, 2, 1, 3, 7, 1},   // 1: 16 x 96 tiles, 2 consumers + 7 producers
    {2, 2, 1, 3, 4, 1},   // 2: 32 x 96 tiles, 4 consumers + 4 producers
    {2, 2, 2, 3, 8, 1},   // 3: 64 x 96 tiles, 4 consumers of 32 x 48 + 8 producers
    {2, 2, 1, 3, 8, 2},   // 4: as 0 with 64-row steps
    {1, 2, 1, 3, 7, 2},   // 5: as 1 with 64-row steps
};

bool bws_supported(const eqlinear_plan* p) {
  if (p->tune.bws_off == 1 || p->dtype != EQL_F16) return false;
  // whole column pairs (16-byte units), column tiles of 96.  Wider layers
  // re-read dy once per column tile and still beat the symmetric
  // matrix-core kernel (measured on MI355X, binary16: 168 -> 45 us at
  // N = 12608, C = 192, D = 384; 5252 -> 911 us at N = 200704, C = 192,
  // D = 768; 1527 -> 496 us for the 448-channel patch layer of the 3 x 3
  // group convolution at 64 x 56 x 56, C = D = 48)
  return p->C % 2 == 0 && p->D % 2 == 0;
}

static int bws_sel(const eqlinear_plan* p) {
  const int sel = p->tune.bws_cfg;
  return (sel < 0 || sel >= (int)(sizeof(kBwsCfgs) / sizeof(kBwsCfgs[0]))) ? 0 : sel;
}

struct BwsDims {
  BwsCfg cfg;
  int64_t S, R, d_pad, c_pad;
  int n_dt, n_ct, per_xcd;
};

static BwsDims bws_dims(const eqlinear_plan* p, int64_t N) {
  BwsDims m;
  m.cfg = kBwsCfgs[bws_sel(p)];
  m.n_dt = (int)((p->D + m.cfg.bd() - 1) / m.cfg.bd());
  m.n_ct = (int)((p->C + m.cfg.bc() - 1) / m.cfg.bc());
  m.d_pad = (int64_t)m.n_dt * m.cfg.bd();
  m.c_pad = (int64_t)m.n_ct * m.cfg.bc();
  const int T = m.n_dt * m.n_ct;
  // about one work-group per CU (one fits per CU), splits of whole 32-row steps
  int64_t S = p->tune.bws_s > 0 ? p->tune.bws_s : (256 / T > 0 ? 256 / T : 1);
  const int64_t srows = 32 * m.cfg.ksub;
  const int64_t steps = (N + srows - 1) / srows;
  if (S > steps) S = steps;
  if (S < 1) S = 1;
  const int64_t steps_per = (steps + S - 1) / S;
  m.R = steps_per * srows;
  m.S = (N + m.R - 1) / m.R;
  if (m.S < 1) m.S = 1;
  m.per_xcd = (int)((m.S * T + 7) / 8);
  return m;
}

size_t bws_workspace(const eqlinear_plan* p, int64_t N) {
  if (N <= 0) return 0;
  const BwsDims m = bws_dims(p, N);
  return (size_t)m.S * (size_t)(4 * m.c_pad * m.d_pad + m.d_pad) * sizeof(float);
}

template <int NWD, int NWC, int DB, int CB, int NP, int KSUB>
static hipError_t launch_bws_t(const BwsDims& m, const eqlinear_plan* p, const void* x, const void* dy,
                               float* part, float* part_b, int64_t N, hipStream_t s) {
  const unsigned blocks = (unsigned)(8 * m.per_xcd);
  hipLaunchKernelGGL((k_bwd_weight_ws<NWD, NWC, DB, CB, NP, KSUB>), dim3(blocks), dim3((NWD * NWC + NP) * 64), 0,
                     s, (const _Float16*)x, (const _Float16*)dy, part, part_b, (int)N, (int)p->C, (int)p->D,
                     (int)m.d_pad, (int)m.c_pad, (int)m.R, m.n_dt, m.n_ct, (int)m.S, m.per_xcd);
  return hipGetLastError();
}

hipError_t launch_bws(const eqlinear_plan* p, const void* x, const void* dy, float* dW, float* dbias,
                      int64_t N, void* ws, hipStream_t s) {
  const BwsDims m = bws_dims(p, N);
  float* part = (float*)ws;
  float* part_b = part + m.S * 4 * m.c_pad * m.d_pad;
  hipError_t e = hipErrorNotSupported;
  switch (bws_sel(p)) {
    case 1: e = launch_bws_t<1, 2, 1, 3, 7, 1>(m, p, x, dy, part, part_b, N, s); break;
    case 2: e = launch_bws_t<2, 2, 1, 3, 4, 1>(m, p, x, dy, part, part_b, N, s); break;
    case 3: e = launch_bws_t<2, 2, 2, 3, 8, 1>(m, p, x, dy, part, part_b, N, s); break;
    case 4: e = launch_bws_t<2, 2, 1, 3, 8, 2>(m, p, x, dy, part, part_b, N, s); break;
    case 5: e = launch_bws_t<1, 2, 1, 3, 7, 2>(m, p, x, dy, part, part_b, N, s); break;
    default: e = launch_bws_t<2, 2, 1, 3, 8, 1>(m, p, x, dy, part, part_b, N, s); break;
  }
  if (e != hipSuccess) return e;
  return launch_bwd_weight_finish(part, part_b, dW, dbias, p->C, p->D, m.d_pad, m.c_pad, m.S, s);
}

}  // namespace eql
