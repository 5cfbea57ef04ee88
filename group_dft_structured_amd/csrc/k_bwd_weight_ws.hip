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
// writes one fp32 partial per plane; the finish kernel sums the S partials in
// split order and applies the inverse butterfly.  Consecutive (split, tile)
// pairs run on one XCD, so the x rows that the tiles of a split all read come
// from that XCD's L2.
//
// Roles inside a work-group, one barrier per 32-row step:
//  * NP producer waves load each step's dy and x rows (range-checked 16-byte
//    buffer loads, one step ahead of the transform), apply the length-4
//    butterfly on the matrix cores (below) into the scaled planes X0/4, X2/4,
//    Xr/2, Xi/2 (eql_device.h) and write them to LDS in matrix-core fragment
//    order with the rows along the fragments' k; dbias is summed in fp32 from
//    the X0 plane before its rounding;
//  * NWD x NWC consumer waves own DB x CB blocks of 16 x 16 outputs and run
//    v_mfma_f32_16x16x32_f16 on fragments read from LDS (k = 32 rows).
#include <type_traits>

#include "eql_device.h"
#include "eql_internal.h"

namespace eql {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_bws(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

}  // namespace

// Producer unit: one 16-byte load per lane covering four rows x 32 channels,
// lane (j, g) reading row g, channels 2j and 2j + 1 (so four consecutive
// lanes read 64 contiguous bytes; a layout with consecutive lanes on
// different rows costs the address unit four times as many cycles).  These
// loads are the B operand of v_mfma_f32_16x16x32_f16 (column j, k = 8g .. 8g+7
// = two channels x four group values of row g); the A operand holds the
// butterfly, A[(p, r)][(g, e', s)] = F[p][s] when g = r and e' = e, for the
// channel e of the pair (two instructions, e = 0, 1), with F the scaled rows
// (1, 1, 1, 1)/4, (1, -1, 1, -1)/4, (1, 0, -1, 0)/2, (0, -1, 0, 1)/2 giving
// X0/4, X2/4, Xr/2, Xi/2.  The result in lane (j, p) is plane p of channel
// 2j + e for the four rows: four consecutive reduction indices of one operand
// column, the layout of the matrix-core operand whose k runs over rows.  Two
// such blocks fill one 16-byte fragment slot (eight rows), written with one
// LDS store.  The products are exact in fp32 and each plane value is rounded
// once to binary16.
template <int NWD, int NWC, int DB, int CB, int NP>
__global__ __launch_bounds__((NWD * NWC + NP) * 64) void k_bwd_weight_ws(
    const _Float16* __restrict__ x, const _Float16* __restrict__ dy, float* __restrict__ part,
    float* __restrict__ part_b, int N, int C, int D, int d_pad, int c_pad, int rows_per_split,
    int n_dt, int n_ct, int S, int per_xcd) {
  constexpr int NC = NWD * NWC;
  constexpr int BD = NWD * DB * 16, BC = NWC * CB * 16;
  constexpr int DBLK = BD / 16, CBLK = BC / 16, NBLK = DBLK + CBLK;
  // 16-column fragments (1 KB) 1040 bytes apart: the 16 lanes of one store
  // (channels 2j + e, j = 0..15, of two blocks) then cover the 64 banks once
  constexpr int FRAG = 520;
  constexpr int PSTR = NBLK * FRAG;         // plane stride (halves)
  constexpr int BUF = 4 * PSTR;             // halves per 32-row step
  static_assert(BD % 32 == 0 && BC % 32 == 0, "32-channel producer units");
  constexpr int DCH = BD / 32, XCH = BC / 32;  // 32-channel units of dy and x per step
  // HALVES producer waves share one 32-channel unit, each taking 8 / HALVES
  // of the four-row blocks of a step
  constexpr int HALVES = NP / (DCH + XCH);
  static_assert(HALVES * (DCH + XCH) == NP && (HALVES == 1 || HALVES == 2), "producer waves per unit");
  constexpr int NBK = 8 / HALVES;  // four-row blocks per producer wave and step
  __shared__ __attribute__((aligned(16))) _Float16 lds[2 * BUF];
  __shared__ float bred[HALVES][BD];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wgid = blockIdx.x, xcd = wgid & 7, slot = wgid >> 3;
  const int T = n_dt * n_ct;
  const int L = xcd * per_xcd + slot;
  if (slot >= per_xcd || L >= S * T) return;  // whole work-group
  const int split = L / T, tile = L % T;
  const int dt = tile / n_ct, ct = tile % n_ct;
  const int d0 = dt * BD, c0 = ct * BC;
  const int r_begin = split * rows_per_split;
  const int r_end = min(N, r_begin + rows_per_split);
  const int nsteps = (r_end - r_begin + 31) / 32;
  const int j = lane & 15, g = lane >> 4;

  if (wave >= NC) {
    // =========================== producer waves ===========================
    const int pw = wave - NC;
    auto produce = [&](auto dy_c) {
      constexpr bool IS_DY = decltype(dy_c)::value;
      const int width = IS_DY ? D : C;
      const int pu = pw / HALVES, hp = pw % HALVES;  // unit and part of it
      const int o = IS_DY ? pu : pu - DCH;           // unit within the operand's tile columns
      // butterfly operand (A) of lane (i16 = j, g) for channel e = 0, 1 of each pair
      half8 bf[2];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int pl = j >> 2, rr = j & 3, sv = t & 3;
          float v = 0.f;
          if (g == rr && (t >> 2) == e) {
            if (pl == 0) v = 0.25f;
            else if (pl == 1) v = (sv & 1) ? -0.25f : 0.25f;
            else if (pl == 2) v = sv == 0 ? 0.5f : sv == 2 ? -0.5f : 0.f;
            else v = sv == 3 ? 0.5f : sv == 1 ? -0.5f : 0.f;
          }
          bf[e][t] = (_Float16)v;
        }
      // the lane's load: row g of each four-row block, channels 2j, 2j + 1 of
      // the unit (an out-of-range offset past the channels)
      const int col = (IS_DY ? d0 : c0) + 32 * o + 2 * j;
      const uint32_t blk_off = 4u * (uint32_t)width * 8u;  // next four-row block
      const uint32_t goff =
          col < width ? (uint32_t)(g * width + col) * 8u + (uint32_t)(hp * NBK) * blk_off : 0x7FFFFFF0u;
      // LDS slot of lane (j, p = g), channel 2j + e, slot 0 (slot q adds q * 16 * 8)
      int lslot[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int cc = 32 * o + 2 * j + e;
        const int blk = (IS_DY ? 0 : DBLK) + (cc >> 4);
        lslot[e] = g * PSTR + blk * FRAG + (hp * (NBK / 2) * 16 + (cc & 15)) * 8;
      }
      const _Float16* const src = IS_DY ? dy : x;
      auto load_step = [&](half8 (&raw)[NBK], int st) {
        const int r0 = r_begin + st * 32;
        const int rows = r0 < r_end ? min(32, r_end - r0) : 0;
        const int64_t rb0 = rows > 0 ? r0 : 0;
        const __amdgpu_buffer_rsrc_t rs =
            rsrc_bws(src + rb0 * width * 4, (uint32_t)rows * (uint32_t)width * 8u);
#pragma unroll
        for (int bk = 0; bk < NBK; ++bk)
          raw[bk] = __builtin_bit_cast(
              half8, __builtin_amdgcn_raw_buffer_load_b128(rs, goff + (uint32_t)bk * blk_off, 0, 0));
      };
      float bsum[2] = {0.f, 0.f};
      auto store_step = [&](const half8 (&raw)[NBK], _Float16* buf) {
#pragma unroll
        for (int q = 0; q < NBK / 2; ++q) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const f32x4 t0 = mma16(bf[e], raw[2 * q], f32x4{});
            const f32x4 t1 = mma16(bf[e], raw[2 * q + 1], f32x4{});
            if constexpr (IS_DY)  // plane 0 (lanes g = 0): G0/4 of the eight rows, fp32
              bsum[e] += ((t0[0] + t0[1]) + (t0[2] + t0[3])) + ((t1[0] + t1[1]) + (t1[2] + t1[3]));
            half8 v;
            v[0] = (_Float16)t0[0]; v[1] = (_Float16)t0[1]; v[2] = (_Float16)t0[2]; v[3] = (_Float16)t0[3];
            v[4] = (_Float16)t1[0]; v[5] = (_Float16)t1[1]; v[6] = (_Float16)t1[2]; v[7] = (_Float16)t1[3];
            *reinterpret_cast<half8*>(buf + lslot[e] + q * 128) = v;
          }
        }
      };
      // Two steps in registers.  Between barriers i and i+1 the producers
      // transform step i+1 (loaded in the previous interval) into buffer
      // (i+1) % 2, then request step i+2 into the slot step i left, so each
      // load has one interval to arrive.  Measured at 12608 x 96 x 384
      // (partials kernel, back-to-back launches): requests issued before the
      // transform instead of after it held the transform back (+0.9 us), and
      // prefetching two or three steps ahead was slower (+0.3 and +1.0 us;
      // more requests in flight per CU, with the transform waiting behind
      // them).  No scheduling fence separates the transform and
      // the requests (one there cost half of the load-order gain).  Steps
      // past the split load as zeros.
      half8 ra[NBK], rb[NBK];
      load_step(ra, 0);
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0)
      load_step(rb, 1);
      store_step(ra, lds);
      __syncthreads();  // barrier 0: step 0 is in buffer 0
      __builtin_amdgcn_sched_barrier(0);
      int i = 0;
      for (; i + 2 <= nsteps - 1; i += 2) {
        store_step(rb, lds + BUF);
        load_step(ra, i + 2);
        __syncthreads();  // barrier i+1
        __builtin_amdgcn_sched_barrier(0);
        store_step(ra, lds);
        load_step(rb, i + 3);
        __syncthreads();  // barrier i+2
        __builtin_amdgcn_sched_barrier(0);
      }
      if (nsteps - 1 - i > 0) {  // one step left, in rb, for buffer 1
        store_step(rb, lds + BUF);
        __syncthreads();
      }
      if constexpr (IS_DY) {
        // bias partial of this split: lane (j, 0) holds channels 2j, 2j + 1
        // for the wave's rows
        if (ct == 0 && g == 0) {
          const int cc = 32 * o + 2 * j;
          bred[hp][cc] = bsum[0];
          bred[hp][cc + 1] = bsum[1];
        }
      }
    };
    if (pw / HALVES < DCH) produce(std::true_type{});
    else produce(std::false_type{});
  } else {
    // =========================== consumer waves ===========================
    const int wd = wave / NWC, wc = wave % NWC;
    f32x4 acc[DB][CB][4], accn[DB][CB];
#pragma unroll
    for (int a = 0; a < DB; ++a)
#pragma unroll
      for (int b = 0; b < CB; ++b) {
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[a][b][p] = f32x4{};
        accn[a][b] = f32x4{};
      }
    half8 ga[DB][4], xb[CB][4];
    auto read_step = [&](half8 (&ga)[DB][4], half8 (&xb)[CB][4], const _Float16* buf) {
#pragma unroll
      for (int a = 0; a < DB; ++a)
#pragma unroll
        for (int p = 0; p < 4; ++p)
          ga[a][p] = *reinterpret_cast<const half8*>(buf + p * PSTR + (wd * DB + a) * FRAG + lane * 8);
#pragma unroll
      for (int b = 0; b < CB; ++b)
#pragma unroll
        for (int p = 0; p < 4; ++p)
          xb[b][p] = *reinterpret_cast<const half8*>(buf + p * PSTR + (DBLK + wc * CB + b) * FRAG + lane * 8);
    };
    auto mma_step = [&](const half8 (&ga)[DB][4], const half8 (&xb)[CB][4]) {
#pragma unroll
      for (int b = 0; b < CB; ++b)
#pragma unroll
        for (int a = 0; a < DB; ++a) {
          acc[a][b][0] = mma16(ga[a][0], xb[b][0], acc[a][b][0]);
          acc[a][b][2] = mma16(ga[a][2], xb[b][2], acc[a][b][2]);
          acc[a][b][1] = mma16(ga[a][1], xb[b][1], acc[a][b][1]);
          acc[a][b][3] = mma16(ga[a][3], xb[b][2], acc[a][b][3]);
          acc[a][b][2] = mma16(ga[a][3], xb[b][3], acc[a][b][2]);
          accn[a][b] = mma16(ga[a][2], xb[b][3], accn[a][b]);
        }
    };
    for (int st = 0; st < nsteps; ++st) {
      __syncthreads();  // barrier st: step st is in buffer st % 2
      read_step(ga, xb, lds + (st & 1) * BUF);
      mma_step(ga, xb);
    }
    // partial planes part[split][p][d][c] (c contiguous): lane (j, g) holds
    // rows d 4g..4g+3 of column c j of each 16 x 16 block; sixteen lanes store
    // 64 contiguous bytes per row
    const int64_t plane = (int64_t)c_pad * d_pad;
    float* pout = part + (int64_t)split * 4 * plane;
#pragma unroll
    for (int a = 0; a < DB; ++a)
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        const int d = d0 + (wd * DB + a) * 16 + 4 * g;
        const int c = c0 + (wc * CB + b) * 16 + j;
        acc[a][b][3] -= accn[a][b];
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
          for (int r = 0; r < 4; ++r) pout[p * plane + (int64_t)(d + r) * c_pad + c] = acc[a][b][p][r];
      }
  }

  // ---- bias partial: the producer parts summed in a fixed order ------------
  if (ct == 0) {
    __syncthreads();
    for (int jj = tid; jj < BD; jj += (NC + NP) * 64) {
      float sb = bred[0][jj];
      if constexpr (HALVES == 2) sb += bred[1][jj];
      part_b[(int64_t)split * d_pad + d0 + jj] = 4.0f * sb;
    }
  }
}

// Sum of the S partials [S][4][d_pad][c_pad] (c contiguous) and [S][d_pad],
// inverse butterfly, dW and dbias.  Work-group = 8 waves over 256
// consecutive (d, c) elements of a plane (64 lanes x 4 c); wave w sums the
// splits s = w, w + 8, ... in increasing order and wave 0 adds the eight wave
// sums in wave order: a fixed summation tree, so the result is
// deterministic.  Loads and the stores of dW [D][C][4] are contiguous across
// lanes.  The last ceil(d_pad / 256) work-groups sum the bias partials.
constexpr int FIN_WAVES = 8;
__global__ __launch_bounds__(64 * FIN_WAVES) void k_bwd_weight_finish(
    const float* __restrict__ part, const float* __restrict__ part_b, float* __restrict__ dW,
    float* __restrict__ dbias, int C, int D, int d_pad, int c_pad, int S, int n_main) {
  __shared__ f32x4 red[FIN_WAVES][4][64];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t plane = (int64_t)c_pad * d_pad;
  if ((int)blockIdx.x >= n_main) {  // bias: 256 consecutive d per work-group
    if (dbias == nullptr) return;    // whole work-group
    const int d = ((int)blockIdx.x - n_main) * 256 + 4 * lane;
    f32x4 b = {};
    if (d < d_pad)  // d_pad is a multiple of 32
      for (int s = w; s < S; s += FIN_WAVES) b += *reinterpret_cast<const f32x4*>(part_b + (int64_t)s * d_pad + d);
    red[w][0][lane] = b;
    __syncthreads();
    if (w == 0) {
      f32x4 q = red[0][0][lane];
#pragma unroll
      for (int ww = 1; ww < FIN_WAVES; ++ww) q += red[ww][0][lane];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (d + k < D) dbias[d + k] = q[k];
    }
    return;
  }
  const int64_t e0 = (int64_t)blockIdx.x * 256 + 4 * lane;  // c_pad is a multiple of 32
  f32x4 P[4] = {};
  if (e0 < plane) {
    constexpr int IT = 4;
    for (int s0 = w; s0 < S; s0 += FIN_WAVES * IT) {
      f32x4 v[IT][4];
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int sp = s0 + FIN_WAVES * it;
        if (sp < S) {
          const float* ps = part + (int64_t)sp * 4 * plane + e0;
#pragma unroll
          for (int p = 0; p < 4; ++p) v[it][p] = *reinterpret_cast<const f32x4*>(ps + p * plane);
        }
      }
#pragma unroll
      for (int it = 0; it < IT; ++it)
        if (s0 + FIN_WAVES * it < S) {
#pragma unroll
          for (int p = 0; p < 4; ++p) P[p] += v[it][p];
        }
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) red[w][p][lane] = P[p];
  __syncthreads();
  if (w == 0 && e0 < plane) {
    f32x4 q[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      q[p] = red[0][p][lane];
#pragma unroll
      for (int ww = 1; ww < FIN_WAVES; ++ww) q[p] += red[ww][p][lane];
    }
    const int d = (int)(e0 / c_pad), c = (int)(e0 % c_pad);
    if (d < D) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c + k < C)
          *reinterpret_cast<floatx4*>(dW + ((int64_t)d * C + c + k) * 4) = idft4(q[0][k], q[1][k], q[2][k], q[3][k]);
    }
  }
}

// ---------------------------------------------------------------------------
// Tiles of 32 (d) x 96 (c) outputs: 4 consumer waves of 16 x 48, 8 producer
// waves (dy: one 32-column unit, x: three, each split over two waves by rows).
// Measured on MI355X at N = 12608, C = 96, D = 384 (binary16, warm): 22.1 us
// for this kernel and the finish against 26.9 us for the vector-unit
// butterfly with 16-byte loads whose lanes walk rows (four times the address
// cycles of lanes along a row) it replaces; 20.4-21.6 us with the producers'
// loads one step ahead, after the transform.
constexpr int BWS_NWD = 2, BWS_NWC = 2, BWS_DB = 1, BWS_CB = 3, BWS_NP = 8;
constexpr int BWS_BD = BWS_NWD * BWS_DB * 16, BWS_BC = BWS_NWC * BWS_CB * 16;

bool bws_supported(const eqlinear_plan* p) {
  if (p->tune.bws_off == 1 || p->dtype != EQL_F16) return false;
  // whole column pairs (16-byte units).  Wider layers re-read dy once per
  // column tile and still beat the tiled kernel of k_bwd_weight.hip.
  return p->C % 2 == 0 && p->D % 2 == 0;
}

struct BwsDims {
  int64_t S, R, d_pad, c_pad;
  int n_dt, n_ct, per_xcd;
};

static BwsDims bws_dims(const eqlinear_plan* p, int64_t N) {
  BwsDims m;
  m.n_dt = (int)((p->D + BWS_BD - 1) / BWS_BD);
  m.n_ct = (int)((p->C + BWS_BC - 1) / BWS_BC);
  m.d_pad = (int64_t)m.n_dt * BWS_BD;
  m.c_pad = (int64_t)m.n_ct * BWS_BC;
  const int T = m.n_dt * m.n_ct;
  // about one work-group per CU (one fits per CU), splits of whole 32-row steps
  int64_t S = p->tune.bws_s > 0 ? p->tune.bws_s : (256 / T > 0 ? 256 / T : 1);
  const int64_t steps = (N + 31) / 32;
  if (S > steps) S = steps;
  if (S < 1) S = 1;
  const int64_t steps_per = (steps + S - 1) / S;
  m.R = steps_per * 32;
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

hipError_t launch_bws(const eqlinear_plan* p, const void* x, const void* dy, float* dW, float* dbias,
                      int64_t N, void* ws, hipStream_t s) {
  const BwsDims m = bws_dims(p, N);
  float* part = (float*)ws;
  float* part_b = part + m.S * 4 * m.c_pad * m.d_pad;
  const unsigned blocks = (unsigned)(8 * m.per_xcd);
  hipLaunchKernelGGL((k_bwd_weight_ws<BWS_NWD, BWS_NWC, BWS_DB, BWS_CB, BWS_NP>), dim3(blocks),
                     dim3((BWS_NWD * BWS_NWC + BWS_NP) * 64), 0, s, (const _Float16*)x, (const _Float16*)dy,
                     part, part_b, (int)N, (int)p->C, (int)p->D, (int)m.d_pad, (int)m.c_pad, (int)m.R, m.n_dt,
                     m.n_ct, (int)m.S, m.per_xcd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_main = (int)((m.d_pad * m.c_pad + 255) / 256);
  const int n_bias = (int)((m.d_pad + 255) / 256);
  hipLaunchKernelGGL(k_bwd_weight_finish, dim3((unsigned)(n_main + n_bias)), dim3(64 * FIN_WAVES), 0, s, part,
                     part_b, dW, dbias, (int)p->C, (int)p->D, (int)m.d_pad, (int)m.c_pad, (int)m.S, n_main);
  return hipGetLastError();
}

}  // namespace eql
