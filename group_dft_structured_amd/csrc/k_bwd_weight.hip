// Backward with respect to the compact weight and the bias.
//
// dW[d,c,r] = sum_{n,t} dy[n,d,t] x[n,c,(t-r) mod 4] is a circular
// cross-correlation along the group axis, summed over rows.  In the group
// Fourier domain (the same p4 transforms as the forward, Flash EQ-Linear
// "Specializzazione per il Gruppo di Rotazione p4") it becomes, per frequency,
// P[k] = sum_n G[n,:,k] conj(X[n,:,k]) with G = DFT_4(dy), X = DFT_4(x):
//     P0 = sum G0^T X0                  P2 = sum G2^T X2
//     Pr = sum (Gr^T Xr + Gi^T Xi)      Pi = sum (Gi^T Xr - Gr^T Xi)
// again six real products, and dW = IDFT_4(P).  dbias[d] = sum_n G0[n,d].
//
// Pass 1 (k_bwd_weight_partial): work-group (split s, d tile, c tile) reduces
// the rows of split s on the matrix cores with fp32 accumulators and writes
// its four fp32 partial planes to the workspace.  Pass 2
// (k_bwd_weight_reduce) sums the partials of every split in a fixed order
// (deterministic, no atomics), applies the inverse butterfly and writes dW
// and dbias.
#include <type_traits>

#include "eql_device.h"
#include "eql_internal.h"

namespace eql {

template <typename T>
struct BwTile {
  static constexpr int BR = 64 / (int)sizeof(T);   // rows per chunk (matrix-core k)
  static constexpr int PAD = 16 / (int)sizeof(T);
  static constexpr int SK = BR + PAD;              // LDS stride (80 B)
  static constexpr int KPL = BR / 2;
  static constexpr int STEPS = BR / Mma<T>::K_STEP;
  static constexpr int RB = 16 / (int)sizeof(T);   // rows per 16-byte LDS write
};

template <typename T>
struct LaneK2 {
  typedef typename std::conditional<std::is_same<T, float>::value, floatx4, half8>::type v16b;
  v16b lo, hi;
};

template <typename T>
__device__ __forceinline__ LaneK2<T> lds_lane_k2(const T* p) {
  LaneK2<T> r;
  r.lo = *reinterpret_cast<const typename LaneK2<T>::v16b*>(p);
  r.hi = *reinterpret_cast<const typename LaneK2<T>::v16b*>(p + BwTile<T>::KPL / 2);
  return r;
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag step_frag2(const LaneK2<T>& v, int s);
template <>
__device__ __forceinline__ half8 step_frag2<_Float16>(const LaneK2<_Float16>& v, int s) {
  return s == 0 ? v.lo : v.hi;
}
template <>
__device__ __forceinline__ float step_frag2<float>(const LaneK2<float>& v, int s) {
  return s < 4 ? v.lo[s] : v.hi[s - 4];
}

// Stage rows [r, r+BR) x features [f0, f0+BF) of a [rows][F][4] tensor,
// transposed, as four scaled spectral planes dst[p][feature][row] (stride
// SK).  Unit = (feature j, block q of RB rows); consecutive threads take
// consecutive features so that the quad loads coalesce.  The fp32 sum of the
// four group values (X0, unscaled) is summed into fsum[it] when SUM is set.
template <typename T, int BF, int NT, bool SUM>
__device__ __forceinline__ void stage_cols_dft(const T* __restrict__ src, int F, int r, int r_end,
                                               int f0, T* __restrict__ dst, float* fsum) {
  constexpr int BR = BwTile<T>::BR, SK = BwTile<T>::SK, RB = BwTile<T>::RB;
  constexpr int UNITS = BF * (BR / RB);
  constexpr int PLANE = BF * SK;
  typedef typename LaneK2<T>::v16b V;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < (UNITS + NT - 1) / NT; ++it) {
    const int u = it * NT + tid;
    if (UNITS % NT != 0 && u >= UNITS) break;
    const int j = u % BF, q = u / BF;
    const int f = f0 + j;
    V o0, o2, orr, oi;
#pragma unroll
    for (int e = 0; e < RB; ++e) {
      const int n = r + q * RB + e;
      floatx4 v = {0.f, 0.f, 0.f, 0.f};
      if (n < r_end && f < F) {
        typedef typename Elem<T>::quad Q;
        v = Elem<T>::unpack(*reinterpret_cast<const Q*>(src + ((int64_t)n * F + f) * 4));
      }
      const Spec4 s = dft4(v[0], v[1], v[2], v[3]);  // scaled planes
      if (SUM) fsum[it] += (v[0] + v[2]) + (v[1] + v[3]);  // unscaled X0 for the bias
      o0[e] = Elem<T>::from_f(s.f0);
      o2[e] = Elem<T>::from_f(s.f2);
      orr[e] = Elem<T>::from_f(s.fr);
      oi[e] = Elem<T>::from_f(s.fi);
    }
    T* d = dst + j * SK + q * RB;
    *reinterpret_cast<V*>(d + 0 * PLANE) = o0;
    *reinterpret_cast<V*>(d + 1 * PLANE) = o2;
    *reinterpret_cast<V*>(d + 2 * PLANE) = orr;
    *reinterpret_cast<V*>(d + 3 * PLANE) = oi;
  }
}

template <typename T, int BD, int BC, int WAVES_D, int WAVES_C>
__global__ __launch_bounds__(64 * WAVES_D* WAVES_C) void k_bwd_weight_partial(
    const T* __restrict__ x,     // [N][C][4]
    const T* __restrict__ dy,    // [N][D][4]
    float* __restrict__ part,    // [S][4][d_pad][c_pad]
    float* __restrict__ part_b,  // [S][d_pad]
    int N, int C, int D, int d_pad, int c_pad, int rows_per_split, int n_dt, int n_ct) {
  constexpr int NT = 64 * WAVES_D * WAVES_C;
  constexpr int BR = BwTile<T>::BR, SK = BwTile<T>::SK, KPL = BwTile<T>::KPL;
  constexpr int STEPS = BwTile<T>::STEPS, RB = BwTile<T>::RB;
  constexpr int WD = BD / WAVES_D, WC = BC / WAVES_C;
  constexpr int MB = WD / 32, NB = WC / 32;
  static_assert(WD % 32 == 0 && WC % 32 == 0, "wave tile must be a multiple of 32");
  constexpr int G_PLANE = BD * SK, X_PLANE = BC * SK;
  constexpr int G_ITERS = (BD * (BR / RB) + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) T lds[4 * G_PLANE + 4 * X_PLANE];
  __shared__ float bred[BR / RB][BD];
  T* Gs = lds;
  T* Xs = lds + 4 * G_PLANE;

  int t = blockIdx.x;
  const int ct = t % n_ct;
  t /= n_ct;
  const int dt = t % n_dt;
  const int split = t / n_dt;
  const int d0 = dt * BD, c0 = ct * BC;
  const int r_begin = split * rows_per_split;
  const int r_end = min(N, r_begin + rows_per_split);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int h = lane >> 5, i32 = lane & 31;
  const int wd = wave / WAVES_C, wc = wave % WAVES_C;

  floatx16 acc[MB][NB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int p = 0; p < 4; ++p) acc[mb][nb][p] = floatx16{};
  float bsum[G_ITERS];
#pragma unroll
  for (int i = 0; i < G_ITERS; ++i) bsum[i] = 0.f;

  for (int r = r_begin; r < r_end; r += BR) {
    stage_cols_dft<T, BD, NT, true>(dy, D, r, r_end, d0, Gs, bsum);
    stage_cols_dft<T, BC, NT, false>(x, C, r, r_end, c0, Xs, nullptr);
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const T* ap = Gs + (wd * WD + mb * 32 + i32) * SK + h * KPL;
      const LaneK2<T> g0 = lds_lane_k2<T>(ap + 0 * G_PLANE);
      const LaneK2<T> g2 = lds_lane_k2<T>(ap + 1 * G_PLANE);
      const LaneK2<T> gr = lds_lane_k2<T>(ap + 2 * G_PLANE);
      const LaneK2<T> gi = lds_lane_k2<T>(ap + 3 * G_PLANE);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const T* bp = Xs + (wc * WC + nb * 32 + i32) * SK + h * KPL;
        const LaneK2<T> x0 = lds_lane_k2<T>(bp + 0 * X_PLANE);
        const LaneK2<T> x2 = lds_lane_k2<T>(bp + 1 * X_PLANE);
        const LaneK2<T> xr = lds_lane_k2<T>(bp + 2 * X_PLANE);
        const LaneK2<T> xi = lds_lane_k2<T>(bp + 3 * X_PLANE);
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
          const auto fg0 = step_frag2<T>(g0, s), fg2 = step_frag2<T>(g2, s);
          const auto fgr = step_frag2<T>(gr, s), fgi = step_frag2<T>(gi, s);
          const auto fx0 = step_frag2<T>(x0, s), fx2 = step_frag2<T>(x2, s);
          const auto fxr = step_frag2<T>(xr, s), fxi = step_frag2<T>(xi, s);
          acc[mb][nb][0] = Mma<T>::mma(fg0, fx0, acc[mb][nb][0]);
          acc[mb][nb][2] = Mma<T>::mma(fgr, fxr, acc[mb][nb][2]);
          acc[mb][nb][1] = Mma<T>::mma(fg2, fx2, acc[mb][nb][1]);
          acc[mb][nb][3] = Mma<T>::mma(fgi, fxr, acc[mb][nb][3]);
          acc[mb][nb][2] = Mma<T>::mma(fgi, fxi, acc[mb][nb][2]);
          acc[mb][nb][3] = Mma<T>::mma(fgr, -fxi, acc[mb][nb][3]);
        }
      }
    }
    __syncthreads();
  }

  // partial planes
  const int64_t plane = (int64_t)d_pad * c_pad;
  float* pout = part + (int64_t)split * 4 * plane;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int c = c0 + wc * WC + nb * 32 + i32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = d0 + wd * WD + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int64_t o = (int64_t)d * c_pad + c;
#pragma unroll
        for (int p = 0; p < 4; ++p) pout[p * plane + o] = acc[mb][nb][p][r];
      }
    }

  // bias partial: fixed-order reduction over the row blocks of each feature
  if (ct == 0) {
    constexpr int UNITS = BD * (BR / RB);
#pragma unroll
    for (int it = 0; it < G_ITERS; ++it) {
      const int u = it * NT + tid;
      if (u < UNITS) bred[u / BD][u % BD] = bsum[it];
    }
    __syncthreads();
    for (int j = tid; j < BD; j += NT) {
      float sacc = 0.f;
#pragma unroll
      for (int q = 0; q < BR / RB; ++q) sacc += bred[q][j];
      part_b[(int64_t)split * d_pad + d0 + j] = sacc;
    }
  }
}

__global__ __launch_bounds__(256) void k_bwd_weight_reduce(const float* __restrict__ part,
                                                           const float* __restrict__ part_b,
                                                           float* __restrict__ dW,
                                                           float* __restrict__ dbias, int C, int D,
                                                           int d_pad, int c_pad, int S) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t pairs = (int64_t)C * D;
  const int64_t plane = (int64_t)d_pad * c_pad;
  if (i < pairs) {
    const int d = (int)(i / C), c = (int)(i % C);
    const int64_t o = (int64_t)d * c_pad + c;
    float P0 = 0.f, P2 = 0.f, Pr = 0.f, Pi = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* ps = part + (int64_t)s * 4 * plane + o;
      P0 += ps[0];
      P2 += ps[plane];
      Pr += ps[2 * plane];
      Pi += ps[3 * plane];
    }
    *reinterpret_cast<floatx4*>(dW + i * 4) = idft4(P0, P2, Pr, Pi);
    return;
  }
  const int64_t d = i - pairs;
  if (dbias != nullptr && d < D) {
    float b = 0.f;
    for (int s = 0; s < S; ++s) b += part_b[(int64_t)s * d_pad + d];
    dbias[d] = b;
  }
}

// Work-group tile of the partial kernel.
constexpr int BW_BD = 64, BW_BC = 64;

// Rows per split: 512, or more when 512-row splits would give over about
// four work-groups per CU (1024 in all): every split writes four fp32
// partial planes that the reduce pass reads back, and the reduce runs one
// thread per output over all splits (at the 448-channel patch layer of the
// 3 x 3 convolution over 200704 pixels, 392 splits of 512 rows wrote 180 MB
// of partials).
int64_t bwd_weight_rows_per_split(const eqlinear_plan* p, int64_t N) {
  const int64_t tiles = (round_up(p->D, BW_BD) / BW_BD) * (round_up(p->C, BW_BC) / BW_BC);
  const int64_t splits = 1024 / tiles > 1 ? 1024 / tiles : 1;
  const int64_t R = round_up((N + splits - 1) / splits, 512);
  return R > 512 ? R : 512;
}

static void bw_dims(const eqlinear_plan* p, int64_t N, int64_t* S, int64_t* d_pad, int64_t* c_pad) {
  const int64_t R = bwd_weight_rows_per_split(p, N);
  *S = N > 0 ? (N + R - 1) / R : 0;
  *d_pad = round_up(p->D, BW_BD);
  *c_pad = round_up(p->C, BW_BC);
}

// The producer/consumer matrix-core kernel handles binary16 with even channel
// counts (16-byte loads of column pairs); everything else, and plans whose
// knobs turn it off, use the tiled kernel below.
static bool use_bws(const eqlinear_plan* p) { return p->tune.bw_tiled != 1 && bws_supported(p); }

size_t bwd_weight_workspace_bytes(const eqlinear_plan* p, int64_t N) {
  if (p->cyclic) return cyc::workspace_bytes(p, N);
  if (use_bws(p)) return bws_workspace(p, N);
  int64_t S, dp, cp;
  bw_dims(p, N, &S, &dp, &cp);
  if (S == 0) return 0;
  return (size_t)S * (size_t)(4 * dp * cp + dp) * sizeof(float);
}

template <typename T>
static hipError_t launch_bw_t(const eqlinear_plan* p, const void* x, const void* dy, float* dW,
                              float* dbias, int64_t N, void* ws, hipStream_t s) {
  int64_t S, dp, cp;
  bw_dims(p, N, &S, &dp, &cp);
  const int64_t R = bwd_weight_rows_per_split(p, N);
  float* part = (float*)ws;
  float* part_b = part + S * 4 * dp * cp;
  const int n_dt = (int)(dp / BW_BD), n_ct = (int)(cp / BW_BC);
  const int64_t blocks = S * n_dt * n_ct;
  hipLaunchKernelGGL((k_bwd_weight_partial<T, BW_BD, BW_BC, 2, 2>), dim3((unsigned)blocks),
                     dim3(256), 0, s, (const T*)x, (const T*)dy, part, part_b, (int)N, (int)p->C,
                     (int)p->D, (int)dp, (int)cp, (int)R, n_dt, n_ct);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = p->C * p->D + p->D;
  hipLaunchKernelGGL(k_bwd_weight_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     part, part_b, dW, dbias, (int)p->C, (int)p->D, (int)dp, (int)cp, (int)S);
  return hipGetLastError();
}

__global__ void k_zero_f32(float* __restrict__ a, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) a[i] = 0.f;
}

hipError_t launch_backward_weight(const eqlinear_plan* p, const void* x, const void* dy, float* dW,
                                  float* dbias, int64_t N, void* ws, hipStream_t s) {
  if (N == 0) {
    const int64_t n = p->C * p->D * p->T;
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dW, n);
    if (dbias)
      hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)((p->D + 255) / 256)), dim3(256), 0, s, dbias,
                         (int64_t)p->D);
    return hipGetLastError();
  }
  if (p->cyclic) return cyc::launch_backward_weight(p, x, dy, dW, dbias, N, ws, s);
  if (use_bws(p)) return launch_bws(p, x, dy, dW, dbias, N, ws, s);
  if (p->dtype == EQL_F16) return launch_bw_t<_Float16>(p, x, dy, dW, dbias, N, ws, s);
  return launch_bw_t<float>(p, x, dy, dW, dbias, N, ws, s);
}

}  // namespace eql
