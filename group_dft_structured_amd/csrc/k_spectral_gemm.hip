// Fused spectral GEMM: forward and backward-input of the p4 EQ-Linear layer.
//
// y[n,:,:] = IDFT_4( What[k] . DFT_4(x[n,:,:]) )  + bias, per frequency k, with
// What the group DFT of the compact weight (Flash EQ-Linear, "Approccio
// Algoritmico" and "Specializzazione per il Gruppo di Rotazione p4"):
//     Y0 = X0 W0                 Y2 = X2 W2
//     Yr = Xr Wr - Xi Wi         Yi = Xr Wi + Xi Wr
// six real products instead of the sixteen of the unrolled block-circulant
// matrix.  The backward input pass is the same kernel run with the conjugate
// transposed spectra (W0^T, W2^T, Wr^T, -Wi^T) on dy, no bias.
//
// One work-group owns a BM x BN tile of (rows, output channels).  Per K chunk
// it stages the x tile through registers, applies the length-4 butterfly in
// fp32, rounds once to the operand type and writes the four spectral planes to
// LDS; the weight planes of the chunk are copied to LDS beside them.  Every
// wave then runs the six products on the matrix cores for its sub-tile with
// fp32 accumulators.  The epilogue applies the inverse butterfly (exact
// power-of-two scalings), adds the bias and stores y with the group index
// fastest.  No spectral intermediate reaches global memory ("Implementazione":
// fused dataflow, Fourier fragments kept in registers / shared memory).
#include "eql_device.h"
#include "eql_internal.h"
#include "gemm_tile.h"

namespace eql {

// Load the group quad x[n][c][0..3] (zeros when out of range).
template <typename T>
__device__ __forceinline__ floatx4 load_quad(const T* __restrict__ base, bool ok) {
  if (!ok) return floatx4{0.f, 0.f, 0.f, 0.f};
  typedef typename Elem<T>::quad Q;
  return Elem<T>::unpack(*reinterpret_cast<const Q*>(base));
}

// Stage rows [r0, r0+ROWS) x channels [k0, k0+BK) of a [rows][K][4] tensor as
// four spectral planes dst[p][row][k] (row stride SK).  4 channels per thread.
template <typename T, int ROWS, int NT>
__device__ __forceinline__ void stage_rows_dft(const T* __restrict__ src, int rows_total, int K,
                                               int r0, int k0, T* __restrict__ dst) {
  constexpr int BK = Tile<T>::BK, SK = Tile<T>::SK;
  constexpr int TPR = BK / 4;  // threads per row
  constexpr int RPP = NT / TPR;
  constexpr int PLANE = ROWS * SK;
  const int tid = threadIdx.x;
  const int cg = (tid % TPR) * 4;
#pragma unroll
  for (int pass = 0; pass < (ROWS + RPP - 1) / RPP; ++pass) {
    const int row = pass * RPP + tid / TPR;
    if (ROWS % RPP != 0 && row >= ROWS) break;
    const int n = r0 + row;
    const bool row_ok = n < rows_total;
    const T* base = src + ((int64_t)n * K + (k0 + cg)) * 4;
    T o0[4], o2[4], orr[4], oi[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const floatx4 q = load_quad<T>(base + 4 * j, row_ok && (k0 + cg + j) < K);
      const Spec4 s = dft4(q[0], q[1], q[2], q[3]);
      o0[j] = Elem<T>::from_f(s.f0);
      o2[j] = Elem<T>::from_f(s.f2);
      orr[j] = Elem<T>::from_f(s.fr);
      oi[j] = Elem<T>::from_f(s.fi);
    }
    typedef typename Elem<T>::quad Q;
    T* d = dst + row * SK + cg;
    *reinterpret_cast<Q*>(d + 0 * PLANE) = Q{o0[0], o0[1], o0[2], o0[3]};
    *reinterpret_cast<Q*>(d + 1 * PLANE) = Q{o2[0], o2[1], o2[2], o2[3]};
    *reinterpret_cast<Q*>(d + 2 * PLANE) = Q{orr[0], orr[1], orr[2], orr[3]};
    *reinterpret_cast<Q*>(d + 3 * PLANE) = Q{oi[0], oi[1], oi[2], oi[3]};
  }
}

template <typename T, int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M* WAVES_N) void k_spectral_gemm(
    const T* __restrict__ x,        // [N][K][4]
    const T* __restrict__ spec,     // 4 planes [n_pad][k_pad]
    const float* __restrict__ bias, // [n_pad] fp32
    T* __restrict__ y,              // [N][n_out][4]
    int N, int K, int k_pad, int n_out, int n_pad, int n_col_tiles) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int BK = Tile<T>::BK, SK = Tile<T>::SK, KPL = Tile<T>::KPL, STEPS = Tile<T>::STEPS;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int MB = WM / 32, NB = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  constexpr int A_PLANE = BM * SK, B_PLANE = BN * SK;

  __shared__ __attribute__((aligned(16))) T lds[4 * A_PLANE + 4 * B_PLANE];
  T* As = lds;
  T* Bs = lds + 4 * A_PLANE;

  const int tile = blockIdx.x;
  const int col_tile = tile % n_col_tiles;
  const int row_tile = tile / n_col_tiles;
  const int m0 = row_tile * BM;
  const int n0 = col_tile * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int h = lane >> 5, i32 = lane & 31;
  const int wr = wave / WAVES_N, wc = wave % WAVES_N;
  const int64_t plane = (int64_t)n_pad * k_pad;

  floatx16 acc[MB][NB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int p = 0; p < 4; ++p) acc[mb][nb][p] = floatx16{};

  for (int k0 = 0; k0 < k_pad; k0 += BK) {
    // --- stage A (x tile -> four spectral planes) -------------------------
    stage_rows_dft<T, BM, NT>(x, N, K, m0, k0, As);
    // --- stage B (weight spectra chunk) -----------------------------------
    {
      constexpr int UNITS = 4 * BN * 4;  // 16-byte units: plane x row x 4
      constexpr int EPU = 16 / (int)sizeof(T);
#pragma unroll
      for (int u0 = 0; u0 < UNITS; u0 += NT) {
        const int u = u0 + tid;
        if (UNITS % NT != 0 && u >= UNITS) break;
        const int p = u / (BN * 4), rem = u % (BN * 4);
        const int j = rem / 4, q = rem % 4;
        const uint4 v = *reinterpret_cast<const uint4*>(spec + p * plane + (int64_t)(n0 + j) * k_pad +
                                                        k0 + q * EPU);
        *reinterpret_cast<uint4*>(Bs + p * B_PLANE + j * SK + q * EPU) = v;
      }
    }
    __syncthreads();

    // --- six real products on the matrix cores ----------------------------
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const T* ap = As + (wr * WM + mb * 32 + i32) * SK + h * KPL;
      const LaneK<T> a0 = lds_lane_k<T>(ap + 0 * A_PLANE);
      const LaneK<T> a2 = lds_lane_k<T>(ap + 1 * A_PLANE);
      const LaneK<T> ar = lds_lane_k<T>(ap + 2 * A_PLANE);
      const LaneK<T> ai = lds_lane_k<T>(ap + 3 * A_PLANE);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const T* bp = Bs + (wc * WN + nb * 32 + i32) * SK + h * KPL;
        const LaneK<T> b0 = lds_lane_k<T>(bp + 0 * B_PLANE);
        const LaneK<T> b2 = lds_lane_k<T>(bp + 1 * B_PLANE);
        const LaneK<T> br = lds_lane_k<T>(bp + 2 * B_PLANE);
        const LaneK<T> bi = lds_lane_k<T>(bp + 3 * B_PLANE);
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
          const auto fa0 = step_frag<T>(a0, s), fa2 = step_frag<T>(a2, s);
          const auto far = step_frag<T>(ar, s), fai = step_frag<T>(ai, s);
          const auto fb0 = step_frag<T>(b0, s), fb2 = step_frag<T>(b2, s);
          const auto fbr = step_frag<T>(br, s), fbi = step_frag<T>(bi, s);
          acc[mb][nb][0] = Mma<T>::mma(fa0, fb0, acc[mb][nb][0]);
          acc[mb][nb][2] = Mma<T>::mma(far, fbr, acc[mb][nb][2]);
          acc[mb][nb][1] = Mma<T>::mma(fa2, fb2, acc[mb][nb][1]);
          acc[mb][nb][3] = Mma<T>::mma(far, fbi, acc[mb][nb][3]);
          acc[mb][nb][2] = Mma<T>::mma(fai, neg_frag<T>(fbi), acc[mb][nb][2]);
          acc[mb][nb][3] = Mma<T>::mma(fai, fbr, acc[mb][nb][3]);
        }
      }
    }
    __syncthreads();
  }

  // --- epilogue: inverse butterfly, bias, store ------------------------------
  typedef typename Elem<T>::quad Q;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = n0 + wc * WN + nb * 32 + i32;
      const float bcol = bias[col];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wr * WM + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < N && col < n_out) {
          floatx4 o = idft4(acc[mb][nb][0][r], acc[mb][nb][1][r], acc[mb][nb][2][r],
                            acc[mb][nb][3][r]);
          o[0] += bcol;
          o[1] += bcol;
          o[2] += bcol;
          o[3] += bcol;
          *reinterpret_cast<Q*>(y + ((int64_t)row * n_out + col) * 4) = Elem<T>::pack(o);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launch configuration.  Tile shapes are compile-time; a plan picks one by
// dtype and shape (EQL_GEMM_TILE=<index> overrides it, for tuning sweeps).
struct GemmCfg {
  int bm, bn;
};

template <typename T, int BM, int BN, int WM_, int WN_>
static hipError_t launch_gemm_t(const T* a, const T* spec, const float* bias, T* out, int64_t N,
                                int K, int k_pad, int n_out, int n_pad, hipStream_t s) {
  const int ncol = (n_out + BN - 1) / BN;
  const int64_t nrow = (N + BM - 1) / BM;
  const int64_t blocks = nrow * ncol;
  hipLaunchKernelGGL((k_spectral_gemm<T, BM, BN, WM_, WN_>), dim3((unsigned)blocks),
                     dim3(64 * WM_ * WN_), 0, s, a, spec, bias, out, (int)N, K, k_pad, n_out, n_pad,
                     ncol);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_gemm(int cfg, const T* a, const T* spec, const float* bias, T* out,
                              int64_t N, int K, int k_pad, int n_out, int n_pad, hipStream_t s) {
  switch (cfg) {
    case 0: return launch_gemm_t<T, 64, 128, 2, 2>(a, spec, bias, out, N, K, k_pad, n_out, n_pad, s);
    case 1: return launch_gemm_t<T, 64, 64, 2, 2>(a, spec, bias, out, N, K, k_pad, n_out, n_pad, s);
    case 2: return launch_gemm_t<T, 32, 128, 1, 4>(a, spec, bias, out, N, K, k_pad, n_out, n_pad, s);
    case 3: return launch_gemm_t<T, 128, 64, 4, 1>(a, spec, bias, out, N, K, k_pad, n_out, n_pad, s);
    case 4: return launch_gemm_t<T, 128, 128, 2, 2>(a, spec, bias, out, N, K, k_pad, n_out, n_pad, s);
    default: return hipErrorInvalidValue;
  }
}

static int pick_cfg(const Tuning& tn, int64_t n_out) {
  if (tn.gemm_tile >= 0) return tn.gemm_tile;
  return n_out <= 64 ? 1 : 0;
}

// In-place pointwise activation, for the forward kernels without a fused one.
template <typename T>
__global__ __launch_bounds__(256) void k_activate(T* __restrict__ y, int64_t n, int act) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    y[i] = (T)activate((float)y[i], act);
}

// The general fallback: any channel counts, both dtypes.
static hipError_t launch_forward_plain(const eqlinear_plan* p, const void* x, void* y, int64_t N,
                                       hipStream_t s) {
  const int cfg = pick_cfg(p->tune, p->D);
  if (p->dtype == EQL_F16)
    return launch_gemm<_Float16>(cfg, (const _Float16*)x, (const _Float16*)p->spec_fwd, p->bias_f32,
                                 (_Float16*)y, N, (int)p->C, (int)p->fwd.k_pad, (int)p->D,
                                 (int)p->fwd.n_pad, s);
  return launch_gemm<float>(cfg, (const float*)x, (const float*)p->spec_fwd, p->bias_f32, (float*)y,
                            N, (int)p->C, (int)p->fwd.k_pad, (int)p->D, (int)p->fwd.n_pad, s);
}

hipError_t launch_forward(const eqlinear_plan* p, const void* x, void* y, int64_t N, int act,
                          hipStream_t s) {
  if (p->cyclic) return cyc::launch_forward(p, x, y, N, act, s);
  // the producer/consumer kernels apply the activation in their epilogue
  hipError_t e = launch_ws(p->tune, p->dtype, x, p->frag_fwd, p->bias_f32, y, N, (int)p->C,
                           (int)p->fwd.k_pad, (int)p->D, (int)p->fwd.n_pad, false, act, s);
  if (e != hipErrorNotSupported) return e;
  e = launch_ws32(p->tune, p->dtype, x, p->frag_fwd, p->bias_f32, y, N, (int)p->C, (int)p->fwd.k_pad,
                  (int)p->D, (int)p->fwd.n_pad, act, s);
  if (e != hipErrorNotSupported) return e;
  // the fallbacks store the linear output; a second pass applies the activation
  e = launch_forward_plain(p, x, y, N, s);
  if (e != hipSuccess || act == ACT_NONE) return e;
  const int64_t n = N * p->D * p->T;
  const int64_t blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
  if (p->dtype == EQL_F16)
    hipLaunchKernelGGL(k_activate<_Float16>, dim3((unsigned)blocks), dim3(256), 0, s, (_Float16*)y, n,
                       act);
  else
    hipLaunchKernelGGL(k_activate<float>, dim3((unsigned)blocks), dim3(256), 0, s, (float*)y, n, act);
  return hipGetLastError();
}

hipError_t launch_backward_input(const eqlinear_plan* p, const void* dy, void* dx, int64_t N,
                                 hipStream_t s) {
  if (p->cyclic) return cyc::launch_backward_input(p, dy, dx, N, s);
  hipError_t e = launch_ws(p->tune, p->dtype, dy, p->frag_adj, p->zeros_f32, dx, N, (int)p->D,
                           (int)p->adj.k_pad, (int)p->C, (int)p->adj.n_pad, true, ACT_NONE, s);
  if (e != hipErrorNotSupported) return e;
  const int cfg = pick_cfg(p->tune, p->C);
  if (p->dtype == EQL_F16)
    return launch_gemm<_Float16>(cfg, (const _Float16*)dy, (const _Float16*)p->spec_adj,
                                 p->zeros_f32, (_Float16*)dx, N, (int)p->D, (int)p->adj.k_pad,
                                 (int)p->C, (int)p->adj.n_pad, s);
  return launch_gemm<float>(cfg, (const float*)dy, (const float*)p->spec_adj, p->zeros_f32,
                            (float*)dx, N, (int)p->D, (int)p->adj.k_pad, (int)p->C,
                            (int)p->adj.n_pad, s);
}

}  // namespace eql
