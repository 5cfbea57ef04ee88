// EQ-Linear for a cyclic rotation group of any size 2 <= T <= 16: weight
// spectra, forward, backward_input and backward_weight.
//
// Flash EQ-Linear ("Approccio Algoritmico"): the layer is a circular
// convolution along the group axis composed with a linear map along the
// channels, so a DFT of length T along the group axis turns it into one
// product per frequency, and conjugate symmetry of the real DFT keeps only
// the frequencies k <= T/2.  Per row that is 2T - 2 real matrix products for
// even T and 2T - 1 for odd T, against T^2 for the unrolled dense weight
// (about 2/T of the dense multiply-accumulates, the pages' count).  The
// frequency layout, the forward DFT and its inverse are in cyc_device.h.
//
// The p4 group (T = 4) has its own tuned kernels; these kernels serve every
// other T (and T = 4 when a plan asks for them, which the tests use).
//
// Kernels:
//  * k_cyc_spectra: the DFT of every W[d,c,:] (in double, rounded once to
//    binary32 and then to the plan dtype) into T planes [D_pad][C_pad] for
//    the forward and their conjugate transposes [C_pad][D_pad] for
//    backward_input.
//  * k_cyc_gemm: forward, or backward_input with the conjugate spectra.  A
//    work-group computes a tile of rows x output channels for all T planes.
//    Per chunk of reduction channels it loads (row, channel) group vectors
//    with range-checked buffer loads, applies the DFT in fp32, writes the T
//    planes to LDS in matrix-core fragment order next to the weight chunk,
//    and runs the per-frequency products on the matrix cores (fp32
//    accumulate).  The minus sign of the complex product is a sign flip of
//    the imaginary fragment.  The epilogue applies the inverse DFT and the
//    bias in fp32 and stores T contiguous values per (row, channel).
//  * k_cyc_bwp + k_cyc_bwf: backward_weight.  Per split of rows and tile of
//    (d, c): the DFT of dy and x, transposed into LDS so that rows are the
//    reduction index, and the planes P[k] = sum_n G[k] conj(X[k]) on the
//    matrix cores; fp32 partials per split.  The finish kernel sums the
//    splits in order, applies the inverse DFT (dW[r] is the inverse DFT of
//    P at r) and sums the bias partials (dbias = sum_n G[0]).
#include <stdlib.h>

#include "cyc_device.h"
#include "eql_device.h"
#include "eql_internal.h"

namespace eql {
namespace cyc {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Out-of-range offset: a buffer load there returns zeros, a store is dropped.
constexpr uint32_t OOB = 0x7FFFFFF0u;
constexpr int64_t MAX_RECORDS = 0x7FFFFF00;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int64_t b = bytes < MAX_RECORDS ? bytes : MAX_RECORDS;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)b, 0x00020000);
}

// Matrix-core fragments: one lane holds 16 bytes of a 64-byte row slice of
// an operand (8 binary16 or 4 binary32 reduction values), lane group
// g = lane / 16 owning bytes [16 g, 16 g + 16).  The binary32 product runs
// four 16x16x4 steps, step e taking value e of each lane; both operands use
// the same order, so the reduction is over the same index set.
template <typename DT>
struct Tr;

template <>
struct Tr<_Float16> {
  static constexpr int KC = 32;  // reduction values per 64-byte row slice
  typedef half8 frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag neg(frag a) {
    u32x4 u = __builtin_bit_cast(u32x4, a);
    u ^= 0x80008000u;
    return __builtin_bit_cast(frag, u);
  }
};

template <>
struct Tr<float> {
  static constexpr int KC = 16;
  typedef f32x4 frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ frag neg(frag a) {
    u32x4 u = __builtin_bit_cast(u32x4, a);
    u ^= 0x80000000u;
    return __builtin_bit_cast(frag, u);
  }
};

// Product step and sign flip of one fragment, as functors for the group
// descriptors' product schedules.
template <typename DT>
struct MmaOp {
  __device__ __forceinline__ f32x4 operator()(typename Tr<DT>::frag a, typename Tr<DT>::frag b,
                                              f32x4 c) const {
    return Tr<DT>::mma(a, b, c);
  }
};
template <typename DT>
struct NegOp {
  __device__ __forceinline__ typename Tr<DT>::frag operator()(typename Tr<DT>::frag a) const {
    return Tr<DT>::neg(a);
  }
};

// One group vector (T contiguous values) in global memory.  Its byte offset
// is a multiple of T * sizeof(DT) from a 16-byte aligned base, so it is
// moved in pieces of the largest power of two dividing that size (<= 16).
template <int T, typename DT>
struct Unit {
  static constexpr int BYTES = T * (int)sizeof(DT);
  static constexpr int PIECE = BYTES % 16 == 0 ? 16 : BYTES % 8 == 0 ? 8 : BYTES % 4 == 0 ? 4 : 2;
  static constexpr int NPIECE = BYTES / PIECE;
};

template <int T, typename DT>
__device__ __forceinline__ void load_unit(__amdgpu_buffer_rsrc_t r, uint32_t off, DT (&v)[T]) {
  typedef Unit<T, DT> U;
  static_for<0, U::NPIECE>([&](auto pp) {
    constexpr int p = decltype(pp)::value;
    const uint32_t o = off == OOB ? OOB : off + p * U::PIECE;
    if constexpr (U::PIECE == 16) {
      const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0);
      __builtin_memcpy(reinterpret_cast<char*>(v) + p * 16, &q, 16);
    } else if constexpr (U::PIECE == 8) {
      const u32x2 q = __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, 0);
      __builtin_memcpy(reinterpret_cast<char*>(v) + p * 8, &q, 8);
    } else if constexpr (U::PIECE == 4) {
      const uint32_t q = __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0);
      __builtin_memcpy(reinterpret_cast<char*>(v) + p * 4, &q, 4);
    } else {
      const unsigned short q = __builtin_amdgcn_raw_buffer_load_b16(r, o, 0, 0);
      __builtin_memcpy(reinterpret_cast<char*>(v) + p * 2, &q, 2);
    }
  });
}

template <int T, typename DT>
__device__ __forceinline__ void store_unit(__amdgpu_buffer_rsrc_t r, uint32_t off, const DT (&v)[T]) {
  typedef Unit<T, DT> U;
  static_for<0, U::NPIECE>([&](auto pp) {
    constexpr int p = decltype(pp)::value;
    const uint32_t o = off == OOB ? OOB : off + p * U::PIECE;
    if constexpr (U::PIECE == 16) {
      u32x4 q;
      __builtin_memcpy(&q, reinterpret_cast<const char*>(v) + p * 16, 16);
      __builtin_amdgcn_raw_buffer_store_b128(q, r, o, 0, 0);
    } else if constexpr (U::PIECE == 8) {
      u32x2 q;
      __builtin_memcpy(&q, reinterpret_cast<const char*>(v) + p * 8, 8);
      __builtin_amdgcn_raw_buffer_store_b64(q, r, o, 0, 0);
    } else if constexpr (U::PIECE == 4) {
      uint32_t q;
      __builtin_memcpy(&q, reinterpret_cast<const char*>(v) + p * 4, 4);
      __builtin_amdgcn_raw_buffer_store_b32(q, r, o, 0, 0);
    } else {
      unsigned short q;
      __builtin_memcpy(&q, reinterpret_cast<const char*>(v) + p * 2, 2);
      __builtin_amdgcn_raw_buffer_store_b16(q, r, o, 0, 0);
    }
  });
}

template <typename DT>
__device__ __forceinline__ float to_f(DT v) {
  return (float)v;
}

// ---- weight spectra --------------------------------------------------------
template <typename G, typename DT>
__global__ __launch_bounds__(256) void k_cyc_spectra(
    const DT* __restrict__ W, const DT* __restrict__ bias, DT* __restrict__ spec_fwd,
    DT* __restrict__ spec_adj, float* __restrict__ bias_f32, float* __restrict__ zeros_f32, int C,
    int D, int fwd_n, int fwd_k, int adj_n, int adj_k) {
  constexpr int T = G::T;
  const int64_t fwd_elems = (int64_t)fwd_n * fwd_k;
  const int64_t adj_elems = (int64_t)adj_n * adj_k;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  auto spectrum = [&](int d, int c, double (&X)[T]) {
    for (int j = 0; j < T; ++j) X[j] = 0.0;
    if (d < D && c < C) {
      double w[T];
      const DT* src = W + ((int64_t)d * C + c) * T;
      for (int s = 0; s < T; ++s) w[s] = (double)to_f(src[s]);
      G::template fwd<double>(w, X);
      G::template scale<double>(X);
    }
  };
  if (i < fwd_elems) {
    const int d = (int)(i / fwd_k), c = (int)(i % fwd_k);
    double X[T];
    spectrum(d, c, X);
    static_for<0, T>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      spec_fwd[j * fwd_elems + i] = (DT)(float)X[j];
    });
    return;
  }
  const int64_t k = i - fwd_elems;
  if (k < adj_elems) {
    const int c = (int)(k / adj_k), d = (int)(k % adj_k);
    double X[T];
    spectrum(d, c, X);
    static_for<0, T>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      const float v = (float)X[G::adj_src(j)];
      spec_adj[j * adj_elems + k] = (DT)(G::adj_neg(j) ? -v : v);
    });
    return;
  }
  const int64_t b = k - adj_elems;
  if (b < fwd_n) {
    bias_f32[b] = (bias != nullptr && b < D) ? to_f(bias[b]) : 0.f;
    return;
  }
  const int64_t z = b - fwd_n;
  if (z < adj_n) zeros_f32[z] = 0.f;
}

// ---- forward / backward_input ---------------------------------------------
// Tile BM rows x BN output channels, 4 waves as 2 x 2, each wave (BM/2) x
// (BN/2) in 16 x 16 blocks.  LDS per chunk: T planes of the a-tile [BM][64 B]
// and of the weight tile [BN][64 B].
template <typename G, typename DT, int BM, int BN, bool ACT>
__global__ __launch_bounds__(256) void k_cyc_gemm(const DT* __restrict__ a,
                                                  const DT* __restrict__ spec,
                                                  const float* __restrict__ bias,
                                                  DT* __restrict__ out, int N, int K, int k_pad,
                                                  int n_out, int n_pad, int row_tiles,
                                                  int col_tiles, int per_xcd, int act) {
  typedef Tr<DT> F;
  typedef typename F::frag frag;
  constexpr int T = G::T;
  constexpr int KC = F::KC;
  constexpr int RB = BM / 32, NB = BN / 32;
  constexpr int UX = BM * KC / 256;      // group vectors per thread per chunk
  constexpr int WP = T * BN * 4;           // 16-byte weight pieces per chunk
  constexpr int UW = (WP + 255) / 256;     // per thread (the last round may be partial)
  static_assert(UX * 256 == BM * KC, "tile does not divide");
  __shared__ __attribute__((aligned(16))) unsigned char lds[T * (BM + BN) * 64];
  unsigned char* const lx = lds;
  unsigned char* const lw = lds + T * BM * 64;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int i16 = lane & 15, g = lane >> 4;

  // The column tiles of one row tile are consecutive tiles of one XCD
  // (work-group i runs on XCD i % 8), so they share its L2.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int tile = xcd * per_xcd + slot;
  if (tile >= row_tiles * col_tiles) return;
  const int rt = tile / col_tiles, ct = tile - rt * col_tiles;
  const int row0 = rt * BM, d0 = ct * BN;
  const int rows = min(BM, N - row0);
  const __amdgpu_buffer_rsrc_t rx =
      rsrc(a + (int64_t)row0 * K * T, (int64_t)rows * K * T * (int64_t)sizeof(DT));
  const unsigned char* const wbase = reinterpret_cast<const unsigned char*>(spec);

  DT xv[UX][T];
  u32x4 wv[UW];
  auto load_chunk = [&](int kc) {
#pragma unroll
    for (int i = 0; i < UX; ++i) {
      const int u = tid + 256 * i, r = u / KC, ch = kc * KC + u % KC;
      const uint32_t off = ch < K ? (uint32_t)(((int64_t)r * K + ch) * T * (int64_t)sizeof(DT)) : OOB;
      load_unit<T, DT>(rx, off, xv[i]);
    }
#pragma unroll
    for (int i = 0; i < UW; ++i) {
      const int p = tid + 256 * i, j = p / (BN * 4), rem = p % (BN * 4);
      if (WP % 256 == 0 || p < WP) {
        const int64_t e = ((int64_t)j * n_pad + d0 + (rem >> 2)) * k_pad + (int64_t)kc * KC;
        wv[i] = *reinterpret_cast<const u32x4*>(wbase + e * (int64_t)sizeof(DT) + (rem & 3) * 16);
      }
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int i = 0; i < UX; ++i) {
      const int u = tid + 256 * i, r = u / KC, c = u % KC;
      float xf[T], X[T];
#pragma unroll
      for (int s = 0; s < T; ++s) xf[s] = to_f(xv[i][s]);
      G::template fwd<float>(xf, X);
      G::template scale<float>(X);
#pragma unroll
      for (int j = 0; j < T; ++j)
        *reinterpret_cast<DT*>(lx + (j * BM + r) * 64 + c * (int)sizeof(DT)) = (DT)X[j];
    }
#pragma unroll
    for (int i = 0; i < UW; ++i) {
      const int p = tid + 256 * i, j = p / (BN * 4), rem = p % (BN * 4);
      if (WP % 256 == 0 || p < WP)
        *reinterpret_cast<u32x4*>(lw + (j * BN + (rem >> 2)) * 64 + (rem & 3) * 16) = wv[i];
    }
  };

  f32x4 acc[RB][NB][T];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < T; ++j) acc[rb][nb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&]() {
    frag bw[NB][T];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < T; ++j)
        bw[nb][j] = *reinterpret_cast<const frag*>(
            lw + (j * BN + wn * NB * 16 + nb * 16 + i16) * 64 + g * 16);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      frag ax[T];
#pragma unroll
      for (int j = 0; j < T; ++j)
        ax[j] = *reinterpret_cast<const frag*>(
            lx + (j * BM + wm * RB * 16 + rb * 16 + i16) * 64 + g * 16);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        G::fwd_mma(acc[rb][nb], ax, bw[nb], MmaOp<DT>{}, NegOp<DT>{});
    }
  };

  const int nk = (K + KC - 1) / KC;
  load_chunk(0);
  for (int kc = 0; kc < nk; ++kc) {
    if (kc) __syncthreads();  // every wave is done reading the previous chunk
    store_chunk();
    __syncthreads();
    if (kc + 1 < nk) load_chunk(kc + 1);
    compute();
  }

  // epilogue: inverse DFT and bias in fp32, T contiguous values per (row, d)
  const __amdgpu_buffer_rsrc_t ro =
      rsrc(out + (int64_t)row0 * n_out * T, (int64_t)rows * n_out * T * (int64_t)sizeof(DT));
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int d = d0 + wn * NB * 16 + nb * 16 + i16;  // < n_pad: bias is padded
    const float b = bias[d];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = wm * RB * 16 + rb * 16 + 4 * g + r;
        float Q[T], y[T];
#pragma unroll
        for (int j = 0; j < T; ++j) Q[j] = acc[rb][nb][j][r];
        G::template inv<float>(Q, y);
        DT o[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
          float v = y[t] + b;
          if constexpr (ACT) v = activate(v, act);
          o[t] = (DT)v;
        }
        const uint32_t off =
            d < n_out ? (uint32_t)(((int64_t)rr * n_out + d) * T * (int64_t)sizeof(DT)) : OOB;
        store_unit<T, DT>(ro, off, o);
      }
    }
  }
}

// ---- backward_weight -------------------------------------------------------
// Tile TD (d) x TC (c), 4 waves as 2 x 2.  Per step of KC rows: the DFT of
// dy and x, written to LDS transposed ([column][rows], rows contiguous, an
// 80-byte pitch that spreads the column-wise writes over the banks).
template <typename G, typename DT, int TD, int TC>
__global__ __launch_bounds__(256) void k_cyc_bwp(const DT* __restrict__ x,
                                                 const DT* __restrict__ dy,
                                                 float* __restrict__ part,
                                                 float* __restrict__ part_b, int N, int C, int D,
                                                 int rows_per_split, int d_pad, int c_pad,
                                                 int d_tiles, int c_tiles, int n_tiles,
                                                 int per_xcd) {
  typedef Tr<DT> F;
  typedef typename F::frag frag;
  constexpr int T = G::T;
  constexpr int RS = F::KC;  // rows per step
  constexpr int PITCH = 80;
  constexpr int RB = TD / 32, NB = TC / 32;
  constexpr int GD = 256 / TD, GC = 256 / TC;        // row-pair groups
  constexpr int PD = RS / 2 / GD, PC = RS / 2 / GC;  // row pairs per thread
  static_assert(PD * GD * 2 == RS && PC * GC * 2 == RS, "tile does not divide");
  __shared__ __attribute__((aligned(16))) unsigned char lds[T * (TD + TC) * PITCH];
  __shared__ float bred[GD][TD];
  unsigned char* const lg = lds;
  unsigned char* const lxs = lds + T * TD * PITCH;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int i16 = lane & 15, g = lane >> 4;

  // the tiles of one split are consecutive tiles of one XCD: they read the
  // same rows of x and dy through its L2
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int tile = xcd * per_xcd + slot;
  if (tile >= n_tiles) return;
  const int per_split = d_tiles * c_tiles;
  const int s = tile / per_split, rem = tile - s * per_split;
  const int dt = rem / c_tiles, ct = rem - dt * c_tiles;
  const int d0 = dt * TD, c0 = ct * TC;
  const int64_t r_begin = (int64_t)s * rows_per_split;
  const int64_t r_end = min((int64_t)N, r_begin + rows_per_split);
  const int nsteps = r_begin < r_end ? (int)((r_end - r_begin + RS - 1) / RS) : 0;

  const int dcol = tid % TD, dgrp = tid / TD;
  const int ccol = tid % TC, cgrp = tid / TC;
  const bool d_ok = d0 + dcol < D, c_ok = c0 + ccol < C;

  DT gv[PD][2][T], xv[PC][2][T];
  auto load_step = [&](int st) {
    const int64_t r0 = r_begin + (int64_t)st * RS;
    const int64_t nr = min((int64_t)RS, r_end - r0);
    const __amdgpu_buffer_rsrc_t rd = rsrc(dy + r0 * D * T, nr * D * T * (int64_t)sizeof(DT));
    const __amdgpu_buffer_rsrc_t rc = rsrc(x + r0 * C * T, nr * C * T * (int64_t)sizeof(DT));
#pragma unroll
    for (int i = 0; i < PD; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 2 * (dgrp + GD * i) + h;
        const uint32_t off =
            d_ok ? (uint32_t)(((int64_t)r * D + d0 + dcol) * T * (int64_t)sizeof(DT)) : OOB;
        load_unit<T, DT>(rd, off, gv[i][h]);
      }
#pragma unroll
    for (int i = 0; i < PC; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 2 * (cgrp + GC * i) + h;
        const uint32_t off =
            c_ok ? (uint32_t)(((int64_t)r * C + c0 + ccol) * T * (int64_t)sizeof(DT)) : OOB;
        load_unit<T, DT>(rc, off, xv[i][h]);
      }
  };

  float bsum = 0.f;  // sum over this thread's rows of G[0] at column dcol
  auto store_step = [&]() {
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      float Gs[2][T];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float v[T];
#pragma unroll
        for (int t = 0; t < T; ++t) v[t] = to_f(gv[i][h][t]);
        G::template fwd<float>(v, Gs[h]);
      }
      // plane 0 before its scaling is the sum over the group
      bsum += Gs[0][0];
      bsum += Gs[1][0];
      G::template scale<float>(Gs[0]);
      G::template scale<float>(Gs[1]);
      const int rp = dgrp + GD * i;
#pragma unroll
      for (int j = 0; j < T; ++j) {
        DT two[2] = {(DT)Gs[0][j], (DT)Gs[1][j]};
        __builtin_memcpy(lg + (j * TD + dcol) * PITCH + rp * 2 * (int)sizeof(DT), two, sizeof(two));
      }
    }
#pragma unroll
    for (int i = 0; i < PC; ++i) {
      float X[2][T];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float v[T];
#pragma unroll
        for (int t = 0; t < T; ++t) v[t] = to_f(xv[i][h][t]);
        G::template fwd<float>(v, X[h]);
        G::template scale<float>(X[h]);
      }
      const int rp = cgrp + GC * i;
#pragma unroll
      for (int j = 0; j < T; ++j) {
        DT two[2] = {(DT)X[0][j], (DT)X[1][j]};
        __builtin_memcpy(lxs + (j * TC + ccol) * PITCH + rp * 2 * (int)sizeof(DT), two, sizeof(two));
      }
    }
  };

  f32x4 acc[RB][NB][T];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < T; ++j) acc[rb][nb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&]() {
    frag xb[NB][T];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < T; ++j)
        xb[nb][j] = *reinterpret_cast<const frag*>(
            lxs + (j * TC + wn * NB * 16 + nb * 16 + i16) * PITCH + g * 16);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      frag ga[T];
#pragma unroll
      for (int j = 0; j < T; ++j)
        ga[j] = *reinterpret_cast<const frag*>(
            lg + (j * TD + wm * RB * 16 + rb * 16 + i16) * PITCH + g * 16);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        G::bw_mma(acc[rb][nb], ga, xb[nb], MmaOp<DT>{}, NegOp<DT>{});
    }
  };

  if (nsteps > 0) load_step(0);
  for (int st = 0; st < nsteps; ++st) {
    if (st) __syncthreads();
    store_step();
    __syncthreads();
    if (st + 1 < nsteps) load_step(st + 1);
    compute();
  }

  // partial planes of this split: part[s][j][d][c]
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int c = c0 + wn * NB * 16 + nb * 16 + i16;
#pragma unroll
      for (int j = 0; j < T; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = d0 + wm * RB * 16 + rb * 16 + 4 * g + r;
          part[(((int64_t)s * T + j) * d_pad + d) * c_pad + c] = acc[rb][nb][j][r];
        }
    }
  if (ct == 0) {
    bred[dgrp][dcol] = bsum;
    __syncthreads();
    if (tid < TD) {
      float b = 0.f;
#pragma unroll
      for (int q = 0; q < GD; ++q) b += bred[q][tid];
      part_b[(int64_t)s * d_pad + d0 + tid] = b;
    }
  }
}

template <typename G>
__global__ __launch_bounds__(256) void k_cyc_bwf(const float* __restrict__ part,
                                                 const float* __restrict__ part_b,
                                                 float* __restrict__ dW, float* __restrict__ dbias,
                                                 int C, int D, int d_pad, int c_pad, int S) {
  constexpr int T = G::T;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t DC = (int64_t)D * C;
  if (i < DC) {
    const int d = (int)(i / C), c = (int)(i % C);
    float P[T];
#pragma unroll
    for (int j = 0; j < T; ++j) P[j] = 0.f;
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int j = 0; j < T; ++j) P[j] += part[(((int64_t)s * T + j) * d_pad + d) * c_pad + c];
    float w[T];
    G::template inv<float>(P, w);
#pragma unroll
    for (int r = 0; r < T; ++r) dW[i * T + r] = w[r];
  } else if (dbias != nullptr && i < DC + D) {
    const int d = (int)(i - DC);
    float b = 0.f;
    for (int s = 0; s < S; ++s) b += part_b[(int64_t)s * d_pad + d];
    dbias[d] = b;
  }
}

// ---- host side -------------------------------------------------------------
struct BwDims {
  int64_t S, rows_per_split;
  int TD, d_pad, c_pad, d_tiles, c_tiles;
};

BwDims bw_dims(const eqlinear_plan* p, int64_t N) {
  BwDims b;
  b.TD = p->cyc_bw_tile;
  b.d_tiles = (int)((p->D + b.TD - 1) / b.TD);
  b.c_tiles = (int)((p->C + b.TD - 1) / b.TD);
  b.d_pad = b.d_tiles * b.TD;
  b.c_pad = b.c_tiles * b.TD;
  const int64_t tiles = (int64_t)b.d_tiles * b.c_tiles;
  // about cyc_bw_wgs work-groups (two per compute unit by default), at least
  // 128 rows per split
  int64_t S = (p->cyc_bw_wgs + tiles - 1) / tiles;
  const int64_t smax = N / 128 > 1 ? N / 128 : 1;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  b.rows_per_split = (N + S - 1) / S;
  b.rows_per_split = round_up(b.rows_per_split < 1 ? 1 : b.rows_per_split, 32);
  b.S = N > 0 ? (N + b.rows_per_split - 1) / b.rows_per_split : 0;
  return b;
}

template <typename G, typename DT, int BM, int BN, bool ACT = false>
hipError_t launch_gemm_tile(const void* a, const void* spec, const float* bias, void* out,
                            int64_t N, int K, int k_pad, int n_out, int n_pad, int act,
                            hipStream_t s) {
  const int64_t row_tiles = (N + BM - 1) / BM;
  const int col_tiles = (n_out + BN - 1) / BN;
  const int64_t tiles = row_tiles * col_tiles;
  if (tiles > (int64_t)1 << 31) return hipErrorInvalidValue;
  const int64_t per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL((k_cyc_gemm<G, DT, BM, BN, ACT>), dim3((unsigned)(per_xcd * 8)), dim3(256), 0, s,
                     (const DT*)a, (const DT*)spec, bias, (DT*)out, (int)N, K, k_pad, n_out, n_pad,
                     (int)row_tiles, col_tiles, (int)per_xcd, act);
  return hipGetLastError();
}

// Tile shapes (rows x output channels): 0 = 64x64, 1 = 64x32, 2 = 32x64,
// 3 = 32x32 (EQL_CYC_TILE overrides the default).
template <typename G, typename DT>
hipError_t launch_gemm_t(const Tuning& tn, const void* a, const void* spec, const float* bias,
                         void* out, int64_t N, int K, int k_pad, int n_out, int n_pad, int act,
                         hipStream_t s) {
  constexpr int T = G::T;
  const bool wide = T <= 8 && sizeof(DT) == 2;
  if (act != ACT_NONE) {  // fused activation: the default tile only
    if (wide)
      return launch_gemm_tile<G, DT, 32, 64, true>(a, spec, bias, out, N, K, k_pad, n_out, n_pad,
                                                   act, s);
    return launch_gemm_tile<G, DT, 32, 32, true>(a, spec, bias, out, N, K, k_pad, n_out, n_pad, act,
                                                 s);
  }
  int cfg = tn.cyc_tile >= 0 ? tn.cyc_tile : (wide ? 2 : 3);
  if (T > 8 && cfg == 0) cfg = 3;
  switch (cfg) {
    case 0:
      if constexpr (T <= 8)
        return launch_gemm_tile<G, DT, 64, 64>(a, spec, bias, out, N, K, k_pad, n_out, n_pad, act, s);
      return hipErrorInvalidValue;
    case 1: return launch_gemm_tile<G, DT, 64, 32>(a, spec, bias, out, N, K, k_pad, n_out, n_pad, act, s);
    case 2: return launch_gemm_tile<G, DT, 32, 64>(a, spec, bias, out, N, K, k_pad, n_out, n_pad, act, s);
    case 3: return launch_gemm_tile<G, DT, 32, 32>(a, spec, bias, out, N, K, k_pad, n_out, n_pad, act, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename G, typename DT, int TD>
hipError_t launch_bw_tile(const eqlinear_plan* p, const void* x, const void* dy, float* dW,
                          float* dbias, int64_t N, void* ws, hipStream_t s) {
  constexpr int T = G::T;
  const BwDims b = bw_dims(p, N);
  if (b.TD != TD) return hipErrorInvalidValue;
  float* part = (float*)ws;
  float* part_b = part + b.S * T * (int64_t)b.d_pad * b.c_pad;
  const int64_t n_tiles = b.S * b.d_tiles * b.c_tiles;
  const int64_t per_xcd = (n_tiles + 7) / 8;
  hipLaunchKernelGGL((k_cyc_bwp<G, DT, TD, TD>), dim3((unsigned)(per_xcd * 8)), dim3(256), 0, s,
                     (const DT*)x, (const DT*)dy, part, part_b, (int)N, (int)p->C, (int)p->D,
                     (int)b.rows_per_split, b.d_pad, b.c_pad, b.d_tiles, b.c_tiles, (int)n_tiles,
                     (int)per_xcd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = p->D * p->C + p->D;
  hipLaunchKernelGGL(k_cyc_bwf<G>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part,
                     part_b, dW, dbias, (int)p->C, (int)p->D, b.d_pad, b.c_pad, (int)b.S);
  return hipGetLastError();
}

template <typename G, typename DT>
hipError_t launch_bw_t(const eqlinear_plan* p, const void* x, const void* dy, float* dW,
                       float* dbias, int64_t N, void* ws, hipStream_t s) {
  if constexpr (G::T <= 8) {
    if (p->cyc_bw_tile == 64) return launch_bw_tile<G, DT, 64>(p, x, dy, dW, dbias, N, ws, s);
  }
  return launch_bw_tile<G, DT, 32>(p, x, dy, dW, dbias, N, ws, s);
}

template <typename G, typename DT>
hipError_t launch_spectra_t(const eqlinear_plan* p, const void* W, const void* bias,
                            hipStream_t s) {
  const int64_t total = (int64_t)p->fwd.plane_elems() + (int64_t)p->adj.plane_elems() +
                        p->fwd.n_pad + p->adj.n_pad;
  hipLaunchKernelGGL((k_cyc_spectra<G, DT>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     s, (const DT*)W, (const DT*)bias, (DT*)p->spec_fwd, (DT*)p->spec_adj,
                     p->bias_f32, p->zeros_f32, (int)p->C, (int)p->D, (int)p->fwd.n_pad,
                     (int)p->fwd.k_pad, (int)p->adj.n_pad, (int)p->adj.k_pad);
  return hipGetLastError();
}

// Instantiates CALL(G, DT) for the plan's group (cyclic C_T or dihedral D_n,
// n = T / 2) and dtype, and returns its result.
#define EQL_DT(G_, CALL) (p->dtype == EQL_F16 ? CALL(G_, _Float16) : CALL(G_, float))
#define EQL_GROUP_DISPATCH(CALL)                                   \
  if (p->group == EQL_GROUP_DIHEDRAL) {                            \
    switch (p->T / 2) {                                            \
      case 2: return EQL_DT(Dihedral<2>, CALL);                    \
      case 3: return EQL_DT(Dihedral<3>, CALL);                    \
      case 4: return EQL_DT(Dihedral<4>, CALL);                    \
      case 5: return EQL_DT(Dihedral<5>, CALL);                    \
      case 6: return EQL_DT(Dihedral<6>, CALL);                    \
      case 7: return EQL_DT(Dihedral<7>, CALL);                    \
      case 8: return EQL_DT(Dihedral<8>, CALL);                    \
      default: return hipErrorInvalidValue;                        \
    }                                                              \
  }                                                                \
  switch (p->T) {                                                  \
    case 2: return EQL_DT(Cyclic<2>, CALL);                        \
    case 3: return EQL_DT(Cyclic<3>, CALL);                        \
    case 4: return EQL_DT(Cyclic<4>, CALL);                        \
    case 5: return EQL_DT(Cyclic<5>, CALL);                        \
    case 6: return EQL_DT(Cyclic<6>, CALL);                        \
    case 7: return EQL_DT(Cyclic<7>, CALL);                        \
    case 8: return EQL_DT(Cyclic<8>, CALL);                        \
    case 9: return EQL_DT(Cyclic<9>, CALL);                        \
    case 10: return EQL_DT(Cyclic<10>, CALL);                      \
    case 11: return EQL_DT(Cyclic<11>, CALL);                      \
    case 12: return EQL_DT(Cyclic<12>, CALL);                      \
    case 13: return EQL_DT(Cyclic<13>, CALL);                      \
    case 14: return EQL_DT(Cyclic<14>, CALL);                      \
    case 15: return EQL_DT(Cyclic<15>, CALL);                      \
    case 16: return EQL_DT(Cyclic<16>, CALL);                      \
    default: return hipErrorInvalidValue;                          \
  }

}  // namespace

size_t workspace_bytes(const eqlinear_plan* p, int64_t N) {
  if (N <= 0) return 0;
  const BwDims b = bw_dims(p, N);
  return (size_t)(b.S * p->T * (int64_t)b.d_pad * b.c_pad + b.S * (int64_t)b.d_pad) * sizeof(float);
}

hipError_t launch_spectra(const eqlinear_plan* p, const void* W, const void* bias, hipStream_t s) {
#define EQL_CALL(G_, DT_) launch_spectra_t<G_, DT_>(p, W, bias, s)
  EQL_GROUP_DISPATCH(EQL_CALL)
#undef EQL_CALL
}

hipError_t launch_forward(const eqlinear_plan* p, const void* x, void* y, int64_t N, int act,
                          hipStream_t s) {
#define EQL_CALL(G_, DT_)                                                                    \
  launch_gemm_t<G_, DT_>(p->tune, x, p->spec_fwd, p->bias_f32, y, N, (int)p->C, (int)p->fwd.k_pad, \
                         (int)p->D, (int)p->fwd.n_pad, act, s)
  EQL_GROUP_DISPATCH(EQL_CALL)
#undef EQL_CALL
}

hipError_t launch_backward_input(const eqlinear_plan* p, const void* dy, void* dx, int64_t N,
                                 hipStream_t s) {
#define EQL_CALL(G_, DT_)                                                                      \
  launch_gemm_t<G_, DT_>(p->tune, dy, p->spec_adj, p->zeros_f32, dx, N, (int)p->D, (int)p->adj.k_pad, \
                         (int)p->C, (int)p->adj.n_pad, ACT_NONE, s)
  EQL_GROUP_DISPATCH(EQL_CALL)
#undef EQL_CALL
}

hipError_t launch_backward_weight(const eqlinear_plan* p, const void* x, const void* dy, float* dW,
                                  float* dbias, int64_t N, void* ws, hipStream_t s) {
#define EQL_CALL(G_, DT_) launch_bw_t<G_, DT_>(p, x, dy, dW, dbias, N, ws, s)
  EQL_GROUP_DISPATCH(EQL_CALL)
#undef EQL_CALL
}

}  // namespace cyc
}  // namespace eql
