// p4 group convolution on the plane, through rotation-aware patches.
//
// The pages name equivariant convolutions as the next operator for their
// principle (Flash EQ-Linear, gist.science summary, "Limitazioni e Lavoro
// Futuro").  On fields f[P = N*H*W][C][4] over the plane and p4 (the group
// index fastest, so every pixel is one EQ-Linear row) the layer is
//     y[p, d, t] = b[d] + sum_{c, s, v} psi[d, c, R^-t v, (t - s) mod 4] f[p + v, c, s]
// over the k x k offsets v (zero padding), R the quarter turn
// R(a, b) = (-b, a) of (row, column) offsets.
//
// Identity used here.  The nonzero offsets fall into orbits {R^j u} of four
// under the quarter turn; take the representative u with row >= 1 and column
// >= 0.  For an orbit, substituting v = R^j u and s = (j + e) mod 4 gives
//     sum_j sum_e psi[d, c, R^(j-t) u, (t - j) - e] f[p + R^j u, c, j + e],
// which depends on t and j only through t - j: an EQ-Linear layer (circular
// convolution along the group axis, "Intuizione Centrale") on the patch
// channels (u, c, e) with
//     x'[p, (u, c, e), j] = f[p + R^j u, c, (j + e) mod 4]
//     W'[d, (u, c, e), m] = psi[d, c, R^-m u, (m - e) mod 4],
// and the centre tap is the EQ-Linear layer with W'[d, c, m] = psi[d, c, 0, m].
// So the convolution is one EQ-Linear layer with k^2 C input channels, and
// the p4 transform ("Specializzazione per il Gruppo di Rotazione p4") applies
// with its six real products per channel pair: 6 k^2 C D against 16 k^2 C D.
// Each filter entry appears exactly once in W', so W' is a permutation of
// psi and the weight gradient folds back by the same map.
//
// Patch channel order: the C centre channels, then per orbit (representatives
// row-major over rows 1..h, columns 0..h) the 4C channels c*4 + e.  Four
// consecutive patch channels (c, e = 0..3) read the same four neighbour
// quads f[p + R^j u, c, 0..3], j = 0..3, so a gather of four channels costs
// four 4-element loads, as a plain row does.
//
// The backward input pass is the same convolution with the adjoint filter
//     psi*[c, d, w, r] = psi[d, c, -R^r w, (-r) mod 4]
// (K(v)^T shifted to -v is again of the group-convolution form), and runs the
// same kernel on dy.
//
// Kernels in this file (each is described where it is defined):
//  * k_conv_rd_f16: binary16 forward and backward input for 4 to 24
//    reduction steps: weights in VGPRs, every lane gathering and
//    transforming its own matrix-core fragment, the steps split over four
//    waves that combine their partial spectra through LDS;
//  * k_conv_gemm32: binary32, an LDS-tiled spectral GEMM with 16x16x4
//    steps and output tiles of 16 to 64 channels;
//  * k_conv_gemm: the LDS-tiled spectral GEMM with 32x32 steps for the
//    binary16 shapes outside the register-direct range;
//  * k_conv_gather8_f16 / k_conv_gather: the patches written out for the
//    filter gradient; k_conv_patch_weights and k_conv_fold: the permutation
//    between the filter and the patch weight, both ways.
// All of them share the gather rule below: four 4-value loads give four
// patch channels, a centre pixel's own channels or (c, e = 0..3) of an orbit.
#include <utility>

#include "eql_device.h"
#include "eql_internal.h"
#include "gemm_tile.h"

namespace eql {

namespace {

// R^j (a, b) for the quarter turn R(a, b) = (-b, a), j in 0..3.
__host__ __device__ __forceinline__ void turn(int a, int b, int j, int& ra, int& rb) {
  switch (j & 3) {
    case 0: ra = a; rb = b; break;
    case 1: ra = -b; rb = a; break;
    case 2: ra = -a; rb = -b; break;
    default: ra = b; rb = -a; break;
  }
}

__host__ __device__ __forceinline__ int centre_width(int Cs) { return conv_centre_width(Cs); }
__host__ __device__ __forceinline__ int patch_width(int Cs, int k) { return conv_patch_width(Cs, k); }

// Place of the filter entry psi[., c, w, r] (w = (wa, wb) a centred offset)
// in the patch weight W'[., cp, m] for a field of Cs channels.
__host__ __device__ __forceinline__ void patch_place(int c, int wa, int wb, int r, int Cs, int h,
                                                     int& cp, int& m) {
  if (wa == 0 && wb == 0) {
    cp = c;
    m = r;
    return;
  }
  // the one turn m with R^m w in the representative quadrant (row >= 1,
  // column >= 0); then w = R^-m u
  int ua = 0, ub = 0;
  m = 0;
  for (int j = 0; j < 4; ++j) {
    int ra, rb;
    turn(wa, wb, j, ra, rb);
    if (ra >= 1 && rb >= 0) {
      m = j;
      ua = ra;
      ub = rb;
    }
  }
  const int o = (ua - 1) * (h + 1) + ub;
  const int e = (m - r) & 3;
  cp = centre_width(Cs) + o * 4 * Cs + 4 * c + e;
}

}  // namespace

// ---------------------------------------------------------------------------
// Gathered operand: the field, its geometry and the patch width.
struct PatchSrc {
  const void* f;  // [P][Cs][4]
  int H, W, Cs;
  int h;   // kernel half-width (k = 2h + 1)
  int Cc;  // centre width, Cs rounded up to 32
  int K;   // patch channels, Cc + (k^2 - 1) Cs
  int P;   // pixels, N*H*W
};

// Four patch channels starting at cp (a multiple of 4) of one pixel, as four
// raw quads and the mode that turns them into group vectors:
//   mode 0: centre channels cp..cp+3 of the pixel itself, vector e = quad e;
//   mode 1: orbit channels (c, e = 0..3), quad j = f[p + R^j u, c, 0..3],
//           vector e = (quad j element (j + e) mod 4)_j;
//   mode 2: the centre padding or beyond the patch width, zeros.
template <typename T>
struct PatchQuads {
  typedef typename Elem<T>::quad Q;
  Q q[4];
};

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes): loads at an offset past the end
// return zeros, which gives the zero padding of the image border without a
// branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t conv_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t OOB = 0x7FFFFFF0u;

template <typename T>
__device__ __forceinline__ typename Elem<T>::quad load_q(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ half4 load_q<_Float16>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(half4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
template <>
__device__ __forceinline__ floatx4 load_q<float>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <typename T>
__device__ __forceinline__ void patch_mode(const PatchSrc& s, int cp, int& mode, int& c, int& ua,
                                           int& ub) {
  if (cp >= s.K || (cp >= s.Cs && cp < s.Cc)) {
    mode = 2;
  } else if (cp < s.Cc) {
    mode = 0;
    c = cp;
  } else {
    mode = 1;
    const int rem = cp - s.Cc;
    const int o = rem / (4 * s.Cs);
    c = (rem - o * 4 * s.Cs) >> 2;
    ua = 1 + o / (s.h + 1);
    ub = o % (s.h + 1);
  }
}

// The four quads of a pixel's patch channels, read through the resource r
// whose first pixel is pix0 (pix = -1: a row past the end, zeros).
template <typename T>
__device__ __forceinline__ PatchQuads<T> patch_load(const PatchSrc& s, __amdgpu_buffer_rsrc_t r,
                                                    int pix0, int pix, int pi, int pj, int mode, int c,
                                                    int ua, int ub) {
  constexpr int QB = 4 * (int)sizeof(T);  // bytes per quad
  PatchQuads<T> out;
  const bool live = pix >= 0 && mode != 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t off = OOB;
    if (mode == 0) {
      off = (uint32_t)(((pix - pix0) * s.Cs + c + j) * QB);
    } else {
      int va, vb;
      turn(ua, ub, j, va, vb);
      const int ii = pi + va, jj = pj + vb;
      if (ii >= 0 && ii < s.H && jj >= 0 && jj < s.W)
        off = (uint32_t)(((pix + va * s.W + vb - pix0) * s.Cs + c) * QB);
    }
    out.q[j] = load_q<T>(r, live ? off : OOB);
  }
  return out;
}

// Group vector e (0..3) of the four patch channels.
template <typename T>
__device__ __forceinline__ floatx4 patch_vector(const PatchQuads<T>& r, int mode, int e) {
  if (mode == 0) return Elem<T>::unpack(r.q[e]);
  floatx4 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const floatx4 u = Elem<T>::unpack(r.q[j]);
    v[j] = u[(j + e) & 3];
  }
  return v;
}

// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M* WAVES_N) void k_conv_gemm(
    const PatchSrc src,
    const T* __restrict__ spec,      // 4 planes [n_pad][k_pad]
    const float* __restrict__ bias,  // [n_pad] fp32
    T* __restrict__ y,               // [P][n_out][4]
    int k_pad, int n_out, int n_pad, int n_col_tiles, int n_tiles, int act) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int BK = Tile<T>::BK, SK = Tile<T>::SK, KPL = Tile<T>::KPL, STEPS = Tile<T>::STEPS;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int MB = WM / 32, NB = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  constexpr int A_PLANE = BM * SK, B_PLANE = BN * SK;
  constexpr int TPR = BK / 4;                 // staging threads per row
  constexpr int RPP = NT / TPR;               // rows per staging pass
  constexpr int PASSES = (BM + RPP - 1) / RPP;
  constexpr int UNITS = 4 * BN * 4;           // 16-byte weight units per chunk
  constexpr int UPT = (UNITS + NT - 1) / NT;  // per thread
  constexpr int EPU = 16 / (int)sizeof(T);
  static_assert(BK * (int)sizeof(T) == 64, "a chunk row is four 16-byte units");

  __shared__ __attribute__((aligned(16))) T lds[4 * A_PLANE + 4 * B_PLANE];
  T* As = lds;
  T* Bs = lds + 4 * A_PLANE;

  // Work-groups that are dispatched to one XCD (every eighth) take a
  // contiguous run of tiles, so the halo rows they share sit in one L2.
  const int per_xcd = (n_tiles + 7) / 8;
  const int tile = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (tile >= n_tiles) return;
  const int col_tile = tile % n_col_tiles;
  const int row_tile = tile / n_col_tiles;
  const int m0 = row_tile * BM;
  const int n0 = col_tile * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, i32 = lane & 31;
  const int wr = wave / WAVES_N, wc = wave % WAVES_N;
  const int64_t plane = (int64_t)n_pad * k_pad;

  // the field rows this tile reads: its pixels and a halo of h image rows
  // and h pixels on each side
  const int halo = src.h * src.W + src.h;
  const int pix0 = m0 - halo > 0 ? m0 - halo : 0;
  const int pix1 = m0 + BM + halo < src.P ? m0 + BM + halo : src.P;
  const __amdgpu_buffer_rsrc_t rf =
      conv_rsrc((const T*)src.f + (int64_t)pix0 * src.Cs * 4,
                (uint32_t)((int64_t)(pix1 - pix0) * src.Cs * 4 * (int)sizeof(T)));

  // staging rows of this thread and their image coordinates
  const int cg = (tid % TPR) * 4;
  int pix[PASSES], pi[PASSES], pj[PASSES];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int row = ps * RPP + tid / TPR;
    const int m = m0 + row;
    const bool ok = row < BM && m < src.P;
    pix[ps] = ok ? m : -1;
    pj[ps] = ok ? m % src.W : 0;
    pi[ps] = ok ? (m / src.W) % src.H : 0;
  }

  PatchQuads<T> qa[PASSES];
  u32x4v qb[UPT];
  int mode = 2;
  auto load_chunk = [&](int k0) {
    int c = 0, ua = 0, ub = 0;
    patch_mode<T>(src, k0 + cg, mode, c, ua, ub);
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps)
      qa[ps] = patch_load<T>(src, rf, pix0, pix[ps], pi[ps], pj[ps], mode, c, ua, ub);
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = i * NT + tid;
      if (UNITS % NT == 0 || u < UNITS) {
        const int p = u / (BN * 4), rem = u % (BN * 4);
        const int j = rem / 4, q = rem % 4;
        qb[i] = *reinterpret_cast<const u32x4v*>(spec + p * plane + (int64_t)(n0 + j) * k_pad + k0 +
                                                 q * EPU);
      }
    }
  };
  auto store_chunk = [&]() {
    typedef typename Elem<T>::quad Q;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int row = ps * RPP + tid / TPR;
      if (BM % RPP != 0 && row >= BM) break;
      T o0[4], o2[4], orr[4], oi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const floatx4 v = patch_vector<T>(qa[ps], mode, e);
        const Spec4 s = dft4(v[0], v[1], v[2], v[3]);
        o0[e] = Elem<T>::from_f(s.f0);
        o2[e] = Elem<T>::from_f(s.f2);
        orr[e] = Elem<T>::from_f(s.fr);
        oi[e] = Elem<T>::from_f(s.fi);
      }
      T* d = As + row * SK + cg;
      *reinterpret_cast<Q*>(d + 0 * A_PLANE) = Q{o0[0], o0[1], o0[2], o0[3]};
      *reinterpret_cast<Q*>(d + 1 * A_PLANE) = Q{o2[0], o2[1], o2[2], o2[3]};
      *reinterpret_cast<Q*>(d + 2 * A_PLANE) = Q{orr[0], orr[1], orr[2], orr[3]};
      *reinterpret_cast<Q*>(d + 3 * A_PLANE) = Q{oi[0], oi[1], oi[2], oi[3]};
    }
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = i * NT + tid;
      if (UNITS % NT == 0 || u < UNITS) {
        const int p = u / (BN * 4), rem = u % (BN * 4);
        const int j = rem / 4, q = rem % 4;
        *reinterpret_cast<u32x4v*>(Bs + p * B_PLANE + j * SK + q * EPU) = qb[i];
      }
    }
  };

  floatx16 acc[MB][NB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int p = 0; p < 4; ++p) acc[mb][nb][p] = floatx16{};

  load_chunk(0);
  for (int k0 = 0; k0 < k_pad; k0 += BK) {
    store_chunk();
    __syncthreads();
    if (k0 + BK < k_pad) load_chunk(k0 + BK);  // in flight during the products

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
          // Y0 = X0 W0, Y2 = X2 W2, Yr = Xr Wr - Xi Wi, Yi = Xr Wi + Xi Wr
          acc[mb][nb][0] = Mma<T>::mma(fa0, fb0, acc[mb][nb][0]);
          acc[mb][nb][1] = Mma<T>::mma(fa2, fb2, acc[mb][nb][1]);
          acc[mb][nb][2] = Mma<T>::mma(far, fbr, acc[mb][nb][2]);
          acc[mb][nb][3] = Mma<T>::mma(far, fbi, acc[mb][nb][3]);
          acc[mb][nb][2] = Mma<T>::mma(fai, neg_frag<T>(fbi), acc[mb][nb][2]);
          acc[mb][nb][3] = Mma<T>::mma(fai, fbr, acc[mb][nb][3]);
        }
      }
    }
    __syncthreads();
  }

  // --- epilogue: inverse butterfly, bias, activation, store -------------------
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
        if (row < src.P && col < n_out) {
          floatx4 o = idft4(acc[mb][nb][0][r], acc[mb][nb][1][r], acc[mb][nb][2][r],
                            acc[mb][nb][3][r]);
#pragma unroll
          for (int t = 0; t < 4; ++t) o[t] = activate(o[t] + bcol, act);
          *reinterpret_cast<Q*>(y + ((int64_t)row * n_out + col) * 4) = Elem<T>::pack(o);
        }
      }
    }
  }
}

// Binary32 variant with 16x16x4 matrix-core steps: output tiles of 64
// pixels x 16*NBN channels (NBN = 3 fits 48 channels exactly, where 32x32
// steps would pad to 64), four waves of 16 pixels each.  Within a 16-channel
// chunk the reduction index is permuted the same way for both operands: in
// step s lane group g supplies channel 4g + s, so a lane reads its four
// steps' operands as one 16-byte LDS read per plane.
template <int NBN>
__global__ __launch_bounds__(256) void k_conv_gemm32(
    const PatchSrc src,
    const float* __restrict__ spec,  // 4 planes [n_pad][k_pad]
    const float* __restrict__ bias,  // [n_pad]
    float* __restrict__ y,           // [P][n_out][4]
    int k_pad, int n_out, int n_pad, int n_col_tiles, int n_tiles, int act) {
  typedef float T;
  constexpr int BM = 64, BN = 16 * NBN, NT = 256;
  constexpr int BK = Tile<T>::BK, SK = Tile<T>::SK;  // 16 channels, 20-float rows
  constexpr int A_PLANE = BM * SK, B_PLANE = BN * SK;
  constexpr int TPR = BK / 4;                 // staging threads per row
  constexpr int RPP = NT / TPR;               // rows per staging pass
  constexpr int PASSES = (BM + RPP - 1) / RPP;
  constexpr int UNITS = 4 * BN * 4;           // 16-byte weight units per chunk
  constexpr int UPT = (UNITS + NT - 1) / NT;
  static_assert(BK == 16 && SK % 4 == 0, "16-channel chunks, 16-byte aligned rows");

  __shared__ __attribute__((aligned(16))) T lds[4 * A_PLANE + 4 * B_PLANE];
  T* As = lds;
  T* Bs = lds + 4 * A_PLANE;

  const int per_xcd = (n_tiles + 7) / 8;
  const int tile = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (tile >= n_tiles) return;
  const int col_tile = tile % n_col_tiles;
  const int row_tile = tile / n_col_tiles;
  const int m0 = row_tile * BM;
  const int n0 = col_tile * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, g = lane >> 4;
  const int64_t plane = (int64_t)n_pad * k_pad;

  const int halo = src.h * src.W + src.h;
  const int pix0 = m0 - halo > 0 ? m0 - halo : 0;
  const int pix1 = m0 + BM + halo < src.P ? m0 + BM + halo : src.P;
  const __amdgpu_buffer_rsrc_t rf =
      conv_rsrc((const T*)src.f + (int64_t)pix0 * src.Cs * 4,
                (uint32_t)((int64_t)(pix1 - pix0) * src.Cs * 4 * (int)sizeof(T)));

  const int cg = (tid % TPR) * 4;
  int pix[PASSES], pi[PASSES], pj[PASSES];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int row = ps * RPP + tid / TPR;
    const int m = m0 + row;
    const bool ok = row < BM && m < src.P;
    pix[ps] = ok ? m : -1;
    pj[ps] = ok ? m % src.W : 0;
    pi[ps] = ok ? (m / src.W) % src.H : 0;
  }

  PatchQuads<T> qa[PASSES];
  u32x4v qb[UPT];
  int mode = 2;
  auto load_chunk = [&](int k0) {
    int c = 0, ua = 0, ub = 0;
    patch_mode<T>(src, k0 + cg, mode, c, ua, ub);
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps)
      qa[ps] = patch_load<T>(src, rf, pix0, pix[ps], pi[ps], pj[ps], mode, c, ua, ub);
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = i * NT + tid;
      qb[i] = u32x4v{};
      if (UNITS % NT == 0 || u < UNITS) {
        const int p = u / (BN * 4), rem = u % (BN * 4);
        const int j = rem / 4, q = rem % 4;
        // output tiles of 48 channels can reach past the padded planes
        if (n0 + j < n_pad)
          qb[i] = *reinterpret_cast<const u32x4v*>(spec + p * plane + (int64_t)(n0 + j) * k_pad + k0 +
                                                   q * 4);
      }
    }
  };
  auto store_chunk = [&]() {
    typedef typename Elem<T>::quad Q;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int row = ps * RPP + tid / TPR;
      if (BM % RPP != 0 && row >= BM) break;
      T o0[4], o2[4], orr[4], oi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const floatx4 v = patch_vector<T>(qa[ps], mode, e);
        const Spec4 sp = dft4(v[0], v[1], v[2], v[3]);
        o0[e] = sp.f0;
        o2[e] = sp.f2;
        orr[e] = sp.fr;
        oi[e] = sp.fi;
      }
      T* d = As + row * SK + cg;
      *reinterpret_cast<Q*>(d + 0 * A_PLANE) = Q{o0[0], o0[1], o0[2], o0[3]};
      *reinterpret_cast<Q*>(d + 1 * A_PLANE) = Q{o2[0], o2[1], o2[2], o2[3]};
      *reinterpret_cast<Q*>(d + 2 * A_PLANE) = Q{orr[0], orr[1], orr[2], orr[3]};
      *reinterpret_cast<Q*>(d + 3 * A_PLANE) = Q{oi[0], oi[1], oi[2], oi[3]};
    }
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = i * NT + tid;
      if (UNITS % NT == 0 || u < UNITS) {
        const int p = u / (BN * 4), rem = u % (BN * 4);
        const int j = rem / 4, q = rem % 4;
        *reinterpret_cast<u32x4v*>(Bs + p * B_PLANE + j * SK + q * 4) = qb[i];
      }
    }
  };

  // acc[nb][plane]: lane (i16, g) register r is pixel m0 + 16 wave + 4g + r,
  // channel n0 + 16nb + i16 (16x16x4 result layout)
  floatx4 acc[NBN][4];
#pragma unroll
  for (int nb = 0; nb < NBN; ++nb)
#pragma unroll
    for (int pl = 0; pl < 4; ++pl) acc[nb][pl] = floatx4{};

  load_chunk(0);
  for (int k0 = 0; k0 < k_pad; k0 += BK) {
    store_chunk();
    __syncthreads();
    if (k0 + BK < k_pad) load_chunk(k0 + BK);  // in flight during the products

    floatx4 a[4];
#pragma unroll
    for (int pl = 0; pl < 4; ++pl)
      a[pl] = *reinterpret_cast<const floatx4*>(As + pl * A_PLANE + (wave * 16 + i16) * SK + 4 * g);
    floatx4 b[NBN][4];
#pragma unroll
    for (int nb = 0; nb < NBN; ++nb)
#pragma unroll
      for (int pl = 0; pl < 4; ++pl)
        b[nb][pl] = *reinterpret_cast<const floatx4*>(Bs + pl * B_PLANE + (nb * 16 + i16) * SK + 4 * g);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      // Y0 = X0 W0, Y2 = X2 W2, Yr = Xr Wr - Xi Wi, Yi = Xr Wi + Xi Wr; the
      // two products into Yr (and Yi) are issued apart
#pragma unroll
      for (int nb = 0; nb < NBN; ++nb) {
        acc[nb][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0][st], b[nb][0][st], acc[nb][0], 0, 0, 0);
        acc[nb][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1][st], b[nb][1][st], acc[nb][1], 0, 0, 0);
        acc[nb][2] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2][st], b[nb][2][st], acc[nb][2], 0, 0, 0);
        acc[nb][3] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2][st], b[nb][3][st], acc[nb][3], 0, 0, 0);
      }
#pragma unroll
      for (int nb = 0; nb < NBN; ++nb) {
        acc[nb][2] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3][st], -b[nb][3][st], acc[nb][2], 0, 0, 0);
        acc[nb][3] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3][st], b[nb][2][st], acc[nb][3], 0, 0, 0);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int nb = 0; nb < NBN; ++nb) {
    const int col = n0 + nb * 16 + i16;
    if (col >= n_out) continue;
    const float bcol = bias[col];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wave * 16 + 4 * g + r;
      if (row < src.P) {
        floatx4 o = idft4(acc[nb][0][r], acc[nb][1][r], acc[nb][2][r], acc[nb][3][r]);
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] = activate(o[t] + bcol, act);
        *reinterpret_cast<floatx4*>(y + ((int64_t)row * n_out + col) * 4) = o;
      }
    }
  }
}

template <int NBN>
static hipError_t launch_conv32_t(const PatchSrc& src, const float* spec, const float* bias, float* out,
                                  int k_pad, int n_out, int n_pad, int act, hipStream_t s) {
  constexpr int BN = 16 * NBN;
  const int ncol = (n_out + BN - 1) / BN;
  const int64_t nrow = ((int64_t)src.P + 63) / 64;
  const int64_t tiles = nrow * ncol;
  if (tiles > (int64_t)0x7fffffff / 2) return hipErrorInvalidValue;
  const int64_t grid = (tiles + 7) / 8 * 8;
  hipLaunchKernelGGL((k_conv_gemm32<NBN>), dim3((unsigned)grid), dim3(256), 0, s, src, spec, bias, out,
                     k_pad, n_out, n_pad, ncol, (int)tiles, act);
  return hipGetLastError();
}

// Output tiles of 16, 32, 48 or 64 channels: the fewest padded channels,
// then the widest tile.
static hipError_t launch_conv32(const PatchSrc& src, const float* spec, const float* bias, float* out,
                                int k_pad, int n_out, int n_pad, int act, hipStream_t s) {
  int best = 4, waste = 1 << 30;
  for (int nbn = 4; nbn >= 1; --nbn) {
    const int bn = 16 * nbn, wst = (n_out + bn - 1) / bn * bn - n_out;
    if (wst < waste) {
      waste = wst;
      best = nbn;
    }
  }
  switch (best) {
    case 1: return launch_conv32_t<1>(src, spec, bias, out, k_pad, n_out, n_pad, act, s);
    case 2: return launch_conv32_t<2>(src, spec, bias, out, k_pad, n_out, n_pad, act, s);
    case 3: return launch_conv32_t<3>(src, spec, bias, out, k_pad, n_out, n_pad, act, s);
    default: return launch_conv32_t<4>(src, spec, bias, out, k_pad, n_out, n_pad, act, s);
  }
}

// Patches of a binary32 field written out, x'[P][K][4] (the weight-gradient
// operand).  One thread per (pixel, four patch channels): 64 bytes of output,
// consecutive for consecutive threads, staged through LDS so that each of a
// wave's four stores writes 1 KB contiguously (non-temporal: streamed).
template <typename T>
__global__ __launch_bounds__(256) void k_conv_gather(const PatchSrc src, T* __restrict__ xp) {
  static_assert(sizeof(T) == 4, "four binary32 quads per thread");
  __shared__ __attribute__((aligned(16))) floatx4 stage[4][256];
  const int blocks4 = src.K / 4;
  const int64_t total = (int64_t)src.P * blocks4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x & 63, wbase = threadIdx.x & ~63;
  floatx4 out[4] = {};
  if (i < total) {
    const int pix = (int)(i / blocks4);
    const int cp = (int)(i % blocks4) * 4;
    int mode = 2, c = 0, ua = 0, ub = 0;
    patch_mode<T>(src, cp, mode, c, ua, ub);
    const int halo = src.h * src.W + src.h;
    const int pix0 = pix - halo > 0 ? pix - halo : 0;
    const int pix1 = pix + 1 + halo < src.P ? pix + 1 + halo : src.P;
    const __amdgpu_buffer_rsrc_t rf =
        conv_rsrc((const T*)src.f + (int64_t)pix0 * src.Cs * 4,
                  (uint32_t)((int64_t)(pix1 - pix0) * src.Cs * 4 * (int)sizeof(T)));
    const PatchQuads<T> r =
        patch_load<T>(src, rf, pix0, pix, (pix / src.W) % src.H, pix % src.W, mode, c, ua, ub);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = patch_vector<T>(r, mode, e);
  }
  floatx4* const run = &stage[0][0] + wbase * 4;  // the wave's 4 KB in output order
#pragma unroll
  for (int e = 0; e < 4; ++e) run[4 * lane + e] = out[e];
  __syncthreads();
  const int64_t i0 = (int64_t)blockIdx.x * 256 + wbase;
  floatx4* const dst = reinterpret_cast<floatx4*>(xp) + i0 * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int slot = 64 * e + lane;
    if (i0 + slot / 4 < total) __builtin_nontemporal_store(run[slot], &dst[slot]);
  }
}

// Orbit representative o (row-major over rows 1..h, columns 0..h).
__device__ __forceinline__ void orbit_rep(int o, int h, int& ua, int& ub) {
  ua = 1 + o / (h + 1);
  ub = o % (h + 1);
}

// Patch weights of the forward layer, W'[d, cp, m] over [D][Kf][4], and of
// the adjoint layer, W*'[c, cp, m] over [C][Ka][4], one thread per entry:
//     centre:  W'[d, c, m] = psi[d, c, 0, m]
//     orbit:   W'[d, (u, c, e), m] = psi[d, c, R^-m u, (m - e) mod 4]
// and the same for the adjoint filter psi*[c, d, w, r] = psi[d, c, -R^r w,
// (-r) mod 4].  The centre padding gets zeros.
template <typename T>
__global__ __launch_bounds__(256) void k_conv_patch_weights(const T* __restrict__ psi,
                                                            T* __restrict__ wf, T* __restrict__ wa,
                                                            int C, int D, int k) {
  const int h = k / 2;
  const int Kf = patch_width(C, k), Ka = patch_width(D, k);
  const int64_t nf = (int64_t)D * Kf * 4, na = (int64_t)C * Ka * 4;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool adj = i >= nf;
  if (adj) i -= nf;
  if (i >= (adj ? na : nf)) return;
  const int m = (int)(i & 3);
  const int K = adj ? Ka : Kf, Cs = adj ? D : C;  // patch width, gathered channels
  const int cp = (int)((i >> 2) % K);
  const int o_ch = (int)((i >> 2) / K);           // output channel of the patch layer
  int src_ch = 0, wa_ = 0, wb_ = 0, r = 0;
  bool zero = false;
  if (cp < centre_width(Cs)) {
    src_ch = cp;
    zero = cp >= Cs;
    r = m;
  } else {
    const int rem = cp - centre_width(Cs);
    const int o = rem / (4 * Cs);
    src_ch = (rem - o * 4 * Cs) >> 2;
    const int e = rem & 3;
    int ua, ub;
    orbit_rep(o, h, ua, ub);
    turn(ua, ub, (-m) & 3, wa_, wb_);
    r = (m - e) & 3;
  }
  T v = (T)0.f;
  if (!zero) {
    // forward: psi[d = o_ch, c = src_ch, w, r];
    // adjoint: psi*[c = o_ch, d = src_ch, w, r] = psi[d, c, -R^r w, -r]
    int d = o_ch, c = src_ch, pa = wa_, pb = wb_, q = r;
    if (adj) {
      d = src_ch;
      c = o_ch;
      int ta, tb;
      turn(wa_, wb_, r, ta, tb);
      pa = -ta;
      pb = -tb;
      q = (-r) & 3;
    }
    v = psi[((((int64_t)d * C + c) * k + (pa + h)) * k + (pb + h)) * 4 + q];
  }
  (adj ? wa : wf)[i] = v;
}

// Filter gradient from the patch-weight gradient dW' [D][Kf][4] (fp32):
// each filter entry has one place in W' (the inverse of the map of
// k_conv_patch_weights).
__global__ __launch_bounds__(256) void k_conv_fold(const float* __restrict__ dwp,
                                                   float* __restrict__ dpsi, int C, int D, int k) {
  const int64_t total = (int64_t)D * C * k * k * 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int h = k / 2;
  const int q = (int)(i & 3);
  int64_t rest = i >> 2;
  const int b = (int)(rest % k) - h;
  rest /= k;
  const int a = (int)(rest % k) - h;
  rest /= k;
  const int c = (int)(rest % C);
  const int d = (int)(rest / C);
  int cp, m;
  patch_place(c, a, b, q, C, h, cp, m);
  dpsi[i] = dwp[((int64_t)d * patch_width(C, k) + cp) * 4 + m];
}

// ---------------------------------------------------------------------------
// Register-direct binary16 kernel.  A work-group of four waves (one per
// SIMD) owns NB blocks of 16 output channels and walks 16-pixel tiles.  The
// reduction steps (32 patch channels each) are split over the four waves;
// each wave keeps the weight-spectrum fragments of its steps for all NB
// blocks in VGPRs (A operand of v_mfma_f32_16x16x32_f16).  The x operand
// needs no staging: lane (i16, g) of the B fragment of a step is pixel i16
// and 8 consecutive patch channels, whose four group values it loads itself
// (four 16-byte loads: 8 channels of the pixel for a centre step, or 2
// channels of each of the four turned neighbours for an orbit step), so the
// group DFT along the group axis is a butterfly inside the lane.  Loads run
// one step ahead.  At the end of a tile the waves combine their partial
// spectra through LDS; wave b finishes block b (inverse butterfly, bias,
// activation, store).
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ uint32_t pack2h(float a, float b) {
  const f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace

// First reduction step of each of the four waves (and the step count).
struct WaveSplit {
  int start[5];
};

template <int NB, int KSW, bool UNI>
__global__ __launch_bounds__(256, 1) void k_conv_rd_f16(
    const PatchSrc src, const _Float16* __restrict__ spec, const float* __restrict__ bias,
    _Float16* __restrict__ y, const WaveSplit split, int k_pad, int n_out, int n_pad, int n_ranges,
    int n_tiles, int Qx, int act) {
  // partial spectra of every wave: wave x block x plane x lane (f32x4),
  // double buffered
  constexpr int WAVES = 4;
  constexpr int RED = WAVES * NB * 4 * 64;
  __shared__ __attribute__((aligned(16))) f32x4 red[2 * RED];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, g = lane >> 4;
  // work-group -> (channel range j, XCD x, worker w); the XCD's workers take
  // interleaved tiles of one contiguous run, so the halo rows they share
  // stay in that XCD's L2
  const int wgid = blockIdx.x, xcd = wgid & 7, slot = wgid >> 3;
  const int j = slot % n_ranges, w = slot / n_ranges;
  const int per = (n_tiles + 7) / 8;
  const int t_begin = xcd * per + w;
  const int t_end = (xcd + 1) * per < n_tiles ? (xcd + 1) * per : n_tiles;
  const int n_my = t_begin < t_end ? (t_end - t_begin - 1) / Qx + 1 : 0;
  if (n_my == 0) return;  // whole work-group

  // this wave's reduction steps [ks0, ks0 + cnt), 1 <= cnt <= KSW (host
  // split, balanced against the end-of-tile work of the finishing waves)
  const int ks0 = split.start[wave], cnt = split.start[wave + 1] - ks0;
  const int d0 = j * NB * 16;

  // weight fragments: channel d0 + 16nb + i16, patch channels 32s + 8g .. + 7
  half8 w0[NB][KSW], w2[NB][KSW], wr[NB][KSW], wi[NB][KSW];
  {
    const uint32_t plane_bytes = (uint32_t)n_pad * k_pad * 2;
    const int64_t plane = (int64_t)n_pad * k_pad;
    const __amdgpu_buffer_rsrc_t r0 = conv_rsrc(spec, plane_bytes), r2 = conv_rsrc(spec + plane, plane_bytes);
    const __amdgpu_buffer_rsrc_t rr = conv_rsrc(spec + 2 * plane, plane_bytes);
    const __amdgpu_buffer_rsrc_t ri = conv_rsrc(spec + 3 * plane, plane_bytes);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int s = 0; s < KSW; ++s) {
        const int row = d0 + nb * 16 + i16;
        const uint32_t off = s < cnt && row < n_pad
                                 ? (uint32_t)(row * k_pad + 32 * (ks0 + s) + 8 * g) * 2
                                 : OOB;
        w0[nb][s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r0, off, 0, 0));
        w2[nb][s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r2, off, 0, 0));
        wr[nb][s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, 0));
        wi[nb][s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(ri, off, 0, 0));
      }
  }

  // bias of the four output channels this lane finishes (wave nb < NB
  // finishes block nb), loaded once instead of in every tile's epilogue
  float bl[4] = {0.f, 0.f, 0.f, 0.f};
  if (wave < NB) {
    const int col = d0 + wave * 16 + 4 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) bl[r] = col + r < n_out ? bias[col + r] : 0.f;
  }

  // per-step constants of this lane's 8 patch channels, packed in one
  // register per step: the source channel (centre steps: first of 8; orbit
  // steps: first of 2) in bits 0-15, the orbit representative in bits 16-18
  // and 19-21, and in bit 22 whether the channels exist (past the patch
  // width they read zeros)
  uint32_t kst[KSW];
#pragma unroll
  for (int s = 0; s < KSW; ++s) {
    const int cp = 32 * (ks0 + s) + 8 * g;
    int ch = 0, ra = 0, rb = 0;
    const bool lv = s < cnt && cp < src.K;
    if (cp < src.Cc) {
      ch = cp;
    } else if (lv) {
      const int rem = cp - src.Cc;
      const int o = rem / (4 * src.Cs);
      ch = (rem - o * 4 * src.Cs) >> 2;  // even
      orbit_rep(o, src.h, ra, rb);
    }
    kst[s] = (uint32_t)ch | ((uint32_t)ra << 16) | ((uint32_t)rb << 19) | ((lv ? 1u : 0u) << 22);
  }
  // With a channel count that is a multiple of 8 (UNI) the patch width is a
  // whole number of steps and every step lies inside the centre segment or
  // inside one orbit for all lanes: its first channel and orbit
  // representative are the same for the whole wave, kept per step in one
  // scalar (channel in bits 0-15, representative in bits 16-19 and 20-23),
  // and the neighbour offsets are scalar arithmetic
  uint32_t ust[KSW];
  if constexpr (UNI) {
#pragma unroll
    for (int s = 0; s < KSW; ++s) {
      const int cp0 = 32 * (ks0 + s);
      int cst = cp0, ua = 0, ub = 0;
      if (cp0 >= src.Cc) {
        const int rem = cp0 - src.Cc;
        const int o = rem / (4 * src.Cs);
        cst = (rem - o * 4 * src.Cs) >> 2;
        orbit_rep(o, src.h, ua, ub);
      }
      ust[s] = (uint32_t)cst | ((uint32_t)ua << 16) | ((uint32_t)ub << 20);
    }
  }

  // tile state of the gather (the gather runs ahead of the products)
  int g_ti = -1, p = 0, pi = 0, pj = 0, lo = 0;
  uint32_t cbase = 0, obase = 0;  // UNI: byte offsets of the lane's centre / orbit channels
  bool pix_ok = false;
  __amdgpu_buffer_rsrc_t rf = conv_rsrc(src.f, 0);
  const int halo = src.h * src.W + src.h;

  // loads of step S of this worker's tile ti; tiles past the end load zeros
  // (an empty resource)
  auto gather = [&](u32x4v (&raw)[4], int ti, auto s_c) {
    constexpr int S = decltype(s_c)::value;
    if (ti != g_ti) {
      g_ti = ti;
      const int t = t_begin + ti * Qx;
      const bool tile_ok = ti < n_my;
      p = t * 16 + i16;
      pix_ok = tile_ok && p < src.P;
      pj = p % src.W;
      pi = (p / src.W) % src.H;
      lo = t * 16 - halo > 0 ? t * 16 - halo : 0;
      const int hi = t * 16 + 16 + halo < src.P ? t * 16 + 16 + halo : src.P;
      rf = conv_rsrc((const _Float16*)src.f + (int64_t)(tile_ok ? lo : 0) * src.Cs * 4,
                     tile_ok && hi > lo ? (uint32_t)((int64_t)(hi - lo) * src.Cs * 8) : 0u);
      if constexpr (UNI) {
        obase = (uint32_t)(((p - lo) * src.Cs + 2 * g) * 8);
        cbase = obase + 48u * (uint32_t)g;
        if (!pix_ok) pi = -(1 << 20);  // every neighbour out of range
      }
    }
    uint32_t off[4];
    if constexpr (UNI) {
      const int cst = (int)(ust[S] & 0xFFFFu);
      if (32 * (ks0 + S) < src.Cc) {
        const bool ok = pix_ok && cst + 8 * g < src.Cs;
        const uint32_t base = cbase + (uint32_t)cst * 8u;
#pragma unroll
        for (int e = 0; e < 4; ++e) off[e] = ok ? base + 16 * e : OOB;
      } else {
        const int ua = (int)((ust[S] >> 16) & 15u), ub = (int)((ust[S] >> 20) & 15u);
        const int row_b = src.W * src.Cs * 8, pix_b = src.Cs * 8;
        const uint32_t base = obase + (uint32_t)cst * 8u;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          int va, vb;
          turn(ua, ub, jj, va, vb);
          const bool in = (unsigned)(pi + va) < (unsigned)src.H && (unsigned)(pj + vb) < (unsigned)src.W;
          off[jj] = in ? base + (uint32_t)(va * row_b + vb * pix_b) : OOB;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) raw[e] = __builtin_amdgcn_raw_buffer_load_b128(rf, off[e], 0, 0);
      return;
    }
    const int c = (int)(kst[S] & 0xFFFFu);
    const int ua = (int)((kst[S] >> 16) & 7u), ub = (int)((kst[S] >> 19) & 7u);
    const bool lv = (kst[S] >> 22) & 1u;
    const uint32_t base = (uint32_t)(((p - lo) * src.Cs + c) * 8);
    if (32 * (ks0 + S) < src.Cc) {
      // centre step: channel pairs c + 2e of the pixel; pairs past Cs are zeros
#pragma unroll
      for (int e = 0; e < 4; ++e) off[e] = pix_ok && c + 2 * e < src.Cs ? base + 16 * e : OOB;
    } else {
      // orbit step: channels c, c + 1 of the four turned neighbours
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        int va, vb;
        turn(ua, ub, jj, va, vb);
        const bool in = (unsigned)(pi + va) < (unsigned)src.H && (unsigned)(pj + vb) < (unsigned)src.W;
        off[jj] = pix_ok && lv && in ? base + (uint32_t)((va * src.W + vb) * src.Cs * 8) : OOB;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) raw[e] = __builtin_amdgcn_raw_buffer_load_b128(rf, off[e], 0, 0);
  };

  // butterfly of two channels' group vectors (a0..a3, b0..b3) into packed
  // binary16 pairs of the scaled planes (X0/4, X2/4, Xr/2, -Xi/2): X0, X2
  // from fp32 pair sums, scaled and rounded once; (Xr, -Xi)/2 =
  // (x0 - x2, x1 - x3)/2 from one packed fused multiply-add
  float one = 1.0f;
  asm volatile("" : "+v"(one));
  auto bfly = [&](const half8& w, uint32_t& o0, uint32_t& o2, uint32_t& orr, uint32_t& oi) {
    const float sa = __builtin_fmaf((float)w[0], one, (float)w[2]);
    const float ta = __builtin_fmaf((float)w[1], one, (float)w[3]);
    const float sb = __builtin_fmaf((float)w[4], one, (float)w[6]);
    const float tb = __builtin_fmaf((float)w[5], one, (float)w[7]);
    o0 = __builtin_bit_cast(uint32_t, f16x2{quarter_h(sa + ta), quarter_h(sb + tb)});
    o2 = __builtin_bit_cast(uint32_t, f16x2{quarter_h(sa - ta), quarter_h(sb - tb)});
    const f16x2 a01 = {w[0], w[1]}, a23 = {w[2], w[3]};
    const f16x2 b01 = {w[4], w[5]}, b23 = {w[6], w[7]};
    const f16x2 da = half_diff(a01, a23), db = half_diff(b01, b23);
    orr = __builtin_bit_cast(uint32_t, f16x2{da[0], db[0]});
    oi = __builtin_bit_cast(uint32_t, f16x2{da[1], db[1]});
  };

  struct Frag {
    half8 x0, x2, xr, xn, xi;  // xn = -Xi, xi = Xi
  };
  // group DFT of step S's loads into the four B fragments
  auto transform = [&](const u32x4v (&raw)[4], auto s_c) {
    constexpr int S = decltype(s_c)::value;
    u32x4v v0, v2, vr, vi;
    if (32 * (ks0 + S) < src.Cc) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t t0, t2, tr, tq;
        bfly(__builtin_bit_cast(half8, raw[e]), t0, t2, tr, tq);
        v0[e] = t0;
        v2[e] = t2;
        vr[e] = tr;
        vi[e] = tq;
      }
    } else {
      // orbit step: patch channels (c, e = 0..3), (c + 1, e = 0..3); the
      // group vector of (ch, e) over the turns jj is neighbour jj's value
      // (jj + e) mod 4 of channel c + ch
      // (ch, e) over the turns jj is neighbour jj's value (jj + e) mod 4 of
      // channel c + ch.  Every sum and difference is one mixed-precision fma
      // on the loaded binary16 halves (no repacking of the loads); the
      // scaled planes X0/4, X2/4, Xr/2, -Xi/2 are rounded once to binary16.
      const half8 L[4] = {__builtin_bit_cast(half8, raw[0]), __builtin_bit_cast(half8, raw[1]),
                          __builtin_bit_cast(half8, raw[2]), __builtin_bit_cast(half8, raw[3])};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int ch = e2 >> 1, ea = 2 * (e2 & 1), eb = ea + 1;
        float a[4], b[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          a[jj] = (float)L[jj][4 * ch + ((jj + ea) & 3)];
          b[jj] = (float)L[jj][4 * ch + ((jj + eb) & 3)];
        }
        const float sa = __builtin_fmaf(a[0], one, a[2]), ta = __builtin_fmaf(a[1], one, a[3]);
        const float sb = __builtin_fmaf(b[0], one, b[2]), tb = __builtin_fmaf(b[1], one, b[3]);
        const float ra = __builtin_fmaf(a[2], -one, a[0]), qa = __builtin_fmaf(a[3], -one, a[1]);
        const float rb = __builtin_fmaf(b[2], -one, b[0]), qb = __builtin_fmaf(b[3], -one, b[1]);
        v0[e2] = __builtin_bit_cast(uint32_t, f16x2{quarter_h(sa + ta), quarter_h(sb + tb)});
        v2[e2] = __builtin_bit_cast(uint32_t, f16x2{quarter_h(sa - ta), quarter_h(sb - tb)});
        vr[e2] = pack2h(ra * SCALE1, rb * SCALE1);
        vi[e2] = pack2h(qa * SCALE1, qb * SCALE1);
      }
    }
    Frag F;
    F.x0 = __builtin_bit_cast(half8, v0);
    F.x2 = __builtin_bit_cast(half8, v2);
    F.xr = __builtin_bit_cast(half8, vr);
    F.xn = __builtin_bit_cast(half8, vi);
    F.xi = __builtin_bit_cast(half8, vi ^ 0x80008000u);
    return F;
  };

  // four accumulators per block: Y0, Y2, Yr = Wr Xr + Wi (-Xi) and
  // Yi = Wi Xr + Wr Xi; the two products into Yr (and Yi) are issued apart
  struct Acc {
    f32x4 c0[NB], c2[NB], cr[NB], ci[NB];
  };
  Acc acc;

  // products of step S; the first step of a tile starts from a zero
  // accumulator operand (no register clearing)
  auto products = [&](const Frag& F, auto s_c) {
    constexpr int S = decltype(s_c)::value;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      acc.c0[nb] = mma16(w0[nb][S], F.x0, S == 0 ? f32x4{} : acc.c0[nb]);
      acc.cr[nb] = mma16(wr[nb][S], F.xr, S == 0 ? f32x4{} : acc.cr[nb]);
      acc.c2[nb] = mma16(w2[nb][S], F.x2, S == 0 ? f32x4{} : acc.c2[nb]);
      acc.ci[nb] = mma16(wi[nb][S], F.xr, S == 0 ? f32x4{} : acc.ci[nb]);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      acc.cr[nb] = mma16(wi[nb][S], F.xn, acc.cr[nb]);
      acc.ci[nb] = mma16(wr[nb][S], F.xi, acc.ci[nb]);
    }
  };

  // end of a tile: combine the waves' partial spectra; wave nb < NB
  // finishes channel block nb
  auto finish = [&](int ti) {
    f32x4* const buf = red + (ti & 1) * RED;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4* const q = buf + ((wave * NB + nb) * 4) * 64 + lane;
      q[0 * 64] = acc.c0[nb];
      q[1 * 64] = acc.c2[nb];
      q[2 * 64] = acc.cr[nb];
      q[3 * 64] = acc.ci[nb];
    }
    __syncthreads();
    if (wave < NB) {
      const int nb = wave;
      f32x4 Y[4];
#pragma unroll
      for (int pl = 0; pl < 4; ++pl) {
        Y[pl] = buf[((0 * NB + nb) * 4 + pl) * 64 + lane];
#pragma unroll
        for (int ww = 1; ww < WAVES; ++ww) Y[pl] += buf[((ww * NB + nb) * 4 + pl) * 64 + lane];
      }
      // lane (i16, g), register r: output channel d0 + 16nb + 4g + r, pixel
      // 16t + i16; the four channels' group vectors are 32 contiguous bytes
      const int t = t_begin + ti * Qx;
      const int px = t * 16 + i16;
      const int col = d0 + nb * 16 + 4 * g;
      if (px < src.P && col < n_out) {
        float v[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const floatx4 o = idft4_bias(Y[0][r], Y[1][r], Y[2][r], Y[3][r], bl[r]);
          v[r][0] = o[0];
          v[r][1] = o[1];
          v[r][2] = o[2];
          v[r][3] = o[3];
        }
        // one uniform branch for the activation, not one per value
        if (act != ACT_NONE) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) v[r][q] = activate(v[r][q], act);
        }
        uint32_t o[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o[2 * r] = pack2h(v[r][0], v[r][1]);
          o[2 * r + 1] = pack2h(v[r][2], v[r][3]);
        }
        u32x4v* const dst = reinterpret_cast<u32x4v*>(y + ((int64_t)px * n_out + col) * 4);
        dst[0] = u32x4v{o[0], o[1], o[2], o[3]};
        dst[1] = u32x4v{o[4], o[5], o[6], o[7]};
      }
    }
  };

  // Software pipeline over this wave's items (tile-major, CNT steps per
  // tile, CNT = cnt fixed at compile time): the products of item i are
  // issued before the butterfly of item i + 1, so the matrix cores work
  // while the same wave runs the butterfly's VALU instructions; loads run
  // two items ahead.  Before item i: F holds its fragments, ring[(i+1)%2]
  // the loads of item i+1 and ring[i%2] those of item i+2.  Tiles are
  // unrolled in pairs so that every ring slot and step index is a
  // compile-time index.
  auto run = [&](auto cnt_c) {
    constexpr int CNT = decltype(cnt_c)::value;
    typedef std::integral_constant<int, 0> s0_t;
    typedef std::integral_constant<int, 1 % CNT> s1_t;
    typedef std::integral_constant<int, 2 % CNT> s2_t;
    u32x4v ring[2][4];
    gather(ring[0], 0, s0_t{});
    gather(ring[1], 1 / CNT, s1_t{});
    Frag F = transform(ring[0], s0_t{});
    gather(ring[0], 2 / CNT, s2_t{});
    auto body = [&](int ti, auto par_c) {
      constexpr int PAR = decltype(par_c)::value;
      static_for<CNT>([&](auto s_c) {
        constexpr int S = decltype(s_c)::value;
        constexpr int I = PAR * CNT + S;  // item index mod 2
        products(F, s_c);
        F = transform(ring[(I + 1) % 2], std::integral_constant<int, (S + 1) % CNT>{});
        if (S == CNT - 1) finish(ti);
        gather(ring[(I + 1) % 2], ti + (S + 3) / CNT, std::integral_constant<int, (S + 3) % CNT>{});
      });
    };
    for (int ti = 0; ti < n_my; ti += 2) {
      body(ti, std::integral_constant<int, 0>{});
      if (ti + 1 < n_my) body(ti + 1, std::integral_constant<int, 1>{});
    }
  };
  static_for<KSW>([&](auto c_c) {
    if (cnt == decltype(c_c)::value + 1) run(std::integral_constant<int, decltype(c_c)::value + 1>{});
  });
}

template <int NB, int KSW, bool UNI>
static hipError_t launch_rd_t(const PatchSrc& src, const _Float16* spec, const float* bias,
                              _Float16* out, int k_pad, int n_out, int n_pad, int act, hipStream_t s) {
  const int KS = (src.K + 31) / 32;
  const int n_ranges = (n_out + NB * 16 - 1) / (NB * 16);
  const int n_tiles = (src.P + 15) / 16;
  const int per = (n_tiles + 7) / 8;
  const int Qx = per < 32 ? per : 32;  // workers per XCD and channel range
  const int64_t grid = (int64_t)8 * Qx * n_ranges;
  // Steps per wave: the contiguous ranges (1 to KSW steps each) that even
  // out the estimated time per tile.  Measured at the stage shape, in units
  // of 1/20 of an orbit step: a centre step costs 15, the end-of-tile work
  // of a wave that finishes a channel block 23 (LDS exchange, inverse
  // butterfly, stores) and 40 more with an activation, of a wave that only
  // hands over its partial spectra 7.
  const int n_centre = src.Cc / 32;
  const int fin = act != ACT_NONE ? 63 : 23;
  auto range_cost = [&](int a, int b, bool finishes) {
    const int nc = (n_centre < b ? n_centre : b) - a;
    const int centre = nc > 0 ? nc : 0;
    return 15 * centre + 20 * (b - a - centre) + (finishes ? fin : 7);
  };
  WaveSplit sp;
  int best = -1;
  for (int a = 1; a <= KSW && a < KS; ++a)
    for (int b = a + 1; b - a <= KSW && b < KS; ++b)
      for (int c = b + 1; c - b <= KSW && c < KS; ++c) {
        if (KS - c > KSW) continue;
        const int bounds[5] = {0, a, b, c, KS};
        int worst = 0;
        for (int w = 0; w < 4; ++w) {
          const int t = range_cost(bounds[w], bounds[w + 1], w < NB);
          worst = t > worst ? t : worst;
        }
        if (best < 0 || worst < best) {
          best = worst;
          for (int w = 0; w < 5; ++w) sp.start[w] = bounds[w];
        }
      }
  if (best < 0) return hipErrorNotSupported;
  hipLaunchKernelGGL((k_conv_rd_f16<NB, KSW, UNI>), dim3((unsigned)grid), dim3(256), 0, s, src, spec, bias,
                     out, sp, k_pad, n_out, n_pad, n_ranges, n_tiles, Qx, act);
  return hipGetLastError();
}

// Register-direct kernel when the steps of a wave fit its weight registers
// (at least four reduction steps, at most 24); hipErrorNotSupported
// otherwise.  A wave takes at most KSW steps, one more than an even share.
static hipError_t launch_rd(const Tuning& tn, const PatchSrc& src, const _Float16* spec,
                            const float* bias, _Float16* out, int k_pad, int n_out, int n_pad,
                            int act, hipStream_t s) {
  if (tn.conv_rd == 0) return hipErrorNotSupported;
  const int KS = (src.K + 31) / 32;
  if (KS < 4) return hipErrorNotSupported;
  // Eight waves (two per SIMD, fewer weight registers each) measured 7x
  // slower at the 448-channel patch width: the compiler spills to scratch
  // within 256 registers.  Four waves, one per SIMD.
  // three channel blocks up to 16 steps (room for one step more than an even
  // share per wave), two blocks up to 24
  const bool uni = src.Cs % 8 == 0;
  switch ((KS + 3) / 4) {
    case 1: return uni ? launch_rd_t<3, 2, true>(src, spec, bias, out, k_pad, n_out, n_pad, act, s)
                   : launch_rd_t<3, 2, false>(src, spec, bias, out, k_pad, n_out, n_pad, act, s);
    case 2: return uni ? launch_rd_t<3, 3, true>(src, spec, bias, out, k_pad, n_out, n_pad, act, s)
                   : launch_rd_t<3, 3, false>(src, spec, bias, out, k_pad, n_out, n_pad, act, s);
    case 3: return uni ? launch_rd_t<3, 4, true>(src, spec, bias, out, k_pad, n_out, n_pad, act, s)
                   : launch_rd_t<3, 4, false>(src, spec, bias, out, k_pad, n_out, n_pad, act, s);
    case 4: return uni ? launch_rd_t<3, 5, true>(src, spec, bias, out, k_pad, n_out, n_pad, act, s)
                   : launch_rd_t<3, 5, false>(src, spec, bias, out, k_pad, n_out, n_pad, act, s);
    case 5: return uni ? launch_rd_t<2, 5, true>(src, spec, bias, out, k_pad, n_out, n_pad, act, s)
                   : launch_rd_t<2, 5, false>(src, spec, bias, out, k_pad, n_out, n_pad, act, s);
    case 6: return uni ? launch_rd_t<2, 6, true>(src, spec, bias, out, k_pad, n_out, n_pad, act, s)
                   : launch_rd_t<2, 6, false>(src, spec, bias, out, k_pad, n_out, n_pad, act, s);
    default: return hipErrorNotSupported;
  }
}

// Patches of a binary16 field written out, x'[P][K][4], one thread per
// (pixel, 8 patch channels): the four 16-byte loads of the register-direct
// kernel's gather.  Consecutive threads own consecutive 64-byte pieces of
// the output, so a wave's 64 pieces are 4 KB in one run; they go through
// LDS so that each of the wave's four stores writes 1 KB contiguously
// instead of 16 bytes every 64.  The patches (k^2 times the field) are
// streamed: non-temporal stores.
__global__ __launch_bounds__(256) void k_conv_gather8_f16(const PatchSrc src,
                                                          _Float16* __restrict__ xp) {
  __shared__ __attribute__((aligned(16))) u32x4v stage[4][256];  // [piece part][thread]
  const int units = src.K / 8;
  const int64_t total = (int64_t)src.P * units;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x & 63, wbase = threadIdx.x & ~63;
  u32x4v out[4] = {};
  if (i < total) {
    const int p = (int)(i / units);
    const int cp = (int)(i - (int64_t)p * units) * 8;
    const int halo = src.h * src.W + src.h;
    const int lo = p - halo > 0 ? p - halo : 0;
    const int hi = p + 1 + halo < src.P ? p + 1 + halo : src.P;
    const __amdgpu_buffer_rsrc_t r = conv_rsrc((const _Float16*)src.f + (int64_t)lo * src.Cs * 4,
                                               (uint32_t)((int64_t)(hi - lo) * src.Cs * 8));
    const bool centre = cp < src.Cc;
    uint32_t off[4];
    if (centre) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        off[e] = cp + 2 * e < src.Cs ? (uint32_t)(((p - lo) * src.Cs + cp + 2 * e) * 8) : OOB;
    } else {
      const int rem = cp - src.Cc;
      const int o = rem / (4 * src.Cs);
      const int c = (rem - o * 4 * src.Cs) >> 2;
      int ua, ub;
      orbit_rep(o, src.h, ua, ub);
      const int pj = p % src.W, pi = (p / src.W) % src.H;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        int va, vb;
        turn(ua, ub, jj, va, vb);
        const bool in = (unsigned)(pi + va) < (unsigned)src.H && (unsigned)(pj + vb) < (unsigned)src.W;
        off[jj] = in ? (uint32_t)(((p + va * src.W + vb - lo) * src.Cs + c) * 8) : OOB;
      }
    }
    u32x4v raw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) raw[e] = __builtin_amdgcn_raw_buffer_load_b128(r, off[e], 0, 0);
    if (centre) {
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = raw[e];
    } else {
      // patch channels (c, e = 0..3), (c + 1, e = 0..3): the group vector
      // of (ch, e) over the turns jj is neighbour jj's value (jj + e) mod 4
      // of channel c + ch
      const half8 L0 = __builtin_bit_cast(half8, raw[0]), L1 = __builtin_bit_cast(half8, raw[1]);
      const half8 L2 = __builtin_bit_cast(half8, raw[2]), L3 = __builtin_bit_cast(half8, raw[3]);
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int ch = e2 >> 1, ea = 2 * (e2 & 1), eb = ea + 1;
        half8 wv;
        wv[0] = L0[4 * ch + ((0 + ea) & 3)];
        wv[1] = L1[4 * ch + ((1 + ea) & 3)];
        wv[2] = L2[4 * ch + ((2 + ea) & 3)];
        wv[3] = L3[4 * ch + ((3 + ea) & 3)];
        wv[4] = L0[4 * ch + ((0 + eb) & 3)];
        wv[5] = L1[4 * ch + ((1 + eb) & 3)];
        wv[6] = L2[4 * ch + ((2 + eb) & 3)];
        wv[7] = L3[4 * ch + ((3 + eb) & 3)];
        out[e2] = __builtin_bit_cast(u32x4v, wv);
      }
    }
  }
  // the wave's output run in LDS in output order (piece part e of thread t
  // at 16-byte slot 4t + e of the wave's 4 KB), read back as four 1 KB rows
  u32x4v* const run = &stage[0][0] + wbase * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) run[4 * lane + e] = out[e];
  __syncthreads();
  const int64_t i0 = (int64_t)blockIdx.x * 256 + wbase;  // first piece of the wave
  u32x4v* const dst = reinterpret_cast<u32x4v*>(xp) + i0 * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int slot = 64 * e + lane;  // 16-byte slot of the wave's run
    if (i0 + slot / 4 < total) __builtin_nontemporal_store(run[slot], &dst[slot]);
  }
}

// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int WM_, int WN_>
static hipError_t launch_conv_t(const PatchSrc& src, const T* spec, const float* bias, T* out,
                                int k_pad, int n_out, int n_pad, int act, hipStream_t s) {
  const int ncol = (n_out + BN - 1) / BN;
  const int64_t nrow = ((int64_t)src.P + BM - 1) / BM;
  const int64_t tiles = nrow * ncol;
  if (tiles > (int64_t)0x7fffffff / 2) return hipErrorInvalidValue;
  const int64_t grid = (tiles + 7) / 8 * 8;
  hipLaunchKernelGGL((k_conv_gemm<T, BM, BN, WM_, WN_>), dim3((unsigned)grid), dim3(64 * WM_ * WN_),
                     0, s, src, spec, bias, out, k_pad, n_out, n_pad, ncol, (int)tiles, act);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_conv_cfg(int cfg, const PatchSrc& src, const T* spec, const float* bias,
                                  T* out, int k_pad, int n_out, int n_pad, int act, hipStream_t s) {
  switch (cfg) {
    case 0: return launch_conv_t<T, 64, 64, 2, 2>(src, spec, bias, out, k_pad, n_out, n_pad, act, s);
    case 1: return launch_conv_t<T, 64, 128, 2, 2>(src, spec, bias, out, k_pad, n_out, n_pad, act, s);
    case 2: return launch_conv_t<T, 128, 64, 2, 2>(src, spec, bias, out, k_pad, n_out, n_pad, act, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv(const Tuning& tn, eqlinear_dtype_t dt, const void* f, int H, int W, int Cs,
                       int k, int64_t P, const void* spec, const float* bias, void* out, int k_pad,
                       int n_out, int n_pad, int act, hipStream_t s) {
  if (P <= 0) return hipSuccess;
  PatchSrc src{f, H, W, Cs, k / 2, centre_width(Cs), patch_width(Cs, k), (int)P};
  // a tile shape set by its knob selects the LDS-tiled kernel
  const bool tiled = tn.conv_tile >= 0;
  const int cfg = tiled ? tn.conv_tile : (n_out <= 64 ? 0 : 1);
  if (dt == EQL_F16) {
    if (!tiled) {
      const hipError_t e = launch_rd(tn, src, (const _Float16*)spec, bias, (_Float16*)out, k_pad,
                                     n_out, n_pad, act, s);
      if (e != hipErrorNotSupported) return e;
    }
    return launch_conv_cfg<_Float16>(cfg, src, (const _Float16*)spec, bias, (_Float16*)out, k_pad,
                                     n_out, n_pad, act, s);
  }
  if (!tiled && tn.conv_f32_16 != 0)
    return launch_conv32(src, (const float*)spec, bias, (float*)out, k_pad, n_out, n_pad, act, s);
  return launch_conv_cfg<float>(cfg, src, (const float*)spec, bias, (float*)out, k_pad, n_out, n_pad,
                                act, s);
}

hipError_t launch_conv_gather(eqlinear_dtype_t dt, const void* f, int H, int W, int Cs, int k,
                              int64_t P, void* xp, hipStream_t s) {
  if (P <= 0) return hipSuccess;
  PatchSrc src{f, H, W, Cs, k / 2, centre_width(Cs), patch_width(Cs, k), (int)P};
  const int64_t n = P * ((src.K + 3) / 4);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (dt == EQL_F16) {
    const int64_t n8 = P * (src.K / 8);
    hipLaunchKernelGGL(k_conv_gather8_f16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, src,
                       (_Float16*)xp);
  } else
    hipLaunchKernelGGL(k_conv_gather<float>, dim3(blocks), dim3(256), 0, s, src, (float*)xp);
  return hipGetLastError();
}

hipError_t launch_conv_patch_weights(eqlinear_dtype_t dt, const void* psi, void* wf, void* wa,
                                     int C, int D, int k, hipStream_t s) {
  const int64_t n = ((int64_t)D * patch_width(C, k) + (int64_t)C * patch_width(D, k)) * 4;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (dt == EQL_F16)
    hipLaunchKernelGGL(k_conv_patch_weights<_Float16>, dim3(blocks), dim3(256), 0, s,
                       (const _Float16*)psi, (_Float16*)wf, (_Float16*)wa, C, D, k);
  else
    hipLaunchKernelGGL(k_conv_patch_weights<float>, dim3(blocks), dim3(256), 0, s, (const float*)psi,
                       (float*)wf, (float*)wa, C, D, k);
  return hipGetLastError();
}

hipError_t launch_conv_fold(const float* dwp, float* dpsi, int C, int D, int k, hipStream_t s) {
  const int64_t n = (int64_t)D * C * k * k * 4;
  hipLaunchKernelGGL(k_conv_fold, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dwp, dpsi, C, D,
                     k);
  return hipGetLastError();
}

}  // namespace eql
