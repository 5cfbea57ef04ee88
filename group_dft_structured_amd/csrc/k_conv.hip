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
// Forward kernel: an LDS-tiled spectral GEMM over (pixels x output channels)
// whose reduction operand is gathered from the field.  Per chunk of BK patch
// channels each thread loads the quads of four channels for its rows,
// butterflies them in fp32 and writes the four spectral planes to LDS; the
// weight spectra of the chunk are copied beside them.  The loads of chunk
// i + 1 are issued before the matrix-core work of chunk i.  The epilogue
// applies the inverse butterfly, bias and activation in fp32.
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
  cp = Cs + o * 4 * Cs + 4 * c + e;
}

}  // namespace

// ---------------------------------------------------------------------------
// Gathered operand: the field, its geometry and the patch width.
struct PatchSrc {
  const void* f;  // [P][Cs][4]
  int H, W, Cs;
  int h;  // kernel half-width (k = 2h + 1)
  int K;  // patch channels, k^2 Cs
  int P;  // pixels, N*H*W
};

// Four patch channels starting at cp (a multiple of 4) of one pixel, as four
// raw quads and the mode that turns them into group vectors:
//   mode 0: centre channels cp..cp+3 of the pixel itself, vector e = quad e;
//   mode 1: orbit channels (c, e = 0..3), quad j = f[p + R^j u, c, 0..3],
//           vector e = (quad j element (j + e) mod 4)_j;
//   mode 2: beyond the patch width, zeros.
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
  if (cp >= s.K) {
    mode = 2;
  } else if (cp < s.Cs) {
    mode = 0;
    c = cp;
  } else {
    mode = 1;
    const int rem = cp - s.Cs;
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

// Patches of a field written out, x'[P][K][4] (the weight-gradient operand).
// One thread per (pixel, four patch channels).
template <typename T>
__global__ __launch_bounds__(256) void k_conv_gather(const PatchSrc src, T* __restrict__ xp) {
  typedef typename Elem<T>::quad Q;
  const int blocks4 = (src.K + 3) / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)src.P * blocks4) return;
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
  T* out = xp + ((int64_t)pix * src.K + cp) * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (cp + e < src.K) *reinterpret_cast<Q*>(out + 4 * e) = Elem<T>::pack(patch_vector<T>(r, mode, e));
}

// Patch weights of the forward (W' [D][k^2 C][4]) and of the adjoint layer
// (W*' [C][k^2 D][4], from psi*[c, d, w, r] = psi[d, c, -R^r w, (-r) mod 4]),
// one thread per filter entry psi[d][c][a][b][q]; and the bias copy is left
// to the inner plans.
template <typename T>
__global__ __launch_bounds__(256) void k_conv_patch_weights(const T* __restrict__ psi,
                                                            T* __restrict__ wf, T* __restrict__ wa,
                                                            int C, int D, int k) {
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
  const T v = psi[i];
  int cp, m;
  patch_place(c, a, b, q, C, h, cp, m);
  wf[((int64_t)d * (k * k * C) + cp) * 4 + m] = v;
  // position in the adjoint filter: r = -q, w = -R^q (a, b)
  int ta, tb;
  turn(a, b, q, ta, tb);
  patch_place(d, -ta, -tb, (-q) & 3, D, h, cp, m);
  wa[((int64_t)c * (k * k * D) + cp) * 4 + m] = v;
}

// Filter gradient from the patch-weight gradient dW' [D][k^2 C][4] (fp32):
// each entry has one place in W' (the map of k_conv_patch_weights).
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
  dpsi[i] = dwp[((int64_t)d * (k * k * C) + cp) * 4 + m];
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

hipError_t launch_conv(eqlinear_dtype_t dt, const void* f, int H, int W, int Cs, int k, int64_t P,
                       const void* spec, const float* bias, void* out, int k_pad, int n_out,
                       int n_pad, int act, hipStream_t s) {
  if (P <= 0) return hipSuccess;
  PatchSrc src{f, H, W, Cs, k / 2, k * k * Cs, (int)P};
  int cfg = n_out <= 64 ? 0 : 1;
  const char* env = getenv("EQL_CONV_TILE");
  if (env != nullptr && *env) cfg = atoi(env);
  if (dt == EQL_F16)
    return launch_conv_cfg<_Float16>(cfg, src, (const _Float16*)spec, bias, (_Float16*)out, k_pad,
                                     n_out, n_pad, act, s);
  return launch_conv_cfg<float>(cfg, src, (const float*)spec, bias, (float*)out, k_pad, n_out, n_pad,
                                act, s);
}

hipError_t launch_conv_gather(eqlinear_dtype_t dt, const void* f, int H, int W, int Cs, int k,
                              int64_t P, void* xp, hipStream_t s) {
  if (P <= 0) return hipSuccess;
  PatchSrc src{f, H, W, Cs, k / 2, k * k * Cs, (int)P};
  const int64_t n = P * ((src.K + 3) / 4);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (dt == EQL_F16)
    hipLaunchKernelGGL(k_conv_gather<_Float16>, dim3(blocks), dim3(256), 0, s, src, (_Float16*)xp);
  else
    hipLaunchKernelGGL(k_conv_gather<float>, dim3(blocks), dim3(256), 0, s, src, (float*)xp);
  return hipGetLastError();
}

hipError_t launch_conv_patch_weights(eqlinear_dtype_t dt, const void* psi, void* wf, void* wa,
                                     int C, int D, int k, hipStream_t s) {
  const int64_t n = (int64_t)D * C * k * k * 4;
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
