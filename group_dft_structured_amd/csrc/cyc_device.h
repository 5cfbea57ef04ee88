// Device helpers for the generic group kernels: the real DFT of length T
// along the group axis and its inverse, for any group size 2 <= T <= 16, and
// the group descriptors (cyclic C_T, dihedral D_n) built on it.
//
// Flash EQ-Linear, "Approccio Algoritmico": the EQ-Linear layer is a
// circular convolution along the group axis composed with a linear map
// along the channels, so after a DFT of length T along the group axis it
// becomes one product per frequency.  Inputs and weights are real, so
// frequency T - k is the conjugate of frequency k and only k <= T/2 is kept.
// With omega = exp(-2 pi i / T) and X[k] = sum_s x[s] omega^(k s), the kept
// frequencies are stored as T real planes:
//     plane 0          X[0]                      (real)
//     planes 2k-1, 2k  Re X[k], Im X[k]          for 1 <= k < T - k
//     plane T-1        X[T/2]                    (real, even T only)
// and the inverse, written with the kept frequencies only, is
//     y[t] = (1/T) (Y[0] + (-1)^t Y[T/2] + 2 sum_k Re(Y[k] omega^(-k t))).
// For T = 4 this is the p4 specialisation of the same pages (the
// coefficients reduce to 0, +-1, +-1/2, +-1/4).
//
// Every coefficient is a compile-time constant: the loops below run over
// std::integral_constant indices, and terms whose coefficient is 0 or +-1
// compile to nothing or to a plain add.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace eql {
namespace cyc {

constexpr int TMAX = 16;

// number of complex frequencies kept (1 <= k < T - k)
template <int T>
constexpr int NCX = (T - 1) / 2;
template <int T>
constexpr bool HAS_NYQ = (T % 2) == 0;
// real matrix products per row, channel pair: one per real frequency, four
// per complex frequency
template <int T>
constexpr int PRODUCTS = 1 + 4 * NCX<T> + (HAS_NYQ<T> ? 1 : 0);

// ---- twiddles evaluated at compile time -----------------------------------
constexpr double kPi = 3.14159265358979323846264338327950288;

// Taylor series on [0, pi/2]; 30 terms are far below double rounding there.
constexpr double cos_q(double x) {
  double t = 1.0, s = 1.0;
  for (int n = 1; n < 30; ++n) {
    t *= -x * x / ((2.0 * n - 1.0) * (2.0 * n));
    s += t;
  }
  return s;
}
constexpr double sin_q(double x) {
  double t = x, s = x;
  for (int n = 1; n < 30; ++n) {
    t *= -x * x / ((2.0 * n) * (2.0 * n + 1.0));
    s += t;
  }
  return s;
}
// cos(2 pi m / T), reduced by quarter turns in integers so that the axes give
// exactly 0 and +-1
constexpr double cos_turn(int m, int T) {
  m %= T;
  if (m < 0) m += T;
  const int q = (4 * m) / T, r = 4 * m - q * T;
  const double b = kPi / 2.0 * r / T;
  return q == 0 ? cos_q(b) : q == 1 ? -sin_q(b) : q == 2 ? -cos_q(b) : sin_q(b);
}
// sin(2 pi m / T) = cos(2 pi m / T - pi / 2)
constexpr double sin_turn(int m, int T) { return cos_turn(4 * m - T, 4 * T); }

template <int T, int M>
struct Cos {
  static constexpr double value = cos_turn(M, T);
};
template <int T, int M>
struct Sin {
  static constexpr double value = sin_turn(M, T);
};
// a coefficient scaled by A/T (the inverse uses 1/T and 2/T)
template <int T, int A, typename CT>
struct Scaled {
  static constexpr double value = CT::value * A / T;
};
template <typename CT>
struct Neg {
  static constexpr double value = -CT::value;
};
struct One {
  static constexpr double value = 1.0;
};

// acc + c * v with c a compile-time constant (float or double arithmetic)
template <typename CT, typename R>
__host__ __device__ __forceinline__ R cmad(R acc, R v) {
  constexpr R c = (R)CT::value;
  if constexpr (c == (R)0) {
    return acc;
  } else if constexpr (c == (R)1) {
    return acc + v;
  } else if constexpr (c == (R)-1) {
    return acc - v;
  } else if constexpr (std::is_same<R, float>::value) {
    return __builtin_fmaf(c, v, acc);
  } else {
    return __builtin_fma(c, v, acc);
  }
}

template <int I, int N, typename F>
__host__ __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Forward real DFT of one group vector into the T kept planes.  Inputs at s
// and T - s are paired first (their cosines agree and their sines differ in
// sign), which halves the products.
template <int T, typename R>
__host__ __device__ __forceinline__ void dft_fwd(const R (&x)[T], R (&X)[T]) {
  constexpr int H = NCX<T>;
  R u[H + 1], v[H + 1];
  static_for<1, H + 1>([&](auto ss) {
    constexpr int s = decltype(ss)::value;
    u[s] = x[s] + x[T - s];
    v[s] = x[s] - x[T - s];
  });
  // frequency 0
  R a = x[0];
  if constexpr (HAS_NYQ<T>) a = a + x[T / 2];
  static_for<1, H + 1>([&](auto ss) { a = a + u[decltype(ss)::value]; });
  X[0] = a;
  static_for<1, H + 1>([&](auto kk) {
    constexpr int k = decltype(kk)::value;
    R re = x[0];
    if constexpr (HAS_NYQ<T> && (k % 2) == 1) re = re - x[T / 2];
    if constexpr (HAS_NYQ<T> && (k % 2) == 0) re = re + x[T / 2];
    R im = (R)0;
    static_for<1, H + 1>([&](auto ss) {
      constexpr int s = decltype(ss)::value;
      re = cmad<Cos<T, k * s>>(re, u[s]);
      im = cmad<Neg<Sin<T, k * s>>>(im, v[s]);
    });
    X[2 * k - 1] = re;
    X[2 * k] = im;
  });
  if constexpr (HAS_NYQ<T>) {
    R n = x[0];
    if constexpr ((T / 2) % 2 == 1) n = n - x[T / 2];
    if constexpr ((T / 2) % 2 == 0) n = n + x[T / 2];
    static_for<1, H + 1>([&](auto ss) {
      constexpr int s = decltype(ss)::value;
      if constexpr (s % 2 == 1) n = n - u[s];
      if constexpr (s % 2 == 0) n = n + u[s];
    });
    X[T - 1] = n;
  }
}

// Inverse: the T kept planes back to T group values, with the 1/T and 2/T
// scalings times MUL (a power of two that undoes the plane scalings of the
// operands).  Outputs t and T - t share their cosine part and differ in the
// sign of their sine part.
template <int T, typename R, int MUL = 1>
__host__ __device__ __forceinline__ void dft_inv(const R (&Q)[T], R (&y)[T]) {
  constexpr int H = NCX<T>;
  static_for<0, T / 2 + 1>([&](auto tt) {
    constexpr int t = decltype(tt)::value;
    R a = cmad<Scaled<T, MUL, One>>((R)0, Q[0]);
    if constexpr (HAS_NYQ<T> && (t % 2) == 1) a = cmad<Scaled<T, -MUL, One>>(a, Q[T - 1]);
    if constexpr (HAS_NYQ<T> && (t % 2) == 0) a = cmad<Scaled<T, MUL, One>>(a, Q[T - 1]);
    R b = (R)0;
    static_for<1, H + 1>([&](auto kk) {
      constexpr int k = decltype(kk)::value;
      a = cmad<Scaled<T, 2 * MUL, Cos<T, k * t>>>(a, Q[2 * k - 1]);
      b = cmad<Scaled<T, -2 * MUL, Sin<T, k * t>>>(b, Q[2 * k]);
    });
    if constexpr (t == 0 || 2 * t == T) {
      y[t] = a;
    } else {
      y[t] = a + b;
      y[T - t] = a - b;
    }
  });
}

// Plane scaling of a group of order n: 2^-ceil(log2 n).  Every transform
// plane of a vector of n values is a signed sum of them with coefficients of
// modulus at most 1, so the scaled planes are bounded by the largest input
// magnitude and no binary16 plane overflows while its inputs are finite.
// Both operands of every product carry the scaling (input planes and weight
// spectra; upstream-gradient and input planes in the weight gradient), so
// the inverse multiplies by 1/scale^2, a power of two (exact).
constexpr double plane_scale(int n) {
  double s = 1.0;
  for (int m = 1; m < n; m *= 2) s *= 0.5;
  return s;
}
constexpr int inverse_mul(int n) {
  int v = 1;
  for (int m = 1; m < n; m *= 2) v *= 4;
  return v;
}

// ---- group descriptors ------------------------------------------------------
// The kernels of k_cyclic.hip are written once over a descriptor G that
// gives the group order T (values per group vector and spectral planes),
// the forward transform of one group vector into its T planes, their
// scaling (scale), the inverse of products of two scaled operands (with the
// 1/|G| scalings), the plane map of the adjoint spectrum, and the
// matrix-core products of the forward (input planes times weight planes)
// and of the weight gradient (upstream-gradient planes against input
// planes, summed over rows).  Each product step takes a functor
// mma(a, b, c) = c + a b over fragments of the two operands (and neg(a) =
// -a), so the same schedule serves matrix-core fragments and scalars.

// Cyclic group C_T: the real DFT above.  Frequency k > 0 below T/2 is a
// complex product (Xr + i Xi)(Wr + i Wi), four real products; the adjoint
// spectrum is the complex conjugate (imaginary planes negated).
template <int TT>
struct Cyclic {
  static constexpr int T = TT;
  static constexpr int PRODUCTS = 1 + 4 * NCX<T> + (HAS_NYQ<T> ? 1 : 0);
  template <typename R>
  static __host__ __device__ __forceinline__ void fwd(const R (&x)[T], R (&X)[T]) {
    dft_fwd<T, R>(x, X);
  }
  template <typename R>
  static __host__ __device__ __forceinline__ void scale(R (&X)[T]) {
    static_for<0, T>([&](auto jj) { X[decltype(jj)::value] *= (R)plane_scale(T); });
  }
  template <typename R>
  static __host__ __device__ __forceinline__ void inv(const R (&Q)[T], R (&y)[T]) {
    dft_inv<T, R, inverse_mul(T)>(Q, y);
  }
  static constexpr __host__ __device__ int adj_src(int j) { return j; }
  static constexpr __host__ __device__ bool adj_neg(int j) {
    return j >= 2 && j <= 2 * NCX<T> && (j % 2) == 0;
  }
  // c += A W per frequency; the minus sign of the real part is a sign flip of
  // the imaginary input fragment (neg)
  template <typename Acc, typename Frag, typename Mma, typename Neg>
  static __host__ __device__ __forceinline__ void fwd_mma(Acc (&c)[T], const Frag (&a)[T],
                                                          const Frag (&b)[T], Mma mma, Neg neg) {
    c[0] = mma(a[0], b[0], c[0]);
    static_for<1, NCX<T> + 1>([&](auto kk) {
      constexpr int k = decltype(kk)::value, re = 2 * k - 1, im = 2 * k;
      // (Xr + i Xi)(Wr + i Wi) = (Xr Wr - Xi Wi) + i (Xr Wi + Xi Wr)
      c[re] = mma(a[re], b[re], c[re]);
      c[re] = mma(neg(a[im]), b[im], c[re]);
      c[im] = mma(a[re], b[im], c[im]);
      c[im] = mma(a[im], b[re], c[im]);
    });
    if constexpr (HAS_NYQ<T>) c[T - 1] = mma(a[T - 1], b[T - 1], c[T - 1]);
  }
  // c += G conj(X) per frequency (the weight gradient before the inverse)
  template <typename Acc, typename Frag, typename Mma, typename Neg>
  static __host__ __device__ __forceinline__ void bw_mma(Acc (&c)[T], const Frag (&g)[T],
                                                         const Frag (&x)[T], Mma mma, Neg neg) {
    c[0] = mma(g[0], x[0], c[0]);
    static_for<1, NCX<T> + 1>([&](auto kk) {
      constexpr int k = decltype(kk)::value, re = 2 * k - 1, im = 2 * k;
      // G conj(X) = (Gr Xr + Gi Xi) + i (Gi Xr - Gr Xi)
      c[re] = mma(g[re], x[re], c[re]);
      c[re] = mma(g[im], x[im], c[re]);
      c[im] = mma(g[im], x[re], c[im]);
      c[im] = mma(neg(g[re]), x[im], c[im]);
    });
    if constexpr (HAS_NYQ<T>) c[T - 1] = mma(g[T - 1], x[T - 1], c[T - 1]);
  }
};

// Dihedral group D_n of order T = 2n, elements rho^r sigma^m at index
// m n + r (rho the rotation by 2 pi / n, sigma a reflection,
// sigma rho sigma = rho^-1), read as the reflection groups the pages name as
// the next step ("Limitazioni e Lavoro Futuro"; p4m is D_4).  The layer is
// the group convolution y[g] = sum_h W[h^-1 g] x[h]; its group Fourier
// transform over the real irreducible representations pi,
// x^(pi) = sum_h x[h] pi(h), turns it into y^(pi) = x^(pi) W^(pi):
//  * one-dimensional representations rho -> a, sigma -> b with a = +-1 (-1
//    only for even n) and b = +-1: one real product each;
//  * two-dimensional pi_k (1 <= k <= (n-1)/2): rho -> rotation by
//    2 pi k / n, sigma -> diag(1, -1); a 2 x 2 block product, eight real
//    products.
// Both transforms need the length-n DFT of the two cosets only:
// sum_r u[r] pi_k(rho^r) = [[a, -b], [b, a]] with a + i(-b) the DFT of u at
// k, and the reflection coset is multiplied by diag(1, -1) on the right.
// Planes: 0: (+,+) = S0 + S1, 1: (+,-) = S0 - S1, and for even n 2: (-,+) =
// A0 + A1, 3: (-,-) = A0 - A1 (S_m, A_m the DFT of coset m at 0 and n/2);
// then four planes per pi_k, the block entries 00, 01, 10, 11.  The
// inversion y[g] = (1/2n) sum_pi dim(pi) tr(y^(pi) pi(g)^T) is, per coset,
// a length-n inverse DFT of combined planes.
template <int NN>
struct Dihedral {
  static constexpr int n = NN, T = 2 * NN;
  static constexpr int N1 = (NN % 2 == 0) ? 4 : 2;  // one-dimensional representations
  static constexpr int N2 = (NN - 1) / 2;            // two-dimensional representations
  static constexpr int PRODUCTS = N1 + 8 * N2;
  template <typename R>
  static __host__ __device__ __forceinline__ void fwd(const R (&x)[T], R (&X)[T]) {
    R u0[n], u1[n], U0[n], U1[n];
    static_for<0, n>([&](auto ss) {
      constexpr int s = decltype(ss)::value;
      u0[s] = x[s];
      u1[s] = x[n + s];
    });
    dft_fwd<n, R>(u0, U0);
    dft_fwd<n, R>(u1, U1);
    X[0] = U0[0] + U1[0];
    X[1] = U0[0] - U1[0];
    if constexpr (n % 2 == 0) {
      X[2] = U0[n - 1] + U1[n - 1];
      X[3] = U0[n - 1] - U1[n - 1];
    }
    static_for<1, N2 + 1>([&](auto kk) {
      constexpr int k = decltype(kk)::value, p = N1 + 4 * (k - 1);
      // a_m = Re U_m[k], b_m = -Im U_m[k]
      X[p] = U0[2 * k - 1] + U1[2 * k - 1];       // a0 + a1
      X[p + 1] = U0[2 * k] - U1[2 * k];           // -b0 + b1
      X[p + 2] = -(U0[2 * k] + U1[2 * k]);        // b0 + b1
      X[p + 3] = U0[2 * k - 1] - U1[2 * k - 1];   // a0 - a1
    });
  }
  template <typename R>
  static __host__ __device__ __forceinline__ void scale(R (&X)[T]) {
    static_for<0, T>([&](auto jj) { X[decltype(jj)::value] *= (R)plane_scale(T); });
  }
  template <typename R>
  static __host__ __device__ __forceinline__ void inv(const R (&Q)[T], R (&y)[T]) {
    const R h = (R)(0.5 * inverse_mul(T));
    R V0[n], V1[n], y0[n], y1[n];
    V0[0] = (Q[0] + Q[1]) * h;
    V1[0] = (Q[0] - Q[1]) * h;
    if constexpr (n % 2 == 0) {
      V0[n - 1] = (Q[2] + Q[3]) * h;
      V1[n - 1] = (Q[2] - Q[3]) * h;
    }
    static_for<1, N2 + 1>([&](auto kk) {
      constexpr int k = decltype(kk)::value, p = N1 + 4 * (k - 1);
      // rotation coset: tr(Y R^T) = cos (Y00 + Y11) + sin (Y10 - Y01);
      // reflection coset: tr(Y (R F)^T) = cos (Y00 - Y11) + sin (Y01 + Y10)
      V0[2 * k - 1] = (Q[p] + Q[p + 3]) * h;
      V0[2 * k] = (Q[p + 1] - Q[p + 2]) * h;
      V1[2 * k - 1] = (Q[p] - Q[p + 3]) * h;
      V1[2 * k] = -(Q[p + 1] + Q[p + 2]) * h;
    });
    dft_inv<n, R>(V0, y0);
    dft_inv<n, R>(V1, y1);
    static_for<0, n>([&](auto ss) {
      constexpr int s = decltype(ss)::value;
      y[s] = y0[s];
      y[n + s] = y1[s];
    });
  }
  // adjoint (transposed) layer: W*[c, d, v] = W[d, c, v^-1] has spectrum
  // W^(pi)^T, so the off-diagonal block entries swap
  static constexpr __host__ __device__ int adj_src(int j) {
    return j < N1 ? j : ((j - N1) % 4 == 1 ? j + 1 : (j - N1) % 4 == 2 ? j - 1 : j);
  }
  static constexpr __host__ __device__ bool adj_neg(int) { return false; }
  // c += x^ W^ per representation
  template <typename Acc, typename Frag, typename Mma, typename Neg>
  static __host__ __device__ __forceinline__ void fwd_mma(Acc (&c)[T], const Frag (&a)[T],
                                                          const Frag (&b)[T], Mma mma, Neg) {
    static_for<0, N1>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      c[j] = mma(a[j], b[j], c[j]);
    });
    static_for<1, N2 + 1>([&](auto kk) {
      constexpr int p = N1 + 4 * (decltype(kk)::value - 1);
      c[p] = mma(a[p], b[p], c[p]);                  // Y00 = X00 W00 + X01 W10
      c[p] = mma(a[p + 1], b[p + 2], c[p]);
      c[p + 1] = mma(a[p], b[p + 1], c[p + 1]);      // Y01 = X00 W01 + X01 W11
      c[p + 1] = mma(a[p + 1], b[p + 3], c[p + 1]);
      c[p + 2] = mma(a[p + 2], b[p], c[p + 2]);      // Y10 = X10 W00 + X11 W10
      c[p + 2] = mma(a[p + 3], b[p + 2], c[p + 2]);
      c[p + 3] = mma(a[p + 2], b[p + 1], c[p + 3]);  // Y11 = X10 W01 + X11 W11
      c[p + 3] = mma(a[p + 3], b[p + 3], c[p + 3]);
    });
  }
  // c += x^(pi)^T g^(pi) per representation: the spectrum of the weight
  // gradient, sum_h x[h] pi(h)^T times sum_v dy[v] pi(v)
  template <typename Acc, typename Frag, typename Mma, typename Neg>
  static __host__ __device__ __forceinline__ void bw_mma(Acc (&c)[T], const Frag (&g)[T],
                                                         const Frag (&x)[T], Mma mma, Neg) {
    static_for<0, N1>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      c[j] = mma(g[j], x[j], c[j]);
    });
    static_for<1, N2 + 1>([&](auto kk) {
      constexpr int p = N1 + 4 * (decltype(kk)::value - 1);
      c[p] = mma(g[p], x[p], c[p]);                  // P00 = X00 G00 + X10 G10
      c[p] = mma(g[p + 2], x[p + 2], c[p]);
      c[p + 1] = mma(g[p + 1], x[p], c[p + 1]);      // P01 = X00 G01 + X10 G11
      c[p + 1] = mma(g[p + 3], x[p + 2], c[p + 1]);
      c[p + 2] = mma(g[p], x[p + 1], c[p + 2]);      // P10 = X01 G00 + X11 G10
      c[p + 2] = mma(g[p + 2], x[p + 3], c[p + 2]);
      c[p + 3] = mma(g[p + 1], x[p + 1], c[p + 3]);  // P11 = X01 G01 + X11 G11
      c[p + 3] = mma(g[p + 3], x[p + 3], c[p + 3]);
    });
  }
};

}  // namespace cyc
}  // namespace eql
