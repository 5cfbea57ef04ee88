// Device helpers for the cyclic-group kernels: the real DFT of length T
// along the group axis and its inverse, for any group size 2 <= T <= 16.
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
// scalings.  Outputs t and T - t share their cosine part and differ in the
// sign of their sine part.
template <int T, typename R>
__host__ __device__ __forceinline__ void dft_inv(const R (&Q)[T], R (&y)[T]) {
  constexpr int H = NCX<T>;
  static_for<0, T / 2 + 1>([&](auto tt) {
    constexpr int t = decltype(tt)::value;
    R a = cmad<Scaled<T, 1, One>>((R)0, Q[0]);
    if constexpr (HAS_NYQ<T> && (t % 2) == 1) a = cmad<Scaled<T, -1, One>>(a, Q[T - 1]);
    if constexpr (HAS_NYQ<T> && (t % 2) == 0) a = cmad<Scaled<T, 1, One>>(a, Q[T - 1]);
    R b = (R)0;
    static_for<1, H + 1>([&](auto kk) {
      constexpr int k = decltype(kk)::value;
      a = cmad<Scaled<T, 2, Cos<T, k * t>>>(a, Q[2 * k - 1]);
      b = cmad<Scaled<T, -2, Sin<T, k * t>>>(b, Q[2 * k]);
    });
    if constexpr (t == 0 || 2 * t == T) {
      y[t] = a;
    } else {
      y[t] = a + b;
      y[T - t] = a - b;
    }
  });
}

}  // namespace cyc
}  // namespace eql
