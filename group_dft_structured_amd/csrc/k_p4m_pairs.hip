// p4m (the dihedral group D_4) on the p4 kernels, by pairing channels.
//
// With the group index g = 4m + r of rho^r sigma^m, a p4m tensor
// [N][C][8] is, byte for byte, a p4 tensor [N][2C][4] whose channel 2c + m
// holds coset m (rotations m = 0, reflections m = 1) of channel c.  Splitting
// the group convolution y[g] = sum_h W[h^-1 g] x[h] by cosets (h^-1 g for
// h = rho^s sigma^mh, g = rho^t sigma^mg is rho^(t-s) sigma^mg when mh = 0
// and rho^(s-t) sigma^(1-mg) when mh = 1) gives a p4 layer on the paired
// channels:
//     y_0 = conv(W_0, x_0) + conv(rev W_1, x_1)
//     y_1 = conv(W_1, x_0) + conv(rev W_0, x_1)
// with W_m[r] = W[4m + r], (rev V)[r] = V[(-r) mod 4] and conv the p4
// circular convolution.  The paired weight is therefore
//     W'[2d + mo][2c + mi][r] = W[d][c][src(mo, mi, r)],
//     src = 4 mo + r (mi = 0),  4 (1 - mo) + (-r mod 4) (mi = 1),
// and the bias b'[2d + m] = b[d].  The weight gradient folds back as the sum
// of every paired entry that holds a given W[d][c][u]:
//     dW[d][c][r]     = dW'[2d][2c][r]     + dW'[2d+1][2c+1][-r mod 4]
//     dW[d][c][4 + r] = dW'[2d+1][2c][r]   + dW'[2d][2c+1][-r mod 4]
//     dbias[d]        = dbias'[2d] + dbias'[2d+1].
// This spends 24 real products per (n, c, d) where the group Fourier
// transform spends 12, on the tuned p4 kernels; binary16 p4m at moderate
// widths is bound by HBM bytes, not by the matrix cores, so it is the faster
// path there (the library selects it by shape; the generic kernels serve the
// rest).
#include "eql_internal.h"

namespace eql {

namespace {

__global__ __launch_bounds__(256) void k_p4m_pair_weight(const _Float16* __restrict__ W,
                                                         const _Float16* __restrict__ bias,
                                                         _Float16* __restrict__ Wp,
                                                         _Float16* __restrict__ bp, int C, int D) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)16 * C * D;  // [2D][2C][4]
  if (i < total) {
    const int r = (int)(i & 3);
    const int64_t dc = i >> 2;
    const int cp = (int)(dc % (2 * C)), dp = (int)(dc / (2 * C));
    const int c = cp >> 1, mi = cp & 1, d = dp >> 1, mo = dp & 1;
    const int src = mi == 0 ? 4 * mo + r : 4 * (1 - mo) + ((4 - r) & 3);
    Wp[i] = W[((int64_t)d * C + c) * 8 + src];
  } else if (i < total + 2 * D) {
    const int dp = (int)(i - total);
    bp[dp] = bias != nullptr ? bias[dp >> 1] : (_Float16)0.f;
  }
}

__global__ __launch_bounds__(256) void k_p4m_fold(const float* __restrict__ dWp,
                                                  const float* __restrict__ dbp,
                                                  float* __restrict__ dW,
                                                  float* __restrict__ dbias, int C, int D) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)8 * C * D;  // [D][C][8]
  if (i < total) {
    const int g = (int)(i & 7);
    const int64_t dc = i >> 3;
    const int c = (int)(dc % C), d = (int)(dc / C);
    const int m = g >> 2, r = g & 3, rn = (4 - r) & 3;
    const int64_t C2 = 2 * (int64_t)C;
    // paired entry [dp][cp][r] at (dp * 2C + cp) * 4 + r
    auto at = [&](int dp, int cp, int rr) { return dWp[((int64_t)dp * C2 + cp) * 4 + rr]; };
    dW[i] = m == 0 ? at(2 * d, 2 * c, r) + at(2 * d + 1, 2 * c + 1, rn)
                   : at(2 * d + 1, 2 * c, r) + at(2 * d, 2 * c + 1, rn);
  } else if (dbias != nullptr && i < total + D) {
    const int d = (int)(i - total);
    dbias[d] = dbp[2 * d] + dbp[2 * d + 1];
  }
}

}  // namespace

hipError_t launch_p4m_pair_weight(const void* W, const void* bias, void* Wp, void* bp, int64_t C,
                                  int64_t D, hipStream_t s) {
  const int64_t n = 16 * C * D + 2 * D;
  hipLaunchKernelGGL(k_p4m_pair_weight, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const _Float16*)W, (const _Float16*)bias, (_Float16*)Wp, (_Float16*)bp, (int)C,
                     (int)D);
  return hipGetLastError();
}

hipError_t launch_p4m_fold(const float* dWp, const float* dbp, float* dW, float* dbias, int64_t C,
                           int64_t D, hipStream_t s) {
  const int64_t n = 8 * C * D + D;
  hipLaunchKernelGGL(k_p4m_fold, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dWp, dbp, dW,
                     dbias, (int)C, (int)D);
  return hipGetLastError();
}

}  // namespace eql
