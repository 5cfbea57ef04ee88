// Weight-spectrum precompute: the group DFT of every W[d,c,:] (length 4),
// written once per weight update in the two operand layouts the matrix-core
// kernels read.
//
// Flash EQ-Linear ("Approccio Algoritmico", "Specializzazione per il Gruppo di
// Rotazione p4"): after the DFT along the group axis the convolution becomes a
// product per frequency; the weights are real, so frequency 3 is the
// conjugate of frequency 1 and only {W0, W2, Wr + i Wi} are kept.
//
// Forward operand  (reduction over c):  planes {W0, W2, Wr, Wi}, [D_pad][C_pad]
// Adjoint operand  (reduction over d):  planes {W0, W2, Wr, -Wi} transposed,
//                                       [C_pad][D_pad]  (conj(W)^T per frequency)
// Padding entries are written as zeros, so the GEMM kernels read padded planes
// without bounds checks.
#include "eql_device.h"
#include "eql_internal.h"

namespace eql {

template <typename T>
__global__ __launch_bounds__(256) void k_weight_spectra(
    const T* __restrict__ W, const T* __restrict__ bias, T* __restrict__ spec_fwd,
    T* __restrict__ spec_adj, float* __restrict__ bias_f32, float* __restrict__ zeros_f32,
    int C, int D, int fwd_n, int fwd_k, int adj_n, int adj_k) {
  const int64_t fwd_elems = (int64_t)fwd_n * fwd_k;
  const int64_t adj_elems = (int64_t)adj_n * adj_k;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < fwd_elems) {
    const int d = (int)(i / fwd_k), c = (int)(i % fwd_k);
    Spec4 s = {0.f, 0.f, 0.f, 0.f};
    if (d < D && c < C) {
      const T* w = W + ((int64_t)d * C + c) * 4;
      s = dft4(Elem<T>::to_f(w[0]), Elem<T>::to_f(w[1]), Elem<T>::to_f(w[2]), Elem<T>::to_f(w[3]));
    }
    spec_fwd[0 * fwd_elems + i] = Elem<T>::from_f(s.f0);
    spec_fwd[1 * fwd_elems + i] = Elem<T>::from_f(s.f2);
    spec_fwd[2 * fwd_elems + i] = Elem<T>::from_f(s.fr);
    spec_fwd[3 * fwd_elems + i] = Elem<T>::from_f(s.fi);
    return;
  }
  const int64_t j = i - fwd_elems;
  if (j < adj_elems) {
    const int c = (int)(j / adj_k), d = (int)(j % adj_k);
    Spec4 s = {0.f, 0.f, 0.f, 0.f};
    if (d < D && c < C) {
      const T* w = W + ((int64_t)d * C + c) * 4;
      s = dft4(Elem<T>::to_f(w[0]), Elem<T>::to_f(w[1]), Elem<T>::to_f(w[2]), Elem<T>::to_f(w[3]));
    }
    spec_adj[0 * adj_elems + j] = Elem<T>::from_f(s.f0);
    spec_adj[1 * adj_elems + j] = Elem<T>::from_f(s.f2);
    spec_adj[2 * adj_elems + j] = Elem<T>::from_f(s.fr);
    spec_adj[3 * adj_elems + j] = Elem<T>::from_f(-s.fi);
    return;
  }
  const int64_t k = j - adj_elems;
  if (k < fwd_n) {
    const int d = (int)k;
    bias_f32[d] = (bias != nullptr && d < D) ? Elem<T>::to_f(bias[d]) : 0.f;
    return;
  }
  const int64_t z = k - fwd_n;
  if (z < adj_n) zeros_f32[z] = 0.f;
}

// One operand (four planes [n_pad][k_pad]) rewritten in matrix-core fragment
// order: for plane p, 16-row block b and 32-column step s, the 1 KB fragment
// ((p * n_pad / 16 + b) * k_pad / 32 + s) holds lane l = (i, g) = (l % 16, l / 16)
// at 16 l bytes: row 16 b + i, columns 32 s + 8 g .. + 7.  A wave then loads
// a whole fragment as 1 KB of consecutive 16-byte lanes; in the row-major
// planes its lanes walk 16 rows, which costs the address unit about four
// times as many cycles.  One thread per 16-byte slot.
__global__ __launch_bounds__(256) void k_spectra_frag(const _Float16* __restrict__ spec,
                                                      _Float16* __restrict__ frag, int n_pad, int k_pad) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t plane = (int64_t)n_pad * k_pad;
  if (t >= 4 * plane / 8) return;
  const int l = (int)(t & 63);
  const int64_t f = t >> 6;
  const int ks = k_pad / 32, nblk = n_pad / 16;
  const int s = (int)(f % ks);
  const int b = (int)((f / ks) % nblk);
  const int p = (int)(f / ((int64_t)ks * nblk));
  const _Float16* src = spec + p * plane + (int64_t)(16 * b + (l & 15)) * k_pad + 32 * s + 8 * (l >> 4);
  *reinterpret_cast<u32x4*>(frag + 8 * t) = *reinterpret_cast<const u32x4*>(src);
}

hipError_t launch_spectra(const eqlinear_plan* p, const void* W, const void* bias, hipStream_t s) {
  if (p->cyclic) return cyc::launch_spectra(p, W, bias, s);
  const int64_t total = (int64_t)p->fwd.plane_elems() + (int64_t)p->adj.plane_elems() +
                        p->fwd.n_pad + p->adj.n_pad;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (p->dtype == EQL_F16) {
    hipLaunchKernelGGL(k_weight_spectra<_Float16>, dim3((unsigned)blocks), dim3(threads), 0, s,
                       (const _Float16*)W, (const _Float16*)bias, (_Float16*)p->spec_fwd,
                       (_Float16*)p->spec_adj, p->bias_f32, p->zeros_f32, (int)p->C, (int)p->D,
                       (int)p->fwd.n_pad, (int)p->fwd.k_pad, (int)p->adj.n_pad, (int)p->adj.k_pad);
    if (p->frag_fwd != nullptr) {
      const int64_t nf = 4 * (int64_t)p->fwd.plane_elems() / 8, na = 4 * (int64_t)p->adj.plane_elems() / 8;
      hipLaunchKernelGGL(k_spectra_frag, dim3((unsigned)((nf + 255) / 256)), dim3(256), 0, s,
                         (const _Float16*)p->spec_fwd, (_Float16*)p->frag_fwd, (int)p->fwd.n_pad,
                         (int)p->fwd.k_pad);
      hipLaunchKernelGGL(k_spectra_frag, dim3((unsigned)((na + 255) / 256)), dim3(256), 0, s,
                         (const _Float16*)p->spec_adj, (_Float16*)p->frag_adj, (int)p->adj.n_pad,
                         (int)p->adj.k_pad);
    }
  } else {
    hipLaunchKernelGGL(k_weight_spectra<float>, dim3((unsigned)blocks), dim3(threads), 0, s,
                       (const float*)W, (const float*)bias, (float*)p->spec_fwd,
                       (float*)p->spec_adj, p->bias_f32, p->zeros_f32, (int)p->C, (int)p->D,
                       (int)p->fwd.n_pad, (int)p->fwd.k_pad, (int)p->adj.n_pad, (int)p->adj.k_pad);
  }
  return hipGetLastError();
}

}  // namespace eql
