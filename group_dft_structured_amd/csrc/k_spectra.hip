// Weight-spectrum precompute: the group DFT of every W[d,c,:] (length 4),
// written once per weight update in the two operand layouts the matrix-core
// kernels read, and for p4 plans also in the fragment order of the
// producer/consumer kernels (binary16: both operands; binary32: the forward
// operand).
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

// Position of plane element (row, col) of an [n_pad][k_pad] plane in
// matrix-core fragment order: for 16-row block b and 32-column step s the
// 1 KB fragment (b * k_pad / 32 + s) holds lane l = (i, g) = (l % 16, l / 16)
// at 16 l bytes: row 16 b + i and k-slice g of the step, which holds the
// column pairs g, g + 4, g + 8, g + 12 (the reduction order the
// producer/consumer kernels stage x in; k_fwd_ws.hip).  A wave then loads a
// whole fragment as 1 KB of consecutive 16-byte lanes; in the row-major
// planes its lanes walk 16 rows, which costs the address unit about four
// times as many cycles.
__device__ __forceinline__ int64_t frag_index(int row, int col, int k_pad) {
  const int b = row >> 4, i = row & 15, s = col >> 5;
  const int q = (col & 31) >> 1;           // column pair within the step
  const int g = q & 3, e = ((q >> 2) << 1) | (col & 1);
  return ((int64_t)b * (k_pad >> 5) + s) * 512 + (g * 16 + i) * 8 + e;
}

// The binary32 operand of k_fwd_ws32.hip in fragment order: for 16-row block
// b and 16-column block jb, the 1 KB fragment (b * k_pad / 16 + jb) holds lane
// l = (i, g) at 16 l bytes: row 16 b + i and the columns g, g + 4, g + 8,
// g + 12 of the block (the reduction order that kernel stages x in).
__device__ __forceinline__ int64_t frag_index32(int row, int col, int k_pad) {
  const int b = row >> 4, i = row & 15, jb = col >> 4, c = col & 15;
  return ((int64_t)b * (k_pad >> 4) + jb) * 256 + ((c & 3) * 16 + i) * 4 + (c >> 2);
}

template <typename T>
__device__ __forceinline__ int64_t frag_pos(int row, int col, int k_pad) {
  if constexpr (sizeof(T) == 2) return frag_index(row, col, k_pad);
  else return frag_index32(row, col, k_pad);
}

template <typename T>
__global__ __launch_bounds__(256) void k_weight_spectra(
    const T* __restrict__ W, const T* __restrict__ bias, T* __restrict__ spec_fwd,
    T* __restrict__ spec_adj, T* __restrict__ frag_fwd, T* __restrict__ frag_adj,
    float* __restrict__ bias_f32, float* __restrict__ zeros_f32,
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
    if (frag_fwd != nullptr) {
      const int64_t f = frag_pos<T>(d, c, fwd_k);
      frag_fwd[0 * fwd_elems + f] = Elem<T>::from_f(s.f0);
      frag_fwd[1 * fwd_elems + f] = Elem<T>::from_f(s.f2);
      frag_fwd[2 * fwd_elems + f] = Elem<T>::from_f(s.fr);
      frag_fwd[3 * fwd_elems + f] = Elem<T>::from_f(s.fi);
    }
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
    if (frag_adj != nullptr) {
      const int64_t f = frag_pos<T>(c, d, adj_k);
      frag_adj[0 * adj_elems + f] = Elem<T>::from_f(s.f0);
      frag_adj[1 * adj_elems + f] = Elem<T>::from_f(s.f2);
      frag_adj[2 * adj_elems + f] = Elem<T>::from_f(s.fr);
      frag_adj[3 * adj_elems + f] = Elem<T>::from_f(-s.fi);
    }
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

hipError_t launch_spectra(const eqlinear_plan* p, const void* W, const void* bias, hipStream_t s) {
  if (p->cyclic) return cyc::launch_spectra(p, W, bias, s);
  const int64_t total = (int64_t)p->fwd.plane_elems() + (int64_t)p->adj.plane_elems() +
                        p->fwd.n_pad + p->adj.n_pad;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (p->dtype == EQL_F16) {
    hipLaunchKernelGGL(k_weight_spectra<_Float16>, dim3((unsigned)blocks), dim3(threads), 0, s,
                       (const _Float16*)W, (const _Float16*)bias, (_Float16*)p->spec_fwd,
                       (_Float16*)p->spec_adj, (_Float16*)p->frag_fwd, (_Float16*)p->frag_adj, p->bias_f32,
                       p->zeros_f32, (int)p->C, (int)p->D, (int)p->fwd.n_pad, (int)p->fwd.k_pad,
                       (int)p->adj.n_pad, (int)p->adj.k_pad);
  } else {
    hipLaunchKernelGGL(k_weight_spectra<float>, dim3((unsigned)blocks), dim3(threads), 0, s,
                       (const float*)W, (const float*)bias, (float*)p->spec_fwd,
                       (float*)p->spec_adj, (float*)p->frag_fwd, (float*)p->frag_adj, p->bias_f32, p->zeros_f32,
                       (int)p->C, (int)p->D,
                       (int)p->fwd.n_pad, (int)p->fwd.k_pad, (int)p->adj.n_pad, (int)p->adj.k_pad);
  }
  return hipGetLastError();
}

}  // namespace eql
