// Host-side internals of libeqlinear: the plan object and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/eqlinear.h"

namespace eql {

// Padding of the spectra planes.  A plane used as the matrix-core B operand
// with "k" = reduction channel and "n" = output channel is stored [n][k] with
// k contiguous; k is padded to KPAD and n to NPAD with zeros so that the
// kernels never bounds-check weight reads.
constexpr int KPAD = 32;
constexpr int NPAD = 128;

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// The integer a C caller passed for an enumeration parameter.  A C caller may
// pass any int; reading such a value through the C++ enumeration type is
// undefined when it lies outside the enumeration's range, so the C ABI
// validates its enumeration arguments through their bytes.
template <typename E>
inline int enum_value(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "enumerations of the C ABI are int-sized");
  int v;
  __builtin_memcpy(&v, &e, sizeof(v));
  return v;
}

struct SpectraLayout {
  int64_t n_pad;  // padded output-channel count (rows of a plane)
  int64_t k_pad;  // padded reduction-channel count (contiguous)
  size_t plane_elems() const { return (size_t)(n_pad * k_pad); }
};

}  // namespace eql

namespace eql {

// Launch choices of a plan, read once from EQL_* environment variables when
// the plan is created and range-checked there (-1: unset or out of range,
// which keeps the shape-based default).  They let tests force one kernel path
// and let tuning sweeps vary tile shapes; the workspace query and every
// launch of a plan see the same values, also inside a captured HIP graph.
struct Tuning {
  // producer/consumer binary16 kernel (forward and backward_input)
  int ws_off;       // EQL_NO_WS=1: the general tiled kernel instead
  int ws_nc, ws_np, ws_nb, ws_wpc, ws_qx;  // consumer and producer waves, 16-channel
                                           // blocks per consumer, work-groups per CU,
                                           // workers per XCD
  int ws_g8;        // 8-channel producer units (0/1)
  int ws_pipe;      // software-pipelined activation epilogue (0/1)
  int ws_out;       // 1: consumers store their fragments (streaming)
  int ws_split;     // split producer/consumer stores beyond the cache (0/1)
  int ws_wfirst;    // consumers' weight fragments before the second and third tiles (0/1)
  int ws_ksplit;    // 0: backward_input over 384 channels without split-reduction consumers
  int64_t ws_small_bytes;  // outputs up to this size take the write-through producer stores
  // producer/consumer binary32 forward
  int ws32_off, ws32_nc, ws32_np, ws32_qx, ws32_stream, ws32_pst;
  int ws32_tail;  // split last round of tiles into (tile, block) units (0/1)
  // general tiled kernel: tile shape
  int gemm_tile;
  // backward_weight: producer/consumer kernel off, tiled kernel forced,
  // split count
  int bws_off, bw_tiled, bws_s;
  // generic group kernels: tile shape; p4 through them; weight-gradient
  // tile edge and work-group target; p4m on the p4 kernels
  int cyc_tile, cyclic_p4, cyc_bw_tile, cyc_bw_wgs, p4m_pairs;
  // group convolution: register-direct kernel (0/1), tile shape, binary32 kernel
  int conv_rd, conv_tile, conv_f32_16;
};

// Reads and range-checks every knob (host only, no HIP call).
Tuning read_tuning();

}  // namespace eql

struct eqlinear_plan {
  int64_t C, D;
  int T;        // group order: values per group vector (2..16)
  eqlinear_group_t group;  // cyclic C_T or dihedral D_{T/2}
  bool cyclic;  // served by the generic group kernels (every group but p4, or on request)
  // cyclic backward_weight: tile edge (64 or 32) and work-group target, fixed
  // at plan creation so that workspace size and launch always agree
  int cyc_bw_tile, cyc_bw_wgs;
  eql::Tuning tune;  // launch choices, fixed at plan creation
  eqlinear_dtype_t dtype;
  size_t esize;  // bytes per element of the plan dtype
  int device;    // device of the spectra, -1 before the first set_weight
  bool has_weight;
  // Forward operand: T planes, each [D_pad][C_pad]: for the p4 kernels
  // {W0, W2, Wr, Wi}, for the generic kernels the order of the group
  // descriptor in cyc_device.h.
  eql::SpectraLayout fwd;
  // Backward-input operand: the spectra of the adjoint layer (conjugate or
  // block-transposed), each [C_pad][D_pad].
  eql::SpectraLayout adj;
  void* spec_fwd;     // device, plan dtype
  void* spec_adj;     // device, plan dtype
  // p4 plans: the operands of the producer/consumer kernels again in their
  // matrix-core fragment order (k_spectra.hip): both in binary16, the forward
  // one in binary32 (frag_adj nullptr); nullptr for the generic groups.
  void* frag_fwd;
  void* frag_adj;
  float* bias_f32;    // device, [fwd.n_pad], zeros where no bias
  float* zeros_f32;   // device, [adj.n_pad] zeros (bias of backward_input)
  // p4m (D_4) in binary16 at widths the p4 producer/consumer kernels take:
  // served by this p4 plan on paired channels (2C -> 2D, k_p4m_pairs.hip);
  // nullptr otherwise.  pair_w holds the paired weight [2D][2C][4] and bias
  // [2D] (plan dtype) between set_weight's two launches.
  eqlinear_plan* inner;
  void* pair_w;
};

namespace eql {

// Backward-weight split over rows: each work-group reduces ROWS_PER_SPLIT rows.
int64_t bwd_weight_rows_per_split(const eqlinear_plan* p, int64_t N);
size_t bwd_weight_workspace_bytes(const eqlinear_plan* p, int64_t N);


// Producer/consumer backward-weight path (binary16, even channel counts).
bool bws_supported(const eqlinear_plan* p);
size_t bws_workspace(const eqlinear_plan* p, int64_t N);
hipError_t launch_bws(const eqlinear_plan* p, const void* x, const void* dy, float* dW, float* dbias,
                      int64_t N, void* ws, hipStream_t s);

hipError_t launch_spectra(const eqlinear_plan* p, const void* W, const void* bias, hipStream_t s);
// Producer/consumer spectral kernel (binary16): the forward, or with the
// conjugate-transposed spectra (adjoint = true) the backward-input pass.
// `spec` is an operand in fragment order (frag_fwd or frag_adj).
// act: pointwise activation of the forward epilogue (0 none, 1 GELU, 2 GELU
// with the tanh approximation); 0 for backward_input.
hipError_t launch_ws(const Tuning& tn, eqlinear_dtype_t dt, const void* x, const void* spec,
                     const float* bias, void* y, int64_t N, int K, int k_pad, int n_out, int n_pad,
                     bool adjoint, int act, hipStream_t s);
// Producer/consumer forward kernel, binary32 (reduction width a multiple of 16, <= 192);
// `spec` is the forward operand in its fragment order (frag_fwd).
hipError_t launch_ws32(const Tuning& tn, eqlinear_dtype_t dt, const void* x, const void* spec,
                       const float* bias, void* y, int64_t N, int K, int k_pad, int n_out, int n_pad,
                       int act, hipStream_t s);
hipError_t launch_forward(const eqlinear_plan* p, const void* x, void* y, int64_t N, int act,
                          hipStream_t s);
hipError_t launch_backward_input(const eqlinear_plan* p, const void* dy, void* dx, int64_t N,
                                 hipStream_t s);
hipError_t launch_backward_weight(const eqlinear_plan* p, const void* x, const void* dy, float* dW,
                                  float* dbias, int64_t N, void* ws, hipStream_t s);

// p4m on the p4 kernels (k_p4m_pairs.hip): paired weight and bias from W
// [D][C][8], and the fold of the paired weight gradient [2D][2C][4] (+ bias
// gradient [2D]) back into dW [D][C][8] (+ dbias [D]).
hipError_t launch_p4m_pair_weight(const void* W, const void* bias, void* Wp, void* bp, int64_t C,
                                  int64_t D, hipStream_t s);
hipError_t launch_p4m_fold(const float* dWp, const float* dbp, float* dW, float* dbias, int64_t C,
                           int64_t D, hipStream_t s);

// p4 group convolution through rotation-aware patches (k_conv.hip).  launch_conv
// runs the patch layer whose spectra [n_pad][k_pad] are given, gathering from
// a field [P][Cs][4] of H x W images with a k x k kernel; launch_conv_gather
// writes the patches [P][k^2 Cs][4]; launch_conv_patch_weights writes the
// forward [D][k^2 C][4] and adjoint [C][k^2 D][4] patch weights of psi
// [D][C][k][k][4]; launch_conv_fold takes dpsi from the patch-weight gradient.
// Patch channel layout of a field of Cs channels and a k x k kernel: the
// centre channels padded to a multiple of 32 (a 32-channel reduction step is
// then either centre or orbit channels), then 4 Cs channels per orbit of
// offsets under the quarter turn, (k^2 - 1) / 4 orbits.
__host__ __device__ inline int conv_centre_width(int Cs) { return (Cs + 31) / 32 * 32; }
__host__ __device__ inline int conv_patch_width(int Cs, int k) {
  return conv_centre_width(Cs) + (k * k - 1) * Cs;
}
hipError_t launch_conv(const Tuning& tn, eqlinear_dtype_t dt, const void* f, int H, int W, int Cs,
                       int k, int64_t P, const void* spec, const float* bias, void* out, int k_pad,
                       int n_out, int n_pad, int act, hipStream_t s);
hipError_t launch_conv_gather(eqlinear_dtype_t dt, const void* f, int H, int W, int Cs, int k,
                              int64_t P, void* xp, hipStream_t s);
hipError_t launch_conv_patch_weights(eqlinear_dtype_t dt, const void* psi, void* wf, void* wa,
                                     int C, int D, int k, hipStream_t s);
hipError_t launch_conv_fold(const float* dwp, float* dpsi, int C, int D, int k, hipStream_t s);

// Cyclic-group kernels (k_cyclic.hip), any group size 2 <= T <= 16.
namespace cyc {
size_t workspace_bytes(const eqlinear_plan* p, int64_t N);
hipError_t launch_spectra(const eqlinear_plan* p, const void* W, const void* bias, hipStream_t s);
hipError_t launch_forward(const eqlinear_plan* p, const void* x, void* y, int64_t N, int act,
                          hipStream_t s);
hipError_t launch_backward_input(const eqlinear_plan* p, const void* dy, void* dx, int64_t N,
                                 hipStream_t s);
hipError_t launch_backward_weight(const eqlinear_plan* p, const void* x, const void* dy, float* dW,
                                  float* dbias, int64_t N, void* ws, hipStream_t s);
}  // namespace cyc

}  // namespace eql
