// C ABI of the p4 group convolution (include/eqconv.h): argument validation,
// the plan object and dispatch.  A convolution plan holds two p4 EQ-Linear
// plans over rotation-aware patches (k_conv.hip): the forward layer
// (k^2 C -> D) and the adjoint layer (k^2 D -> C) of the backward input
// pass.  Every check that can run without a GPU runs before the first HIP
// call.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "../../include/eqconv.h"
#include "eql_internal.h"

struct eqconv_plan {
  int64_t C, D, k;
  eqlinear_dtype_t dtype;
  size_t esize;
  eqlinear_plan* fwd;  // patch layer k^2 C -> D
  eqlinear_plan* adj;  // adjoint patch layer k^2 D -> C
  void* wbuf;          // patch weights [D][k^2 C][4] then [C][k^2 D][4], plan dtype
  bool has_weight;
};

namespace {

constexpr int64_t MAX_PATCH_CHANNELS = 1 << 16;
constexpr int64_t MAX_PIXELS = ((int64_t)1 << 31) - 1;
constexpr int64_t MAX_K = 7;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t ru256(size_t v) { return (v + 255) / 256 * 256; }

// pixel count, or -1 when a size is negative or the count does not fit
int64_t pixels(int64_t N, int64_t H, int64_t W) {
  if (N < 0 || H < 0 || W < 0) return -1;
  if (N == 0 || H == 0 || W == 0) return 0;
  if (H > MAX_PIXELS / W) return -1;
  const int64_t hw = H * W;
  if (N > MAX_PIXELS / hw) return -1;
  return N * hw;
}

eqlinear_status_t make_inner(int64_t K, int64_t n_out, eqlinear_dtype_t dt, eqlinear_plan** out) {
  eqlinear_status_t st = eqlinear_plan_create(K, n_out, 4, dt, out);
  // the convolution kernels read the p4 spectra layout {W0, W2, Wr, Wi}
  if (st == EQL_OK) (*out)->cyclic = false;
  return st;
}

size_t ws_patches(const eqconv_plan* p, int64_t P) {
  return ru256((size_t)P * (size_t)eql::conv_patch_width((int)p->C, (int)p->k) * 4 * p->esize);
}
size_t ws_inner(const eqconv_plan* p, int64_t P) {
  return ru256(eqlinear_backward_weight_workspace(p->fwd, P));
}
size_t ws_dwp(const eqconv_plan* p) {
  return ru256((size_t)p->D * eql::conv_patch_width((int)p->C, (int)p->k) * 4 * sizeof(float));
}

// A kernel reads the rows of one tile and a halo of h image rows and h
// pixels on each side through one buffer resource (offsets below 2^31).
bool span_fits(const eqconv_plan* p, int64_t Cs, int64_t W) {
  const int64_t h = p->k / 2;
  const int64_t span = 2 * h * W + 2 * h + 128;  // pixels, largest tile
  return span * Cs * 4 * (int64_t)p->esize < ((int64_t)1 << 31) - 64;
}

eqlinear_status_t hip_status(const char* what, hipError_t e) {
  if (e == hipSuccess) return EQL_OK;
  fprintf(stderr, "eqconv: %s: %s\n", what, hipGetErrorString(e));
  return EQL_ERR_HIP;
}

}  // namespace

extern "C" {

eqlinear_status_t eqconv_plan_create(int64_t C, int64_t D, int64_t k, eqlinear_dtype_t dtype_arg,
                                     eqconv_plan_t* out) {
  if (out == nullptr) return EQL_ERR_INVALID_ARG;
  *out = nullptr;
  if (C <= 0 || D <= 0) return EQL_ERR_INVALID_ARG;
  const int dv = eql::enum_value(dtype_arg);
  if (dv != EQL_F32 && dv != EQL_F16) return EQL_ERR_UNSUPPORTED;
  const eqlinear_dtype_t dtype = (eqlinear_dtype_t)dv;
  if (k < 1 || k > MAX_K || k % 2 == 0) return EQL_ERR_UNSUPPORTED;
  if (C % 4 != 0 || D % 4 != 0) return EQL_ERR_UNSUPPORTED;
  if (C > MAX_PATCH_CHANNELS || D > MAX_PATCH_CHANNELS) return EQL_ERR_UNSUPPORTED;
  if (eql::conv_patch_width((int)C, (int)k) > MAX_PATCH_CHANNELS ||
      eql::conv_patch_width((int)D, (int)k) > MAX_PATCH_CHANNELS)
    return EQL_ERR_UNSUPPORTED;
  eqconv_plan* p = new (std::nothrow) eqconv_plan;
  if (p == nullptr) return EQL_ERR_ALLOC;
  memset(p, 0, sizeof(*p));
  p->C = C;
  p->D = D;
  p->k = k;
  p->dtype = dtype;
  p->esize = dtype == EQL_F16 ? 2 : 4;
  eqlinear_status_t st = make_inner(eql::conv_patch_width((int)C, (int)k), D, dtype, &p->fwd);
  if (st == EQL_OK) st = make_inner(eql::conv_patch_width((int)D, (int)k), C, dtype, &p->adj);
  if (st != EQL_OK) {
    eqlinear_plan_destroy(p->fwd);
    eqlinear_plan_destroy(p->adj);
    delete p;
    return st;
  }
  *out = p;
  return EQL_OK;
}

eqlinear_status_t eqconv_plan_destroy(eqconv_plan_t p) {
  if (p == nullptr) return EQL_OK;
  eqlinear_status_t st = eqlinear_plan_destroy(p->fwd);
  eqlinear_status_t st2 = eqlinear_plan_destroy(p->adj);
  if (st == EQL_OK) st = st2;
  if (p->wbuf != nullptr) {
    hipError_t e = hipFree(p->wbuf);
    if (e != hipSuccess && st == EQL_OK) st = hip_status("hipFree", e);
  }
  delete p;
  return st;
}

eqlinear_status_t eqconv_set_weight(eqconv_plan_t p, const void* psi, const void* bias,
                                    void* stream) {
  if (p == nullptr || psi == nullptr) return EQL_ERR_INVALID_ARG;
  if (!aligned16(psi) || !aligned16(bias)) return EQL_ERR_MISALIGNED;
  const size_t wf_bytes =
      ru256((size_t)p->D * eql::conv_patch_width((int)p->C, (int)p->k) * 4 * p->esize);
  const size_t wa_bytes =
      ru256((size_t)p->C * eql::conv_patch_width((int)p->D, (int)p->k) * 4 * p->esize);
  if (p->wbuf == nullptr) {
    hipError_t e = hipMalloc(&p->wbuf, wf_bytes + wa_bytes);
    if (e != hipSuccess) {
      p->wbuf = nullptr;
      fprintf(stderr, "eqconv: hipMalloc(patch weights): %s\n", hipGetErrorString(e));
      return EQL_ERR_ALLOC;
    }
  }
  void* wf = p->wbuf;
  void* wa = (char*)p->wbuf + wf_bytes;
  eqlinear_status_t st =
      hip_status("patch weight launch",
                 eql::launch_conv_patch_weights(p->dtype, psi, wf, wa, (int)p->C, (int)p->D,
                                                (int)p->k, (hipStream_t)stream));
  if (st != EQL_OK) return st;
  st = eqlinear_set_weight(p->fwd, wf, bias, stream);
  if (st == EQL_OK) st = eqlinear_set_weight(p->adj, wa, nullptr, stream);
  if (st == EQL_OK) p->has_weight = true;
  return st;
}

static eqlinear_status_t run_conv(const eqlinear_plan* inner, const eqconv_plan* p, const void* src,
                                  int64_t Cs, void* out, int64_t n_out, int64_t N, int64_t H,
                                  int64_t W, int act, void* stream) {
  const int64_t P = pixels(N, H, W);
  if (P < 0) return EQL_ERR_INVALID_ARG;
  if (!p->has_weight) return EQL_ERR_NO_WEIGHT;
  if (P == 0) return EQL_OK;
  if (src == nullptr || out == nullptr) return EQL_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(out)) return EQL_ERR_MISALIGNED;
  if (!span_fits(p, Cs, W)) return EQL_ERR_UNSUPPORTED;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != inner->device) return EQL_ERR_INVALID_ARG;
  return hip_status("convolution launch",
                    eql::launch_conv(inner->tune, p->dtype, src, (int)H, (int)W, (int)Cs, (int)p->k, P,
                                     inner->spec_fwd, inner->bias_f32, out, (int)inner->fwd.k_pad,
                                     (int)n_out, (int)inner->fwd.n_pad, act,
                                     (hipStream_t)stream));
}

eqlinear_status_t eqconv_forward(eqconv_plan_t p, const void* f, void* y, int64_t N, int64_t H,
                                 int64_t W, eqlinear_act_t act_arg, void* stream) {
  if (p == nullptr) return EQL_ERR_INVALID_ARG;
  const int av = eql::enum_value(act_arg);
  if (av != EQL_ACT_NONE && av != EQL_ACT_GELU && av != EQL_ACT_GELU_TANH) return EQL_ERR_INVALID_ARG;
  return run_conv(p->fwd, p, f, p->C, y, p->D, N, H, W, av, stream);
}

eqlinear_status_t eqconv_backward_input(eqconv_plan_t p, const void* dy, void* df, int64_t N,
                                        int64_t H, int64_t W, void* stream) {
  if (p == nullptr) return EQL_ERR_INVALID_ARG;
  return run_conv(p->adj, p, dy, p->D, df, p->C, N, H, W, 0, stream);
}

size_t eqconv_backward_weight_workspace(eqconv_plan_t p, int64_t N, int64_t H, int64_t W) {
  if (p == nullptr) return 0;
  const int64_t P = pixels(N, H, W);
  if (P < 0) return 0;
  return ws_patches(p, P) + ws_inner(p, P) + ws_dwp(p);
}

eqlinear_status_t eqconv_backward_weight(eqconv_plan_t p, const void* f, const void* dy,
                                         float* dpsi, float* dbias, int64_t N, int64_t H,
                                         int64_t W, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  if (p == nullptr || dpsi == nullptr) return EQL_ERR_INVALID_ARG;
  const int64_t P = pixels(N, H, W);
  if (P < 0) return EQL_ERR_INVALID_ARG;
  if (P > 0 && (f == nullptr || dy == nullptr)) return EQL_ERR_INVALID_ARG;
  if (!aligned16(f) || !aligned16(dy) || !aligned16(dpsi) || !aligned16(dbias) ||
      !aligned16(workspace))
    return EQL_ERR_MISALIGNED;
  const size_t need = eqconv_backward_weight_workspace(p, N, H, W);
  if (workspace == nullptr || workspace_bytes < need) return EQL_ERR_WORKSPACE;
  if (P > 0 && !span_fits(p, p->C, W)) return EQL_ERR_UNSUPPORTED;
  char* ws = (char*)workspace;
  void* xp = ws;
  void* inner_ws = ws + ws_patches(p, P);
  float* dwp = (float*)(ws + ws_patches(p, P) + ws_inner(p, P));
  eqlinear_status_t st = hip_status(
      "patch gather launch", eql::launch_conv_gather(p->dtype, f, (int)H, (int)W, (int)p->C,
                                                     (int)p->k, P, xp, (hipStream_t)stream));
  if (st != EQL_OK) return st;
  st = eqlinear_backward_weight(p->fwd, xp, dy, dwp, dbias, P, inner_ws, ws_inner(p, P), stream);
  if (st != EQL_OK) return st;
  return hip_status("filter fold launch",
                    eql::launch_conv_fold(dwp, dpsi, (int)p->C, (int)p->D, (int)p->k,
                                          (hipStream_t)stream));
}

eqlinear_status_t eqconv_mac_counts(eqconv_plan_t p, int64_t N, int64_t H, int64_t W,
                                    int64_t* spectral_macs, int64_t* dense_macs) {
  if (p == nullptr) return EQL_ERR_INVALID_ARG;
  const int64_t P = pixels(N, H, W);
  if (P < 0) return EQL_ERR_INVALID_ARG;
  const int64_t per = p->k * p->k * p->C * p->D * P;
  if (spectral_macs) *spectral_macs = 6 * per;
  if (dense_macs) *dense_macs = 16 * per;
  return EQL_OK;
}

}  // extern "C"
