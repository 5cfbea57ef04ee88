/*
 * eqconv.h -- C ABI of the p4 group convolution on the plane in libeqlinear
 * (AMD MI355X, gfx950).
 *
 * The operation.  The pages name equivariant convolutions as the next
 * operator for the Flash EQ-Linear principle without defining one (gist.science
 * summary of Flash EQ-Linear, "Limitazioni e Lavoro Futuro").  The layer here
 * is the k x k convolution of fields over the plane and the rotation group p4
 * whose taps turn together with the cyclic shift of the group axis, so that
 * it commutes with turning the image a quarter turn together with that shift,
 * and whose 1 x 1 case is the EQ-Linear layer of eqlinear.h ("Intuizione
 * Centrale": circular convolution along the group axis composed with a
 * linear map along channels):
 *
 *   y[n,i,j,d,t] = bias[d] + sum_{c<C} sum_{s<4} sum_{(a,b)}
 *                  psi[d,c,h+a',h+b',(t-s) mod 4] * f[n,i+a,j+b,c,s]
 *
 * over the offsets (a, b) in [-h, h]^2 (k = 2h + 1), with (a', b') = R^-t (a, b)
 * for the quarter turn R(a, b) = (-b, a) of (row, column) offsets, and
 * f = 0 outside the image (zero padding, stride 1, output the input's size).
 *
 * How it is computed.  The nonzero offsets fall into orbits of four under
 * R; within an orbit the dependence on the output group element t and the
 * orbit member j is through t - j only, so the convolution is exactly one
 * EQ-Linear layer with k^2 C input channels applied to rotation-aware patches
 * (the C channels of the pixel itself, and per orbit the 4C values
 * f[p + R^j u, c, (j + e) mod 4] over (c, e) as group vectors over j).  The
 * kernels gather those patches on chip and run the p4 transform with its
 * six real products per channel pair: 6 k^2 C D real multiplies per pixel
 * against 16 k^2 C D for the unrolled convolution, the same 3/8.
 *
 * Layouts (dense, row-major, group index fastest; every pointer 16-byte
 * aligned, EQL_ERR_MISALIGNED otherwise):
 *     f, df : [N][H][W][C][4]      y, dy : [N][H][W][D][4]
 *     psi : [D][C][k][k][4] (spatial index = offset + h)      bias : [D]
 *     dpsi : [D][C][k][k][4] binary32      dbias : [D] binary32
 * f, y, df, dy, psi and bias hold the plan's dtype.
 *
 * Ownership, streams, errors and concurrency are as in eqlinear.h: buffers
 * belong to the caller; the plan owns its patch weights and spectra (set by
 * eqconv_set_weight, which keeps no pointer to psi); every call is
 * asynchronous on the given HIP stream and returns a status code, with
 * arguments checked on the host before any HIP call.
 */
#ifndef EQCONV_H
#define EQCONV_H

#include <stddef.h>
#include <stdint.h>

#include "eqlinear.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct eqconv_plan* eqconv_plan_t; /* opaque */

/* Create a plan for C input and D output channels per group element and an
 * odd kernel size k (1 <= k <= 7).  C and D must be multiples of 4 (a gather
 * of four patch channels reads four whole group vectors), and the patch
 * width of each (the channel count rounded up to 32, plus k^2 - 1 times the
 * channel count) at most 65536; otherwise EQL_ERR_UNSUPPORTED (k even or out
 * of range, channel counts) or EQL_ERR_INVALID_ARG (C, D <= 0, out == NULL).
 * Host-only: allocates no device memory. */
eqlinear_status_t eqconv_plan_create(int64_t C, int64_t D, int64_t k, eqlinear_dtype_t dtype,
                                     eqconv_plan_t* out);

/* Destroy a plan and free its device buffers (NULL is a no-op). */
eqlinear_status_t eqconv_plan_destroy(eqconv_plan_t plan);

/* Filter update: reads psi[D][C][k][k][4] and bias[D] (NULL = no bias) in the
 * plan dtype and writes the plan's patch weights (a permutation of psi, for
 * the forward and for the adjoint layer) and their spectra.  Allocates on the
 * first call, on the current device (EQL_ERR_ALLOC on failure). */
eqlinear_status_t eqconv_set_weight(eqconv_plan_t plan, const void* psi, const void* bias,
                                    void* stream);

/* Forward y = conv(f) (+ bias), then act (eqlinear_act_t) on every output
 * value in binary32 before the one rounding to the plan dtype.  One kernel:
 * the patch gather, the group DFT, the real products on the matrix cores with
 * fp32 accumulation, the inverse DFT, bias and activation.  N*H*W = 0 is a
 * successful no-op; N, H, W < 0 or N*H*W >= 2^31 return
 * EQL_ERR_INVALID_ARG; before set_weight, EQL_ERR_NO_WEIGHT.  A tile of
 * pixels and its halo of k/2 image rows on each side must span under 2 GiB
 * of the field ((k - 1) * W * C * 4 elements, roughly), else
 * EQL_ERR_UNSUPPORTED. */
eqlinear_status_t eqconv_forward(eqconv_plan_t plan, const void* f, void* y, int64_t N,
                                 int64_t H, int64_t W, eqlinear_act_t act, void* stream);

/* Backward with respect to the input: df = the transpose of the forward map
 * applied to dy,
 *     df[n,q,c,s] = sum_{v,d,t} psi[d,c,h+R^-t v,(t-s) mod 4] dy[n,q-v,d,t]
 * computed as the convolution of dy with the adjoint filter
 * psi*[c,d,w,r] = psi[d,c,-R^r w,(-r) mod 4] on the same kernel.  Arguments
 * as eqconv_forward, no bias or activation. */
eqlinear_status_t eqconv_backward_input(eqconv_plan_t plan, const void* dy, void* df, int64_t N,
                                        int64_t H, int64_t W, void* stream);

/* Bytes of device workspace eqconv_backward_weight needs (0 for an invalid
 * plan or size): the patches of f (N*H*W times the patch width times 4
 * elements of the plan dtype), the EQ-Linear weight-gradient workspace of the patch layer and
 * the patch-weight gradient (binary32). */
size_t eqconv_backward_weight_workspace(eqconv_plan_t plan, int64_t N, int64_t H, int64_t W);

/* Backward with respect to the filter and bias:
 *     dpsi[d,c,h+w,r] = sum_{n,p,t} dy[n,p,d,t] f[n,p+R^t w,c,(t-r) mod 4]
 *     dbias[d] = sum_{n,p,t} dy[n,p,d,t]
 * (binary32, overwritten; dbias NULL = not wanted).  The patches of f are
 * written to the workspace, the EQ-Linear weight gradient of the patch layer
 * is reduced over pixels in a fixed order, and each filter entry takes its
 * one place in it.  N*H*W = 0 writes zeros.  Needs no prior set_weight. */
eqlinear_status_t eqconv_backward_weight(eqconv_plan_t plan, const void* f, const void* dy,
                                         float* dpsi, float* dbias, int64_t N, int64_t H,
                                         int64_t W, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* Real multiply-accumulates of one forward over N*H*W pixels: 6 k^2 C D per
 * pixel as computed, 16 k^2 C D for the unrolled convolution. */
eqlinear_status_t eqconv_mac_counts(eqconv_plan_t plan, int64_t N, int64_t H, int64_t W,
                                    int64_t* spectral_macs, int64_t* dense_macs);

#ifdef __cplusplus
}
#endif

#endif /* EQCONV_H */
