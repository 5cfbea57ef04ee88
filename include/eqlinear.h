/*
 * eqlinear.h -- C ABI of libeqlinear, the equivariant linear layer
 * (EQ-Linear) of a cyclic rotation group of order T, 2 <= T <= 16, or of a
 * dihedral group (rotations and reflections) of order T = 2n, 2 <= n <= 8,
 * on AMD MI355X (gfx950); the p4 group (cyclic, T = 4) has its own
 * specialised kernels.
 *
 * The operation.  Flash EQ-Linear: Accelerating Equivariant Linear Layers via
 * Group-wise Discrete Fourier Transform (gist.science technical summary,
 * "Intuizione Centrale"; authors' English abstract on the arxivdaily page):
 * an EQ-Linear layer is a circular convolution along the group axis composed
 * with a linear map along channels.  With C input and D output channels per
 * group element,
 *
 *     y[n,d,t] = sum_{c<C} sum_{s<T} W[d,c,(t-s) mod T] * x[n,c,s]  + bias[d]
 *
 * It is the dense product with the unrolled group-circulant matrix
 * ("Problematica"), computed exactly through a real DFT along the group axis
 * ("Approccio Algoritmico": one product per kept frequency k <= T/2, 2T - 2
 * real matrix products for even T and 2T - 1 for odd T;
 * "Specializzazione per il Gruppo di Rotazione p4": for T = 4 the transforms
 * are adds/subtracts and there are six real matrix products).
 *
 * Reflection groups.  The pages' kernels cover p4 only and name reflection
 * groups as the next step ("Limitazioni e Lavoro Futuro").  For the
 * dihedral group D_n (n rotations rho^r and n reflections rho^r sigma,
 * sigma rho sigma = rho^-1; p4m is D_4) the layer is read as the group
 * convolution of the same construction,
 *
 *     y[n,d,g] = sum_{c<C} sum_{h<T} W[d,c,h^-1 g] * x[n,c,h]  + bias[d]
 *
 * with group index g = m*n + r for rho^r sigma^m (rotations first); for the
 * cyclic group h^-1 g = (t - s) mod T and this is the formula above.  It is
 * computed exactly through the group Fourier transform over the real
 * irreducible representations: one real product per one-dimensional
 * representation and a 2 x 2 block product (eight real products) per
 * two-dimensional one, 12 real products against 64 for p4m.
 *
 * Layouts.  Every tensor is dense, row-major, with the group index fastest:
 *     x, dx : [N][C][T]      y, dy : [N][D][T]      W, dW : [D][C][T]
 *     bias, dbias : [D]
 * x, y, dx, dy, W and bias hold the plan's dtype (EQL_F32 = IEEE binary32,
 * EQL_F16 = IEEE binary16); dW and dbias are always binary32.  Every pointer
 * must be 16-byte aligned (EQL_ERR_MISALIGNED otherwise).
 *
 * Ownership.  Buffers passed in belong to the caller and are only read or
 * written during the stream-ordered execution of the call.  The plan owns a
 * small device copy of the weight spectra (set by eqlinear_set_weight, which
 * keeps no pointer to W) and frees it in eqlinear_plan_destroy.
 *
 * Streams and errors.  Every device call is asynchronous on the given HIP
 * stream (NULL = the null stream) and never synchronises.  Arguments are
 * validated on the host before any HIP call, so the validation paths run
 * without a GPU.  A call returns a status code; it never aborts.  Launch
 * failures are reported as EQL_ERR_HIP with the HIP message available from
 * eqlinear_last_error().  Faults inside kernels surface at the caller's next
 * synchronisation, as with any HIP library.
 *
 * Concurrency.  forward, backward_input and backward_weight only read the
 * plan, so they may run concurrently on different streams.  Ordering
 * set_weight against calls in flight is the caller's responsibility.
 */
#ifndef EQLINEAR_H
#define EQLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct eqlinear_plan* eqlinear_plan_t; /* opaque */

typedef enum { EQL_F32 = 0, EQL_F16 = 1 } eqlinear_dtype_t;

/* Symmetry group of the group axis. */
typedef enum {
  EQL_GROUP_CYCLIC = 0,   /* C_T, T = order, 2 <= T <= 16 */
  EQL_GROUP_DIHEDRAL = 1  /* D_n, n = number of rotations, 2 <= n <= 8, T = 2n */
} eqlinear_group_t;

typedef enum {
  EQL_OK = 0,
  EQL_ERR_INVALID_ARG = 1, /* NULL pointer, C/D <= 0, N < 0, size overflow */
  EQL_ERR_UNSUPPORTED = 2, /* group, group order or dtype without kernels */
  EQL_ERR_NO_WEIGHT = 3,   /* forward/backward before set_weight */
  EQL_ERR_MISALIGNED = 4,  /* a buffer is not 16-byte aligned */
  EQL_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  EQL_ERR_ALLOC = 6,       /* hipMalloc of the plan's spectra failed */
  EQL_ERR_HIP = 7          /* another HIP runtime error */
} eqlinear_status_t;

/* Create a plan for C input and D output channels per group element, group
 * size T, and dtype.  T = 4 (the p4 group) runs the specialised p4 kernels;
 * every other T in [2, 16] runs the cyclic-group kernels (the general method
 * of "Approccio Algoritmico", of which the pages' own implementation covers
 * p4 only, "Limitazioni e Lavoro Futuro").  Other T return
 * EQL_ERR_UNSUPPORTED.  Host-only: allocates no device memory.  On success
 * *out holds a new plan. */
eqlinear_status_t eqlinear_plan_create(int64_t C, int64_t D, int64_t T,
                                       eqlinear_dtype_t dtype,
                                       eqlinear_plan_t* out);

/* Create a plan for a given symmetry group: EQL_GROUP_CYCLIC with n = T (as
 * eqlinear_plan_create), or EQL_GROUP_DIHEDRAL with n rotations, 2 <= n <= 8,
 * whose tensors then have T = 2n group values per channel (index m*n + r of
 * rho^r sigma^m).  The dihedral groups run the generic group kernels (their
 * group Fourier transform is the length-n DFT of the rotation and of the
 * reflection half of each group vector, combined into the one- and
 * two-dimensional representations).  One exception: p4m (n = 4) in EQL_F16
 * at widths the p4 producer/consumer kernels take (2C a multiple of 32 up
 * to 192, or 256 or 384) runs as the p4 layer on paired channels: a p4m
 * tensor [N][C][8] is the p4 tensor [N][2C][4] with channel 2c + m holding
 * coset m, and the layer is a p4 layer with a rearranged weight.  That
 * path spends 24 real products per (n, c, d) instead of 12, on kernels
 * bound by HBM bytes rather than by the matrix cores at these widths; the
 * environment variable EQL_P4M_PAIRS=0, read at plan creation, selects the
 * generic kernels instead.  Other groups or orders return
 * EQL_ERR_UNSUPPORTED.  Host-only, as eqlinear_plan_create (a p4m plan on
 * paired channels also creates its inner p4 plan). */
eqlinear_status_t eqlinear_plan_create_group(int64_t C, int64_t D, eqlinear_group_t group,
                                             int64_t n, eqlinear_dtype_t dtype,
                                             eqlinear_plan_t* out);

/* Destroy a plan and free its device spectra (NULL is a no-op).  The caller
 * must ensure no call using the plan is still in flight. */
eqlinear_status_t eqlinear_plan_destroy(eqlinear_plan_t plan);

/* Weight-spectrum precompute (once per weight update).  Reads W[D][C][T] and
 * bias[D] (NULL = no bias) in the plan dtype and writes the plan's spectra:
 * the length-T real DFT of every W[d,c,:], frequencies k <= T/2 only (real
 * and imaginary parts as T real planes; the others are conjugates,
 * "Approccio Algoritmico": conjugate symmetry of the real DFT), or for a
 * dihedral plan its group Fourier transform (T real planes: the
 * one-dimensional representations and the 2 x 2 blocks), in the layouts the
 * forward and backward kernels read.  On the first call it allocates the
 * spectra on the current device (EQL_ERR_ALLOC on failure); later calls
 * must run on the same device. */
eqlinear_status_t eqlinear_set_weight(eqlinear_plan_t plan, const void* W,
                                      const void* bias, void* stream);

/* Forward: y[N][D][T] from x[N][C][T] (formula above, with the bias given to
 * set_weight).  One fused kernel: group DFT of x on chip, the real products
 * of every kept frequency on the matrix cores (fp32 accumulation; binary16
 * operands for EQL_F16, binary32 for EQL_F32), inverse DFT, bias and the
 * store.  N = 0 is a successful no-op. */
eqlinear_status_t eqlinear_forward(eqlinear_plan_t plan, const void* x, void* y,
                                   int64_t N, void* stream);

/* Pointwise activation fused into the forward epilogue. */
typedef enum {
  EQL_ACT_NONE = 0,      /* y as above */
  EQL_ACT_GELU = 1,      /* GELU: v * Phi(v) = (v/2) (1 + erf(v / sqrt 2)) */
  EQL_ACT_GELU_TANH = 2  /* GELU, tanh form: (v/2)(1 + tanh(sqrt(2/pi)(v + 0.044715 v^3))) */
} eqlinear_act_t;

/* Forward followed by a pointwise activation: y = act(forward(x)), with act
 * applied to every output value after the bias, in binary32, before the one
 * rounding to the plan dtype.  The pages' fused dataflow ("Implementazione":
 * no intermediate written to global memory) carried one step further, for
 * the EQ-Linear -> GELU -> EQ-Linear chain of the equivariant transformers
 * the layer serves ("Livello di Rete").  A pointwise map commutes with the
 * group action, so the result stays equivariant.  The default kernels apply
 * the activation in their epilogue; shapes served by the fallback kernels
 * get a second in-place pass over y.  act outside eqlinear_act_t returns
 * EQL_ERR_INVALID_ARG; otherwise as eqlinear_forward (which is
 * eqlinear_forward_act with EQL_ACT_NONE). */
eqlinear_status_t eqlinear_forward_act(eqlinear_plan_t plan, const void* x, void* y,
                                       int64_t N, eqlinear_act_t act, void* stream);

/* Backward with respect to the input ("Implementazione": forward and backward
 * passes): dx[n,c,s] = sum_{d,t} W[d,c,(t-s) mod T] * dy[n,d,t] (dihedral:
 * dx[n,c,h] = sum_{d,g} W[d,c,h^-1 g] * dy[n,d,g]), i.e. the transpose of
 * the forward map, computed with the adjoint weight spectra (conjugate, or
 * with the 2 x 2 blocks transposed).
 * dx has the plan dtype.  N = 0 is a successful no-op. */
eqlinear_status_t eqlinear_backward_input(eqlinear_plan_t plan, const void* dy,
                                          void* dx, int64_t N, void* stream);

/* Bytes of device workspace eqlinear_backward_weight needs for N rows
 * (0 for an invalid plan or N < 0). */
size_t eqlinear_backward_weight_workspace(eqlinear_plan_t plan, int64_t N);

/* Backward with respect to the weight and bias ("Implementazione": forward
 * and backward passes; "Intuizione Centrale": the dense matrix replicates one
 * set of shared weights, so each weight's gradient is the sum over its
 * replicas; computed per kept frequency with the transforms of
 * "Specializzazione per il Gruppo di Rotazione p4"):
 *     dW[d,c,r] = sum_{n,t} dy[n,d,t] * x[n,c,(t-r) mod T]   (binary32)
 *     dbias[d]  = sum_{n,t} dy[n,d,t]                          (binary32)
 * (dihedral: dW[d,c,u] = sum_{n,h} dy[n,d,h u] * x[n,c,h])
 * i.e. the gradient of every replica of a shared weight summed back onto it.
 * dW and dbias (NULL = not wanted) are overwritten, not accumulated into.
 * The reduction over N runs in binary32 in a fixed order (deterministic).
 * workspace must hold eqlinear_backward_weight_workspace(plan, N) bytes
 * (EQL_ERR_WORKSPACE otherwise).  N = 0 writes zeros.  Needs no prior
 * set_weight. */
eqlinear_status_t eqlinear_backward_weight(eqlinear_plan_t plan, const void* x,
                                           const void* dy, float* dW, float* dbias,
                                           int64_t N, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* Size of the device scratch array of eqlinear_backward_weight_noalloc:
 * 32 MiB per GPU the library runs on, held until the process ends. */
#define EQL_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* eqlinear_backward_weight without a workspace argument and without any
 * device allocation, for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * workspace is a static device array of EQL_NOALLOC_SCRATCH_BYTES in the
 * library (one per GPU); the first call on a device looks up its address
 * (hipGetSymbolAddress, no stream work).  Shapes whose workspace
 * (eqlinear_backward_weight_workspace) exceeds it return EQL_ERR_WORKSPACE
 * with the sizes in eqlinear_last_error(); host validation runs first, as
 * for eqlinear_backward_weight.  Results are those of
 * eqlinear_backward_weight (same kernels, same order).  Every call on a GPU
 * uses that GPU's one array, and each call writes the parts it reads before
 * reading them: calls that overlap on one GPU (different streams or
 * threads) race and must be ordered by the caller. */
eqlinear_status_t eqlinear_backward_weight_noalloc(eqlinear_plan_t plan, const void* x,
                                                   const void* dy, float* dW, float* dbias,
                                                   int64_t N, void* stream);

/* Static description of a status code. */
const char* eqlinear_status_string(eqlinear_status_t st);

/* Message of the last EQL_ERR_HIP / EQL_ERR_ALLOC on the calling thread
 * ("" if none). */
const char* eqlinear_last_error(void);

/* Real multiply-accumulates of one forward over N rows as computed by the
 * library ((2T - 2)*N*C*D for even T, (2T - 1)*N*C*D for odd T; 6*N*C*D for
 * p4; dihedral D_n: (4n - 4)*N*C*D for even n, (4n - 2)*N*C*D for odd n,
 * 12*N*C*D for p4m, 24*N*C*D for p4m on paired channels) and of the dense
 * unrolled product (T*T*N*C*D); for even
 * cyclic T the ratio is 2(T-1)/T^2, 3/8 at T = 4 (authors' abstract).
 * Either pointer may be NULL. */
eqlinear_status_t eqlinear_mac_counts(eqlinear_plan_t plan, int64_t N,
                                      int64_t* spectral_macs, int64_t* dense_macs);

#ifdef __cplusplus
}
#endif

#endif /* EQLINEAR_H */
