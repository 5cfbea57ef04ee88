// Host-only stand-ins for the launchers of the largest kernel files of
// libeqlinear (the producer/consumer forward kernels, the generic group
// kernels and the group convolution), so that the rest of the library's host
// code (plan objects, argument validation, workspace sizing, dispatch, the
// no-allocation scratch lookup) builds quickly with AddressSanitizer and
// UndefinedBehaviorSanitizer and runs without a GPU.  Each stand-in reports
// hipErrorNotSupported (the dispatch then falls back) or a plausible size.
#include "../../group_dft_structured_amd/csrc/eql_internal.h"

namespace eql {
hipError_t launch_ws(const Tuning&, eqlinear_dtype_t, const void*, const void*, const float*, void*,
                     int64_t, int, int, int, int, bool, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_ws32(const Tuning&, eqlinear_dtype_t, const void*, const void*, const float*, void*,
                       int64_t, int, int, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_conv(const Tuning&, eqlinear_dtype_t, const void*, int, int, int, int, int64_t,
                       const void*, const float*, void*, int, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_conv_gather(eqlinear_dtype_t, const void*, int, int, int, int, int64_t, void*,
                              hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_conv_patch_weights(eqlinear_dtype_t, const void*, void*, void*, int, int, int,
                                     hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_conv_fold(const float*, float*, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
namespace cyc {
size_t workspace_bytes(const eqlinear_plan* p, int64_t N) {
  return N > 0 ? (size_t)p->T * (size_t)p->C * (size_t)p->D * 64 : 0;
}
hipError_t launch_spectra(const eqlinear_plan*, const void*, const void*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_forward(const eqlinear_plan*, const void*, void*, int64_t, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_backward_input(const eqlinear_plan*, const void*, void*, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_backward_weight(const eqlinear_plan*, const void*, const void*, float*, float*,
                                  int64_t, void*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace cyc
}  // namespace eql
