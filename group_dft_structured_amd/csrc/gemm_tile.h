// LDS tile geometry and matrix-core operand reads shared by the LDS-tiled
// spectral GEMM kernels (k_spectral_gemm.hip, k_conv.hip).  Each spectral
// plane is staged in LDS as [rows][SK] with the reduction index contiguous; a
// lane of the 32x32 matrix-core step reads its KPL contiguous elements of one
// row per chunk.
#pragma once

#include <type_traits>

#include "eql_device.h"

namespace eql {

template <typename T>
struct Tile {
  static constexpr int BK = 64 / (int)sizeof(T);   // reduction channels per chunk (64 B per row)
  static constexpr int PAD = 16 / (int)sizeof(T);  // LDS row padding (16 B)
  static constexpr int SK = BK + PAD;              // LDS row stride in elements (80 B)
  static constexpr int KPL = BK / 2;               // contiguous k per lane and plane per chunk
  static constexpr int STEPS = BK / Mma<T>::K_STEP;
};

// A chunk of the matrix-core operand for one 32-row block, one plane, as read
// by this lane: KPL contiguous elements (32 B).
template <typename T>
struct LaneK {
  typedef typename std::conditional<std::is_same<T, float>::value, floatx4, half8>::type v16b;
  v16b lo, hi;
};

template <typename T>
__device__ __forceinline__ LaneK<T> lds_lane_k(const T* p) {
  LaneK<T> r;
  r.lo = *reinterpret_cast<const typename LaneK<T>::v16b*>(p);
  r.hi = *reinterpret_cast<const typename LaneK<T>::v16b*>(p + Tile<T>::KPL / 2);
  return r;
}

// Operand of matrix-core step s (0 <= s < STEPS) taken from a lane's chunk.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag step_frag(const LaneK<T>& v, int s);

template <>
__device__ __forceinline__ half8 step_frag<_Float16>(const LaneK<_Float16>& v, int s) {
  return s == 0 ? v.lo : v.hi;
}
template <>
__device__ __forceinline__ float step_frag<float>(const LaneK<float>& v, int s) {
  return s < 4 ? v.lo[s] : v.hi[s - 4];
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag neg_frag(typename Mma<T>::frag a) {
  return -a;
}

}  // namespace eql
