// K-streaming spectral GEMM (binary16) for wide reduction and narrow output:
// the backward-input pass of the p4 EQ-Linear layer (reduction over the D
// output channels of the forward, C outputs), and any pass of that shape.
//
// Arithmetic, with the conjugate-transposed weight spectra B = (W0^T, W2^T,
// Wr^T, -Wi^T) and G = DFT_4(dy) (Flash EQ-Linear, "Approccio Algoritmico":
// per-frequency products, conjugate symmetry):
//     dX0 = G0 B0   dX2 = G2 B2   dXr = Gr Br - Gi Bi   dXi = Gr Bi + Gi Br
// followed by the inverse length-4 butterfly.
//
// Organisation on CDNA4:
//  * a persistent work-group owns BN = 16*NOB output channels and keeps their
//    weight spectra for the whole reduction (K up to ~380 channels) in LDS;
//  * each wave owns 16-row tiles and streams them through the reduction in
//    32-channel steps: range-checked buffer loads run three steps ahead in a
//    register ring, the butterfly happens in registers (X0/X2 exact in fp32
//    via v_dot2, Xr/-Xi by packed subtraction), and the 6*NOB products of a
//    step use weight fragments read from LDS, so the dy stream overlaps the
//    matrix-core work even when a wave has a single tile;
//  * the epilogue writes 32 contiguous bytes per lane.
#include "eql_device.h"
#include "eql_internal.h"

namespace eql {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_ks(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t pack2h(float a, float b) {
  const f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

}  // namespace

template <int NOB, int NW, int KCAP>
__global__ __launch_bounds__(NW * 64) void k_gemm_kstream_f16(
    const _Float16* __restrict__ a, const _Float16* __restrict__ spec, const float* __restrict__ bias,
    _Float16* __restrict__ out, int N, int K, int n_out, int n_pad, int k_pad, int n_ct, int Qx) {
  constexpr int NT = NW * 64;
  constexpr int BN = NOB * 16;
  constexpr int SKB = KCAP + 8;  // LDS row stride (halves): 16-lane reads hit distinct banks
  constexpr int PL = BN * SKB;
  __shared__ __attribute__((aligned(16))) _Float16 Bs[4 * PL];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar registers)
  const int i16 = lane & 15, g = lane >> 4;
  const int wgid = blockIdx.x, xcd = wgid & 7, slot = wgid >> 3;
  const int j = slot % n_ct;
  const int q = (slot / n_ct) * 8 + xcd, Q = Qx * 8;
  const int col0 = j * BN;
  const int ks = k_pad / 32;
  const int n_rt = (N + 15) / 16;
  const int64_t row_elems = (int64_t)K * 4;

  // loads of step s of tile t: lane (i16, g) reads row t*16+i16, channels s*32+8g..+7
  auto load_step = [&](half8 (&r)[4], int t, int s) {
    const int64_t r0 = (int64_t)t * 16;
    const int64_t rows = r0 < N ? (N - r0 < 16 ? N - r0 : 16) : 0;
    const __amdgpu_buffer_rsrc_t ra = rsrc_ks(a + r0 * row_elems, (uint32_t)(rows * row_elems * 2));
    const uint32_t off = (uint32_t)((i16 * row_elems + (s * 32 + 8 * g) * 4) * 2);
#pragma unroll
    for (int v = 0; v < 4; ++v)
      r[v] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(ra, off + 16 * v, 0, 0));
  };

  // first tile's first steps are requested before the weight staging
  int t = q * NW + wave;
  half8 rA[4], rB[4], rC[4];
  load_step(rA, t, 0);
  load_step(rB, t, 1);
  load_step(rC, t, 2);

  // ---- weight spectra of the range into LDS (rows past n_pad read as zeros) ----
  // A fixed, fully unrolled count of 16-byte units per thread: every load is
  // in flight before the first LDS store (a load-store-load loop would pay
  // the memory latency once per unit).
  {
    const uint32_t plane_bytes = (uint32_t)n_pad * k_pad * 2;
    const int64_t plane = (int64_t)n_pad * k_pad;
    const int upr = k_pad / 8;  // 16-byte units per row
    const int total = 4 * BN * upr;
    constexpr int SU = (4 * BN * (KCAP / 8) + NT - 1) / NT;  // units per thread, at most
    u32x4 v[SU];
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = i * NT + tid;
      const int p = u / (BN * upr), rem = u % (BN * upr);
      const int c = rem / upr, k = (rem % upr) * 8;
      const __amdgpu_buffer_rsrc_t rp = rsrc_ks(spec + (p < 4 ? p : 0) * plane, plane_bytes);
      const uint32_t off = u < total ? (uint32_t)(((col0 + c) * k_pad + k) * 2) : 0x7FFFFFF0u;
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int u = i * NT + tid;
      if (u < total) {
        const int p = u / (BN * upr), rem = u % (BN * upr);
        const int c = rem / upr, k = (rem % upr) * 8;
        *reinterpret_cast<u32x4*>(Bs + p * PL + c * SKB + k) = v[i];
      }
    }
  }
  float bc[NOB][4];
  {
    const __amdgpu_buffer_rsrc_t rb = rsrc_ks(bias, (uint32_t)n_pad * 4);
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        bc[ob][r] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rb, (col0 + ob * 16 + 4 * g + r) * 4, 0, 0));
  }
  __syncthreads();

  const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
  const f16x2 pm = {(_Float16)1.f, (_Float16)-1.f};
  const _Float16* wb = Bs + i16 * SKB + 8 * g;

  // one k-step: butterfly of the loaded rows, 6*NOB products
  auto do_step = [&](const half8 (&r)[4], int s, f32x4 (&c0)[NOB], f32x4 (&c2)[NOB],
                     f32x4 (&cr)[NOB], f32x4 (&ci)[NOB]) {
    half8 x0, x2, xr, xi, xq;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const half8& w = r[e >> 1];
      const int o = (e & 1) * 4;
      const f16x2 p01 = {w[o], w[o + 1]}, p23 = {w[o + 2], w[o + 3]};
      const float f0 = __builtin_amdgcn_fdot2(p01, ones, __builtin_amdgcn_fdot2(p23, ones, 0.f, false), false);
      const float f2 = __builtin_amdgcn_fdot2(p01, pm, __builtin_amdgcn_fdot2(p23, pm, 0.f, false), false);
      const f16x2 d = p01 - p23;  // (Xr, -Xi)
      x0[e] = (_Float16)f0;
      x2[e] = (_Float16)f2;
      xr[e] = d[0];
      xq[e] = d[1];
    }
    xi = -xq;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
      const _Float16* wp = wb + ob * 16 * SKB + s * 32;
      const half8 w0 = *reinterpret_cast<const half8*>(wp + 0 * PL);
      const half8 w2 = *reinterpret_cast<const half8*>(wp + 1 * PL);
      const half8 wr = *reinterpret_cast<const half8*>(wp + 2 * PL);
      const half8 wi = *reinterpret_cast<const half8*>(wp + 3 * PL);
      c0[ob] = mma16(w0, x0, c0[ob]);
      cr[ob] = mma16(wr, xr, cr[ob]);
      c2[ob] = mma16(w2, x2, c2[ob]);
      ci[ob] = mma16(wi, xr, ci[ob]);
      cr[ob] = mma16(wi, xq, cr[ob]);
      ci[ob] = mma16(wr, xi, ci[ob]);
    }
  };

  while (t < n_rt) {
    f32x4 c0[NOB], c2[NOB], cr[NOB], ci[NOB];
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) c0[ob] = c2[ob] = cr[ob] = ci[ob] = f32x4{};
    const int tn = t + Q * NW;  // this wave's next tile
    // steps s, s+1, s+2 live in rA, rB, rC; each slot is refilled with the
    // step three ahead (running into the next tile's first steps)
    // (ks is a multiple of three: the launcher checks it)
    for (int s = 0; s < ks; s += 3) {
      do_step(rA, s, c0, c2, cr, ci);
      load_step(rA, s + 3 < ks ? t : tn, s + 3 < ks ? s + 3 : s + 3 - ks);
      do_step(rB, s + 1, c0, c2, cr, ci);
      load_step(rB, s + 4 < ks ? t : tn, s + 4 < ks ? s + 4 : s + 4 - ks);
      do_step(rC, s + 2, c0, c2, cr, ci);
      load_step(rC, s + 5 < ks ? t : tn, s + 5 < ks ? s + 5 : s + 5 - ks);
    }
    // epilogue: lane holds channels col0 + 16ob + 4g + r of row t*16 + i16
    const int64_t r0 = (int64_t)t * 16;
    const int64_t rows = N - r0 < 16 ? N - r0 : 16;
    const __amdgpu_buffer_rsrc_t ro = rsrc_ks(out + r0 * n_out * 4, (uint32_t)(rows * n_out * 8));
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
      uint32_t o[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const floatx4 v = idft4(c0[ob][r], c2[ob][r], cr[ob][r], ci[ob][r]);
        o[2 * r] = pack2h(v[0] + bc[ob][r], v[1] + bc[ob][r]);
        o[2 * r + 1] = pack2h(v[2] + bc[ob][r], v[3] + bc[ob][r]);
      }
      const int col = col0 + ob * 16 + 4 * g;
      const uint32_t off = col < n_out ? (uint32_t)((i16 * n_out + col) * 8) : 0x7FFFFFF0u;
      const u32x4 lo = {o[0], o[1], o[2], o[3]}, hi = {o[4], o[5], o[6], o[7]};
      __builtin_amdgcn_raw_buffer_store_b128(lo, ro, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(hi, ro, off + 16, 0, 0);
    }
    t = tn;
  }
}

// ---------------------------------------------------------------------------
static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

template <int NOB, int NW, int KCAP>
static hipError_t launch_ks_t(const void* a, const void* spec, const float* bias, void* out,
                              int64_t N, int K, int k_pad, int n_out, int n_pad, hipStream_t s) {
  constexpr int BN = NOB * 16;
  const int n_ct = (n_out + BN - 1) / BN;
  const int64_t n_rt = (N + 15) / 16;
  // one work-group per CU (the weight spectra fill most of the LDS); waves
  // without a tile exit at once, so only cap by the number of row tiles
  int qx = 256 / (8 * n_ct);
  if (qx < 1) qx = 1;
  const int64_t max_qx = (n_rt + 7) / 8;
  if (qx > max_qx) qx = (int)(max_qx < 1 ? 1 : max_qx);
  qx = env_int("EQL_KS_QX", qx);
  const unsigned blocks = (unsigned)(8 * n_ct * qx);
  hipLaunchKernelGGL((k_gemm_kstream_f16<NOB, NW, KCAP>), dim3(blocks), dim3(NW * 64), 0, s,
                     (const _Float16*)a, (const _Float16*)spec, bias, (_Float16*)out, (int)N, K,
                     n_out, n_pad, k_pad, n_ct, qx);
  return hipGetLastError();
}

// hipErrorNotSupported when outside this kernel's limits.
hipError_t launch_kstream(eqlinear_dtype_t dt, const void* a, const void* spec, const float* bias,
                          void* out, int64_t N, int K, int k_pad, int n_out, int n_pad,
                          hipStream_t s) {
  if (env_int("EQL_NO_KSTREAM", 0) || dt != EQL_F16) return hipErrorNotSupported;
  // the three-slot load ring hands step 0 of the next tile to slot 0, which
  // needs a multiple of three 32-channel steps
  if (K != k_pad || K % 96 != 0 || n_out % 4 != 0) return hipErrorNotSupported;
  if ((int64_t)n_pad * k_pad * 2 >= (1LL << 31)) return hipErrorNotSupported;
  const int nob = env_int("EQL_KS_NOB", 3);
  const int nw = env_int("EQL_KS_NW", 8);
#define EQL_KS_CASE(NOB_, NW_, KCAP_)                                                       \
  if (nob == NOB_ && nw == NW_ && k_pad <= KCAP_ && 4 * NOB_ * 16 * (KCAP_ + 8) * 2 <= 160 * 1024) \
    return launch_ks_t<NOB_, NW_, KCAP_>(a, spec, bias, out, N, K, k_pad, n_out, n_pad, s);
  EQL_KS_CASE(3, 8, 384)
  EQL_KS_CASE(3, 4, 384)
  EQL_KS_CASE(2, 8, 384)
  EQL_KS_CASE(2, 4, 384)
  EQL_KS_CASE(2, 8, 576)
  EQL_KS_CASE(1, 8, 1152)
#undef EQL_KS_CASE
  return hipErrorNotSupported;
}

}  // namespace eql
