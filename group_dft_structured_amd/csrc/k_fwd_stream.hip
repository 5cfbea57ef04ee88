// Streaming spectral GEMM for reduction widths that fit a work-group's LDS:
// forward of the p4 EQ-Linear layer (and any pass with the same shape).
//
// Same arithmetic as the tiled kernel (Flash EQ-Linear, "Approccio
// Algoritmico" / "Specializzazione per il Gruppo di Rotazione p4"):
//     Y0 = X0 W0   Y2 = X2 W2   Yr = Xr Wr - Xi Wi   Yi = Xr Wi + Xi Wr
// organised for HBM streaming on CDNA4:
//  * a persistent work-group owns BN output channels and copies their weight
//    spectra (all K reduction channels) into LDS once;
//  * every wave streams 16-row tiles: it loads its rows of x straight into
//    registers in the matrix-core operand layout and applies the length-4
//    butterfly there (no LDS round trip for x).  X0 and X2 come out of
//    v_dot2_f32_f16 with +-1 coefficients (exact in fp32, one rounding to
//    binary16); Xr and -Xi come out of one packed binary16 subtraction,
//    correctly rounded.  -Xi is kept as a fifth operand plane so that no
//    weight fragment ever needs negating;
//  * the six products run on 16x16 matrix-core tiles with the weights as the
//    A operand and x as the B operand, so each lane ends with 4 consecutive
//    output channels of one row: the epilogue (inverse butterfly, bias) writes
//    32 contiguous bytes per lane (binary16; 64 for binary32), one 16-channel
//    block at a time, overlapping the next block's products.
// Work-groups that own different channel ranges of the same row tiles are
// placed on the same XCD (work-group id modulo 8), so the x tile they share
// is served from that XCD's L2.
#include "eql_device.h"
#include "eql_internal.h"

namespace eql {

namespace {

typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx4_t mma16_f16(half8 a, half8 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4_t mma16_f32(float a, float b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Work-group -> (output channel range j, worker q).  Work-groups with the
// same worker id live on the same XCD.
struct WgMap {
  int j, q, Q;
};
__device__ __forceinline__ WgMap map_wg(int n_ct, int Qx) {
  const int wg = blockIdx.x, xcd = wg & 7, slot = wg >> 3;
  WgMap m;
  m.j = slot % n_ct;
  m.q = (slot / n_ct) * 8 + xcd;
  m.Q = Qx * 8;
  return m;
}

// Copy 4 weight planes [n_pad][k_pad] rows [col0, col0+BN) into LDS
// Bs[p][col][k] with row stride SKB elements, and the bias of the range.
template <typename T, int BN, int NT>
__device__ __forceinline__ void stage_weights(const T* __restrict__ spec, const float* __restrict__ bias,
                                              int n_pad, int k_pad, int col0, int SKB,
                                              T* __restrict__ Bs, float* __restrict__ bs) {
  constexpr int EPU = 16 / (int)sizeof(T);
  const int upr = k_pad / EPU;  // 16-byte units per row
  const int units = 4 * BN * upr;
  const int64_t plane = (int64_t)n_pad * k_pad;
  for (int u = threadIdx.x; u < units; u += NT) {
    const int p = u / (BN * upr), rem = u % (BN * upr);
    const int c = rem / upr, k = (rem % upr) * EPU;
    const uint4 v = *reinterpret_cast<const uint4*>(spec + p * plane + (int64_t)(col0 + c) * k_pad + k);
    *reinterpret_cast<uint4*>(Bs + (p * BN + c) * SKB + k) = v;
  }
  for (int c = threadIdx.x; c < BN; c += NT) bs[c] = bias[col0 + c];
}

// Inverse butterfly + bias for one (row, channel): 4 outputs.
__device__ __forceinline__ floatx4 epilogue4(float Y0, float Y2, float Yr, float Yi, float b) {
  const float u = __builtin_fmaf(Y0, 0.25f, b);
  const float p = __builtin_fmaf(Y2, 0.25f, u);   // (Y0 + Y2)/4 + b
  const float m = __builtin_fmaf(Y2, -0.25f, u);  // (Y0 - Y2)/4 + b
  floatx4 o;
  o[0] = __builtin_fmaf(Yr, 0.5f, p);
  o[1] = __builtin_fmaf(Yi, -0.5f, m);
  o[2] = __builtin_fmaf(Yr, -0.5f, p);
  o[3] = __builtin_fmaf(Yi, 0.5f, m);
  return o;
}

}  // namespace

// ---------------------------------------------------------------------------
// binary16, 16x16x32 matrix-core tiles.  In k-step s, lane (i16 = l % 16,
// g = l / 16) holds row i16 of the x tile and reduction channels
// s*32 + 8g .. +7; the weight fragment of the same lane is output channel i16
// of the 16-channel block and the same reduction channels.
template <int BN, int NW, int KS>
__global__ __launch_bounds__(NW * 64) void k_fwd_stream_f16(
    const _Float16* __restrict__ x, const _Float16* __restrict__ spec, const float* __restrict__ bias,
    _Float16* __restrict__ y, int N, int K, int n_out, int n_pad, int n_ct, int Qx) {
  constexpr int NT = NW * 64;
  constexpr int NB = BN / 16;
  constexpr int KP = KS * 32;       // padded reduction width
  constexpr int SKB = KP + 8;       // LDS row stride (elements)
  constexpr int PL = BN * SKB;      // LDS plane stride
  __shared__ __attribute__((aligned(16))) _Float16 Bs[4 * PL];
  __shared__ float bs[BN];
  const WgMap m = map_wg(n_ct, Qx);
  const int col0 = m.j * BN;
  stage_weights<_Float16, BN, NT>(spec, bias, n_pad, KP, col0, SKB, Bs, bs);
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i16 = lane & 15, g = lane >> 4;
  const int n_rt = (N + 15) / 16;
  const _Float16* wbase = Bs + i16 * SKB + 8 * g;
  const half2_t ones = {(_Float16)1.f, (_Float16)1.f};
  const half2_t pm = {(_Float16)1.f, (_Float16)-1.f};

  for (int t = m.q * NW + wave; t < n_rt; t += m.Q * NW) {
    const int row = t * 16 + i16;
    const bool row_ok = row < N;
    // x fragments: xs[s][v] holds channels s*32 + 8g + 2v, +1 (4 group elements each)
    half8 xs[KS][4];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int c = s * 32 + 8 * g;
      if (row_ok && c < K) {
        const half8* src = reinterpret_cast<const half8*>(x + ((int64_t)row * K + c) * 4);
#pragma unroll
        for (int v = 0; v < 4; ++v) xs[s][v] = src[v];
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) xs[s][v] = half8{};
      }
    }
    // butterfly -> planes X0, X2, Xr, Xi, Xq = -Xi
    half8 a0[KS], a2[KS], ar[KS], ai[KS], aq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const half8& w = xs[s][e >> 1];
        const int o = (e & 1) * 4;
        const half2_t x01 = {w[o], w[o + 1]}, x23 = {w[o + 2], w[o + 3]};
        const float f0 = __builtin_amdgcn_fdot2(x01, ones, __builtin_amdgcn_fdot2(x23, ones, 0.f, false), false);
        const float f2 = __builtin_amdgcn_fdot2(x01, pm, __builtin_amdgcn_fdot2(x23, pm, 0.f, false), false);
        const half2_t d = x01 - x23;  // (x0 - x2, x1 - x3) = (Xr, -Xi)
        a0[s][e] = (_Float16)f0;
        a2[s][e] = (_Float16)f2;
        ar[s][e] = d[0];
        aq[s][e] = d[1];
      }
      ai[s] = -aq[s];
    }
    // one 16-channel block per iteration: kept rolled so that only one
    // block's weight fragments are live (the x planes stay in registers)
#pragma unroll 1
    for (int nb = 0; nb < NB; ++nb) {
      floatx4_t c0 = {}, c2 = {}, cr = {}, ci = {};
      const _Float16* wp = wbase + nb * 16 * SKB;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const half8 w0 = *reinterpret_cast<const half8*>(wp + 0 * PL + s * 32);
        const half8 w2 = *reinterpret_cast<const half8*>(wp + 1 * PL + s * 32);
        const half8 wr = *reinterpret_cast<const half8*>(wp + 2 * PL + s * 32);
        const half8 wi = *reinterpret_cast<const half8*>(wp + 3 * PL + s * 32);
        c0 = mma16_f16(w0, a0[s], c0);
        cr = mma16_f16(wr, ar[s], cr);
        c2 = mma16_f16(w2, a2[s], c2);
        ci = mma16_f16(wi, ar[s], ci);
        cr = mma16_f16(wi, aq[s], cr);
        ci = mma16_f16(wr, ai[s], ci);
      }
      // lane holds output channels col0 + nb*16 + 4g + r (r = 0..3) of row `row`
      const int cl = nb * 16 + 4 * g;
      const int col = col0 + cl;
      if (row_ok && col < n_out) {
        _Float16* dst = y + ((int64_t)row * n_out + col) * 4;
        half8 o01, o23;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const floatx4 o = epilogue4(c0[r], c2[r], cr[r], ci[r], bs[cl + r]);
          half8& h = r < 2 ? o01 : o23;
          const int b = (r & 1) * 4;
          h[b + 0] = (_Float16)o[0];
          h[b + 1] = (_Float16)o[1];
          h[b + 2] = (_Float16)o[2];
          h[b + 3] = (_Float16)o[3];
        }
        // 16-byte stores need an even channel count (row starts 16-byte aligned)
        if ((n_out & 1) == 0 && col + 4 <= n_out) {
          __builtin_nontemporal_store(o01, reinterpret_cast<half8*>(dst));
          __builtin_nontemporal_store(o23, reinterpret_cast<half8*>(dst + 8));
        } else {
          // odd channel count or ragged last block: 8-byte stores of the
          // channels that exist
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (col + r < n_out) {
              const half8& h = r < 2 ? o01 : o23;
              const int b = (r & 1) * 4;
              half4 q = {h[b], h[b + 1], h[b + 2], h[b + 3]};
              *reinterpret_cast<half4*>(dst + 4 * r) = q;
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// binary32, 16x16x4 matrix-core tiles.  Lane (i16, g) holds row i16 and, in
// k-step e, reduction channel g*(KP/4) + e, so each lane reads a contiguous
// run of channels of its row.
template <int BN, int NW, int KS>
__global__ __launch_bounds__(NW * 64) void k_fwd_stream_f32(
    const float* __restrict__ x, const float* __restrict__ spec, const float* __restrict__ bias,
    float* __restrict__ y, int N, int K, int n_out, int n_pad, int n_ct, int Qx) {
  constexpr int NT = NW * 64;
  constexpr int NB = BN / 16;
  constexpr int KP = KS * 32;
  constexpr int CPL = KP / 4;   // channels per lane
  constexpr int SKB = KP + 4;
  constexpr int PL = BN * SKB;
  __shared__ __attribute__((aligned(16))) float Bs[4 * PL];
  __shared__ float bs[BN];
  const WgMap m = map_wg(n_ct, Qx);
  const int col0 = m.j * BN;
  stage_weights<float, BN, NT>(spec, bias, n_pad, KP, col0, SKB, Bs, bs);
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i16 = lane & 15, g = lane >> 4;
  const int n_rt = (N + 15) / 16;
  const float* wbase = Bs + i16 * SKB + g * CPL;

  for (int t = m.q * NW + wave; t < n_rt; t += m.Q * NW) {
    const int row = t * 16 + i16;
    const bool row_ok = row < N;
    float a0[CPL], a2[CPL], ar[CPL], ai[CPL], aq[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const int c = g * CPL + e;
      floatx4 v = {0.f, 0.f, 0.f, 0.f};
      if (row_ok && c < K) v = *reinterpret_cast<const floatx4*>(x + ((int64_t)row * K + c) * 4);
      const float s02 = v[0] + v[2], s13 = v[1] + v[3];
      a0[e] = s02 + s13;
      a2[e] = s02 - s13;
      ar[e] = v[0] - v[2];
      ai[e] = v[3] - v[1];
      aq[e] = v[1] - v[3];
    }
#pragma unroll 1
    for (int nb = 0; nb < NB; ++nb) {
      floatx4_t c0 = {}, c2 = {}, cr = {}, ci = {};
      const float* wp = wbase + nb * 16 * SKB;
#pragma unroll
      for (int e4 = 0; e4 < CPL; e4 += 4) {
        const floatx4 w0 = *reinterpret_cast<const floatx4*>(wp + 0 * PL + e4);
        const floatx4 w2 = *reinterpret_cast<const floatx4*>(wp + 1 * PL + e4);
        const floatx4 wr = *reinterpret_cast<const floatx4*>(wp + 2 * PL + e4);
        const floatx4 wi = *reinterpret_cast<const floatx4*>(wp + 3 * PL + e4);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = e4 + u;
          c0 = mma16_f32(w0[u], a0[e], c0);
          cr = mma16_f32(wr[u], ar[e], cr);
          c2 = mma16_f32(w2[u], a2[e], c2);
          ci = mma16_f32(wi[u], ar[e], ci);
          cr = mma16_f32(wi[u], aq[e], cr);
          ci = mma16_f32(wr[u], ai[e], ci);
        }
      }
      const int cl = nb * 16 + 4 * g;
      const int col = col0 + cl;
      if (row_ok) {
        float* dst = y + ((int64_t)row * n_out + col) * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (col + r < n_out) {
            const floatx4 o = epilogue4(c0[r], c2[r], cr[r], ci[r], bs[cl + r]);
            __builtin_nontemporal_store(o, reinterpret_cast<floatx4*>(dst + 4 * r));
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

template <typename T>
static hipError_t launch_stream_kernel(void (*kern)(const T*, const T*, const float*, T*, int, int,
                                                    int, int, int, int),
                                       int nw, int n_ct, int Qx, const void* a, const void* spec,
                                       const float* bias, void* out, int64_t N, int K, int n_out,
                                       int n_pad, hipStream_t s) {
  const unsigned blocks = (unsigned)(8 * n_ct * Qx);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * nw), 0, s, (const T*)a, (const T*)spec, bias,
                     (T*)out, (int)N, K, n_out, n_pad, n_ct, Qx);
  return hipGetLastError();
}

// Workers per XCD and channel range: about `wg_per_cu` work-groups per CU,
// fewer when there are not enough row tiles to share.
static int pick_qx(int64_t N, int n_ct, int nw, int wg_per_cu) {
  const int64_t tiles = (N + 15) / 16;
  int qx = (256 * wg_per_cu) / (8 * n_ct);
  if (qx < 1) qx = 1;
  const int64_t max_qx = (tiles + 8LL * nw - 1) / (8LL * nw);
  if (qx > max_qx) qx = (int)(max_qx < 1 ? 1 : max_qx);
  return env_int("EQL_STREAM_QX", qx);
}

// Output-channel range per work-group: the listed width that wastes the
// fewest padded channels (ties go to the wider range).
static int pick_bn(int n_out, const int* opts, int n_opts) {
  int best = opts[0];
  int64_t best_waste = -1;
  for (int i = 0; i < n_opts; ++i) {
    const int bn = opts[i];
    const int64_t waste = (int64_t)((n_out + bn - 1) / bn) * bn - n_out;
    if (best_waste < 0 || waste < best_waste || (waste == best_waste && bn > best)) {
      best = bn;
      best_waste = waste;
    }
  }
  return env_int("EQL_STREAM_BN", best);
}

#define EQL_STREAM_CASE(KERN, T, BN_, NW_, KS_)                                                  \
  if (bn == BN_ && nw == NW_ && ks == KS_)                                                       \
    return launch_stream_kernel<T>(KERN<BN_, NW_, KS_>, NW_, n_ct, qx, a, spec, bias, out, N, K, \
                                   n_out, n_pad, s);

// Returns hipErrorNotSupported when the shape is outside the streaming
// kernel's limits (the caller then uses the tiled kernel).
hipError_t launch_stream(eqlinear_dtype_t dt, const void* a, const void* spec, const float* bias,
                         void* out, int64_t N, int K, int k_pad, int n_out, int n_pad, hipStream_t s) {
  if (env_int("EQL_NO_STREAM", 0)) return hipErrorNotSupported;
  if (K % 8 != 0 || k_pad % 32 != 0) return hipErrorNotSupported;
  const int ks = k_pad / 32;
  const int nw = env_int("EQL_STREAM_NW", 8);
  const int wpc = env_int("EQL_STREAM_WPC", 1);
  if (dt == EQL_F16) {
    static const int opts96[] = {128, 96, 64};
    static const int opts192[] = {96, 64};
    const int bn = ks <= 3 ? pick_bn(n_out, opts96, 3) : pick_bn(n_out, opts192, 2);
    const int n_ct = (n_out + bn - 1) / bn;
    const int qx = pick_qx(N, n_ct, nw, wpc);
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 128, 8, 3)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 96, 8, 3)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 64, 8, 3)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 128, 4, 3)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 64, 4, 3)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 128, 8, 2)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 96, 8, 2)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 64, 8, 2)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 128, 8, 1)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 96, 8, 1)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 64, 8, 1)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 96, 8, 6)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 64, 8, 6)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 96, 4, 6)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 64, 4, 6)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 96, 8, 4)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 64, 8, 4)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 96, 8, 5)
    EQL_STREAM_CASE(k_fwd_stream_f16, _Float16, 64, 8, 5)
    return hipErrorNotSupported;
  }
  static const int opts_f32[] = {96, 64, 32};
  const int bn = pick_bn(n_out, opts_f32, 3);
  const int n_ct = (n_out + bn - 1) / bn;
  const int qx = pick_qx(N, n_ct, nw, wpc);
  EQL_STREAM_CASE(k_fwd_stream_f32, float, 96, 8, 3)
  EQL_STREAM_CASE(k_fwd_stream_f32, float, 64, 8, 3)
  EQL_STREAM_CASE(k_fwd_stream_f32, float, 32, 8, 3)
  EQL_STREAM_CASE(k_fwd_stream_f32, float, 96, 4, 3)
  EQL_STREAM_CASE(k_fwd_stream_f32, float, 64, 4, 3)
  EQL_STREAM_CASE(k_fwd_stream_f32, float, 96, 8, 2)
  EQL_STREAM_CASE(k_fwd_stream_f32, float, 64, 8, 2)
  EQL_STREAM_CASE(k_fwd_stream_f32, float, 32, 8, 2)
  EQL_STREAM_CASE(k_fwd_stream_f32, float, 96, 8, 1)
  EQL_STREAM_CASE(k_fwd_stream_f32, float, 64, 8, 1)
  EQL_STREAM_CASE(k_fwd_stream_f32, float, 32, 8, 1)
  return hipErrorNotSupported;
}
#undef EQL_STREAM_CASE

}  // namespace eql
