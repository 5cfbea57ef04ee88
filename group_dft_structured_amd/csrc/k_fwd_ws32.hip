// Forward of the p4 EQ-Linear layer in binary32 with producer and consumer
// waves (reduction widths that are multiples of 16 channels, up to 192).
//
// Arithmetic (Flash EQ-Linear, "Approccio Algoritmico" and "Specializzazione
// per il Gruppo di Rotazione p4"): with the group DFT of x and of the weight,
//     Y0 = X0 W0   Y2 = X2 W2   Yr = Xr Wr - Xi Wi   Yi = Xr Wi + Xi Wr
// six real products, then the inverse length-4 butterfly and the bias; all
// in fp32 (the transforms are sums of four values, the products run on
// v_mfma_f32_16x16x4_f32).
//
// Organisation on CDNA4, as for the binary16 kernel: a persistent work-group
// owns BN = 16*NC output channels and walks 16-row tiles of x;
//  * NP producer waves load each tile three tiles ahead (16-byte buffer
//    loads in a register ring), apply the length-4 butterfly and write the
//    four planes to LDS in matrix-core fragment order (double buffered);
//  * NC consumer waves keep the weight spectra of 16 output channels in
//    VGPRs, run the products from LDS and store 64 contiguous bytes per lane
//    (four output channels of one row), or leave the tile in LDS for the
//    producers to store (PST, below).
// The reduction index is permuted identically for both operands so that a
// lane's four consecutive k-steps read 16 contiguous bytes: within a block
// of 16 channels, lane group g at k-step e handles channel 4g + e.  Its
// weights are then one 16-byte load per plane and block, and its x values
// one 16-byte LDS read per plane and block.
#include "eql_device.h"
#include "eql_internal.h"

namespace eql {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// inverse butterfly of one (row, channel) with its bias, fp32
__device__ __forceinline__ f32x4 epi4_32(float Y0, float Y2, float Yr, float Yi, float b) {
  const float u = __builtin_fmaf(Y0, 0.25f, b);
  const float p = __builtin_fmaf(Y2, 0.25f, u);   // (Y0 + Y2)/4 + b
  const float m = __builtin_fmaf(Y2, -0.25f, u);  // (Y0 - Y2)/4 + b
  f32x4 o;
  o[0] = __builtin_fmaf(Yr, 0.5f, p);
  o[1] = __builtin_fmaf(Yi, -0.5f, m);
  o[2] = __builtin_fmaf(Yr, -0.5f, p);
  o[3] = __builtin_fmaf(Yi, 0.5f, m);
  return o;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc32(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

}  // namespace

// LDS per buffer: plane p, channel block j (16 channels): 1 KB at
// (p*KB + j)*256 floats; lane (i16, g) reads the 16 bytes at (g*16 + i16)*4
// floats = row i16, channels 16j + 4g .. 16j + 4g + 3.
//
// PST: the consumers leave each output tile in LDS (rows of BN channels x 16
// bytes, a 16-byte pad per row so that 8 consecutive lanes' 16-byte writes
// of 8 rows land on distinct banks; double buffered) and the producers write
// it out as whole rows during the next tile, so the consumers' matrix-core
// stream never waits on a store.
template <int NC, int NP, int KB, int YP, bool ACT = false, bool PST = false>
__global__ __launch_bounds__((NC + NP) * 64) void k_fwd_ws_f32(
    const float* __restrict__ x, const float* __restrict__ spec, const float* __restrict__ bias,
    float* __restrict__ y, int N, int K, int n_out, int n_pad, int n_ct, int Qx, int act) {
  constexpr int BN = NC * 16;
  constexpr int KP = KB * 16;                 // reduction channels
  constexpr int FRAG = 256;                   // floats per fragment block
  constexpr int PS = KB * FRAG;               // plane stride (floats)
  constexpr int BUF = 4 * PS;                 // floats per buffer
  constexpr int PT = NP * 64;                 // producer threads
  constexpr int UNITS = 16 * (KP / 4);        // (row, 4 channels) units per tile
  constexpr int UPT = (UNITS + PT - 1) / PT;  // per producer thread
  constexpr int LPT = 4 * UPT;                // 16-byte loads per producer thread
  constexpr int DUMMY = (UNITS % PT != 0) ? 4 * PT : 0;  // floats
  constexpr int OPITCH = BN * 4 + 4;  // floats per staged output row
  constexpr int OBUF = 16 * OPITCH;   // floats per staged output tile
  __shared__ __attribute__((aligned(16))) float xs[2 * BUF + DUMMY + (PST ? 2 * OBUF : 0)];
  float* const obuf = xs + 2 * BUF + DUMMY;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wgid = blockIdx.x, xcd = wgid & 7, slot = wgid >> 3;
  const int j = slot % n_ct;
  const int q = (slot / n_ct) * 8 + xcd, Q = Qx * 8;
  const int n_rt = (N + 15) / 16;
  const int n_my = q < n_rt ? (n_rt - 1 - q) / Q + 1 : 0;  // tiles of this worker
  if (n_my == 0) return;  // whole work-group

  if (wave >= NC) {
    // =========================== producer waves ===========================
    const int ptid = tid - NC * 64;
    const int64_t row_elems = (int64_t)K * 4;
    // unit u -> (row = u % 16, 4-channel group c4 = u / 16): four 16-byte
    // loads (one channel's four group values each), contiguous in the row
    auto load_tile = [&](f32x4 (&raw)[LPT], int i) {
      const int64_t r0 = (int64_t)(q + (int64_t)i * Q) * 16;
      const int64_t rows = r0 < N ? (N - r0 < 16 ? N - r0 : 16) : 0;
      const __amdgpu_buffer_rsrc_t rx = rsrc32(x + (r0 < N ? r0 : 0) * row_elems, (uint32_t)(rows * row_elems * 4));
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const int u = k * PT + ptid;
        const int row = u % 16, c4 = u / 16;
        const bool real = UNITS % PT == 0 || u < UNITS;
        const uint32_t off = (uint32_t)(row * row_elems + 16 * c4) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          raw[4 * k + e] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, real ? off + 16 * e : 0x7FFFFFF0u, 0, 0));
      }
    };
    auto store_tile = [&](const f32x4 (&raw)[LPT], float* buf) {
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const int u = k * PT + ptid;
        const int row = u % 16, c4 = u / 16;
        const int jb = c4 >> 2, g = c4 & 3;
        const bool real = UNITS % PT == 0 || u < UNITS;
        f32x4 p0, p2, pr, pi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // channel 4*c4 + e: values t = 0..3
          const f32x4 v = raw[4 * k + e];
          const float s02 = v[0] + v[2], s13 = v[1] + v[3];
          p0[e] = s02 + s13;
          p2[e] = s02 - s13;
          pr[e] = v[0] - v[2];
          pi[e] = v[3] - v[1];
        }
        float* const dummy = xs + 2 * BUF + ptid * 4;
        float* const dst = buf + jb * FRAG + (g * 16 + row) * 4;
        *reinterpret_cast<f32x4*>(real ? dst + 0 * PS : dummy) = p0;
        *reinterpret_cast<f32x4*>(real ? dst + 1 * PS : dummy) = p2;
        *reinterpret_cast<f32x4*>(real ? dst + 2 * PS : dummy) = pr;
        *reinterpret_cast<f32x4*>(real ? dst + 3 * PS : dummy) = pi;
      }
    };
    // PST: write staged output tile t (16 rows x BN channels, 16 bytes = one
    // channel's four group values per lane, whole rows per wave instruction)
    auto store_out = [&](int t) {
      const int64_t r0 = (int64_t)(q + (int64_t)t * Q) * 16;
      const int64_t rows = N - r0 < 16 ? N - r0 : 16;
      const __amdgpu_buffer_rsrc_t ry = rsrc32(y + r0 * n_out * 4, (uint32_t)(rows * n_out * 16));
      const float* const sb = obuf + (t & 1) * OBUF;
      constexpr int CH = 16 * BN;              // 16-byte chunks per tile
      constexpr int SPT = (CH + PT - 1) / PT;  // per producer thread
#pragma unroll
      for (int k = 0; k < SPT; ++k) {
        const int u0 = k * PT + ptid;
        const bool real = CH % PT == 0 || u0 < CH;
        const int u = real ? u0 : 0;
        const int row = u / BN, ch = u % BN;
        const u32x4 v = *reinterpret_cast<const u32x4*>(sb + row * OPITCH + 4 * ch);
        const int col = j * BN + ch;
        const uint32_t off = (real && col < n_out) ? (uint32_t)((row * n_out + col) * 16) : 0x7FFFFFF0u;
        __builtin_amdgcn_raw_buffer_store_b128(v, ry, off, 0, YP);
      }
    };
    // phase p first writes out the tile the consumers staged in phase p - 1
    auto out_step = [&](int p) {
      if (PST && p >= 1) store_out(p - 1);
    };
    // Ring: tile i sits in slot i % 3 from its load until its transform;
    // between barriers i and i+1 the producers transform tile i+1 and load
    // tile i+4 into the slot it frees.  Tiles past the end load as zeros.
    // Every work-group's first tile is requested before any later one.
    f32x4 ra[LPT], rb[LPT], rc[LPT];
    load_tile(ra, 0);
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0): expcnt, lgkmcnt not waited
    load_tile(rb, 1);
    load_tile(rc, 2);
    store_tile(ra, xs);
    load_tile(ra, 3);
    __syncthreads();  // barrier 0: tile 0 is in buffer 0
    __builtin_amdgcn_sched_barrier(0);
    int cur = 1;
    int i = 0;
    for (; i + 3 <= n_my - 1; i += 3) {
      out_step(i);
      store_tile(rb, xs + cur * BUF);
      __builtin_amdgcn_sched_barrier(0);
      load_tile(rb, i + 4);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      cur ^= 1;
      out_step(i + 1);
      store_tile(rc, xs + cur * BUF);
      __builtin_amdgcn_sched_barrier(0);
      load_tile(rc, i + 5);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      cur ^= 1;
      out_step(i + 2);
      store_tile(ra, xs + cur * BUF);
      __builtin_amdgcn_sched_barrier(0);
      load_tile(ra, i + 6);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      cur ^= 1;
    }
    const int rest = n_my - 1 - i;  // 0, 1 or 2 transforms left
    if (rest > 0) {
      out_step(i);
      store_tile(rb, xs + cur * BUF);
      __syncthreads();
      cur ^= 1;
      if (rest > 1) {
        out_step(i + 1);
        store_tile(rc, xs + cur * BUF);
        __syncthreads();
      }
    }
    if (PST) {
      out_step(n_my - 1);
      __syncthreads();  // barrier n_my: the last tile is staged
      store_out(n_my - 1);
    }
  } else {
    // =========================== consumer waves ===========================
    const int i16 = lane & 15, g = lane >> 4;
    const int d0 = j * BN + wave * 16;  // this wave's first output channel
    // weight fragments (A operand): channel d0 + i16, reduction channels
    // 16jb + 4g .. 16jb + 4g + 3 (one per k-step e of block jb)
    f32x4 w0[KB], w2[KB], wr[KB], wi[KB];
    float bc[4];
    {
      const uint32_t plane_bytes = (uint32_t)n_pad * KP * 4;
      const int64_t plane = (int64_t)n_pad * KP;
      const __amdgpu_buffer_rsrc_t r0 = rsrc32(spec, plane_bytes), r2 = rsrc32(spec + plane, plane_bytes);
      const __amdgpu_buffer_rsrc_t rr = rsrc32(spec + 2 * plane, plane_bytes);
      const __amdgpu_buffer_rsrc_t ri = rsrc32(spec + 3 * plane, plane_bytes);
      const __amdgpu_buffer_rsrc_t rb = rsrc32(bias, (uint32_t)n_pad * 4);
      const uint32_t off = (uint32_t)((d0 + i16) * KP + 4 * g) * 4;
#pragma unroll
      for (int jb = 0; jb < KB; ++jb) {
        w0[jb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r0, off + jb * 64, 0, 0));
        w2[jb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r2, off + jb * 64, 0, 0));
        wr[jb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, off + jb * 64, 0, 0));
        wi[jb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ri, off + jb * 64, 0, 0));
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        bc[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, (d0 + 4 * g + r) * 4, 0, 0));
    }
    struct Acc {
      f32x4 c0, c2, cr, ci;
    };
    auto products = [&](Acc& a, const float* buf) {
      a.c0 = a.c2 = a.cr = a.ci = f32x4{};
#pragma unroll
      for (int jb = 0; jb < KB; ++jb) {
        const float* f = buf + jb * FRAG + lane * 4;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(f + 0 * PS);
        const f32x4 x2 = *reinterpret_cast<const f32x4*>(f + 1 * PS);
        const f32x4 xr = *reinterpret_cast<const f32x4*>(f + 2 * PS);
        const f32x4 xi = *reinterpret_cast<const f32x4*>(f + 3 * PS);
        const f32x4 xq = -xi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a.c0 = mma4(w0[jb][e], x0[e], a.c0);
          a.cr = mma4(wr[jb][e], xr[e], a.cr);
          a.c2 = mma4(w2[jb][e], x2[e], a.c2);
          a.ci = mma4(wi[jb][e], xr[e], a.ci);
          a.cr = mma4(wi[jb][e], xq[e], a.cr);
          a.ci = mma4(wr[jb][e], xi[e], a.ci);
        }
      }
    };
    // lane holds channels d0 + 4g + r of row r0 + i16: 64 contiguous bytes
    auto epilogue = [&](int i, const Acc& a) {
      const int64_t r0 = (int64_t)(q + (int64_t)i * Q) * 16;
      const int64_t rows = N - r0 < 16 ? N - r0 : 16;
      const __amdgpu_buffer_rsrc_t ry = rsrc32(y + r0 * n_out * 4, (uint32_t)(rows * n_out * 16));
      const int col = d0 + 4 * g;
      const uint32_t off = col < n_out ? (uint32_t)((i16 * n_out + col) * 16) : 0x7FFFFFF0u;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 v = epi4_32(a.c0[r], a.c2[r], a.cr[r], a.ci[r], bc[r]);
        if constexpr (ACT) {
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = activate(v[t], act);
        }
        if (PST) {
          // row i16, work-group channel wave*16 + 4g + r
          *reinterpret_cast<f32x4*>(obuf + (i & 1) * OBUF + i16 * OPITCH + (wave * 16 + 4 * g + r) * 4) = v;
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ry, off + 16 * r, 0, YP);
        }
      }
    };
    __syncthreads();  // barrier 0
    int cur = 0;
    Acc A;
    for (int i = 0; i < n_my; ++i) {
      products(A, xs + cur * BUF);
      epilogue(i, A);
      cur ^= 1;
      // barrier i+1 (with PST also after the last tile: its staged output is
      // then complete for the producers)
      if (PST || i + 1 < n_my) __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

template <int NC, int NP, int KB>
static hipError_t launch_ws32_t(const void* x, const void* spec, const float* bias, void* y, int64_t N,
                                int K, int n_out, int n_pad, int act, hipStream_t s) {
  constexpr int BN = NC * 16;
  const int n_ct = (n_out + BN - 1) / BN;
  const int64_t n_rt = (N + 15) / 16;
  int qx = 256 / (8 * n_ct);
  if (qx < 1) qx = 1;
  const int64_t max_qx = (n_rt + 7) / 8;
  if (qx > max_qx) qx = (int)(max_qx < 1 ? 1 : max_qx);
  qx = env_int("EQL_WS32_QX", qx);
  const unsigned blocks = (unsigned)(8 * n_ct * qx);
  const int64_t y_bytes = N * (int64_t)n_out * 16;
  const bool stream = env_int("EQL_WS32_STREAM", y_bytes <= (128LL << 20) ? 1 : 0) != 0;
  // Output path (measured on MI355X): outputs inside the memory-side cache
  // are stored by the producers from LDS (C=96, D=96, N=12608: 26.1 us
  // against 30.4 with the consumers storing; 30.8 against 36.0 with GELU);
  // larger ones by the consumers (C=192, D=768: producer stores measured
  // 4038 us against 3690).
  const bool pst = env_int("EQL_WS32_PST", y_bytes <= (128LL << 20) ? 1 : 0) != 0;
  const dim3 grid(blocks), block((NC + NP) * 64);
#define EQL_WS32_LAUNCH(YP_, ACT_, PST_)                                                              \
  hipLaunchKernelGGL((k_fwd_ws_f32<NC, NP, KB, YP_, ACT_, PST_>), grid, block, 0, s, (const float*)x,  \
                     (const float*)spec, bias, (float*)y, (int)N, K, n_out, n_pad, n_ct, qx, act)
#define EQL_WS32_MODES(YP_, ACT_)                      \
  do {                                                 \
    if (pst) EQL_WS32_LAUNCH(YP_, ACT_, true);         \
    else EQL_WS32_LAUNCH(YP_, ACT_, false);            \
  } while (0)
  if (act != ACT_NONE && stream) EQL_WS32_MODES(2, true);
  else if (act != ACT_NONE) EQL_WS32_MODES(0, true);
  else if (stream) EQL_WS32_MODES(2, false);
  else EQL_WS32_MODES(0, false);
#undef EQL_WS32_MODES
#undef EQL_WS32_LAUNCH
  return hipGetLastError();
}

// hipErrorNotSupported when outside this kernel's limits.
hipError_t launch_ws32(eqlinear_dtype_t dt, const void* x, const void* spec, const float* bias, void* y,
                       int64_t N, int K, int k_pad, int n_out, int n_pad, int act, hipStream_t s) {
  if (env_int("EQL_NO_WS32", 0) || dt != EQL_F32) return hipErrorNotSupported;
  // whole 16-channel reduction blocks read without a channel mask, whole
  // 4-channel output groups (64-byte stores)
  if (K != k_pad || K % 16 != 0 || n_out % 4 != 0) return hipErrorNotSupported;
  if ((int64_t)n_pad * k_pad * 4 >= (1LL << 31) || (int64_t)16 * n_out * 16 >= (1LL << 31))
    return hipErrorNotSupported;
  const int kb = k_pad / 16;
  // consumers: one per output block of 16 (up to 8); their weight
  // fragments take 16*kb VGPRs, so long reductions use four
  const int nc_default = (kb > 6 || (kb == 6 && n_out > 96)) ? 4 : (n_out <= 96 ? 6 : 8);
  const int nc = env_int("EQL_WS32_NC", nc_default);
  const int np = env_int("EQL_WS32_NP", kb > 6 ? 4 : 2);
  if ((int64_t)((n_out + 16 * nc - 1) / (16 * nc)) * 16 * nc > n_pad) return hipErrorNotSupported;
#define EQL_WS32_CASE(NC_, NP_, KB_) \
  if (nc == NC_ && np == NP_ && kb == KB_) return launch_ws32_t<NC_, NP_, KB_>(x, spec, bias, y, N, K, n_out, n_pad, act, s);
  EQL_WS32_CASE(6, 2, 6)
  EQL_WS32_CASE(4, 2, 6)
  EQL_WS32_CASE(6, 2, 2)
  EQL_WS32_CASE(6, 2, 4)
  EQL_WS32_CASE(8, 2, 2)
  EQL_WS32_CASE(8, 2, 4)
  EQL_WS32_CASE(4, 4, 8)
  EQL_WS32_CASE(4, 4, 12)
#undef EQL_WS32_CASE
  return hipErrorNotSupported;
}

}  // namespace eql
