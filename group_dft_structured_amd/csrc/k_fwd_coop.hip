// Weight-stationary, software-pipelined spectral GEMM: the forward of the p4
// EQ-Linear layer for reduction widths up to 192 channels.
//
// Arithmetic (Flash EQ-Linear, "Approccio Algoritmico" and "Specializzazione
// per il Gruppo di Rotazione p4"): with the group DFT of x and of the weight,
//     Y0 = X0 W0   Y2 = X2 W2   Yr = Xr Wr - Xi Wi   Yi = Xr Wi + Xi Wr
// six real products, then the inverse length-4 butterfly and the bias.
//
// Organisation on CDNA4:
//  * a persistent work-group of NW waves owns BN = 16*NB*NW output channels;
//    every wave keeps the four weight-spectrum fragments of its 16*NB
//    channels (all K reduction channels) in VGPRs for the whole kernel;
//  * the work-group walks 16*MR-row tiles of x: the tile is read with
//    coalesced 16-byte loads, transformed once by the length-4 butterfly
//    (X0, X2 exact in fp32 via v_dot2 with +-1, rounded once to binary16;
//    Xr and -Xi by one correctly rounded packed subtraction; Xi = -(-Xi)),
//    and written to LDS in matrix-core fragment order, double buffered;
//  * while the matrix cores work on tile i (16x16x32 f16, weights as the A
//    operand, x from LDS as the B operand), the loads of tile i+1 are in
//    flight; the epilogue (inverse butterfly, bias) then writes 32 contiguous
//    bytes per lane: 4 consecutive output channels of one row.
// Work-groups sharing row tiles (different channel ranges) are placed on the
// same XCD so that the x tile they all read is served by that XCD's L2.
#include "eql_device.h"
#include "eql_internal.h"

namespace eql {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 epi4(float Y0, float Y2, float Yr, float Yi, float b) {
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

// Raw buffer resource over [base, base + bytes): the hardware range check
// turns out-of-range loads into zeros and drops out-of-range stores, so the
// kernel needs no bounds branches (and the compiler can keep memory
// operations in flight across iterations with exact wait counts).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Round two fp32 values to a packed pair of binary16 (round to nearest even).
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

}  // namespace

// LDS fragment layout: for plane p (X0, X2, Xr, Xi), k-step s and row block
// mb, one 1 KB fragment; lane (i16, g) of the B operand reads 16 bytes at
// (g*16 + i16)*16, i.e. consecutive lanes read consecutive 16-byte words.
// Each wave owns NB blocks of 16 output channels, so every x fragment read
// from LDS feeds 6*NB matrix-core products (-Xi is formed in registers).
template <int NW, int NB, int KS, int MR>
__global__ __launch_bounds__(NW * 64) void k_fwd_coop_f16(
    const _Float16* __restrict__ x, const _Float16* __restrict__ spec, const float* __restrict__ bias,
    _Float16* __restrict__ y, int N, int K, int n_out, int n_pad, int k_pad, int n_ct, int Qx) {
  constexpr int NT = NW * 64;
  constexpr int BN = NW * NB * 16;
  constexpr int KP = KS * 32;
  constexpr int RT = 16 * MR;                 // rows per tile
  constexpr int FRAG = 512;                   // halves per fragment
  constexpr int PS = KS * MR * FRAG;          // plane stride (halves)
  constexpr int BUF = 4 * PS;                 // halves per buffer
  constexpr int UNITS = RT * (KP / 2);        // 16-byte loads per tile (2 channels each)
  constexpr int UPT = (UNITS + NT - 1) / NT;  // per thread
  // units past the tile (when NT does not divide UNITS) write their
  // butterfly into a per-thread dummy word after the two buffers, so the
  // transform has no data-dependent branch
  constexpr int DUMMY = (UNITS % NT != 0) ? 2 * NT : 0;  // halves
  __shared__ __attribute__((aligned(16))) _Float16 xs[2 * BUF + DUMMY];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar registers)
  const int i16 = lane & 15, g = lane >> 4;
  // work-group -> (channel range j, worker q); equal q share an XCD
  const int wgid = blockIdx.x, xcd = wgid & 7, slot = wgid >> 3;
  const int j = slot % n_ct;
  const int q = (slot / n_ct) * 8 + xcd, Q = Qx * 8;
  const int d0 = j * BN + wave * NB * 16;  // this wave's first output channel

  // ---- weight fragments (A operand): channel d0 + 16*nb + i16, reduction channels s*32 + 8g.. ----
  half8 w0[NB][KS], w2[NB][KS], wr[NB][KS], wi[NB][KS];
  float bc[NB][4];
  {
    const uint32_t plane_bytes = (uint32_t)n_pad * KP * 2;
    const int64_t plane = (int64_t)n_pad * KP;
    const __amdgpu_buffer_rsrc_t r0 = rsrc(spec, plane_bytes), r2 = rsrc(spec + plane, plane_bytes);
    const __amdgpu_buffer_rsrc_t rr = rsrc(spec + 2 * plane, plane_bytes);
    const __amdgpu_buffer_rsrc_t ri = rsrc(spec + 3 * plane, plane_bytes);
    const __amdgpu_buffer_rsrc_t rb = rsrc(bias, (uint32_t)n_pad * 4);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t off = (uint32_t)((d0 + nb * 16 + i16) * KP + 8 * g) * 2;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        w0[nb][s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r0, off + s * 64, 0, 0));
        w2[nb][s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r2, off + s * 64, 0, 0));
        wr[nb][s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(rr, off + s * 64, 0, 0));
        wi[nb][s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(ri, off + s * 64, 0, 0));
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        bc[nb][r] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rb, (d0 + nb * 16 + 4 * g + r) * 4, 0, 0));
    }
  }

  const int n_rt = (N + RT - 1) / RT;
  const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
  const f16x2 pm = {(_Float16)1.f, (_Float16)-1.f};

  // ---- tile loader: unit u -> (row = u % RT, channel pair cp = u / RT) ----
  const int64_t row_elems = (int64_t)K * 4;  // elements per x row (K == KP)
  auto load_tile = [&](half8 (&raw)[UPT], int t) {
    const int64_t r0 = (int64_t)t * RT;
    const int64_t rows = r0 < N ? (N - r0 < RT ? N - r0 : RT) : 0;
    const __amdgpu_buffer_rsrc_t rx = rsrc(x + r0 * row_elems, (uint32_t)(rows * row_elems * 2));
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = k * NT + tid;
      const int row = u % RT, cp = u / RT;
      // units past the tile size read beyond the range and come back as zeros
      const uint32_t off = (UNITS % NT == 0 || u < UNITS) ? (uint32_t)(row * row_elems + 4 * 2 * cp) * 2
                                                         : 0x7FFFFFF0u;
      raw[k] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
    }
  };
  // butterfly of a loaded tile into LDS buffer `buf` (fragment order)
  auto store_tile = [&](const half8 (&raw)[UPT], _Float16* buf) {
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = k * NT + tid;
      const int row = u % RT, cp = u / RT;
      const int c = 2 * cp;
      const int s = c >> 5, gg = (c & 31) >> 3, jj = c & 7;
      const int mb = row >> 4, r16 = row & 15;
      const bool real = UNITS % NT == 0 || u < UNITS;
      const half8 w = raw[k];
      const f16x2 a01 = {w[0], w[1]}, a23 = {w[2], w[3]};  // channel c
      const f16x2 b01 = {w[4], w[5]}, b23 = {w[6], w[7]};  // channel c + 1
      const float x0a = __builtin_amdgcn_fdot2(a01, ones, __builtin_amdgcn_fdot2(a23, ones, 0.f, false), false);
      const float x0b = __builtin_amdgcn_fdot2(b01, ones, __builtin_amdgcn_fdot2(b23, ones, 0.f, false), false);
      const float x2a = __builtin_amdgcn_fdot2(a01, pm, __builtin_amdgcn_fdot2(a23, pm, 0.f, false), false);
      const float x2b = __builtin_amdgcn_fdot2(b01, pm, __builtin_amdgcn_fdot2(b23, pm, 0.f, false), false);
      const f16x2 da = a01 - a23, db = b01 - b23;  // (Xr, -Xi) of each channel
      const f16x2 xr = {da[0], db[0]}, xi = {-da[1], -db[1]};
      // every unit stores unconditionally: units past the tile send their
      // four words to this thread's dummy slot (a select, not a branch)
      uint32_t* const dummy = reinterpret_cast<uint32_t*>(xs + 2 * BUF) + tid;
      _Float16* const dst = buf + (s * MR + mb) * FRAG + (gg * 16 + r16) * 8 + jj;
      *(real ? reinterpret_cast<uint32_t*>(dst + 0 * PS) : dummy) = pack2(x0a, x0b);
      *(real ? reinterpret_cast<uint32_t*>(dst + 1 * PS) : dummy) = pack2(x2a, x2b);
      *(real ? reinterpret_cast<uint32_t*>(dst + 2 * PS) : dummy) = __builtin_bit_cast(uint32_t, xr);
      *(real ? reinterpret_cast<uint32_t*>(dst + 3 * PS) : dummy) = __builtin_bit_cast(uint32_t, xi);
    }
  };
  // products + epilogue of tile t from LDS buffer `buf`
  auto compute_tile = [&](int t, const _Float16* buf) {
    const int64_t r0 = (int64_t)t * RT;
    const int64_t rows = N - r0 < RT ? N - r0 : RT;
    const __amdgpu_buffer_rsrc_t ry = rsrc(y + r0 * n_out * 4, (uint32_t)(rows * n_out * 8));
#pragma unroll
    for (int mb = 0; mb < MR; ++mb) {
      f32x4 c0[NB], c2[NB], cr[NB], ci[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) c0[nb] = c2[nb] = cr[nb] = ci[nb] = f32x4{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const _Float16* f = buf + (s * MR + mb) * FRAG + lane * 8;
        const half8 x0 = *reinterpret_cast<const half8*>(f + 0 * PS);
        const half8 x2 = *reinterpret_cast<const half8*>(f + 1 * PS);
        const half8 xr = *reinterpret_cast<const half8*>(f + 2 * PS);
        const half8 xi = *reinterpret_cast<const half8*>(f + 3 * PS);
        const half8 xq = -xi;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          c0[nb] = mma16(w0[nb][s], x0, c0[nb]);
          cr[nb] = mma16(wr[nb][s], xr, cr[nb]);
          c2[nb] = mma16(w2[nb][s], x2, c2[nb]);
          ci[nb] = mma16(wi[nb][s], xr, ci[nb]);
          cr[nb] = mma16(wi[nb][s], xq, cr[nb]);
          ci[nb] = mma16(wr[nb][s], xi, ci[nb]);
        }
      }
      // lane holds channels d0 + 16nb + 4g + r of row t*RT + mb*16 + i16;
      // rows past N fall outside the tile's store range and are dropped
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        uint32_t o[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4 v = epi4(c0[nb][r], c2[nb][r], cr[nb][r], ci[nb][r], bc[nb][r]);
          o[2 * r] = pack2(v[0], v[1]);
          o[2 * r + 1] = pack2(v[2], v[3]);
        }
        // channel groups past n_out (last range) would alias the next row:
        // give them an offset outside the range so the stores are dropped
        const int col = d0 + nb * 16 + 4 * g;
        const uint32_t off =
            col < n_out ? (uint32_t)(((mb * 16 + i16) * n_out + col) * 8) : 0x7FFFFFF0u;
        const u32x4 lo = {o[0], o[1], o[2], o[3]}, hi = {o[4], o[5], o[6], o[7]};
        __builtin_amdgcn_raw_buffer_store_b128(lo, ry, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(hi, ry, off + 16, 0, 0);
      }
    }
  };

  // Software pipeline, x prefetched three tiles ahead in a register ring:
  // iteration i computes tile t_i from LDS, loads t_{i+3} into the ring slot
  // t_i used, and moves t_{i+1} (already in registers) through the butterfly
  // into the other LDS buffer.  Tiles past the end load as zeros.  The main
  // loop runs whole rounds of the three ring slots and the last one or two
  // tiles follow it, so the loop header is entered only with the same set of
  // loads in flight (no early exit merges into it; the compiler's wait counts
  // stay exact instead of falling back to waiting on the newest loads).
  // Scheduling fences keep the three phases (issue the prefetch, products
  // and stores, butterfly) in program order: interleaving them lets the
  // compiler hoist butterfly arithmetic, and its waits on loads, into the
  // products.
  const int n_my = q < n_rt ? (n_rt - 1 - q) / Q + 1 : 0;  // tiles of this worker
  if (n_my == 0) return;
  // In the loop every tile's loads are followed by one tile's worth of
  // output stores (2*NB*MR per lane).  The prologue issues the same number
  // of stores after each prefetched tile, aimed outside an empty range (the
  // hardware drops them without memory traffic), so that the loop header
  // sees one pending sequence from either side and the compiler can wait on
  // a tile's loads without also waiting on the tile loaded after it.
  constexpr int SPT = 2 * NB * MR;
  const __amdgpu_buffer_rsrc_t rnull = rsrc(y, 0);
  auto dummy_stores = [&](uint32_t base) {  // distinct offsets: none is a dead store
#pragma unroll
    for (int k = 0; k < SPT; ++k) __builtin_amdgcn_raw_buffer_store_b32(0u, rnull, base + 64u * k, 0, 0);
  };
  half8 ra[UPT], rb[UPT], rc[UPT];
  int t = q;
  load_tile(ra, t);
  load_tile(rb, t + Q);
  dummy_stores(0x7FFF0000u);
  load_tile(rc, t + 2 * Q);
  dummy_stores(0x7FFF8000u);
  // The weight, bias and first-tile loads are all in flight together; wait
  // until only the two prefetched tiles and their stores are outstanding.
  static_assert(2 * (UPT + SPT) <= 63, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(((2 * (UPT + SPT)) & 15) | (0x7 << 4) | (0xF << 8) |
                             (((2 * (UPT + SPT)) >> 4) << 14));
  store_tile(ra, xs);
  __syncthreads();
  int cur = 0;
  for (int i = 3; i <= n_my; i += 3) {
    load_tile(ra, t + 3 * Q);
    __builtin_amdgcn_sched_barrier(0);
    compute_tile(t, xs + cur * BUF);
    __builtin_amdgcn_sched_barrier(0);
    store_tile(rb, xs + (cur ^ 1) * BUF);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    cur ^= 1;
    t += Q;
    load_tile(rb, t + 3 * Q);
    __builtin_amdgcn_sched_barrier(0);
    compute_tile(t, xs + cur * BUF);
    __builtin_amdgcn_sched_barrier(0);
    store_tile(rc, xs + (cur ^ 1) * BUF);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    cur ^= 1;
    t += Q;
    load_tile(rc, t + 3 * Q);
    __builtin_amdgcn_sched_barrier(0);
    compute_tile(t, xs + cur * BUF);
    __builtin_amdgcn_sched_barrier(0);
    store_tile(ra, xs + (cur ^ 1) * BUF);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    cur ^= 1;
    t += Q;
  }
  const int rest = n_my % 3;  // tiles left: t (in LDS) and t + Q (in rb)
  if (rest > 0) {
    compute_tile(t, xs + cur * BUF);
    if (rest > 1) {
      store_tile(rb, xs + (cur ^ 1) * BUF);
      __syncthreads();
      compute_tile(t + Q, xs + (cur ^ 1) * BUF);
    }
  }
}

// ---------------------------------------------------------------------------
static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

template <int NW, int NB, int KS, int MR>
static hipError_t launch_coop_t(const void* x, const void* spec, const float* bias, void* y,
                                int64_t N, int K, int n_out, int n_pad, int k_pad, int wpc,
                                hipStream_t s) {
  constexpr int BN = NW * NB * 16;
  const int n_ct = (n_out + BN - 1) / BN;
  const int64_t n_rt = (N + 16 * MR - 1) / (16 * MR);
  int qx = (256 * wpc) / (8 * n_ct);
  if (qx < 1) qx = 1;
  const int64_t max_qx = (n_rt + 7) / 8;
  if (qx > max_qx) qx = (int)(max_qx < 1 ? 1 : max_qx);
  qx = env_int("EQL_COOP_QX", qx);
  const unsigned blocks = (unsigned)(8 * n_ct * qx);
  hipLaunchKernelGGL((k_fwd_coop_f16<NW, NB, KS, MR>), dim3(blocks), dim3(NW * 64), 0, s,
                     (const _Float16*)x, (const _Float16*)spec, bias, (_Float16*)y, (int)N, K, n_out,
                     n_pad, k_pad, n_ct, qx);
  return hipGetLastError();
}

// hipErrorNotSupported when outside this kernel's limits.
hipError_t launch_coop(eqlinear_dtype_t dt, const void* x, const void* spec, const float* bias,
                       void* y, int64_t N, int K, int k_pad, int n_out, int n_pad, hipStream_t s) {
  if (env_int("EQL_NO_COOP", 0) || dt != EQL_F16) return hipErrorNotSupported;
  // exact 32-channel steps (x rows are read without a channel mask) and whole
  // 4-channel output groups (32-byte stores)
  if (K != k_pad || K % 32 != 0 || n_out % 4 != 0) return hipErrorNotSupported;
  // 32-bit buffer offsets: one tile's bytes, and the spectra planes
  if ((int64_t)n_pad * k_pad * 2 >= (1LL << 31)) return hipErrorNotSupported;
  const int ks = k_pad / 32;
  const int nw = env_int("EQL_COOP_NW", 8);
  const int nb = env_int("EQL_COOP_NB", 1);
  const int mr = env_int("EQL_COOP_MR", 1);
  const int wpc = env_int("EQL_COOP_WPC", 1);
#define EQL_COOP_CASE(NW_, NB_, KS_, MR_) \
  if (nw == NW_ && nb == NB_ && ks == KS_ && mr == MR_) \
    return launch_coop_t<NW_, NB_, KS_, MR_>(x, spec, bias, y, N, K, n_out, n_pad, k_pad, wpc, s);
  EQL_COOP_CASE(4, 2, 3, 1)
  EQL_COOP_CASE(4, 2, 3, 2)
  EQL_COOP_CASE(8, 2, 3, 1)
  EQL_COOP_CASE(4, 1, 3, 1)
  EQL_COOP_CASE(8, 1, 3, 1)
  EQL_COOP_CASE(4, 3, 3, 1)
  EQL_COOP_CASE(4, 2, 2, 1)
  EQL_COOP_CASE(4, 2, 1, 1)
  EQL_COOP_CASE(4, 1, 6, 1)
  EQL_COOP_CASE(8, 1, 6, 1)
  EQL_COOP_CASE(4, 2, 6, 1)
  EQL_COOP_CASE(4, 1, 4, 1)
  EQL_COOP_CASE(4, 1, 5, 1)
#undef EQL_COOP_CASE
  return hipErrorNotSupported;
}

}  // namespace eql
