// Forward of the p4 EQ-Linear layer with producer and consumer waves
// (binary16, reduction widths up to 192 channels).
//
// Arithmetic (Flash EQ-Linear, "Approccio Algoritmico" and "Specializzazione
// per il Gruppo di Rotazione p4"): with the group DFT of x and of the weight,
//     Y0 = X0 W0   Y2 = X2 W2   Yr = Xr Wr - Xi Wi   Yi = Xr Wi + Xi Wr
// six real products, then the inverse length-4 butterfly and the bias.
//
// Organisation on CDNA4.  A persistent work-group owns BN = 16*NB*NC output
// channels and walks 16-row tiles of x.  Its waves have one of two roles:
//  * NP producer waves stream x: range-checked 16-byte buffer loads three
//    tiles ahead in a register ring, the length-4 butterfly into the scaled
//    planes X0/4, X2/4 (pair sums in fp32, rounded once to binary16) and
//    Xr/2, -Xi/2 (one packed fused multiply-add per channel), and the write
//    of the four planes to LDS in matrix-core fragment order (double
//    buffered).  They also
//    write the previous tile's output, staged in LDS by the consumers, to
//    memory as whole rows;
//  * NC consumer waves keep the weight-spectrum fragments of their 16*NB
//    channels in VGPRs, multiply the tile from LDS on the matrix cores
//    (16x16x32 f16, fp32 accumulate), apply the inverse butterfly and the
//    bias in fp32 and leave the binary16 result in LDS.
// The two roles run separate loops that meet at one work-group barrier per
// tile, so the butterfly of tile i+1 and the stores of tile i-1 overlap the
// products of tile i.  The consumers never touch global memory in the loop,
// so memory back-pressure never stalls the matrix cores.  Work-groups that
// read the same x tiles (different channel ranges) sit on the same XCD and
// share its L2.
//
// Split reduction (KSPLIT, backward_input over 384 channels): two consumer
// waves per 16-channel output block, each holding the weight fragments of
// half of the reduction steps, so the weights take half the VGPRs, twelve
// waves fit (six producers instead of four) and each producer transforms
// two units per tile instead of three.  The second wave of a pair parks its
// accumulators in LDS; the first adds them in a fixed order one tile later
// and runs the epilogue, so the producers store each tile two phases after
// its products.
#include <type_traits>

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

// inverse butterfly of one (row, channel) with its bias, fp32 (products of
// scaled planes: factors 4 and 2)
__device__ __forceinline__ f32x4 epi4(float Y0, float Y2, float Yr, float Yi, float b) {
  return idft4_bias(Y0, Y2, Yr, Yi, b);
}

// Raw buffer resource over [base, base + bytes): out-of-range loads return
// zeros and out-of-range stores are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Cache policy of the output stores (instruction cache-policy bits): 2 is
// the non-temporal (streaming) hint, 0x11 system scope (sc0 | sc1: written
// through the L2, used with whole-line stores only).  Either shortens the
// write-back of dirty L2 lines after the last wave, several microseconds
// per launch at a few tens of MB; beyond the memory-side cache the
// streaming hint sustains the higher bandwidth.
constexpr int POLICY_STREAM = 2, POLICY_THROUGH = 0x11;

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

}  // namespace

// LDS fragment layout (per buffer): plane p (X0, X2, Xr, Xi) and k-step s
// hold one 1 KB fragment at (p*KS + s)*512 halves; lane (i16, g) of the B
// operand reads the 16 bytes of slot g*16 + (i16 ^ 4g): row i16 and k-slice g.
// The row index is swizzled by 4g so that a producer wave whose sixteen
// lanes hold four rows x four slices writes sixteen distinct banks groups.
// Reduction order inside a 32-channel step: slice g holds the channel pairs
// g, g + 4, g + 8, g + 12 (two channels each, in that order), so that the
// four lanes of a producer quad read 64 contiguous bytes of a row; the
// weight fragments (k_spectra.hip) use the same order.
template <int NC, int NP, int NB, int KS, int YP, bool G8, bool STAGGER, bool PST, bool PIPE,
          bool SPLIT, bool ACT = false, bool KSPLIT = false>
__device__ __forceinline__ void ws_body(
    const _Float16* __restrict__ x, const _Float16* __restrict__ spec, const float* __restrict__ bias,
    _Float16* __restrict__ y, int N, int K, int n_out, int n_pad, int n_ct, int Qx, int act,
    int wfirst) {
  // KSPLIT: two consumer waves per output block, each over half of the
  // reduction steps (wave 2b + h: block b, half h); the second half leaves
  // its accumulators in LDS and the first adds them, in a fixed order, one
  // tile later, before the epilogue
  static_assert(!KSPLIT || (!PIPE && PST && !SPLIT && !ACT && NB == 1 && NC % 2 == 0 && KS % 2 == 0),
                "split reduction: paired waves, staged output, no pipelining");
  constexpr int NCB = KSPLIT ? NC / 2 : NC;  // consumer output blocks of NB x 16 channels
  constexpr int KSH = KSPLIT ? KS / 2 : KS;  // reduction steps per consumer wave
  constexpr int BN = NCB * NB * 16;
  constexpr int KP = KS * 32;
  constexpr int FRAG = 512;                   // halves per fragment
  constexpr int PS = KS * FRAG;               // plane stride (halves)
  constexpr int BUF = 4 * PS;                 // halves per buffer
  constexpr int PT = NP * 64;                 // producer threads
  // producer unit: one row and 8 reduction channels (64 contiguous bytes,
  // four 16-byte loads; its butterfly fills one 16-byte fragment slot per
  // plane) when G8, else one row and 2 channels (one 16-byte load)
  constexpr int CPU = G8 ? 8 : 2;                    // channels per unit
  constexpr int LPU = G8 ? 4 : 1;                    // 16-byte loads per unit
  constexpr int UNITS = 16 * (KP / CPU);             // units per tile
  constexpr int UPT = (UNITS + PT - 1) / PT;         // units per producer thread
  constexpr int LPT = UPT * LPU;                     // loads per producer thread
  constexpr int DUMMY = (UNITS % PT != 0) ? (G8 ? 8 : 2) * PT : 0;  // halves
  // producer-stored output (PST): the consumers leave each output tile in
  // LDS, row-major over the work-group's BN channels, double buffered; the
  // producers write it to memory during the next tile.  The 16-byte pad per
  // row puts the 16-byte writes of 8 consecutive consumer lanes (8 rows) on
  // distinct LDS banks.
  constexpr int OPITCH = BN * 4 + 8;  // halves per staged output row
  constexpr int OBUF = 16 * OPITCH;   // halves per staged output tile
  __shared__ __attribute__((aligned(16))) _Float16 xs[2 * BUF + DUMMY + (PST ? 2 * OBUF : 0)];
  _Float16* const obuf = xs + 2 * BUF + DUMMY;  // PST staging (two tiles)
  // KSPLIT: parked accumulators of the second halves, [2][NCB][6][64] f32x4
  __shared__ __attribute__((aligned(16))) f32x4 park[KSPLIT ? 2 * NCB * 6 * 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar registers)
  // work-group -> (channel range j, worker q); equal q share an XCD
  const int wgid = blockIdx.x, xcd = wgid & 7, slot = wgid >> 3;
  const int j = slot % n_ct;
  const int q = (slot / n_ct) * 8 + xcd, Q = Qx * 8;
  const int n_rt = (N + 15) / 16;
  const int n_my = q < n_rt ? (n_rt - 1 - q) / Q + 1 : 0;  // tiles of this worker
  if (n_my == 0) return;  // whole work-group

  // PST: write rows [ROW0, ROW0 + NROWS) of this worker's staged output tile
  // t (16 rows x BN channels, one 16-byte chunk = 2 channels x 4 group values
  // per lane, whole rows per wave instruction) from staging buffer t % 2,
  // spread over the TPR threads of one role (rt = thread index in the role).
  // SPLIT: the producers write rows 0-7 and the consumers rows 8-15.
  static_assert(!(SPLIT && (PIPE || !PST)), "split stores need producer-side staging, no lag");
  auto store_rows = [&](auto row0_c, auto nrows_c, auto tpr_c, int t, int rt) {
    constexpr int ROW0 = decltype(row0_c)::value, NROWS = decltype(nrows_c)::value;
    constexpr int TPR = decltype(tpr_c)::value;
    const int64_t r0 = (int64_t)(q + (int64_t)t * Q) * 16;
    const int64_t rows = N - r0 < 16 ? N - r0 : 16;
    const __amdgpu_buffer_rsrc_t ry = rsrc(y + r0 * n_out * 4, (uint32_t)(rows * n_out * 8));
    const _Float16* const sb = obuf + (t & 1) * OBUF;
    constexpr int LPR = BN / 2;                 // chunks per row
    constexpr int CH = NROWS * LPR;             // chunks to write
    constexpr int SPT = (CH + TPR - 1) / TPR;   // chunks per thread
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int u0 = k * TPR + rt;
      const bool real = CH % TPR == 0 || u0 < CH;
      const int u = real ? u0 : 0;
      const int row = ROW0 + u / LPR, ch = u % LPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(sb + row * OPITCH + 8 * ch);
      const int col = j * BN + 2 * ch;
      const uint32_t off = (real && col < n_out) ? (uint32_t)((row * n_out + col) * 8) : 0x7FFFFFF0u;
      __builtin_amdgcn_raw_buffer_store_b128(v, ry, off, 0, YP);
    }
  };
  typedef std::integral_constant<int, 0> c0_t;
  typedef std::integral_constant<int, 8> c8_t;
  typedef std::integral_constant<int, SPLIT ? 8 : 16> cprod_rows_t;

  if (wave >= NC) {
    // =========================== producer waves ===========================
    const int ptid = tid - NC * 64;
    const int64_t row_elems = (int64_t)K * 4;
    // unit u -> (row, channels).  Lanes that share a row read contiguous
    // bytes (lanes walking rows would cost the address unit four times the
    // cycles).  With 2-channel units, sixteen lanes take the sixteen channel
    // pairs of one 32-channel step of one row (256 contiguous bytes), so a
    // wave covers four rows; its 4-byte LDS writes (four slices x four words
    // of four swizzled rows) then meet 64 distinct banks.  With 8-channel
    // units, lane l takes row (l / 4) % 16, step u / 64 and slice g = l % 4:
    // load e reads pair 4e + g of the step (four lanes, 64 contiguous
    // bytes), and the four pairs fill the slot of slice g.
    auto unit_pos = [](int u, int& row, int& grp) {
      if (G8) {
        row = (u >> 2) & 15;
        grp = (u >> 6) * 4 + (u & 3);             // (step, slice) = (grp / 4, grp % 4)
      } else {
        row = (u >> 4) & 15;
        grp = ((u >> 8) << 4) | (u & 15);         // channel pair
      }
    };
    auto load_tile = [&](half8 (&raw)[LPT], int i) {
      const int64_t r0 = (int64_t)(q + (int64_t)i * Q) * 16;
      const int64_t rows = r0 < N ? (N - r0 < 16 ? N - r0 : 16) : 0;
      const __amdgpu_buffer_rsrc_t rx = rsrc(x + (r0 < N ? r0 : 0) * row_elems, (uint32_t)(rows * row_elems * 2));
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const int u = k * PT + ptid;
        int row, grp;
        unit_pos(u, row, grp);
        const bool real = UNITS % PT == 0 || u < UNITS;
        // G8: pair 4e + g of step grp / 4 is at byte 256 (grp / 4) + 64 e + 16 g
        const uint32_t off = G8 ? (uint32_t)(row * row_elems * 2 + 256 * (grp >> 2) + 16 * (grp & 3))
                                : (uint32_t)(row * row_elems + 4 * CPU * grp) * 2;
#pragma unroll
        for (int e = 0; e < LPU; ++e)
          raw[k * LPU + e] = __builtin_bit_cast(
              half8, __builtin_amdgcn_raw_buffer_load_b128(rx, real ? off + 64 * e : 0x7FFFFFF0u, 0, 0));
      }
    };
    // butterfly of one 16-byte word (channels c, c + 1, four group values
    // each) into packed binary16 pairs (X0/4, X2/4, Xr/2, -Xi/2) of the two
    // channels (scaled planes, eql_device.h).  X0 and X2 come from the pair
    // sums x0 + x2 and x1 + x3 in fp32, scaled and rounded once to binary16;
    // (Xr, -Xi)/2 = (x0 - x2, x1 - x3)/2 from one packed fused multiply-add
    // per channel.  The fourth plane holds -Xi/2 so that no lane ever negates
    // a fragment; the consumers fold the sign into their sums.  The
    // multiplier 1.0 is made opaque to the optimiser so that each pair sum
    // stays one mixed-precision fma (binary16 operands, fp32 result) instead
    // of two conversions and an add.
    float one = 1.0f;
    asm volatile("" : "+v"(one));
    auto bfly = [&](const half8& w, uint32_t& o0, uint32_t& o2, uint32_t& orr, uint32_t& oi) {
      const float sa = __builtin_fmaf((float)w[0], one, (float)w[2]);
      const float ta = __builtin_fmaf((float)w[1], one, (float)w[3]);
      const float sb = __builtin_fmaf((float)w[4], one, (float)w[6]);
      const float tb = __builtin_fmaf((float)w[5], one, (float)w[7]);
      o0 = __builtin_bit_cast(uint32_t, f16x2{quarter_h(sa + ta), quarter_h(sb + tb)});
      o2 = __builtin_bit_cast(uint32_t, f16x2{quarter_h(sa - ta), quarter_h(sb - tb)});
      const f16x2 a01 = {w[0], w[1]}, a23 = {w[2], w[3]};  // channel c
      const f16x2 b01 = {w[4], w[5]}, b23 = {w[6], w[7]};  // channel c + 1
      const f16x2 da = half_diff(a01, a23), db = half_diff(b01, b23);  // (Xr, -Xi)/2 of each channel
      orr = __builtin_bit_cast(uint32_t, f16x2{da[0], db[0]});
      oi = __builtin_bit_cast(uint32_t, f16x2{da[1], db[1]});
    };
    auto store_tile = [&](const half8 (&raw)[LPT], _Float16* buf) {
#pragma unroll
      for (int k = 0; k < UPT; ++k) {
        const int u = k * PT + ptid;
        int row, grp;
        unit_pos(u, row, grp);
        // fragment slot (step s, slice gg, row) and the word of the pair in it
        int s, gg, jj;
        if (G8) {
          s = grp >> 2;
          gg = grp & 3;
          jj = 0;
        } else {
          const int qp = (grp & 15);  // channel pair within the 32-channel step
          s = grp >> 4;
          gg = qp & 3;
          jj = (qp >> 2) * 2;
        }
        const bool real = UNITS % PT == 0 || u < UNITS;
        // units past the tile send their words to this thread's dummy slot
        _Float16* const dummy = xs + 2 * BUF + ptid * (G8 ? 8 : 2);
        _Float16* const dst = buf + s * FRAG + (gg * 16 + (row ^ (gg << 2))) * 8 + jj;
        if (G8) {
          u32x4 v0, v2, vr, vi;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t t0, t2, tr, ti;
            bfly(raw[k * 4 + e], t0, t2, tr, ti);
            v0[e] = t0;
            v2[e] = t2;
            vr[e] = tr;
            vi[e] = ti;
          }
          *reinterpret_cast<u32x4*>(real ? dst + 0 * PS : dummy) = v0;
          *reinterpret_cast<u32x4*>(real ? dst + 1 * PS : dummy) = v2;
          *reinterpret_cast<u32x4*>(real ? dst + 2 * PS : dummy) = vr;
          *reinterpret_cast<u32x4*>(real ? dst + 3 * PS : dummy) = vi;
        } else {
          uint32_t v0, v2, vr, vi;
          bfly(raw[k], v0, v2, vr, vi);
          *reinterpret_cast<uint32_t*>(real ? dst + 0 * PS : dummy) = v0;
          *reinterpret_cast<uint32_t*>(real ? dst + 1 * PS : dummy) = v2;
          *reinterpret_cast<uint32_t*>(real ? dst + 2 * PS : dummy) = vr;
          *reinterpret_cast<uint32_t*>(real ? dst + 3 * PS : dummy) = vi;
        }
      }
    };
    // PST: the producers' rows of staged output tile t
    auto store_out = [&](int t) {
      store_rows(c0_t{}, cprod_rows_t{}, std::integral_constant<int, PT>{}, t, ptid);
    };
    // phase p (between barriers p and p + 1) first writes out the tile the
    // consumers staged in phase p - 1: tile p - 1, or p - 2 when their
    // epilogue lags their products by one tile (PIPE)
    constexpr int LAG = (PIPE || KSPLIT) ? 2 : 1;
    auto out_step = [&](int p) {
      if (PST && p >= LAG) store_out(p - LAG);
    };
    // Ring: tile i sits in slot i % 3 from its load until its butterfly;
    // between barriers i and i+1 the producers transform tile i+1 and load
    // tile i+4 into the slot it frees.  Only loads are in flight here, so
    // the wait before each transform leaves exactly the two younger tiles
    // (2*LPT loads) outstanding.  Tiles past the end load as zeros.  The
    // scheduling fences stop the compiler from hoisting a later transform's
    // arithmetic (and so its wait on younger loads) above a barrier.
    half8 ra[LPT], rb[LPT], rc[LPT];
    load_tile(ra, 0);
    if (STAGGER) {
      // every work-group's first tile is requested before any second or
      // third one, so the first tiles are not queued behind the whole
      // prefetch burst of the grid
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0): expcnt, lgkmcnt not waited
    }
    if (wfirst) {
      // weights first: tile 0 is transformed, then the producers wait for
      // the consumers' weight fragments to arrive before requesting more
      store_tile(ra, xs);
      __syncthreads();  // barrier W
      load_tile(rb, 1);
      load_tile(rc, 2);
    } else {
      load_tile(rb, 1);
      load_tile(rc, 2);
      store_tile(ra, xs);
    }
    load_tile(ra, 3);
    __syncthreads();  // barrier 0: tile 0 is in buffer 0
    int cur = 1;      // buffer of the next tile
    int i = 0;        // barriers i .. : tile i+1 goes to buffer cur
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
    if (PIPE || KSPLIT) {
      // phase n_my - 1, barrier n_my (the consumers' last products are done),
      // and with PST phase n_my and barrier n_my + 1 (their last epilogue)
      out_step(n_my - 1);
      __syncthreads();
      if (PST) {
        out_step(n_my);
        __syncthreads();
        store_out(n_my - 1);
      }
    } else if (PST) {
      // phase n_my - 1, then barrier n_my (after the consumers' last tile)
      out_step(n_my - 1);
      __syncthreads();
      store_out(n_my - 1);
    }
  } else {
    // =========================== consumer waves ===========================
    const int i16 = lane & 15, g = lane >> 4;
    const int xslot = lane ^ (g << 2);      // LDS slot of row i16, slice g
    const int cw = KSPLIT ? wave >> 1 : wave;  // this wave's output block
    const int kh = KSPLIT ? wave & 1 : 0;      // its half of the reduction (KSPLIT)
    const int d0 = j * BN + cw * NB * 16;      // its first output channel
    // weight fragments (A operand): channel d0 + 16nb + i16, reduction
    // channels 32s + 8g .. 32s + 8g + 7, from the operand in fragment order
    // (1 KB per fragment, lane l at 16 l bytes: one contiguous wave load)
    half8 w0[NB][KSH], w2[NB][KSH], wr[NB][KSH], wi[NB][KSH];
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
        const uint32_t off = (uint32_t)(((d0 / 16 + nb) * KS + kh * KSH) * 1024 + lane * 16);
#pragma unroll
        for (int s = 0; s < KSH; ++s) {
          w0[nb][s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r0, off + s * 1024, 0, 0));
          w2[nb][s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r2, off + s * 1024, 0, 0));
          wr[nb][s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(rr, off + s * 1024, 0, 0));
          wi[nb][s] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(ri, off + s * 1024, 0, 0));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
          bc[nb][r] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(rb, (d0 + nb * 16 + 4 * g + r) * 4, 0, 0));
      }
    }
    // Yr = Wr Xr - Wi Xi and Yi = Wi Xr + Wr Xi with the plane xn = -Xi.
    // Six independent accumulators (Yr = cr + cq, Yi = ci - cn), so no
    // fragment is negated; the pipelined consumers, which hold two sets,
    // use four (Yr in cr, Yi in ci, with Xi = -xn by a sign flip of the
    // fragment) to stay within the register budget.
    constexpr bool ACC4 = PIPE;
    constexpr int NA = ACC4 ? 1 : NB;  // extent of the unused cq, cn in ACC4
    struct Acc {
      f32x4 c0[NB], c2[NB], cr[NB], ci[NB], cq[NA], cn[NA];
    };
    // products of one tile from buffer `buf`
    auto products = [&](Acc& a, const _Float16* buf) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        a.c0[nb] = a.c2[nb] = a.cr[nb] = a.ci[nb] = f32x4{};
        if constexpr (!ACC4) a.cq[nb] = a.cn[nb] = f32x4{};
      }
#pragma unroll
      for (int s = 0; s < KSH; ++s) {
        const _Float16* f = buf + (kh * KSH + s) * FRAG + xslot * 8;
        const half8 x0 = *reinterpret_cast<const half8*>(f + 0 * PS);
        const half8 x2 = *reinterpret_cast<const half8*>(f + 1 * PS);
        const half8 xr = *reinterpret_cast<const half8*>(f + 2 * PS);
        const half8 xn = *reinterpret_cast<const half8*>(f + 3 * PS);
        if constexpr (ACC4) {
          const half8 xi = __builtin_bit_cast(half8, __builtin_bit_cast(u32x4, xn) ^ 0x80008000u);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            a.c0[nb] = mma16(w0[nb][s], x0, a.c0[nb]);
            a.cr[nb] = mma16(wr[nb][s], xr, a.cr[nb]);
            a.ci[nb] = mma16(wi[nb][s], xr, a.ci[nb]);
            a.c2[nb] = mma16(w2[nb][s], x2, a.c2[nb]);
            a.cr[nb] = mma16(wi[nb][s], xn, a.cr[nb]);
            a.ci[nb] = mma16(wr[nb][s], xi, a.ci[nb]);
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            a.c0[nb] = mma16(w0[nb][s], x0, a.c0[nb]);
            a.cr[nb] = mma16(wr[nb][s], xr, a.cr[nb]);
            a.c2[nb] = mma16(w2[nb][s], x2, a.c2[nb]);
            a.ci[nb] = mma16(wi[nb][s], xr, a.ci[nb]);
            a.cq[nb] = mma16(wi[nb][s], xn, a.cq[nb]);
            a.cn[nb] = mma16(wr[nb][s], xn, a.cn[nb]);
          }
        }
      }
    };
    // epilogue of this worker's i-th tile: inverse butterfly, bias and
    // activation (kind ak, a compile-time constant) in fp32, one rounding,
    // then the staged (PST) or direct store
    auto epilogue = [&](auto ak, int i, const Acc& a) {
      constexpr int AK = decltype(ak)::value;
      const int64_t r0 = (int64_t)(q + (int64_t)i * Q) * 16;
      const int64_t rows = N - r0 < 16 ? N - r0 : 16;
      const __amdgpu_buffer_rsrc_t ry = rsrc(y + r0 * n_out * 4, (uint32_t)(rows * n_out * 8));
      // lane holds channels d0 + 16nb + 4g + r of row r0 + i16; rows past N
      // fall outside the store range and are dropped
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        uint32_t o[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float yr = ACC4 ? a.cr[nb][r] : a.cr[nb][r] + a.cq[nb % NA][r];
          const float yi = ACC4 ? a.ci[nb][r] : a.ci[nb][r] - a.cn[nb % NA][r];
          f32x4 v = epi4(a.c0[nb][r], a.c2[nb][r], yr, yi, bc[nb][r]);
          if constexpr (AK != ACT_NONE) {
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = activate_k<AK>(v[t]);
          }
          o[2 * r] = pack2(v[0], v[1]);
          o[2 * r + 1] = pack2(v[2], v[3]);
        }
        const u32x4 lo = {o[0], o[1], o[2], o[3]}, hi = {o[4], o[5], o[6], o[7]};
        if (PST) {
          // row i16, work-group channels cw*16NB + 16nb + 4g .. + 3 (cw: the wave's block)
          _Float16* const sp = obuf + (i & 1) * OBUF + i16 * OPITCH + (cw * NB * 16 + nb * 16 + 4 * g) * 4;
          *reinterpret_cast<u32x4*>(sp) = lo;
          *reinterpret_cast<u32x4*>(sp + 8) = hi;
        } else {
          // channel groups past n_out (last range) would alias the next row:
          // give them an offset outside the range so the stores are dropped
          const int col = d0 + nb * 16 + 4 * g;
          const uint32_t off = col < n_out ? (uint32_t)((i16 * n_out + col) * 8) : 0x7FFFFFF0u;
          __builtin_amdgcn_raw_buffer_store_b128(lo, ry, off, 0, YP);
          __builtin_amdgcn_raw_buffer_store_b128(hi, ry, off + 16, 0, YP);
        }
      }
    };
    typedef std::integral_constant<int, ACT_NONE> ak_none;
    typedef std::integral_constant<int, ACT_GELU> ak_gelu;
    typedef std::integral_constant<int, ACT_GELU_TANH> ak_tanh;
    // epilogue with the activation chosen once per tile (one uniform branch)
    auto epilogue_any = [&](int i, const Acc& a) {
      if constexpr (!ACT) {
        epilogue(ak_none{}, i, a);
      } else if (act == ACT_GELU) {
        epilogue(ak_gelu{}, i, a);
      } else {
        epilogue(ak_tanh{}, i, a);
      }
    };
    // Software pipeline step: the products of the next tile (into `nx`, from
    // buffer `buf`) and the epilogue of tile i (from `cu`) in one basic
    // block, with the scheduler told to alternate them: every fragment read
    // first, then one matrix-core product and VALU instructions of the
    // epilogue in turn.  A wave issues a VALU instruction only every 8-9
    // cycles but a 16x16x32 product every 16, so the epilogue runs in the
    // shadow of the products instead of after them.
    auto pipe_step = [&](Acc& nx, const _Float16* buf, int i, const Acc& cu) {
      auto one = [&](auto ak) {
        products(nx, buf);
        epilogue(ak, i, cu);
        constexpr int NM = 6 * NB * KS;
        constexpr int VPM = (decltype(ak)::value != ACT_NONE ? 80 : 20) * NB / NM + 1;
        // the fragments of step s + 1 are read before the products of step s
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          if (st + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
          for (int k = 0; k < 6 * NB; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
          }
        }
      };
      if constexpr (!ACT) {
        one(ak_none{});
      } else if (act == ACT_GELU) {
        one(ak_gelu{});
      } else {
        one(ak_tanh{});
      }
    };
    if (wfirst) {
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0): the weights are in
      __syncthreads();  // barrier W
    }
    __syncthreads();  // barrier 0
    if constexpr (KSPLIT) {
      // Between barriers i and i+1: the first half of each pair adds the
      // second half's parked accumulators of tile i-1 to its own and runs
      // that tile's epilogue (staged, stored by the producers one phase
      // later), then both halves run the products of tile i over their
      // steps, and the second half parks them (buffer i % 2).
      Acc A;
      f32x4* const pk = park + cw * 6 * 64 + lane;
      auto add_parked = [&](int i) {
        const f32x4* p = pk + (i & 1) * (NCB * 6 * 64);
        A.c0[0] += p[0]; A.c2[0] += p[64]; A.cr[0] += p[128];
        A.ci[0] += p[192]; A.cq[0] += p[256]; A.cn[0] += p[320];
      };
      for (int i = 0; i < n_my; ++i) {
        if (kh == 0 && i > 0) {
          add_parked(i - 1);
          epilogue_any(i - 1, A);
        }
        products(A, xs + (i & 1) * BUF);
        if (kh == 1) {
          f32x4* p = pk + (i & 1) * (NCB * 6 * 64);
          p[0] = A.c0[0]; p[64] = A.c2[0]; p[128] = A.cr[0];
          p[192] = A.ci[0]; p[256] = A.cq[0]; p[320] = A.cn[0];
        }
        __syncthreads();  // barrier i+1
      }
      if (kh == 0) {
        add_parked(n_my - 1);
        epilogue_any(n_my - 1, A);
      }
      __syncthreads();  // barrier n_my + 1: the last tile is staged
    } else if (PIPE) {
      // Software pipeline: between barriers i+1 and i+2 the products of tile
      // i+1 (buffer (i+1) % 2) are issued before the epilogue of tile i, so
      // the matrix cores work while the same wave runs the epilogue's VALU
      // instructions.  Two accumulator sets alternate (loop unrolled twice);
      // the last one or two tiles leave the loop, so no products are issued
      // for a tile past the worker's last.
      Acc A, B;
      products(A, xs);
      int i = 0;
      for (; i + 2 < n_my; i += 2) {
        __syncthreads();  // barrier i+1
        pipe_step(B, xs + BUF, i, A);
        __syncthreads();  // barrier i+2
        pipe_step(A, xs, i + 1, B);
      }
      if (i + 1 < n_my) {  // two tiles left: i (products in A) and i + 1
        __syncthreads();  // barrier i+1
        pipe_step(B, xs + BUF, i, A);
        __syncthreads();  // barrier i+2 = n_my
        epilogue_any(i + 1, B);
      } else {  // one tile left
        __syncthreads();  // barrier n_my
        epilogue_any(i, A);
      }
      if (PST) __syncthreads();  // barrier n_my + 1: the last tile is staged
    } else {
      int cur = 0;
      Acc A;
      typedef std::integral_constant<int, NC * 64> ctpr_t;
      for (int i = 0; i < n_my; ++i) {
        products(A, xs + cur * BUF);
        epilogue_any(i, A);
        // SPLIT: the consumers' rows of the tile staged in the previous
        // phase, after this tile's products (the wait at the barrier would
        // otherwise be idle)
        if (SPLIT && i >= 1) store_rows(c8_t{}, c8_t{}, ctpr_t{}, i - 1, tid);
        cur ^= 1;
        // barrier i+1 (with PST also after the last tile: its staged output
        // is then complete for the producers)
        if (PST || i + 1 < n_my) __syncthreads();
      }
      if (SPLIT) store_rows(c8_t{}, c8_t{}, ctpr_t{}, n_my - 1, tid);
    }
  }
}

// Two entry points share the body so that the passes are told apart in
// kernel traces: the forward (weight spectra) and the backward-input pass
// (conjugate-transposed spectra, zero bias).  PST selects the output path:
// the producers write whole rows staged through LDS (the default), or the
// consumers store their fragments directly.
template <int NC, int NP, int NB, int KS, int YP, bool G8, bool PST, bool PIPE, bool SPLIT,
          bool ACT = false>
__global__ __launch_bounds__((NC + NP) * 64) void k_fwd_ws_f16(
    const _Float16* __restrict__ x, const _Float16* __restrict__ spec, const float* __restrict__ bias,
    _Float16* __restrict__ y, int N, int K, int n_out, int n_pad, int n_ct, int Qx, int act,
    int wfirst) {
  ws_body<NC, NP, NB, KS, YP, G8, true, PST, PIPE, SPLIT, ACT>(x, spec, bias, y, N, K, n_out, n_pad,
                                                               n_ct, Qx, act, wfirst);
}

template <int NC, int NP, int NB, int KS, int YP, bool G8, bool PST, bool PIPE, bool SPLIT,
          bool KSPLIT = false>
__global__ __launch_bounds__((NC + NP) * 64) void k_bwd_input_ws_f16(
    const _Float16* __restrict__ dy, const _Float16* __restrict__ spec, const float* __restrict__ bias,
    _Float16* __restrict__ dx, int N, int K, int n_out, int n_pad, int n_ct, int Qx, int wfirst) {
  ws_body<NC, NP, NB, KS, YP, G8, true, PST, PIPE, SPLIT, false, KSPLIT>(dy, spec, bias, dx, N, K, n_out, n_pad, n_ct,
                                                          Qx, ACT_NONE, wfirst);
}

// ---------------------------------------------------------------------------
// knob value, or the default when the knob is unset (-1)
static int pick(int knob, int dflt) { return knob >= 0 ? knob : dflt; }

template <int NC, int NP, int NB, int KS>
static hipError_t launch_ws_t(const Tuning& tn, const void* x, const void* spec, const float* bias,
                              void* y, int64_t N, int K, int n_out, int n_pad, int wpc, bool adjoint,
                              int act, hipStream_t s) {
  constexpr int BN = NC * NB * 16;
  const int n_ct = (n_out + BN - 1) / BN;
  if ((int64_t)n_ct * BN > n_pad) return hipErrorNotSupported;  // weight reads stay in the planes
  const int64_t n_rt = (N + 15) / 16;
  int qx = (256 * wpc) / (8 * n_ct);
  if (qx < 1) qx = 1;
  const int64_t max_qx = (n_rt + 7) / 8;
  if (qx > max_qx) qx = (int)(max_qx < 1 ? 1 : max_qx);
  qx = pick(tn.ws_qx, qx);
  const unsigned blocks = (unsigned)(8 * n_ct * qx);
  const int wfirst = pick(tn.ws_wfirst, 0);
  // Output path (measured on MI355X, binary16): the producers store whole
  // rows, written through the L2 while the output fits well inside the
  // 256 MB memory-side cache (C=96, D=384, N=12608: 11.2 us against 13.3
  // with streaming consumer stores) and streamed beyond it (C=192, D=768,
  // N=200704: 484 us against 507 written through).
  const int64_t y_bytes = N * (int64_t)n_out * 8;
  const bool small = y_bytes <= tn.ws_small_bytes;
  // 8-channel producer units for long reductions (fewer instructions per
  // tile)
  const bool g8 = pick(tn.ws_g8, KS > 6 ? 1 : 0) != 0;
  const dim3 grid(blocks), block((NC + NP) * 64);
#define EQL_WS_LAUNCH4(YP_, G8_, PST_, SPLIT_)                                                      \
  do {                                                                                              \
    if (adjoint)                                                                                    \
      hipLaunchKernelGGL((k_bwd_input_ws_f16<NC, NP, NB, KS, YP_, G8_, PST_, false, SPLIT_>), grid, block, 0, \
                         s, (const _Float16*)x, (const _Float16*)spec, bias, (_Float16*)y, (int)N, K,   \
                         n_out, n_pad, n_ct, qx, wfirst);                                           \
    else if (act != ACT_NONE)                                                                       \
      hipLaunchKernelGGL((k_fwd_ws_f16<NC, NP, NB, KS, YP_, G8_, PST_, false, SPLIT_, true>), grid, block, \
                         0, s, (const _Float16*)x, (const _Float16*)spec, bias, (_Float16*)y, (int)N, K, \
                         n_out, n_pad, n_ct, qx, act, wfirst);                                      \
    else                                                                                            \
      hipLaunchKernelGGL((k_fwd_ws_f16<NC, NP, NB, KS, YP_, G8_, PST_, false, SPLIT_>), grid, block, 0, \
                         s, (const _Float16*)x, (const _Float16*)spec, bias, (_Float16*)y, (int)N, K,   \
                         n_out, n_pad, n_ct, qx, act, wfirst);                                      \
  } while (0)
#define EQL_WS_LAUNCH(YP_, G8_, PST_) EQL_WS_LAUNCH4(YP_, G8_, PST_, false)
  // Software-pipelined consumers (products of tile i+1 interleaved with the
  // epilogue of tile i, two accumulator sets) for forward outputs inside the
  // memory-side cache and reductions of up to six steps (the second
  // accumulator set fits the register budget there).
  if constexpr (KS <= 6) {
    // With a fused activation the second accumulator set and the
    // activation's registers fit the budget of twelve waves only up to three
    // reduction steps (beyond, the compiler spills); consumer-side stores
    // (EQL_WS_OUT=1) run unpipelined.
    const bool pipe = !adjoint && small && pick(tn.ws_pipe, 1) != 0 && pick(tn.ws_out, 0) != 1 &&
                      (act == ACT_NONE || KS <= 3);
    if (pipe) {
#define EQL_WS_PIPE_LAUNCH(YP_, G8_, PST_, ACT_)                                                       \
  hipLaunchKernelGGL((k_fwd_ws_f16<NC, NP, NB, KS, YP_, G8_, PST_, true, false, ACT_>), grid, block, 0, s, \
                     (const _Float16*)x, (const _Float16*)spec, bias, (_Float16*)y, (int)N, K, n_out,     \
                     n_pad, n_ct, qx, act, wfirst)
      if (act != ACT_NONE) {
        if constexpr (KS <= 3) {
          if (g8) EQL_WS_PIPE_LAUNCH(POLICY_THROUGH, true, true, true);
          else EQL_WS_PIPE_LAUNCH(POLICY_THROUGH, false, true, true);
        }
      } else {
        if (g8) EQL_WS_PIPE_LAUNCH(POLICY_THROUGH, true, true, false);
        else EQL_WS_PIPE_LAUNCH(POLICY_THROUGH, false, true, false);
      }
#undef EQL_WS_PIPE_LAUNCH
      return hipGetLastError();
    }
  }
  // output mode: 0 producer stores (written through small outputs,
  // streamed large ones); 1 consumer stores, streaming
  const int mode = pick(tn.ws_out, 0);
  // Outputs beyond the memory-side cache: the stores of each tile split
  // between producers (rows 0-7) and consumers (rows 8-15).  There the
  // producers set the pace and the consumers wait at the barrier (measured
  // at C=192, D=768: consumers wait 31% of their time, producers 12%);
  // measured 518 -> 499 us.
  const bool split = !small && pick(tn.ws_split, 1) != 0;
  if (mode == 1) {
    if (g8) EQL_WS_LAUNCH(POLICY_STREAM, true, false);
    else EQL_WS_LAUNCH(POLICY_STREAM, false, false);
  } else if (small) {
    if (g8) EQL_WS_LAUNCH(POLICY_THROUGH, true, true);
    else EQL_WS_LAUNCH(POLICY_THROUGH, false, true);
  } else if (split) {
    if (g8) EQL_WS_LAUNCH4(POLICY_STREAM, true, true, true);
    else EQL_WS_LAUNCH4(POLICY_STREAM, false, true, true);
  } else {
    if (g8) EQL_WS_LAUNCH(POLICY_STREAM, true, true);
    else EQL_WS_LAUNCH(POLICY_STREAM, false, true);
  }
#undef EQL_WS_LAUNCH4
#undef EQL_WS_LAUNCH
  return hipGetLastError();
}

// backward_input with split-reduction consumers: NC / 2 output blocks of 16
// channels per work-group, two consumer waves per block over the halves of
// the KS reduction steps, NP producer waves, producer-staged output.
template <int NC, int NP, int KS>
static hipError_t launch_bwi_ksplit(const Tuning& tn, const void* x, const void* spec, const float* bias,
                                    void* y, int64_t N, int K, int n_out, int n_pad, hipStream_t s) {
  constexpr int BN = NC / 2 * 16;
  const int n_ct = (n_out + BN - 1) / BN;
  if ((int64_t)n_ct * BN > n_pad) return hipErrorNotSupported;  // weight reads stay in the planes
  const int64_t n_rt = (N + 15) / 16;
  int qx = 256 / (8 * n_ct);
  if (qx < 1) qx = 1;
  const int64_t max_qx = (n_rt + 7) / 8;
  if (qx > max_qx) qx = (int)(max_qx < 1 ? 1 : max_qx);
  qx = pick(tn.ws_qx, qx);
  const unsigned blocks = (unsigned)(8 * n_ct * qx);
  const int wfirst = pick(tn.ws_wfirst, 0);
  const bool small = N * (int64_t)n_out * 8 <= tn.ws_small_bytes;
  const dim3 grid(blocks), block((NC + NP) * 64);
  if (small)
    hipLaunchKernelGGL((k_bwd_input_ws_f16<NC, NP, 1, KS, POLICY_THROUGH, true, true, false, false, true>), grid,
                       block, 0, s, (const _Float16*)x, (const _Float16*)spec, bias, (_Float16*)y, (int)N, K,
                       n_out, n_pad, n_ct, qx, wfirst);
  else
    hipLaunchKernelGGL((k_bwd_input_ws_f16<NC, NP, 1, KS, POLICY_STREAM, true, true, false, false, true>), grid,
                       block, 0, s, (const _Float16*)x, (const _Float16*)spec, bias, (_Float16*)y, (int)N, K,
                       n_out, n_pad, n_ct, qx, wfirst);
  return hipGetLastError();
}

// hipErrorNotSupported when outside this kernel's limits.
hipError_t launch_ws(const Tuning& tn, eqlinear_dtype_t dt, const void* x, const void* spec,
                     const float* bias, void* y, int64_t N, int K, int k_pad, int n_out, int n_pad,
                     bool adjoint, int act, hipStream_t s) {
  if (tn.ws_off == 1 || dt != EQL_F16) return hipErrorNotSupported;
  // exact 32-channel steps (x rows are read without a channel mask) and whole
  // 4-channel output groups (32-byte stores)
  if (K != k_pad || K % 32 != 0 || n_out % 4 != 0) return hipErrorNotSupported;
  // 32-bit buffer offsets: one tile of x and of y, and the spectra planes
  if ((int64_t)n_pad * k_pad * 2 >= (1LL << 31) || (int64_t)16 * n_out * 8 >= (1LL << 31))
    return hipErrorNotSupported;
  const int ks = k_pad / 32;
  // long reductions: 3 or 4 consumer waves, whichever pads the output
  // channels less (ties go to 4)
  const int pad3 = (n_out + 47) / 48 * 48 - n_out, pad4 = (n_out + 63) / 64 * 64 - n_out;
  // backward_input over 384 channels where 48-channel work-groups pad the
  // output least: split-reduction consumers (six producer waves instead of
  // four; measured at 12608 x 384 -> 96, five alternating runs on one box:
  // 15.0-16.0 against 15.3-16.9 us); shapes it does not take run the
  // organisation below
  if (adjoint && ks == 12 && pad3 < pad4 && pick(tn.ws_ksplit, 1) == 1) {
    const hipError_t e = launch_bwi_ksplit<6, 6, 12>(tn, x, spec, bias, y, N, K, n_out, n_pad, s);
    if (e != hipErrorNotSupported) return e;
  }
  // measured on MI355X: 4 consumer waves of 32 channels for short reductions,
  // 8 consumer waves of 16 channels (fewer VGPRs per wave) up to 192
  // channels, and 4 consumer waves of 16 channels beyond (the weight
  // fragments of a wave grow with the reduction width)
  const bool wide = ks <= 3, deep = ks > 6;
  // with a fused activation the epilogue carries most of the consumers' work:
  // short reductions then take 8 consumer waves of 16 channels (measured at
  // C = 96, D = 384 with GELU: 26.6 us against 37.6 us with 4 waves of 32)
  const bool act_wide = wide && act != 0 && !adjoint;
  const int nc = pick(tn.ws_nc, act_wide ? 8 : wide ? 4 : deep ? (pad3 < pad4 ? 3 : 4) : 8);
  const int np = pick(tn.ws_np, 4);
  const int nb = pick(tn.ws_nb, wide && !act_wide ? 2 : 1);
  const int wpc = pick(tn.ws_wpc, 1);
#define EQL_WS_CASE(NC_, NP_, NB_, KS_) \
  if (nc == NC_ && np == NP_ && nb == NB_ && ks == KS_) \
    return launch_ws_t<NC_, NP_, NB_, KS_>(tn, x, spec, bias, y, N, K, n_out, n_pad, wpc, adjoint, act, s);
  EQL_WS_CASE(4, 4, 2, 1)
  EQL_WS_CASE(4, 4, 2, 2)
  EQL_WS_CASE(4, 4, 2, 3)
  EQL_WS_CASE(8, 4, 1, 4)
  EQL_WS_CASE(8, 4, 1, 5)
  EQL_WS_CASE(8, 4, 1, 6)
  EQL_WS_CASE(8, 4, 1, 1)
  EQL_WS_CASE(8, 4, 1, 2)
  EQL_WS_CASE(8, 4, 1, 3)
  EQL_WS_CASE(4, 4, 1, 8)
  EQL_WS_CASE(4, 4, 1, 12)
  EQL_WS_CASE(3, 4, 1, 8)
  EQL_WS_CASE(3, 4, 1, 12)
#undef EQL_WS_CASE
  return hipErrorNotSupported;
}

}  // namespace eql
