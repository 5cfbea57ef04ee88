// C ABI of libeqlinear: argument validation, the plan object and dispatch.
// Every check that can run without a GPU runs before the first HIP call.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "eql_internal.h"

namespace {

thread_local char g_last_error[256] = "";

void set_error(const char* what, hipError_t e) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Largest channel count and row count accepted (32-bit index arithmetic in
// the kernels stays in range below these).
constexpr int64_t MAX_CHANNELS = 1 << 16;
constexpr int64_t MAX_ROWS = (int64_t)1 << 30;
// Groups with kernels: the cyclic groups C_2 .. C_16 and the dihedral
// groups D_2 .. D_8 (orders 4 .. 16).
constexpr int64_t MIN_T = 2, MAX_T = 16;
constexpr int64_t MIN_DIH = 2, MAX_DIH = 8;

eqlinear_status_t check_device(const eqlinear_plan* p) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) {
    set_error("hipGetDevice", e);
    return EQL_ERR_HIP;
  }
  if (p->device >= 0 && cur != p->device) {
    snprintf(g_last_error, sizeof(g_last_error),
             "plan spectra live on device %d but device %d is current", p->device, cur);
    return EQL_ERR_INVALID_ARG;
  }
  return EQL_OK;
}

// p4m in binary16 runs on the p4 producer/consumer kernels with paired
// channels (2C -> 2D) when they take that width: twice the matrix products of
// the group Fourier transform, on kernels that are bound by HBM bytes, not
// by the matrix cores, at these widths (measured on MI355X at C = 48,
// D = 192: forward 20.9 us on the generic kernels against the p4 kernel's
// 11.7 us at the paired width).  The knob EQL_P4M_PAIRS=0 selects the
// generic kernels.
bool use_p4m_pairs(const eql::Tuning& tn, eqlinear_group_t group, int64_t n,
                   eqlinear_dtype_t dtype, int64_t C, int64_t D) {
  if (group != EQL_GROUP_DIHEDRAL || n != 4 || dtype != EQL_F16) return false;
  if (tn.p4m_pairs == 0) return false;
  const int64_t k = 2 * C;  // reduction width of the paired forward
  const bool ws_width = k % 32 == 0 && (k <= 192 || k == 256 || k == 384);
  return ws_width && (2 * D) % 4 == 0 && 2 * C <= MAX_CHANNELS && 2 * D <= MAX_CHANNELS;
}

// Workspace of a paired plan: the p4 plan's, then the paired weight gradient
// [2D][2C][4] and bias gradient [2D] (fp32), each 256-byte aligned.
size_t pair_ws_inner(const eqlinear_plan* p, int64_t N) {
  return eql::round_up((int64_t)eqlinear_backward_weight_workspace(p->inner, N), 256);
}
size_t pair_ws_dw(const eqlinear_plan* p) {
  return eql::round_up(16 * p->C * p->D * (int64_t)sizeof(float), 256);
}

// One knob: -1 when unset, empty or outside [lo, hi].
int knob(const char* name, int lo, int hi) {
  const char* v = getenv(name);
  if (v == nullptr || *v == 0) return -1;
  char* end = nullptr;
  const long x = strtol(v, &end, 10);
  if (end == v || *end != 0 || x < lo || x > hi) return -1;
  return (int)x;
}

}  // namespace

eql::Tuning eql::read_tuning() {
  Tuning t;
  t.ws_off = knob("EQL_NO_WS", 0, 1);
  t.ws_nc = knob("EQL_WS_NC", 1, 16);
  t.ws_np = knob("EQL_WS_NP", 1, 16);
  t.ws_nb = knob("EQL_WS_NB", 1, 4);
  t.ws_wpc = knob("EQL_WS_WPC", 1, 8);
  t.ws_qx = knob("EQL_WS_QX", 1, 1 << 20);
  t.ws_g8 = knob("EQL_WS_G8", 0, 1);
  t.ws_pipe = knob("EQL_WS_PIPE", 0, 1);
  t.ws_out = knob("EQL_WS_OUT", 0, 1);
  t.ws_split = knob("EQL_WS_SPLIT", 0, 1);
  t.ws_wfirst = knob("EQL_WS_WFIRST", 0, 1);
  t.ws_ksplit = knob("EQL_WS_KSPLIT", 0, 1);
  const int small_mb = knob("EQL_WS_SMALL_MB", 0, 1 << 20);
  t.ws_small_bytes = small_mb >= 0 ? (int64_t)small_mb << 20 : (int64_t)128 << 20;
  t.ws32_off = knob("EQL_NO_WS32", 0, 1);
  t.ws32_nc = knob("EQL_WS32_NC", 1, 16);
  t.ws32_np = knob("EQL_WS32_NP", 1, 16);
  t.ws32_qx = knob("EQL_WS32_QX", 1, 1 << 20);
  t.ws32_stream = knob("EQL_WS32_STREAM", 0, 1);
  t.ws32_pst = knob("EQL_WS32_PST", 0, 1);
  t.ws32_tail = knob("EQL_WS32_TAIL", 0, 1);
  t.gemm_tile = knob("EQL_GEMM_TILE", 0, 4);
  t.bws_off = knob("EQL_NO_BWS", 0, 1);
  t.bw_tiled = knob("EQL_BW_TILED", 0, 1);
  t.bws_s = knob("EQL_BWS_S", 1, 1 << 20);
  t.cyc_tile = knob("EQL_CYC_TILE", 0, 3);
  t.cyclic_p4 = knob("EQL_CYCLIC_P4", 0, 1);
  t.cyc_bw_tile = knob("EQL_CYC_BW_TILE", 32, 64);
  t.cyc_bw_wgs = knob("EQL_CYC_BW_WGS", 1, 1 << 20);
  t.p4m_pairs = knob("EQL_P4M_PAIRS", 0, 1);
  t.conv_rd = knob("EQL_CONV_RD", 0, 1);
  t.conv_tile = knob("EQL_CONV_TILE", 0, 4);
  t.conv_f32_16 = knob("EQL_CONV_F32_16", 0, 1);
  return t;
}

// ---- scratch of the no-allocation weight gradient --------------------------
// One array per GPU the library runs on, in the code object's device memory
// (zero-initialised, held until the process ends).  Host code never uses the
// array's name as an address: each device's address comes from
// hipGetSymbolAddress, once, on that device's first call.
static __device__ __align__(256) unsigned char scratch[EQL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of the current device's scratch array.
eqlinear_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("hipGetDevice", e);
    return EQL_ERR_HIP;
  }
  if (dev < 0 || dev >= MAX_DEVICES) {
    snprintf(g_last_error, sizeof(g_last_error), "device %d beyond the scratch table (%d)", dev,
             MAX_DEVICES);
    return EQL_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      set_error("hipGetSymbolAddress(scratch)", e);
      return EQL_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return EQL_OK;
}

}  // namespace

extern "C" {

const char* eqlinear_status_string(eqlinear_status_t status) {
  switch (eql::enum_value(status)) {
    case EQL_OK: return "ok";
    case EQL_ERR_INVALID_ARG: return "invalid argument";
    case EQL_ERR_UNSUPPORTED: return "unsupported group, group order or dtype";
    case EQL_ERR_NO_WEIGHT: return "no weight set on the plan";
    case EQL_ERR_MISALIGNED: return "buffer not 16-byte aligned";
    case EQL_ERR_WORKSPACE: return "workspace missing or too small";
    case EQL_ERR_ALLOC: return "device allocation failed";
    case EQL_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* eqlinear_last_error(void) { return g_last_error; }

eqlinear_status_t eqlinear_plan_create(int64_t C, int64_t D, int64_t T, eqlinear_dtype_t dtype,
                                       eqlinear_plan_t* out) {
  if (out == nullptr) return EQL_ERR_INVALID_ARG;
  *out = nullptr;
  const int dv = eql::enum_value(dtype);
  if (dv != EQL_F32 && dv != EQL_F16) return EQL_ERR_UNSUPPORTED;
  return eqlinear_plan_create_group(C, D, EQL_GROUP_CYCLIC, T, (eqlinear_dtype_t)dv, out);
}

eqlinear_status_t eqlinear_plan_create_group(int64_t C, int64_t D, eqlinear_group_t group_arg,
                                             int64_t n, eqlinear_dtype_t dtype_arg,
                                             eqlinear_plan_t* out) {
  if (out == nullptr) return EQL_ERR_INVALID_ARG;
  *out = nullptr;
  const int gv = eql::enum_value(group_arg), dv = eql::enum_value(dtype_arg);
  if ((gv != EQL_GROUP_CYCLIC && gv != EQL_GROUP_DIHEDRAL) || (dv != EQL_F32 && dv != EQL_F16))
    return EQL_ERR_UNSUPPORTED;
  const eqlinear_group_t group = (eqlinear_group_t)gv;
  const eqlinear_dtype_t dtype = (eqlinear_dtype_t)dv;
  int64_t T = 0;
  if (group == EQL_GROUP_CYCLIC) {
    if (n < MIN_T || n > MAX_T) return EQL_ERR_UNSUPPORTED;
    T = n;
  } else if (group == EQL_GROUP_DIHEDRAL) {
    if (n < MIN_DIH || n > MAX_DIH) return EQL_ERR_UNSUPPORTED;
    T = 2 * n;
  } else {
    return EQL_ERR_UNSUPPORTED;
  }
  if (C <= 0 || D <= 0 || C > MAX_CHANNELS || D > MAX_CHANNELS) return EQL_ERR_INVALID_ARG;
  eqlinear_plan* p = new (std::nothrow) eqlinear_plan;
  if (p == nullptr) return EQL_ERR_ALLOC;
  memset(p, 0, sizeof(*p));
  p->C = C;
  p->D = D;
  p->T = (int)T;
  p->group = group;
  p->tune = eql::read_tuning();
  // the cyclic T = 4 (p4) runs the p4 kernels unless EQL_CYCLIC_P4 asks for
  // the generic ones; every other group runs the generic ones
  p->cyclic = group != EQL_GROUP_CYCLIC || T != 4 || p->tune.cyclic_p4 == 1;
  p->cyc_bw_tile = (p->tune.cyc_bw_tile == 64 && T <= 8) ? 64 : 32;
  p->cyc_bw_wgs = p->tune.cyc_bw_wgs > 0 ? p->tune.cyc_bw_wgs : 512;
  p->dtype = dtype;
  p->esize = dtype == EQL_F16 ? 2 : 4;
  p->device = -1;
  p->has_weight = false;
  p->fwd.n_pad = eql::round_up(D, eql::NPAD);
  p->fwd.k_pad = eql::round_up(C, eql::KPAD);
  p->adj.n_pad = eql::round_up(C, eql::NPAD);
  p->adj.k_pad = eql::round_up(D, eql::KPAD);
  p->inner = nullptr;
  p->pair_w = nullptr;
  if (use_p4m_pairs(p->tune, group, n, dtype, C, D)) {
    eqlinear_status_t st = eqlinear_plan_create_group(2 * C, 2 * D, EQL_GROUP_CYCLIC, 4, dtype,
                                                      &p->inner);
    if (st != EQL_OK) {
      delete p;
      return st;
    }
  }
  *out = p;
  return EQL_OK;
}

eqlinear_status_t eqlinear_plan_destroy(eqlinear_plan_t p) {
  if (p == nullptr) return EQL_OK;
  eqlinear_status_t st = EQL_OK;
  if (p->inner != nullptr) st = eqlinear_plan_destroy(p->inner);
  if (p->pair_w != nullptr) {
    hipError_t e = hipFree(p->pair_w);
    if (e != hipSuccess) {
      set_error("hipFree", e);
      st = EQL_ERR_HIP;
    }
  }
  if (p->spec_fwd != nullptr) {
    int prev = -1;
    hipGetDevice(&prev);
    if (prev != p->device) hipSetDevice(p->device);
    hipError_t e = hipFree(p->spec_fwd);  // one allocation holds every device buffer
    if (e != hipSuccess) {
      set_error("hipFree", e);
      st = EQL_ERR_HIP;
    }
    if (prev >= 0 && prev != p->device) hipSetDevice(prev);
  }
  delete p;
  return st;
}

eqlinear_status_t eqlinear_set_weight(eqlinear_plan_t p, const void* W, const void* bias,
                                      void* stream) {
  if (p == nullptr || W == nullptr) return EQL_ERR_INVALID_ARG;
  if (!aligned16(W) || !aligned16(bias)) return EQL_ERR_MISALIGNED;
  eqlinear_status_t st = check_device(p);
  if (st != EQL_OK) return st;
  if (p->inner != nullptr) {
    // paired weight and bias, then the p4 plan's spectra of them
    const size_t wbytes = eql::round_up(16 * p->C * p->D * (int64_t)p->esize, 256);
    if (p->pair_w == nullptr) {
      hipError_t e = hipMalloc(&p->pair_w, wbytes + 2 * p->D * p->esize);
      if (e != hipSuccess) {
        p->pair_w = nullptr;
        set_error("hipMalloc(paired weight)", e);
        return EQL_ERR_ALLOC;
      }
      int dev = -1;
      hipGetDevice(&dev);
      p->device = dev;
    }
    void* bp = (char*)p->pair_w + wbytes;
    hipError_t e = eql::launch_p4m_pair_weight(W, bias, p->pair_w, bp, p->C, p->D,
                                              (hipStream_t)stream);
    if (e != hipSuccess) {
      set_error("paired weight launch", e);
      return EQL_ERR_HIP;
    }
    st = eqlinear_set_weight(p->inner, p->pair_w, bias != nullptr ? bp : nullptr, stream);
    if (st == EQL_OK) p->has_weight = true;
    return st;
  }
  if (p->spec_fwd == nullptr) {
    const size_t fwd_bytes = (size_t)p->T * p->fwd.plane_elems() * p->esize;
    const size_t adj_bytes = (size_t)p->T * p->adj.plane_elems() * p->esize;
    const size_t bias_bytes = (size_t)p->fwd.n_pad * sizeof(float);
    const size_t zero_bytes = (size_t)p->adj.n_pad * sizeof(float);
    // p4 plans keep the operands of the producer/consumer kernels a second
    // time in fragment order: both in binary16, the forward one in binary32
    const bool frag = !p->cyclic;
    const bool frag_adj = frag && p->dtype == EQL_F16;
    const size_t frag_bytes = frag ? fwd_bytes + (frag_adj ? adj_bytes : 0) : 0;
    void* mem = nullptr;
    hipError_t e = hipMalloc(&mem, fwd_bytes + adj_bytes + bias_bytes + zero_bytes + frag_bytes);
    if (e != hipSuccess) {
      set_error("hipMalloc(spectra)", e);
      return EQL_ERR_ALLOC;
    }
    int dev = -1;
    hipGetDevice(&dev);
    char* base = (char*)mem;
    p->spec_fwd = base;
    p->spec_adj = base + fwd_bytes;
    p->bias_f32 = (float*)(base + fwd_bytes + adj_bytes);
    p->zeros_f32 = (float*)(base + fwd_bytes + adj_bytes + bias_bytes);
    if (frag) {
      p->frag_fwd = base + fwd_bytes + adj_bytes + bias_bytes + zero_bytes;
      p->frag_adj = frag_adj ? (char*)p->frag_fwd + fwd_bytes : nullptr;
    }
    p->device = dev;
  }
  hipError_t e = eql::launch_spectra(p, W, bias, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("weight spectra launch", e);
    return EQL_ERR_HIP;
  }
  p->has_weight = true;
  return EQL_OK;
}

static eqlinear_status_t check_gemm_args(eqlinear_plan_t p, const void* in, const void* out,
                                         int64_t N) {
  if (p == nullptr) return EQL_ERR_INVALID_ARG;
  if (N < 0 || N > MAX_ROWS) return EQL_ERR_INVALID_ARG;
  if (!p->has_weight) return EQL_ERR_NO_WEIGHT;
  if (N == 0) return EQL_OK;
  if (in == nullptr || out == nullptr) return EQL_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(out)) return EQL_ERR_MISALIGNED;
  return EQL_OK;
}

eqlinear_status_t eqlinear_forward(eqlinear_plan_t p, const void* x, void* y, int64_t N,
                                   void* stream) {
  return eqlinear_forward_act(p, x, y, N, EQL_ACT_NONE, stream);
}

eqlinear_status_t eqlinear_forward_act(eqlinear_plan_t p, const void* x, void* y, int64_t N,
                                       eqlinear_act_t act_arg, void* stream) {
  const int av = eql::enum_value(act_arg);
  if (av != EQL_ACT_NONE && av != EQL_ACT_GELU && av != EQL_ACT_GELU_TANH) return EQL_ERR_INVALID_ARG;
  const eqlinear_act_t act = (eqlinear_act_t)av;
  eqlinear_status_t st = check_gemm_args(p, x, y, N);
  if (st != EQL_OK || N == 0) return st;
  if (p->inner != nullptr) return eqlinear_forward_act(p->inner, x, y, N, act, stream);
  st = check_device(p);
  if (st != EQL_OK) return st;
  hipError_t e = eql::launch_forward(p, x, y, N, (int)act, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("forward launch", e);
    return EQL_ERR_HIP;
  }
  return EQL_OK;
}

eqlinear_status_t eqlinear_backward_input(eqlinear_plan_t p, const void* dy, void* dx, int64_t N,
                                          void* stream) {
  eqlinear_status_t st = check_gemm_args(p, dy, dx, N);
  if (st != EQL_OK || N == 0) return st;
  if (p->inner != nullptr) return eqlinear_backward_input(p->inner, dy, dx, N, stream);
  st = check_device(p);
  if (st != EQL_OK) return st;
  hipError_t e = eql::launch_backward_input(p, dy, dx, N, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("backward_input launch", e);
    return EQL_ERR_HIP;
  }
  return EQL_OK;
}

size_t eqlinear_backward_weight_workspace(eqlinear_plan_t p, int64_t N) {
  if (p == nullptr || N < 0 || N > MAX_ROWS) return 0;
  if (p->inner != nullptr)
    return N == 0 ? 0 : pair_ws_inner(p, N) + pair_ws_dw(p) + 2 * p->D * sizeof(float);
  return eql::bwd_weight_workspace_bytes(p, N);
}

eqlinear_status_t eqlinear_backward_weight(eqlinear_plan_t p, const void* x, const void* dy,
                                           float* dW, float* dbias, int64_t N, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (p == nullptr || dW == nullptr) return EQL_ERR_INVALID_ARG;
  if (N < 0 || N > MAX_ROWS) return EQL_ERR_INVALID_ARG;
  if (N > 0 && (x == nullptr || dy == nullptr)) return EQL_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dW) || !aligned16(dbias) ||
      !aligned16(workspace))
    return EQL_ERR_MISALIGNED;
  const size_t need = eqlinear_backward_weight_workspace(p, N);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return EQL_ERR_WORKSPACE;
  eqlinear_status_t st = check_device(p);
  if (st != EQL_OK) return st;
  if (p->inner != nullptr && N > 0) {
    // the p4 plan's weight gradient of the paired layer, then the fold
    // (N = 0 takes the common path below, which writes zeros)
    const size_t inner_bytes = pair_ws_inner(p, N);
    float* dWp = (float*)((char*)workspace + inner_bytes);
    float* dbp = (float*)((char*)dWp + pair_ws_dw(p));
    st = eqlinear_backward_weight(p->inner, x, dy, dWp, dbias != nullptr ? dbp : nullptr, N,
                                  workspace, inner_bytes, stream);
    if (st != EQL_OK) return st;
    hipError_t e = eql::launch_p4m_fold(dWp, dbp, dW, dbias, p->C, p->D, (hipStream_t)stream);
    if (e != hipSuccess) {
      set_error("weight-gradient fold launch", e);
      return EQL_ERR_HIP;
    }
    return EQL_OK;
  }
  hipError_t e = eql::launch_backward_weight(p, x, dy, dW, dbias, N, workspace, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("backward_weight launch", e);
    return EQL_ERR_HIP;
  }
  return EQL_OK;
}

eqlinear_status_t eqlinear_backward_weight_noalloc(eqlinear_plan_t p, const void* x,
                                                   const void* dy, float* dW, float* dbias,
                                                   int64_t N, void* stream) {
  if (p == nullptr || dW == nullptr) return EQL_ERR_INVALID_ARG;
  if (N < 0 || N > MAX_ROWS) return EQL_ERR_INVALID_ARG;
  if (N > 0 && (x == nullptr || dy == nullptr)) return EQL_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dW) || !aligned16(dbias))
    return EQL_ERR_MISALIGNED;
  const size_t need = eqlinear_backward_weight_workspace(p, N);
  if (need > EQL_NOALLOC_SCRATCH_BYTES) {
    snprintf(g_last_error, sizeof(g_last_error),
             "backward_weight of %lld rows needs %zu bytes of scratch; the no-allocation "
             "entry point holds %zu",
             (long long)N, need, (size_t)EQL_NOALLOC_SCRATCH_BYTES);
    return EQL_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if (need > 0) {
    const eqlinear_status_t st = scratch_address(&ws);
    if (st != EQL_OK) return st;
  }
  return eqlinear_backward_weight(p, x, dy, dW, dbias, N, ws, need, stream);
}

eqlinear_status_t eqlinear_mac_counts(eqlinear_plan_t p, int64_t N, int64_t* spectral_macs,
                                      int64_t* dense_macs) {
  if (p == nullptr || N < 0) return EQL_ERR_INVALID_ARG;
  // Cyclic: real DFT of length T: frequency 0 (and T/2 for even T) is real,
  // one product each; each kept complex frequency 1 <= k < T - k costs four
  // real products; the others are conjugates (free).  p4: 1 + 4 + 1 = 6 of 16.
  // Dihedral D_n: one product per one-dimensional representation (4 for even
  // n, 2 for odd n) and eight per two-dimensional one ((n - 1) / 2 of them).
  const int64_t T = p->T;
  int64_t products = 1 + 4 * ((T - 1) / 2) + (T % 2 == 0 ? 1 : 0);
  if (p->group == EQL_GROUP_DIHEDRAL) {
    const int64_t n = T / 2;
    products = (n % 2 == 0 ? 4 : 2) + 8 * ((n - 1) / 2);
    // p4m on the p4 kernels: six products per paired channel pair, 24 per (c, d)
    if (p->inner != nullptr) products = 24;
  }
  const int64_t ncd = N * p->C * p->D;
  if (spectral_macs) *spectral_macs = products * ncd;
  if (dense_macs) *dense_macs = T * T * ncd;
  return EQL_OK;
}

}  // extern "C"
