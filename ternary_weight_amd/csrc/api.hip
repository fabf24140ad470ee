// C ABI of libbitlinear.so: argument checks, library-owned workspace, and the
// choice of kernels for the BitLinear forward path.  Every check runs before
// any HIP call; every GPU call only enqueues work on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <set>
#include <tuple>
#include <utility>
#include <vector>

#include "../../include/bitlinear.h"
#include "kernels.hpp"

using namespace bl;

namespace {

constexpr size_t kAlign = 256;
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bl_status check_shape(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K <= 0 || N <= 0) return BL_ERR_INVALID_ARGUMENT;
  if (K % 128 != 0 || K > kKMax) return BL_ERR_UNSUPPORTED;
  if (M > INT32_MAX - 256 || N > INT32_MAX - 256) return BL_ERR_UNSUPPORTED;
  if (((M + 127) / 128) * ((N + 127) / 128) > INT32_MAX) return BL_ERR_UNSUPPORTED;
  if (N * (K / 4) > kMaxOffset || M * K > kMaxOffset) return BL_ERR_UNSUPPORTED;
  return BL_OK;
}

bl_status check_eps(float eps) {
  return (std::isfinite(eps) && eps >= 0.0f) ? BL_OK : BL_ERR_INVALID_ARGUMENT;
}

bl_status check_forward(const float* x, const void* norm_w, const uint8_t* packed_w,
                        float w_scale, int64_t M, int64_t K, int64_t N, float eps, const float* y) {
  bl_status st = check_shape(M, K, N);
  if (st != BL_OK) return st;
  if ((st = check_eps(eps)) != BL_OK) return st;
  if (!(std::isfinite(w_scale) && w_scale > 0.0f)) return BL_ERR_INVALID_ARGUMENT;
  if (!packed_w) return BL_ERR_INVALID_ARGUMENT;  // norm_w may be null: no norm
  if (M > 0 && (!x || !y)) return BL_ERR_INVALID_ARGUMENT;
  if (!aligned16(norm_w) || !aligned16(packed_w) || (M > 0 && (!aligned16(x) || !aligned16(y))))
    return BL_ERR_MISALIGNED;
  return BL_OK;
}

// Workspace layout for M rows of width K: xq [M][K] int8, factor [M] f32,
// rowsum [M] i32, each 256-byte aligned.
struct WsLayout {
  size_t xq, factor, rowsum, bytes;
};
WsLayout ws_layout(int64_t M, int64_t K) {
  WsLayout l;
  l.xq = 0;
  l.factor = round_up(static_cast<size_t>(M * K), kAlign);
  l.rowsum = l.factor + round_up(static_cast<size_t>(M) * 4, kAlign);
  l.bytes = l.rowsum + round_up(static_cast<size_t>(M) * 4, kAlign);
  return l;
}

struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
  // Used while its stream was being captured into a graph: the graph holds
  // this address, so the buffer is never freed (growing it retires it).
  bool captured = false;
  // Pinned host staging for bitlinear_forward_batched's launch tables, and
  // an event recorded after the last copy out of it.
  void* host = nullptr;
  size_t host_bytes = 0;
  hipEvent_t host_done = nullptr;
  bool host_pending = false;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
// Buffers retired because a captured graph may still use them; kept until
// the process ends.
std::vector<void*> g_ws_retired;

// Workspace of at least `bytes` for (current device, stream).  During graph
// capture the existing buffer is used (and marked: it is never freed
// afterwards) and growing it is refused.  Outside capture, growing it waits
// for the stream's earlier work and replaces the buffer; the old one is
// freed unless a captured graph may use it.
bl_status acquire_ws(hipStream_t stream, size_t bytes, uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BL_ERR_HIP;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return BL_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& w = g_ws[{dev, stream}];
  if (cs != hipStreamCaptureStatusNone) {
    if (w.bytes < bytes) return BL_ERR_UNSUPPORTED;
    w.captured = true;
  } else if (w.bytes < bytes) {
    if (w.ptr) {
      if (hipStreamSynchronize(stream) != hipSuccess) return BL_ERR_HIP;
      if (w.captured) g_ws_retired.push_back(w.ptr);
      else if (hipFree(w.ptr) != hipSuccess) return BL_ERR_HIP;
      w.ptr = nullptr;
      w.bytes = 0;
      w.captured = false;
    }
    const size_t nb = round_up(bytes, size_t{1} << 20);
    void* p = nullptr;
    if (hipMalloc(&p, nb) != hipSuccess) {
      (void)hipGetLastError();
      return BL_ERR_NOMEM;
    }
    w.ptr = p;
    w.bytes = nb;
  }
  *out = static_cast<uint8_t*>(w.ptr);
  return BL_OK;
}

// Pinned host staging of at least `bytes` for (current device, stream), for
// tables copied to the device asynchronously: waits until the last copy out
// of the previous contents has finished.  Not for use during capture.
bl_status acquire_staging(hipStream_t stream, size_t bytes, uint8_t** out, hipEvent_t* done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BL_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& w = g_ws[{dev, stream}];
  if (w.host_pending) {
    if (hipEventSynchronize(w.host_done) != hipSuccess) return BL_ERR_HIP;
    w.host_pending = false;
  }
  if (!w.host_done && hipEventCreateWithFlags(&w.host_done, hipEventDisableTiming) != hipSuccess) {
    w.host_done = nullptr;
    return BL_ERR_HIP;
  }
  if (w.host_bytes < bytes) {
    if (w.host && hipHostFree(w.host) != hipSuccess) return BL_ERR_HIP;
    w.host = nullptr;
    w.host_bytes = 0;
    const size_t nb = round_up(bytes, size_t{1} << 16);
    void* p = nullptr;
    if (hipHostMalloc(&p, nb, hipHostMallocDefault) != hipSuccess) {
      (void)hipGetLastError();
      return BL_ERR_NOMEM;
    }
    w.host = p;
    w.host_bytes = nb;
  }
  // The caller records host_done after its copy; mark it pending now (the
  // lock is released before the copy is enqueued).
  w.host_pending = true;
  *out = static_cast<uint8_t*>(w.host);
  *done = w.host_done;
  return BL_OK;
}

inline bl_status from_hip(hipError_t e) { return e == hipSuccess ? BL_OK : BL_ERR_HIP; }

ProbSet single_set(const Prob& p, int total) {
  ProbSet s{};
  s.single = p;
  s.probs = nullptr;
  s.units = nullptr;
  s.total = total;
  return s;
}

// Stage 2 for one problem: the decode kernel for M <= kGemvMaxM (fused:
// with stage 1, and the FFN glue when p.act is set, inside it), else the
// tiled MFMA kernel.
hipError_t launch_matmul_single(const Prob& p, bool raw, bool fused, hipStream_t stream) {
  if (p.M <= kGemvMaxM) {
    GemvLaunch L{};
    L.single = p;
    L.units = nullptr;
    L.tiles = gemv_single_tiles(p.N, gemv_bucket(p.K));
    L.total = gemv_units(p.N, gemv_bucket(p.K), L.tiles);
    return launch_gemv(L, raw, gemv_bucket(p.K), p.M, p.K, fused, stream,
                       fused && p.act != kActNone);
  }
  return launch_gemm(single_set(p, gemm_units(p.M, p.N)), raw, stream);
}

}  // namespace

extern "C" {

const char* bl_status_string(bl_status s) {
  switch (s) {
    case BL_OK: return "BL_OK";
    case BL_ERR_INVALID_ARGUMENT: return "BL_ERR_INVALID_ARGUMENT";
    case BL_ERR_UNSUPPORTED: return "BL_ERR_UNSUPPORTED";
    case BL_ERR_MISALIGNED: return "BL_ERR_MISALIGNED";
    case BL_ERR_NONFINITE: return "BL_ERR_NONFINITE";
    case BL_ERR_HIP: return "BL_ERR_HIP";
    case BL_ERR_NOMEM: return "BL_ERR_NOMEM";
    case BL_ERR_INTERNAL: return "BL_ERR_INTERNAL";
    case BL_ERR_NOT_FOUND: return "BL_ERR_NOT_FOUND";
    default: return "BL_ERR_UNKNOWN";
  }
}

int64_t bl_k_max(void) { return kKMax; }

namespace {

// The calls below with a float32 or a float16 norm weight (nw_f16) share these.
bl_status forward_impl(const float* x, const void* norm_w, bool nw_f16, const uint8_t* packed_w,
                       float w_scale, int64_t M, int64_t K, int64_t N, float eps, float* y,
                       void* stream) {
  try {
    bl_status st = check_forward(x, norm_w, packed_w, w_scale, M, K, N, eps, y);
    if (st != BL_OK || M == 0) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Prob p{};
    p.x = x;
    p.norm_w = static_cast<const float*>(norm_w);
    p.nw_f16 = nw_f16 ? 1 : 0;
    p.w = packed_w;
    p.y = y;
    p.acc = nullptr;
    p.w_scale = w_scale;
    p.eps = eps;
    p.M = static_cast<int>(M);
    p.K = static_cast<int>(K);
    p.N = static_cast<int>(N);
    if (p.M <= kGemvSingleFusedMaxM && gemv_fusable(p.M, p.K))
      return from_hip(launch_matmul_single(p, false, true, s));
    const WsLayout l = ws_layout(M, K);
    uint8_t* ws = nullptr;
    if ((st = acquire_ws(s, l.bytes, &ws)) != BL_OK) return st;
    p.xq = reinterpret_cast<int8_t*>(ws + l.xq);
    p.factor = reinterpret_cast<float*>(ws + l.factor);
    p.rowsum = reinterpret_cast<int32_t*>(ws + l.rowsum);
    if ((st = from_hip(launch_quant(single_set(p, quant_units(p.M)), p.K, false, kActNone, s))) !=
        BL_OK)
      return st;
    return from_hip(launch_matmul_single(p, false, false, s));
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

// Prefill with the quantization inside the product's producer: a statistics
// pass (factor, row sum and max|u| per row; no codes) and the prefill kernel
// that codes the fp32 rows itself.  Decode sizes take bitlinear_forward's
// path, which already quantizes inside its kernel when the rows fit.
bl_status forward_pq_impl(const float* x, const void* norm_w, bool nw_f16, const uint8_t* packed_w,
                          float w_scale, int64_t M, int64_t K, int64_t N, float eps, float* y,
                          void* stream) {
  try {
    bl_status st = check_forward(x, norm_w, packed_w, w_scale, M, K, N, eps, y);
    if (st != BL_OK || M == 0) return st;
    if (M <= kGemvMaxM) return forward_impl(x, norm_w, nw_f16, packed_w, w_scale, M, K, N, eps, y, stream);
    if (K > kGemmPqMaxK || M * K * 4 >= (int64_t{1} << 31)) return BL_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Prob p{};
    p.x = x;
    p.norm_w = static_cast<const float*>(norm_w);
    p.nw_f16 = nw_f16 ? 1 : 0;
    p.w = packed_w;
    p.y = y;
    p.acc = nullptr;
    p.xq = nullptr;
    p.w_scale = w_scale;
    p.eps = eps;
    p.M = static_cast<int>(M);
    p.K = static_cast<int>(K);
    p.N = static_cast<int>(N);
    // factor, row sums and max|u|: 12 bytes per row instead of K codes
    const size_t part = round_up(static_cast<size_t>(M) * 4, 256);
    uint8_t* ws = nullptr;
    if ((st = acquire_ws(s, 3 * part, &ws)) != BL_OK) return st;
    p.factor = reinterpret_cast<float*>(ws);
    p.rowsum = reinterpret_cast<int32_t*>(ws + part);
    p.amax = reinterpret_cast<float*>(ws + 2 * part);
    if ((st = from_hip(launch_quant_stats(single_set(p, quant_units(p.M)), p.K, s))) != BL_OK) return st;
    return from_hip(launch_gemm_pq(p, s));
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

bl_status quant_impl(const float* x, const void* norm_w, bool nw_f16, int64_t M, int64_t K,
                     float eps, int8_t* xq, float* x_factor, void* stream) {
  try {
    bl_status st = check_shape(M, K, 1);
    if (st != BL_OK) return st;
    if ((st = check_eps(eps)) != BL_OK) return st;
    if (M > 0 && (!x || !xq || !x_factor)) return BL_ERR_INVALID_ARGUMENT;
    if (!aligned16(norm_w) || (M > 0 && (!aligned16(x) || !aligned16(xq) || !aligned16(x_factor))))
      return BL_ERR_MISALIGNED;
    if (M == 0) return BL_OK;
    Prob p{};
    p.x = x;
    p.norm_w = static_cast<const float*>(norm_w);
    p.nw_f16 = nw_f16 ? 1 : 0;
    p.xq = xq;
    p.factor = x_factor;
    p.rowsum = nullptr;
    p.eps = eps;
    p.M = static_cast<int>(M);
    p.K = static_cast<int>(K);
    p.N = 1;
    return from_hip(
        launch_quant(single_set(p, quant_units(p.M)), p.K, false, kActNone, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

}  // namespace

bl_status bitlinear_matmul_i32(const int8_t* xq, const uint8_t* packed_w, int64_t M, int64_t K,
                               int64_t N, int32_t* acc, void* stream) {
  try {
    bl_status st = check_shape(M, K, N);
    if (st != BL_OK) return st;
    if (!packed_w || (M > 0 && (!xq || !acc))) return BL_ERR_INVALID_ARGUMENT;
    if (!aligned16(packed_w) || (M > 0 && (!aligned16(xq) || !aligned16(acc))))
      return BL_ERR_MISALIGNED;
    if (M == 0) return BL_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = nullptr;
    if ((st = acquire_ws(s, round_up(static_cast<size_t>(M) * 4, kAlign), &ws)) != BL_OK) return st;
    Prob p{};
    p.w = packed_w;
    p.xq = const_cast<int8_t*>(xq);
    p.rowsum = reinterpret_cast<int32_t*>(ws);
    p.acc = acc;
    p.w_scale = 1.0f;
    p.M = static_cast<int>(M);
    p.K = static_cast<int>(K);
    p.N = static_cast<int>(N);
    if ((st = from_hip(launch_rowsum(p, s))) != BL_OK) return st;
    return from_hip(launch_matmul_single(p, true, false, s));
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

namespace {

// ---- FFN glue: the down projection fed by act(gate) * up ------------------

bl_status glu_quant_impl(const float* gate, const float* up, int32_t act, const void* norm_w,
                         bool nw_f16, int64_t M, int64_t K, float eps, int8_t* xq, float* x_factor,
                         void* stream) {
  try {
    bl_status st = check_shape(M, K, 1);
    if (st != BL_OK) return st;
    if ((st = check_eps(eps)) != BL_OK) return st;
    if (act != BL_ACT_SILU && act != BL_ACT_GELU_TANH) return BL_ERR_INVALID_ARGUMENT;
    if (M > 0 && (!gate || !up || !xq || !x_factor)) return BL_ERR_INVALID_ARGUMENT;
    if (!aligned16(norm_w) ||
        (M > 0 && (!aligned16(gate) || !aligned16(up) || !aligned16(xq) || !aligned16(x_factor))))
      return BL_ERR_MISALIGNED;
    if (M == 0) return BL_OK;
    Prob p{};
    p.x = gate;
    p.up = up;
    p.act = act == BL_ACT_SILU ? kActSilu : kActGeluTanh;
    p.norm_w = static_cast<const float*>(norm_w);
    p.nw_f16 = nw_f16 ? 1 : 0;
    p.xq = xq;
    p.factor = x_factor;
    p.rowsum = nullptr;
    p.eps = eps;
    p.M = static_cast<int>(M);
    p.K = static_cast<int>(K);
    p.N = 1;
    return from_hip(launch_quant(single_set(p, quant_units(p.M)), p.K, false, p.act,
                                 static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

bl_status glu_forward_impl(const float* gate, const float* up, int32_t act, const void* norm_w,
                           bool nw_f16, const uint8_t* packed_w, float w_scale, int64_t M,
                           int64_t K, int64_t N, float eps, float* y, void* stream) {
  try {
    bl_status st = check_forward(gate, norm_w, packed_w, w_scale, M, K, N, eps, y);
    if (st != BL_OK) return st;
    if (act != BL_ACT_SILU && act != BL_ACT_GELU_TANH) return BL_ERR_INVALID_ARGUMENT;
    if (M > 0 && !up) return BL_ERR_INVALID_ARGUMENT;
    if (M > 0 && !aligned16(up)) return BL_ERR_MISALIGNED;
    if (M == 0) return BL_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Prob p{};
    p.x = gate;
    p.up = up;
    p.act = act == BL_ACT_SILU ? kActSilu : kActGeluTanh;
    p.norm_w = static_cast<const float*>(norm_w);
    p.nw_f16 = nw_f16 ? 1 : 0;
    p.w = packed_w;
    p.y = y;
    p.acc = nullptr;
    p.w_scale = w_scale;
    p.eps = eps;
    p.M = static_cast<int>(M);
    p.K = static_cast<int>(K);
    p.N = static_cast<int>(N);
    // Decode sizes whose gate and up rows fit on chip: one launch, no workspace.
    if (p.M <= kGemvSingleFusedMaxM && gemv_fusable(p.M, p.K, true))
      return from_hip(launch_matmul_single(p, false, true, s));
    const WsLayout l = ws_layout(M, K);
    uint8_t* ws = nullptr;
    if ((st = acquire_ws(s, l.bytes, &ws)) != BL_OK) return st;
    p.xq = reinterpret_cast<int8_t*>(ws + l.xq);
    p.factor = reinterpret_cast<float*>(ws + l.factor);
    p.rowsum = reinterpret_cast<int32_t*>(ws + l.rowsum);
    if ((st = from_hip(launch_quant(single_set(p, quant_units(p.M)), p.K, false, p.act, s))) != BL_OK)
      return st;
    return from_hip(launch_matmul_single(p, false, false, s));
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

}  // namespace

bl_status bitlinear_forward(const float* x, const float* norm_w, const uint8_t* packed_w,
                            float w_scale, int64_t M, int64_t K, int64_t N, float eps, float* y,
                            void* stream) {
  return forward_impl(x, norm_w, false, packed_w, w_scale, M, K, N, eps, y, stream);
}
bl_status bitlinear_forward_prefill_fused(const float* x, const float* norm_w, const uint8_t* packed_w,
                                          float w_scale, int64_t M, int64_t K, int64_t N, float eps,
                                          float* y, void* stream) {
  return forward_pq_impl(x, norm_w, false, packed_w, w_scale, M, K, N, eps, y, stream);
}
bl_status bitlinear_forward_prefill_fused_nwf16(const float* x, const uint16_t* norm_w,
                                                const uint8_t* packed_w, float w_scale, int64_t M,
                                                int64_t K, int64_t N, float eps, float* y,
                                                void* stream) {
  return forward_pq_impl(x, norm_w, true, packed_w, w_scale, M, K, N, eps, y, stream);
}
bl_status bitlinear_forward_nwf16(const float* x, const uint16_t* norm_w, const uint8_t* packed_w,
                                  float w_scale, int64_t M, int64_t K, int64_t N, float eps,
                                  float* y, void* stream) {
  return forward_impl(x, norm_w, true, packed_w, w_scale, M, K, N, eps, y, stream);
}
bl_status i2s_pack_device(const float* w, int64_t K, int64_t N, uint8_t* packed,
                          size_t packed_bytes, float* w_scale_out, void* stream) {
  try {
    if (!w || !packed || K <= 0 || N <= 0) return BL_ERR_INVALID_ARGUMENT;
    if (K % 128 != 0) return BL_ERR_UNSUPPORTED;
    const size_t need = i2s_packed_bytes(K, N);
    if (need == 0 || N > INT64_MAX / 64 / K) return BL_ERR_UNSUPPORTED;
    if (packed_bytes < need) return BL_ERR_INVALID_ARGUMENT;
    if (!aligned16(w) || !aligned16(packed)) return BL_ERR_MISALIGNED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = nullptr;
    bl_status st = acquire_ws(s, kPackPartials * sizeof(double) + kAlign, &ws);
    if (st != BL_OK) return st;
    float* scale_dev = reinterpret_cast<float*>(ws + kPackPartials * sizeof(double));
    if ((st = from_hip(launch_i2s_pack_device(w, K, N, packed, reinterpret_cast<double*>(ws),
                                              scale_dev, s))) != BL_OK)
      return st;
    if (w_scale_out) {
      float scale = 0.0f;
      if (hipMemcpyAsync(&scale, scale_dev, sizeof(float), hipMemcpyDeviceToHost, s) != hipSuccess ||
          hipStreamSynchronize(s) != hipSuccess)
        return BL_ERR_HIP;
      if (!std::isfinite(scale)) return BL_ERR_NONFINITE;
      *w_scale_out = scale;
    }
    return BL_OK;
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

bl_status bitlinear_quant(const float* x, const float* norm_w, int64_t M, int64_t K, float eps,
                          int8_t* xq, float* x_factor, void* stream) {
  return quant_impl(x, norm_w, false, M, K, eps, xq, x_factor, stream);
}
bl_status bitlinear_quant_nwf16(const float* x, const uint16_t* norm_w, int64_t M, int64_t K,
                                float eps, int8_t* xq, float* x_factor, void* stream) {
  return quant_impl(x, norm_w, true, M, K, eps, xq, x_factor, stream);
}
bl_status bitlinear_glu_quant(const float* gate, const float* up, int32_t act, const float* norm_w,
                              int64_t M, int64_t K, float eps, int8_t* xq, float* x_factor,
                              void* stream) {
  return glu_quant_impl(gate, up, act, norm_w, false, M, K, eps, xq, x_factor, stream);
}
bl_status bitlinear_glu_quant_nwf16(const float* gate, const float* up, int32_t act,
                                    const uint16_t* norm_w, int64_t M, int64_t K, float eps,
                                    int8_t* xq, float* x_factor, void* stream) {
  return glu_quant_impl(gate, up, act, norm_w, true, M, K, eps, xq, x_factor, stream);
}
bl_status bitlinear_glu_forward(const float* gate, const float* up, int32_t act,
                                const float* norm_w, const uint8_t* packed_w, float w_scale,
                                int64_t M, int64_t K, int64_t N, float eps, float* y,
                                void* stream) {
  return glu_forward_impl(gate, up, act, norm_w, false, packed_w, w_scale, M, K, N, eps, y, stream);
}
bl_status bitlinear_glu_forward_nwf16(const float* gate, const float* up, int32_t act,
                                      const uint16_t* norm_w, const uint8_t* packed_w,
                                      float w_scale, int64_t M, int64_t K, int64_t N, float eps,
                                      float* y, void* stream) {
  return glu_forward_impl(gate, up, act, norm_w, true, packed_w, w_scale, M, K, N, eps, y, stream);
}

bl_status bl_release_workspace(void) {
  try {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if (g_ws.empty()) return BL_OK;
    bl_status st = BL_OK;
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return BL_ERR_HIP;
    for (auto& kv : g_ws) {
      Workspace& w = kv.second;
      if (hipSetDevice(kv.first.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        st = BL_ERR_HIP;
        continue;
      }
      // A buffer a captured graph uses stays allocated (retired).
      if (w.ptr && w.captured) g_ws_retired.push_back(w.ptr);
      else if (w.ptr && hipFree(w.ptr) != hipSuccess) st = BL_ERR_HIP;
      if (w.host && hipHostFree(w.host) != hipSuccess) st = BL_ERR_HIP;
      if (w.host_done && hipEventDestroy(w.host_done) != hipSuccess) st = BL_ERR_HIP;
    }
    g_ws.clear();
    if (hipSetDevice(cur) != hipSuccess) st = BL_ERR_HIP;
    return st;
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

}  // extern "C"

// ---------------------------------------------------------------- groups ---

// One stage of a group: a device problem table and one (problem, local unit)
// entry per workgroup.
struct GroupStage {
  const Prob* probs = nullptr;
  const int2* units = nullptr;
  const FatUnit* fat = nullptr;  // decode stages: problem records inline
  int total = 0;
  int count = 0;  // problems
  int max_m = 0, max_k = 0;
  bool fused = false;  // decode stages: stage 1 runs inside the launch
  bool merged = false; // fused decode stage of several superblock counts (one launch)
  bool shared = false; // quantization stages: every unit heads a share set
  int chunks = 0;      // quantization stages: float4 chunks per lane (0: streaming)
  int set_rows = kSetRowsPerWave;  // shared quantization stages: rows per wave
  bool split = false;  // prefill stages: some problem has K splits
  int act = kActNone;  // quantization stages: the FFN glue of every problem (kActNone: none)
  bool glue = false;   // decode stages: fused with the FFN glue (Prob::act per problem)
  size_t shmem = 0;    // fused decode stages: LDS bytes, the largest of the problems' own
};

// Fused decode launches depend on nothing but the caller's earlier work, so
// a group forward runs them side by side: the first on the caller's stream,
// the others on up to kAuxStreams streams of the group (default priority),
// forked from and joined back into the caller's stream with events.  Their
// tails then overlap instead of idling the GPU between launches.
constexpr int kAuxStreams = 3;

struct bl_group {
  int device = 0;
  std::vector<GroupStage> quant;  // quantization launches, per (chunk count, shared)
  GroupStage gemm;
  std::vector<std::pair<int, GroupStage>> gemv;  // per (superblock bucket, fused)
  void* tables = nullptr;     // device: problem tables and unit tables
  void* workspace = nullptr;  // device: per-problem xq, factor, rowsum
  int naux = 0;               // auxiliary streams in use
  hipStream_t aux[kAuxStreams] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[kAuxStreams] = {};
};

namespace {

bl_status group_current_device(const bl_group* g) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BL_ERR_HIP;
  return dev == g->device ? BL_OK : BL_ERR_INVALID_ARGUMENT;
}

ProbSet stage_set(const GroupStage& st) {
  ProbSet s{};
  s.probs = st.probs;
  s.units = st.units;
  s.total = st.total;
  s.split = st.split ? 1 : 0;
  return s;
}

void free_group(bl_group* g) {
  if (!g) return;
  for (int j = 0; j < kAuxStreams; ++j) {
    if (g->join[j]) (void)hipEventDestroy(g->join[j]);
    if (g->aux[j]) (void)hipStreamDestroy(g->aux[j]);
  }
  if (g->fork) (void)hipEventDestroy(g->fork);
  if (g->tables) (void)hipFree(g->tables);
  if (g->workspace) (void)hipFree(g->workspace);
  delete g;
}

// Unit order of the merged decode launch.  Units with the most superblocks
// go first (the longest workgroups start first, the short ones fill the
// end).  Consecutive workgroups are dealt to the XCDs in turn, each with its
// own L2, so the units of one problem are dealt to one XCD: its workgroups
// after the first then find the problem's x and norm weight in that L2.
// Whole problems go to the XCD with the fewest units so far.
void order_merged_units(std::vector<FatUnit>& units) {
  constexpr int kXcd = 8;
  std::stable_sort(units.begin(), units.end(),
                   [](const FatUnit& a, const FatUnit& b) { return a.nsb > b.nsb; });
  std::vector<std::vector<FatUnit>> per_xcd(kXcd);
  for (size_t i = 0; i < units.size();) {
    size_t j = i + 1;
    while (j < units.size() && units[j].p.w == units[i].p.w && units[j].p.y == units[i].p.y) ++j;
    size_t x = 0;
    for (size_t k = 1; k < per_xcd.size(); ++k)
      if (per_xcd[k].size() < per_xcd[x].size()) x = k;
    per_xcd[x].insert(per_xcd[x].end(), units.begin() + i, units.begin() + j);
    i = j;
  }
  std::vector<FatUnit> out;
  out.reserve(units.size());
  for (size_t k = 0; out.size() < units.size(); ++k)
    for (const auto& l : per_xcd)
      if (k < l.size()) out.push_back(l[k]);
  units.swap(out);
}

// Host image of one stage before upload.
struct StageHost {
  bool fat = false;
  size_t shmem = 0;  // fused decode stages: the largest per-problem LDS staging
  std::vector<Prob> probs;
  std::vector<int2> units;
  std::vector<FatUnit> fat_units;
  int max_m = 0, max_k = 0;
  int set_rows = kSetRowsPerWave;  // shared quantization stages: rows per wave
  bool split = false;              // prefill stage: some problem has K splits
  void add(const Prob& p, int nunits, int nsb = 0) {
    ++nprobs;
    const int idx = static_cast<int>(probs.size());
    if (fat) {
      for (int u = 0; u < nunits; ++u) fat_units.push_back(FatUnit{p, u, nsb});
    } else {
      probs.push_back(p);
      for (int u = 0; u < nunits; ++u) units.push_back(int2{idx, u});
    }
    max_m = std::max(max_m, p.M);
    max_k = std::max(max_k, p.K);
  }
  size_t nunits() const { return fat ? fat_units.size() : units.size(); }
  int nprobs = 0;
};

// Quantization stages.  Problems whose rows are the same x (pointer, M, K and
// eps equal) form a share set: they are placed next to each other, the first
// carrying the set's size, and only it gets work units, so one pass over x
// quantizes the rows for every problem of the set.  Sets of two or more go
// to launches of the shared kernel variant, single problems to the plain
// one, each by the register-resident chunk count of their K.  Sets keep the
// order of their first problem.  Glue problems (act(x) * up) never share;
// they go to launches of their own per activation.
constexpr int kQuantMergedChunks = -1;  // QuantKey::chunks of the merged launch

struct QuantKey {
  int chunks;
  bool shared;
  int act;
  bool operator<(const QuantKey& o) const {
    if (chunks != o.chunks) return chunks < o.chunks;
    return shared != o.shared ? shared < o.shared : act < o.act;
  }
};

std::map<QuantKey, StageHost> build_quant_stages(const std::vector<Prob>& probs) {
  std::vector<std::vector<int>> sets;
  for (size_t i = 0; i < probs.size(); ++i) {
    const Prob& p = probs[i];
    int found = -1;
    for (size_t j = 0; j < sets.size() && found < 0; ++j) {
      const Prob& q = probs[sets[j][0]];
      if (p.act == kActNone && q.act == kActNone && q.x == p.x && q.M == p.M && q.K == p.K &&
          q.eps == p.eps)
        found = static_cast<int>(j);
    }
    if (found < 0) {
      found = static_cast<int>(sets.size());
      sets.emplace_back();
    }
    sets[found].push_back(static_cast<int>(i));
  }
  // Sets larger than the register-resident share kernel holds are split
  // (each part reads x once).
  std::vector<std::vector<int>> parts;
  for (const auto& set : sets) {
    const size_t cap = static_cast<size_t>(quant_set_max(quant_chunks(probs[set[0]].K)));
    if (cap == 0 || set.size() <= cap) {
      parts.push_back(set);
      continue;
    }
    for (size_t b = 0; b < set.size(); b += cap)
      parts.emplace_back(set.begin() + b, set.begin() + std::min(set.size(), b + cap));
  }
  // Small groups: every set in one merged launch (one row per wave) when the
  // separate launches would be several, all register-resident and without
  // the glue, and at most kQuantMergeMaxUnits workgroups in all.
  {
    std::set<std::pair<int, bool>> kinds;
    int64_t units = 0;
    bool ok = true;
    for (const auto& set : parts) {
      const Prob& lead = probs[set[0]];
      const int nc = quant_chunks(lead.K);
      if (nc == 0 || lead.act != kActNone) ok = false;
      kinds.insert({nc, set.size() > 1});
      units += quant_units(lead.M);
    }
    if (ok && kinds.size() > 1 && units <= kQuantMergeMaxUnits) {
      std::map<QuantKey, StageHost> out;
      StageHost& h = out[QuantKey{kQuantMergedChunks, false, kActNone}];
      h.set_rows = 1;
      for (const auto& set : parts) {
        const Prob& lead = probs[set[0]];
        const int first = static_cast<int>(h.probs.size());
        for (size_t k = 0; k < set.size(); ++k) {
          Prob p = probs[set[k]];
          p.share = k == 0 ? static_cast<int>(set.size()) : 0;
          h.probs.push_back(p);
          ++h.nprobs;
        }
        for (int u = 0; u < quant_units(lead.M); ++u) h.units.push_back(int2{first, u});
        h.max_m = std::max(h.max_m, lead.M);
        h.max_k = std::max(h.max_k, lead.K);
      }
      return out;
    }
  }
  // Rows per wave of each shared launch: kSetRowsPerWave, unless that leaves
  // the launch fewer than kSetFewUnits workgroups.
  std::map<QuantKey, long> units_at_default;
  for (const auto& set : parts) {
    const Prob& lead = probs[set[0]];
    const int nc = quant_chunks(lead.K);
    if (set.size() > 1 && nc > 0)
      units_at_default[QuantKey{nc, true, lead.act}] += quant_set_units(lead.M, kSetRowsPerWave);
  }
  std::map<QuantKey, StageHost> out;
  for (const auto& set : parts) {
    const Prob& lead = probs[set[0]];
    const int nc = quant_chunks(lead.K);
    const QuantKey key{nc, set.size() > 1, lead.act};
    StageHost& h = out[key];
    if (set.size() > 1 && nc > 0)
      h.set_rows = units_at_default[key] < kSetFewUnits ? 1 : kSetRowsPerWave;
    const int first = static_cast<int>(h.probs.size());
    for (size_t k = 0; k < set.size(); ++k) {
      Prob p = probs[set[k]];
      p.share = k == 0 ? static_cast<int>(set.size()) : 0;
      h.probs.push_back(p);
      ++h.nprobs;
    }
    const int units =
        set.size() > 1 && nc > 0 ? quant_set_units(lead.M, h.set_rows) : quant_units(lead.M);
    for (int u = 0; u < units; ++u) h.units.push_back(int2{first, u});
    h.max_m = std::max(h.max_m, lead.M);
    h.max_k = std::max(h.max_k, lead.K);
  }
  return out;
}

// Prefill work order.  Each problem keeps its own tile order (row block
// major, so a row block's column tiles, which share activation rows, are
// consecutive).  A launch that runs in successive generations of workgroups
// (more tiles than two per CU) takes the problems one after another: the
// kernel's successor prefetch looks one generation ahead in this order.  A
// launch whose tiles all fit at once merges the tile lists of consecutive
// problems whose packed weights fit kGemmWindowBytes in proportion to their
// progress, so that each XCD's share mixes short-K and long-K tiles in the
// same proportions throughout.  Measured: the plain order is 3% faster on
// the 196-problem prefill launch and 11% on the Gemma3-270M layer at M =
// 4096 (it was 2% slower there at M = 512, where every tile fits at once).
//
// The tiles are then dealt to the XCDs.  Consecutive workgroup ids go to the
// 8 XCDs in turn, and every XCD receives the same number of workgroups, but
// tiles of different K take different times: a plain split of the list into
// 8 contiguous ranges gave a launch of three problems (two at K = 1024, one
// at K = 3072) XCDs with only the long tiles, which finished last.  So each
// sequence (a problem, or a merged window) is cut into 8 contiguous slices
// and XCD x takes slice x of every sequence, in order: every XCD gets the
// same mix of tiles, and a slice still holds consecutive tiles of each
// problem (shared activation rows and weights stay in that XCD's L2).  The
// kernel reads the table entry xcd_remap(b, total) for workgroup b (XCD
// b % 8, its (b / 8)-th workgroup), so XCD x's k-th tile is stored at entry
// x*q + min(x, r) + k.
constexpr size_t kGemmWindowBytes = size_t{2} << 20;
constexpr int kXcds = 8;

void deal_gemm_units(StageHost& h, int cus) {
  if (h.units.empty()) return;
  std::vector<int> tiles(h.probs.size(), 0);
  for (const int2& u : h.units) ++tiles[u.x];
  const bool fits = cus > 0 && h.units.size() <= static_cast<size_t>(2 * cus);
  std::vector<std::vector<int2>> seqs;
  size_t p0 = 0;
  while (p0 < h.probs.size()) {
    size_t p1 = p0 + 1, bytes = static_cast<size_t>(h.probs[p0].N) * static_cast<size_t>(h.probs[p0].K / 4);
    while (fits && p1 < h.probs.size()) {
      const size_t wb = static_cast<size_t>(h.probs[p1].N) * static_cast<size_t>(h.probs[p1].K / 4);
      if (bytes + wb > kGemmWindowBytes) break;
      bytes += wb;
      ++p1;
    }
    // Merge: repeatedly take the problem whose next tile is least advanced
    // relative to its tile count (ties to the lower index).
    std::vector<int2> seq;
    std::vector<int> next(p1 - p0, 0);
    for (;;) {
      int best = -1;
      double key = 0.0;
      for (size_t i = 0; i < next.size(); ++i) {
        const int t = tiles[p0 + i];
        if (next[i] >= t) continue;
        const double k = (next[i] + 0.5) / t;
        if (best < 0 || k < key) {
          best = static_cast<int>(i);
          key = k;
        }
      }
      if (best < 0) break;
      seq.push_back(int2{static_cast<int>(p0) + best, next[best]++});
    }
    seqs.push_back(std::move(seq));
    p0 = p1;
  }
  // Deal: slice x of every sequence to XCD x.
  std::vector<std::vector<int2>> xcd(kXcds);
  for (const auto& seq : seqs) {
    const size_t L = seq.size();
    for (int x = 0; x < kXcds; ++x)
      xcd[x].insert(xcd[x].end(), seq.begin() + L * x / kXcds, seq.begin() + L * (x + 1) / kXcds);
  }
  // Exact counts per XCD (q + 1 for the first r): move tiles from the ends
  // of longer lists to the ends of shorter ones.
  const size_t total = h.units.size();
  const size_t q = total / kXcds, r = total % kXcds;
  auto want = [&](int x) { return q + (static_cast<size_t>(x) < r ? 1 : 0); };
  std::vector<int2> spill;
  for (int x = 0; x < kXcds; ++x)
    while (xcd[x].size() > want(x)) {
      spill.push_back(xcd[x].back());
      xcd[x].pop_back();
    }
  for (int x = 0; x < kXcds; ++x)
    while (xcd[x].size() < want(x)) {
      xcd[x].push_back(spill.back());
      spill.pop_back();
    }
  std::vector<int2> out(total);
  for (int x = 0; x < kXcds; ++x) {
    const size_t base = static_cast<size_t>(x) * q + std::min(static_cast<size_t>(x), r);
    std::copy(xcd[x].begin(), xcd[x].end(), out.begin() + static_cast<std::ptrdiff_t>(base));
  }
  h.units.swap(out);
}

// A launch plan over validated descriptors: the stages' host images (problem
// records with their workspace pointers, unit tables), serialized into one
// table image.  Groups upload it once; bitlinear_forward_batched builds one
// per call.
struct Plan {
  std::map<QuantKey, StageHost> hqs;
  StageHost hm;
  // Decode problems by (bucket, fused, glue); fused ones of up to
  // kGemvMergedMaxNsb superblocks without the glue share one merged launch,
  // keyed (0, true, false).
  std::map<std::tuple<int, bool, bool>, StageHost> hv;
  std::vector<uint8_t> image;
  std::vector<std::array<size_t, 3>> offs;  // per stage: probs, units, fat units
};

struct PlanSizes {
  size_t ws_bytes = 0;     // codes, factors and row sums of the unfused problems,
                           // then the split partial tiles and tile counts
  size_t cnt_off = 0;      // the tile counts: [cnt_off, cnt_off + cnt_bytes) of it
  size_t cnt_bytes = 0;
  size_t table_bound = 0;  // upper bound of the table image
};

// K splits of the prefill problems (one factor per descriptor, 1 = none).
// A prefill launch whose tiles all fit on the device at once (cus compute
// units, one workgroup each) runs as long as its longest workgroup, i.e. its
// largest K: so while the launch still fits, the problem with the most K
// blocks per workgroup gets its split doubled, as long as each split keeps
// kGemmMinSplitBlocks blocks.  cus = 0: no splits.
std::vector<int> gemm_splits(const bl_desc* descs, int32_t count, int cus) {
  std::vector<int> sp(static_cast<size_t>(count), 1);
  if (cus <= 0) return sp;
  auto prefill = [&](int32_t i) { return descs[i].M > kGemvMaxM; };
  auto tiles = [&](int32_t i) {
    return static_cast<int64_t>(gemm_units(static_cast<int>(descs[i].M), static_cast<int>(descs[i].N)));
  };
  int64_t total = 0;
  for (int32_t i = 0; i < count; ++i)
    if (prefill(i)) total += tiles(i);
  if (total == 0 || total > cus) return sp;
  for (;;) {
    int32_t best = -1;
    int64_t best_nb = 0, best_s = 1;
    for (int32_t i = 0; i < count; ++i) {
      if (!prefill(i)) continue;
      const int64_t nb = descs[i].K / 128;
      // blocks per workgroup nb / sp[i], compared without division
      if (best < 0 || nb * best_s > best_nb * sp[i]) {
        best = i;
        best_nb = nb;
        best_s = sp[i];
      }
    }
    if (best < 0) break;
    const int64_t ns = 2 * best_s;
    if (best_nb / ns < kGemmMinSplitBlocks) break;
    const int64_t add = tiles(best) * (ns - best_s);
    if (total + add > cus) break;
    total += add;
    sp[best] = static_cast<int>(ns);
  }
  return sp;
}

// Workspace bytes of the partial tiles of a split prefill problem.
size_t split_part_bytes(const bl_desc& d, int split) {
  if (split <= 1) return 0;
  return round_up(static_cast<size_t>(gemm_units(static_cast<int>(d.M), static_cast<int>(d.N))) *
                      static_cast<size_t>(split) * kGemmPartInts * 4,
                  kAlign);
}

bool desc_fused(const bl_desc& d) {
  return d.M <= kGemvMaxM &&
         gemv_fusable(static_cast<int>(d.M), static_cast<int>(d.K), d.up != nullptr, true);
}

// Validates every descriptor (the rules of bitlinear_forward, plus the glue
// and norm-weight kind fields) and sizes the plan.
bl_status plan_sizes(const bl_desc* descs, int32_t count, int cus, PlanSizes* out) {
  if (!descs || count <= 0) return BL_ERR_INVALID_ARGUMENT;
  int64_t units_q = 0, units_v = 0, units_m = 0;
  PlanSizes z;
  for (int32_t i = 0; i < count; ++i) {
    const bl_desc& d = descs[i];
    bl_status st = check_forward(d.x, d.norm_w, d.packed_w, d.w_scale, d.M, d.K, d.N, d.eps, d.y);
    if (st == BL_OK && d.norm_w_f16 != 0 && d.norm_w_f16 != 1) st = BL_ERR_INVALID_ARGUMENT;
    if (st == BL_OK && d.up && d.act != BL_ACT_SILU && d.act != BL_ACT_GELU_TANH)
      st = BL_ERR_INVALID_ARGUMENT;
    if (st == BL_OK && d.M > 0 && d.up && !aligned16(d.up)) st = BL_ERR_MISALIGNED;
    if (st != BL_OK) return st;
    if (d.M == 0) continue;
    const int M = static_cast<int>(d.M), K = static_cast<int>(d.K), N = static_cast<int>(d.N);
    if (M <= kGemvMaxM) {
      const int v = gemv_units(N, gemv_bucket(K));
      units_v += v;
      z.table_bound += static_cast<size_t>(v) * sizeof(FatUnit);
    } else {
      const int u = gemm_units(M, N);
      units_m += u;
      z.table_bound += sizeof(Prob) + static_cast<size_t>(u) * sizeof(int2);
    }
    if (desc_fused(d)) continue;
    units_q += quant_units(M);
    z.table_bound += sizeof(Prob) + static_cast<size_t>(quant_units(M)) * sizeof(int2);
    z.ws_bytes += ws_layout(d.M, d.K).bytes;
  }
  if (units_q > INT32_MAX / 2 || units_v > INT32_MAX / 2 || units_m > INT32_MAX / 2)
    return BL_ERR_UNSUPPORTED;
  // Split prefill problems: partial tiles after the per-problem regions, all
  // tile counts at the end; their units replace the unsplit ones.
  const std::vector<int> sp = gemm_splits(descs, count, cus);
  size_t cnt = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (sp[i] <= 1) continue;
    const bl_desc& d = descs[i];
    const size_t t = static_cast<size_t>(gemm_units(static_cast<int>(d.M), static_cast<int>(d.N)));
    z.ws_bytes += split_part_bytes(d, sp[i]);
    z.table_bound += t * static_cast<size_t>(sp[i] - 1) * sizeof(int2);
    cnt += t * sizeof(unsigned);
  }
  if (cnt > 0) {
    z.cnt_off = z.ws_bytes;
    z.cnt_bytes = round_up(cnt, kAlign);
    z.ws_bytes += z.cnt_bytes;
  }
  // every stage holds at least one problem: at most 1 + 2 * count stages,
  // each with three sections padded to kAlign
  z.table_bound += (1 + 2 * static_cast<size_t>(count)) * 3 * kAlign;
  *out = z;
  return BL_OK;
}

// Stage host images of the plan (workspace pointers from ws), then the table
// image.  Descriptors must have passed plan_sizes.
void plan_build(const bl_desc* descs, int32_t count, int cus, uint8_t* ws, Plan& pl) {
  std::vector<Prob> qprobs;
  size_t off = 0;
  const std::vector<int> sp = gemm_splits(descs, count, cus);
  size_t part_off = 0, cnt_total = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (descs[i].M == 0) continue;
    if (!desc_fused(descs[i])) part_off += ws_layout(descs[i].M, descs[i].K).bytes;
  }
  size_t cnt_off = part_off;
  for (int32_t i = 0; i < count; ++i) cnt_off += split_part_bytes(descs[i], sp[i]);
  for (int32_t i = 0; i < count; ++i) {
    const bl_desc& d = descs[i];
    if (d.M == 0) continue;
    const bool glue = d.up != nullptr;
    const bool fused = desc_fused(d);
    Prob p{};
    p.x = d.x;
    if (glue) {
      p.up = d.up;
      p.act = d.act == BL_ACT_SILU ? kActSilu : kActGeluTanh;
    }
    p.norm_w = static_cast<const float*>(d.norm_w);
    p.nw_f16 = d.norm_w_f16;
    p.w = d.packed_w;
    if (!fused) {
      const WsLayout l = ws_layout(d.M, d.K);
      p.xq = reinterpret_cast<int8_t*>(ws + off + l.xq);
      p.factor = reinterpret_cast<float*>(ws + off + l.factor);
      p.rowsum = reinterpret_cast<int32_t*>(ws + off + l.rowsum);
      off += l.bytes;
    }
    p.y = d.y;
    p.acc = nullptr;
    p.w_scale = d.w_scale;
    p.eps = d.eps;
    p.M = static_cast<int>(d.M);
    p.K = static_cast<int>(d.K);
    p.N = static_cast<int>(d.N);
    if (!fused) qprobs.push_back(p);
    if (p.M <= kGemvMaxM) {
      const int b = gemv_bucket(p.K);
      const bool merge = fused && !glue && b >= 1 && b <= kGemvMergedMaxNsb;
      // (unfused glue problems read their codes like any other: plain stages)
      StageHost& sh = pl.hv[{merge ? 0 : b, fused, fused && glue}];
      sh.fat = true;
      sh.add(p, gemv_units(p.N, b), merge ? b : 0);
      if (fused) sh.shmem = std::max(sh.shmem, gemv_fused_lds_bytes(p.M, p.K, glue));
    } else {
      const int t = gemm_units(p.M, p.N);
      if (sp[i] > 1) {
        p.ksplit = sp[i];
        p.part = reinterpret_cast<int32_t*>(ws + part_off);
        p.tile_cnt = reinterpret_cast<unsigned*>(ws + cnt_off + cnt_total);
        part_off += split_part_bytes(d, sp[i]);
        cnt_total += static_cast<size_t>(t) * sizeof(unsigned);
        pl.hm.split = true;
      }
      pl.hm.add(p, t * (sp[i] > 1 ? sp[i] : 1));
    }
  }
  pl.hqs = build_quant_stages(qprobs);
  {
    auto it = pl.hv.find({0, true, false});
    if (it != pl.hv.end()) order_merged_units(it->second.fat_units);
  }
  deal_gemm_units(pl.hm, cus);

  // Table image, stage order: prefill, quantization stages, decode stages.
  std::vector<const StageHost*> hosts{&pl.hm};
  for (const auto& kv : pl.hqs) hosts.push_back(&kv.second);
  for (const auto& kv : pl.hv) hosts.push_back(&kv.second);
  const size_t nst = hosts.size();
  size_t total = 0;
  pl.offs.assign(nst, {});
  for (size_t k = 0; k < nst; ++k) {
    pl.offs[k][0] = total;
    total += round_up(hosts[k]->probs.size() * sizeof(Prob), kAlign);
    pl.offs[k][1] = total;
    total += round_up(hosts[k]->units.size() * sizeof(int2), kAlign);
    pl.offs[k][2] = total;
    total += round_up(hosts[k]->fat_units.size() * sizeof(FatUnit), kAlign);
  }
  pl.image.assign(std::max<size_t>(total, 1), 0);
  for (size_t k = 0; k < nst; ++k) {
    const StageHost& h = *hosts[k];
    if (!h.probs.empty())
      std::memcpy(pl.image.data() + pl.offs[k][0], h.probs.data(), h.probs.size() * sizeof(Prob));
    if (!h.units.empty())
      std::memcpy(pl.image.data() + pl.offs[k][1], h.units.data(), h.units.size() * sizeof(int2));
    if (!h.fat_units.empty())
      std::memcpy(pl.image.data() + pl.offs[k][2], h.fat_units.data(),
                  h.fat_units.size() * sizeof(FatUnit));
  }
}

// The group's stages over a copy of the plan's table image at `tables`
// (device).
void plan_bind(const Plan& pl, const uint8_t* tables, bl_group* g) {
  g->quant.assign(pl.hqs.size(), GroupStage{});
  g->gemv.assign(pl.hv.size(), std::pair<int, GroupStage>{});
  std::vector<const StageHost*> hosts{&pl.hm};
  std::vector<GroupStage*> stages{&g->gemm};
  size_t qi = 0;
  for (const auto& kv : pl.hqs) {
    g->quant[qi].shared = kv.first.shared;
    g->quant[qi].chunks = kv.first.chunks;
    g->quant[qi].act = kv.first.act;
    hosts.push_back(&kv.second);
    stages.push_back(&g->quant[qi]);
    ++qi;
  }
  size_t bi = 0;
  for (const auto& kv : pl.hv) {
    g->gemv[bi].first = std::get<0>(kv.first);
    g->gemv[bi].second.fused = std::get<1>(kv.first);
    g->gemv[bi].second.glue = std::get<2>(kv.first);
    g->gemv[bi].second.merged = std::get<0>(kv.first) == 0 && std::get<1>(kv.first);
    hosts.push_back(&kv.second);
    stages.push_back(&g->gemv[bi].second);
    ++bi;
  }
  for (size_t k = 0; k < hosts.size(); ++k) {
    stages[k]->probs = reinterpret_cast<const Prob*>(tables + pl.offs[k][0]);
    stages[k]->units = reinterpret_cast<const int2*>(tables + pl.offs[k][1]);
    stages[k]->fat = hosts[k]->fat ? reinterpret_cast<const FatUnit*>(tables + pl.offs[k][2]) : nullptr;
    stages[k]->total = static_cast<int>(hosts[k]->nunits());
    stages[k]->count = hosts[k]->nprobs;
    stages[k]->max_m = hosts[k]->max_m;
    stages[k]->max_k = hosts[k]->max_k;
    stages[k]->shmem = hosts[k]->shmem;
    stages[k]->set_rows = hosts[k]->set_rows;
    stages[k]->split = hosts[k]->split;
  }
}

}  // namespace

extern "C" {

bl_status bl_group_create(const bl_desc* descs, int32_t count, bl_group** out) {
  try {
    if (!out) return BL_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    PlanSizes sz;
    bl_status st = plan_sizes(descs, count, 0, &sz);  // validation first
    if (st != BL_OK) return st;
    int device = 0, cus = 0;
    if (hipGetDevice(&device) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
      return BL_ERR_HIP;
    if ((st = plan_sizes(descs, count, cus, &sz)) != BL_OK) return st;

    bl_group* g = new (std::nothrow) bl_group;
    if (!g) return BL_ERR_NOMEM;
    g->device = device;
    if (sz.ws_bytes > 0 && hipMalloc(&g->workspace, sz.ws_bytes) != hipSuccess) {
      (void)hipGetLastError();
      free_group(g);
      return BL_ERR_NOMEM;
    }
    // split prefill tiles: the counts start at zero (each launch leaves them so)
    if (sz.cnt_bytes > 0 &&
        hipMemset(static_cast<uint8_t*>(g->workspace) + sz.cnt_off, 0, sz.cnt_bytes) != hipSuccess) {
      free_group(g);
      return BL_ERR_HIP;
    }
    Plan pl;
    plan_build(descs, count, cus, static_cast<uint8_t*>(g->workspace), pl);
    if (hipMalloc(&g->tables, pl.image.size()) != hipSuccess) {
      (void)hipGetLastError();
      free_group(g);
      return BL_ERR_NOMEM;
    }
    if (hipMemcpy(g->tables, pl.image.data(), pl.image.size(), hipMemcpyHostToDevice) != hipSuccess) {
      free_group(g);
      return BL_ERR_HIP;
    }
    plan_bind(pl, static_cast<const uint8_t*>(g->tables), g);
    int nfused = 0;
    for (const auto& st2 : g->gemv) nfused += st2.second.fused ? 1 : 0;
    g->naux = std::min(std::max(nfused - 1, 0), kAuxStreams);
    bool ok = g->naux == 0 || hipEventCreateWithFlags(&g->fork, hipEventDisableTiming) == hipSuccess;
    for (int j = 0; ok && j < g->naux; ++j)
      ok = hipStreamCreateWithFlags(&g->aux[j], hipStreamNonBlocking) == hipSuccess &&
           hipEventCreateWithFlags(&g->join[j], hipEventDisableTiming) == hipSuccess;
    if (!ok) {
      (void)hipGetLastError();
      free_group(g);
      return BL_ERR_HIP;
    }
    *out = g;
    return BL_OK;
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

}  // extern "C"

namespace {

bl_status quant_launch(bl_group* g, size_t i, hipStream_t s) {
  const GroupStage& q = g->quant[i];
  if (q.chunks == kQuantMergedChunks) return from_hip(launch_quant_merged(stage_set(q), s));
  return from_hip(launch_quant(stage_set(q), q.max_k, q.shared, q.act, s, q.set_rows));
}

}  // namespace

extern "C" {

bl_status bl_group_quant(bl_group* g, void* stream) {
  try {
    if (!g) return BL_ERR_INVALID_ARGUMENT;
    bl_status st = group_current_device(g);
    for (size_t i = 0; st == BL_OK && i < g->quant.size(); ++i)
      st = quant_launch(g, i, static_cast<hipStream_t>(stream));
    return st;
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

int32_t bl_group_matmul_launches(const bl_group* g) {
  if (!g) return -1;
  return static_cast<int32_t>(g->gemv.size()) + (g->gemm.total > 0 ? 1 : 0);
}

bl_status bl_group_matmul_launch_info(const bl_group* g, int32_t i, int32_t* kind, int32_t* bucket,
                                      int32_t* count) {
  if (!g || i < 0 || i >= bl_group_matmul_launches(g)) return BL_ERR_INVALID_ARGUMENT;
  const bool decode = i < static_cast<int32_t>(g->gemv.size());
  if (kind) {
    const GroupStage* st = decode ? &g->gemv[i].second : nullptr;
    *kind = !decode ? BL_LAUNCH_PREFILL
                    : (!st->fused ? BL_LAUNCH_DECODE
                                  : (st->glue ? BL_LAUNCH_DECODE_FUSED_GLUE
                                                         : BL_LAUNCH_DECODE_FUSED));
  }
  if (bucket) *bucket = decode ? g->gemv[i].first : 0;
  if (count) *count = decode ? g->gemv[i].second.count : g->gemm.count;
  return BL_OK;
}

bl_status bl_group_matmul_launch(bl_group* g, int32_t i, void* stream) {
  try {
    if (!g || i < 0 || i >= bl_group_matmul_launches(g)) return BL_ERR_INVALID_ARGUMENT;
    bl_status st = group_current_device(g);
    if (st != BL_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (i < static_cast<int32_t>(g->gemv.size())) {
      const GroupStage& gs = g->gemv[i].second;
      if (gs.merged) return from_hip(launch_gemv_merged(gs.fat, gs.total, gs.shmem, s));
      GemvLaunch L{};
      L.units = gs.fat;
      L.total = gs.total;
      L.fused_shmem = gs.shmem;
      return from_hip(launch_gemv(L, false, g->gemv[i].first, gs.max_m, gs.max_k, gs.fused, s,
                                  gs.glue));
    }
    return from_hip(launch_gemm(stage_set(g->gemm), false, s));
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

}  // extern "C"

namespace {

// Stage 1 (when asked) and stage 2 of a group on `stream`, with the fused
// decode launches after the first spread over the auxiliary streams.
bl_status group_run(bl_group* g, hipStream_t s, bool with_quant) {
  bl_status st = group_current_device(g);
  if (st != BL_OK) return st;
  const bool fork = g->naux > 0;
  if (fork) {
    if (hipEventRecord(g->fork, s) != hipSuccess) return BL_ERR_HIP;
    for (int j = 0; j < g->naux; ++j)
      if (hipStreamWaitEvent(g->aux[j], g->fork, 0) != hipSuccess) return BL_ERR_HIP;
  }
  if (with_quant && (st = bl_group_quant(g, s)) != BL_OK) return st;
  const int32_t n = bl_group_matmul_launches(g);
  int fused_seen = 0;
  for (int32_t i = 0; i < n; ++i) {
    hipStream_t target = s;
    if (fork && i < static_cast<int32_t>(g->gemv.size()) && g->gemv[i].second.fused &&
        fused_seen++ > 0)
      target = g->aux[(fused_seen - 2) % g->naux];
    if ((st = bl_group_matmul_launch(g, i, target)) != BL_OK) return st;
  }
  if (fork) {
    for (int j = 0; j < g->naux; ++j)
      if (hipEventRecord(g->join[j], g->aux[j]) != hipSuccess ||
          hipStreamWaitEvent(s, g->join[j], 0) != hipSuccess)
        return BL_ERR_HIP;
  }
  return BL_OK;
}

}  // namespace

extern "C" {

bl_status bl_group_matmul(bl_group* g, void* stream) {
  if (!g) return BL_ERR_INVALID_ARGUMENT;
  try {
    return group_run(g, static_cast<hipStream_t>(stream), false);
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

bl_status bl_group_forward(bl_group* g, void* stream) {
  if (!g) return BL_ERR_INVALID_ARGUMENT;
  try {
    return group_run(g, static_cast<hipStream_t>(stream), true);
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

// Forward launches: the quantization launches, then the matmul launches.
int32_t bl_group_forward_launches(const bl_group* g) {
  if (!g) return -1;
  return static_cast<int32_t>(g->quant.size()) + bl_group_matmul_launches(g);
}

bl_status bl_group_forward_launch_info(const bl_group* g, int32_t i, int32_t* kind,
                                       int32_t* bucket, int32_t* count) {
  if (!g || i < 0 || i >= bl_group_forward_launches(g)) return BL_ERR_INVALID_ARGUMENT;
  const int32_t q = static_cast<int32_t>(g->quant.size());
  if (i >= q) return bl_group_matmul_launch_info(g, i - q, kind, bucket, count);
  const bool merged = g->quant[i].chunks == kQuantMergedChunks;
  if (kind)
    *kind = merged ? BL_LAUNCH_QUANT_MERGED
                   : (g->quant[i].shared ? BL_LAUNCH_QUANT_SHARED
                                         : (g->quant[i].act != kActNone ? BL_LAUNCH_QUANT_GLUE
                                                                        : BL_LAUNCH_QUANT));
  if (bucket) *bucket = merged ? 0 : g->quant[i].chunks;
  if (count) *count = g->quant[i].count;
  return BL_OK;
}

bl_status bl_group_forward_launch(bl_group* g, int32_t i, void* stream) {
  if (!g || i < 0 || i >= bl_group_forward_launches(g)) return BL_ERR_INVALID_ARGUMENT;
  const int32_t q = static_cast<int32_t>(g->quant.size());
  if (i >= q) return bl_group_matmul_launch(g, i - q, stream);
  try {
    const bl_status st = group_current_device(g);
    return st != BL_OK ? st : quant_launch(g, static_cast<size_t>(i), static_cast<hipStream_t>(stream));
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

bl_status bl_group_destroy(bl_group* g) {
  try {
    if (!g) return BL_OK;
    bl_status st = BL_OK;
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) st = BL_ERR_HIP;
    if (hipSetDevice(g->device) != hipSuccess || hipDeviceSynchronize() != hipSuccess) st = BL_ERR_HIP;
    free_group(g);
    if (hipSetDevice(cur) != hipSuccess) st = BL_ERR_HIP;
    return st;
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

}  // extern "C"

extern "C" {

bl_status bl_prefill_splits(const bl_desc* descs, int32_t count, int32_t cus, int32_t* splits) {
  try {
    if (!splits || cus < 0) return BL_ERR_INVALID_ARGUMENT;
    PlanSizes sz;
    const bl_status st = plan_sizes(descs, count, 0, &sz);
    if (st != BL_OK) return st;
    const std::vector<int> sp = gemm_splits(descs, count, cus);
    for (int32_t i = 0; i < count; ++i) splits[i] = sp[static_cast<size_t>(i)];
    return BL_OK;
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

}  // extern "C"

// ------------------------------------------------- stateless batched call ---

extern "C" {

bl_status bitlinear_forward_batched(const bl_desc* descs, int32_t count, void* stream) {
  try {
    // No K splits here: the workspace is shared between calls of different
    // plans, so tile counts could not be kept at zero between them.
    PlanSizes sz;
    bl_status st = plan_sizes(descs, count, 0, &sz);
    if (st != BL_OK) return st;
    bool any = false;
    for (int32_t i = 0; i < count; ++i) any = any || descs[i].M > 0;
    if (!any) return BL_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // The tables travel through pinned host staging on every call, which a
    // captured graph could not replay: capture takes a group instead.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return BL_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) return BL_ERR_UNSUPPORTED;
    const size_t ws_part = round_up(sz.ws_bytes, kAlign);
    uint8_t* ws = nullptr;
    if ((st = acquire_ws(s, ws_part + sz.table_bound, &ws)) != BL_OK) return st;
    Plan pl;
    plan_build(descs, count, 0, ws, pl);
    if (pl.image.size() > sz.table_bound) return BL_ERR_INTERNAL;
    uint8_t* host = nullptr;
    hipEvent_t done = nullptr;
    if ((st = acquire_staging(s, pl.image.size(), &host, &done)) != BL_OK) return st;
    std::memcpy(host, pl.image.data(), pl.image.size());
    if (hipMemcpyAsync(ws + ws_part, host, pl.image.size(), hipMemcpyHostToDevice, s) != hipSuccess ||
        hipEventRecord(done, s) != hipSuccess)
      return BL_ERR_HIP;
    bl_group g;
    if (hipGetDevice(&g.device) != hipSuccess) return BL_ERR_HIP;
    plan_bind(pl, ws + ws_part, &g);
    return group_run(&g, s, true);  // no auxiliary streams: every launch on s
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

}  // extern "C"

// ------------------------------------------------ allocation-free forward ---
// bitlinear_forward_noalloc keeps the codes, factors and row sums of an
// unfused call in `scratch`, a static device array: every GPU that loads the
// library holds its own copy until the process ends.  On the host the
// array's name is only a stand-in, not a device address; the address comes
// from hipGetSymbolAddress, resolved once per device (with that device
// current) and kept, and only that address is handed to the kernels.

namespace {

constexpr size_t kScratchBytes = size_t{64} << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mutex;
std::map<int, uint8_t*> g_scratch;  // device -> address of its scratch

bl_status scratch_address(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BL_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return BL_ERR_HIP;
    }
    it = g_scratch.emplace(dev, static_cast<uint8_t*>(p)).first;
  }
  *out = it->second;
  return BL_OK;
}

}  // namespace

extern "C" {

bl_status bitlinear_forward_noalloc(const float* x, const float* norm_w, const uint8_t* packed_w,
                                    float w_scale, int64_t M, int64_t K, int64_t N, float eps,
                                    float* y, void* stream) {
  try {
    bl_status st = check_forward(x, norm_w, packed_w, w_scale, M, K, N, eps, y);
    if (st != BL_OK || M == 0) return st;
    const WsLayout l = ws_layout(M, K);
    const bool fused = M <= kGemvSingleFusedMaxM && gemv_fusable(static_cast<int>(M), static_cast<int>(K));
    if (!fused && l.bytes > kScratchBytes) return BL_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Prob p{};
    p.x = x;
    p.norm_w = norm_w;
    p.w = packed_w;
    p.y = y;
    p.acc = nullptr;
    p.w_scale = w_scale;
    p.eps = eps;
    p.M = static_cast<int>(M);
    p.K = static_cast<int>(K);
    p.N = static_cast<int>(N);
    if (fused) return from_hip(launch_matmul_single(p, false, true, s));
    uint8_t* ws = nullptr;
    if ((st = scratch_address(&ws)) != BL_OK) return st;
    p.xq = reinterpret_cast<int8_t*>(ws + l.xq);
    p.factor = reinterpret_cast<float*>(ws + l.factor);
    p.rowsum = reinterpret_cast<int32_t*>(ws + l.rowsum);
    // The quantization kernel writes every code, factor and row sum of the
    // M rows before the product reads them: nothing needs clearing.
    if ((st = from_hip(launch_quant(single_set(p, quant_units(p.M)), p.K, false, kActNone, s))) !=
        BL_OK)
      return st;
    return from_hip(launch_matmul_single(p, false, false, s));
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

}  // extern "C"
