// C ABI of libbitlinear.so: argument checks, library-owned workspace, and the
// choice of kernels for the BitLinear forward path.  Every check runs before
// any HIP call; every GPU call only enqueues work on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
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
  return BL_OK;
}

bl_status check_eps(float eps) {
  return (std::isfinite(eps) && eps >= 0.0f) ? BL_OK : BL_ERR_INVALID_ARGUMENT;
}

bl_status check_forward(const float* x, const float* norm_w, const uint8_t* packed_w,
                        float w_scale, int64_t M, int64_t K, int64_t N, float eps, const float* y) {
  bl_status st = check_shape(M, K, N);
  if (st != BL_OK) return st;
  if ((st = check_eps(eps)) != BL_OK) return st;
  if (!(std::isfinite(w_scale) && w_scale > 0.0f)) return BL_ERR_INVALID_ARGUMENT;
  if (!norm_w || !packed_w) return BL_ERR_INVALID_ARGUMENT;
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
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

// Workspace of at least `bytes` for (current device, stream).  Growing it
// waits for the stream's earlier work, frees the old buffer and allocates a
// new one; that is refused while the stream is being captured.
bl_status acquire_ws(hipStream_t stream, size_t bytes, uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BL_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& w = g_ws[{dev, stream}];
  if (w.bytes < bytes) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return BL_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) return BL_ERR_UNSUPPORTED;
    if (w.ptr) {
      if (hipStreamSynchronize(stream) != hipSuccess) return BL_ERR_HIP;
      if (hipFree(w.ptr) != hipSuccess) return BL_ERR_HIP;
      w.ptr = nullptr;
      w.bytes = 0;
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

inline bl_status from_hip(hipError_t e) { return e == hipSuccess ? BL_OK : BL_ERR_HIP; }

ProbSet single_set(const Prob& p, int total) {
  ProbSet s;
  s.single = p;
  s.probs = nullptr;
  s.starts = nullptr;
  s.count = 0;
  s.total = total;
  return s;
}

// Stage 2 for one problem: the decode kernel for M <= kGemvMaxM, else the
// tiled MFMA kernel.
hipError_t launch_matmul_single(const Prob& p, bool raw, hipStream_t stream) {
  if (p.M <= kGemvMaxM) return launch_gemv(single_set(p, gemv_units(p.N)), raw, stream);
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
    default: return "BL_ERR_UNKNOWN";
  }
}

int64_t bl_k_max(void) { return kKMax; }

bl_status bitlinear_forward(const float* x, const float* norm_w, const uint8_t* packed_w,
                            float w_scale, int64_t M, int64_t K, int64_t N, float eps, float* y,
                            void* stream) {
  try {
    bl_status st = check_forward(x, norm_w, packed_w, w_scale, M, K, N, eps, y);
    if (st != BL_OK || M == 0) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const WsLayout l = ws_layout(M, K);
    uint8_t* ws = nullptr;
    if ((st = acquire_ws(s, l.bytes, &ws)) != BL_OK) return st;
    Prob p{};
    p.x = x;
    p.norm_w = norm_w;
    p.w = packed_w;
    p.xq = reinterpret_cast<int8_t*>(ws + l.xq);
    p.factor = reinterpret_cast<float*>(ws + l.factor);
    p.rowsum = reinterpret_cast<int32_t*>(ws + l.rowsum);
    p.y = y;
    p.acc = nullptr;
    p.w_scale = w_scale;
    p.eps = eps;
    p.M = static_cast<int>(M);
    p.K = static_cast<int>(K);
    p.N = static_cast<int>(N);
    if ((st = from_hip(launch_quant(single_set(p, quant_units(p.M)), p.K, s))) != BL_OK) return st;
    return from_hip(launch_matmul_single(p, false, s));
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

bl_status bitlinear_quant(const float* x, const float* norm_w, int64_t M, int64_t K, float eps,
                          int8_t* xq, float* x_factor, void* stream) {
  try {
    bl_status st = check_shape(M, K, 1);
    if (st != BL_OK) return st;
    if ((st = check_eps(eps)) != BL_OK) return st;
    if (!norm_w || (M > 0 && (!x || !xq || !x_factor))) return BL_ERR_INVALID_ARGUMENT;
    if (!aligned16(norm_w) || (M > 0 && (!aligned16(x) || !aligned16(xq) || !aligned16(x_factor))))
      return BL_ERR_MISALIGNED;
    if (M == 0) return BL_OK;
    Prob p{};
    p.x = x;
    p.norm_w = norm_w;
    p.xq = xq;
    p.factor = x_factor;
    p.rowsum = nullptr;
    p.eps = eps;
    p.M = static_cast<int>(M);
    p.K = static_cast<int>(K);
    p.N = 1;
    return from_hip(
        launch_quant(single_set(p, quant_units(p.M)), p.K, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

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
    return from_hip(launch_matmul_single(p, true, s));
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

bl_status bl_release_workspace(void) {
  try {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if (g_ws.empty()) return BL_OK;
    bl_status st = BL_OK;
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return BL_ERR_HIP;
    for (auto& kv : g_ws) {
      if (!kv.second.ptr) continue;
      if (hipSetDevice(kv.first.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
          hipFree(kv.second.ptr) != hipSuccess)
        st = BL_ERR_HIP;
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

struct bl_group {
  int device = 0;
  int count = 0;          // problems with M > 0
  int max_k = 0;
  int quant_total = 0, gemv_total = 0, gemm_total = 0;
  int gemv_count = 0, gemm_count = 0;
  void* tables = nullptr;     // device: all probs | gemv probs | gemm probs | 3 start arrays
  void* workspace = nullptr;  // device: per-problem xq, factor, rowsum
  const Prob* d_all = nullptr;
  const Prob* d_gemv = nullptr;
  const Prob* d_gemm = nullptr;
  const int* d_quant_starts = nullptr;
  const int* d_gemv_starts = nullptr;
  const int* d_gemm_starts = nullptr;
};

namespace {

bl_status group_current_device(const bl_group* g) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BL_ERR_HIP;
  return dev == g->device ? BL_OK : BL_ERR_INVALID_ARGUMENT;
}

ProbSet table_set(const Prob* probs, const int* starts, int count, int total) {
  ProbSet s{};
  s.probs = probs;
  s.starts = starts;
  s.count = count;
  s.total = total;
  return s;
}

void free_group(bl_group* g) {
  if (!g) return;
  if (g->tables) (void)hipFree(g->tables);
  if (g->workspace) (void)hipFree(g->workspace);
  delete g;
}

}  // namespace

extern "C" {

bl_status bl_group_create(const bl_desc* descs, int32_t count, bl_group** out) {
  try {
    if (!out) return BL_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    if (!descs || count <= 0) return BL_ERR_INVALID_ARGUMENT;
    int64_t quant_total = 0, gemv_total = 0, gemm_total = 0;
    size_t ws_bytes = 0;
    int max_k = 0;
    for (int32_t i = 0; i < count; ++i) {
      const bl_desc& d = descs[i];
      bl_status st = check_forward(d.x, d.norm_w, d.packed_w, d.w_scale, d.M, d.K, d.N, d.eps, d.y);
      if (st != BL_OK) return st;
      if (d.M == 0) continue;
      quant_total += d.M;
      if (d.M <= kGemvMaxM) gemv_total += gemv_units(static_cast<int>(d.N));
      else gemm_total += gemm_units(static_cast<int>(d.M), static_cast<int>(d.N));
      ws_bytes += ws_layout(d.M, d.K).bytes;
      max_k = d.K > max_k ? static_cast<int>(d.K) : max_k;
    }
    if (quant_total > INT32_MAX / 2 || gemv_total > INT32_MAX / 2 || gemm_total > INT32_MAX / 2)
      return BL_ERR_UNSUPPORTED;

    bl_group* g = new (std::nothrow) bl_group;
    if (!g) return BL_ERR_NOMEM;
    if (hipGetDevice(&g->device) != hipSuccess) {
      delete g;
      return BL_ERR_HIP;
    }
    if (ws_bytes > 0 && hipMalloc(&g->workspace, ws_bytes) != hipSuccess) {
      (void)hipGetLastError();
      free_group(g);
      return BL_ERR_NOMEM;
    }

    std::vector<Prob> all, gemv, gemm;
    std::vector<int> qs{0}, vs{0}, ms{0};
    uint8_t* ws = static_cast<uint8_t*>(g->workspace);
    size_t off = 0;
    for (int32_t i = 0; i < count; ++i) {
      const bl_desc& d = descs[i];
      if (d.M == 0) continue;
      const WsLayout l = ws_layout(d.M, d.K);
      Prob p{};
      p.x = d.x;
      p.norm_w = d.norm_w;
      p.w = d.packed_w;
      p.xq = reinterpret_cast<int8_t*>(ws + off + l.xq);
      p.factor = reinterpret_cast<float*>(ws + off + l.factor);
      p.rowsum = reinterpret_cast<int32_t*>(ws + off + l.rowsum);
      p.y = d.y;
      p.acc = nullptr;
      p.w_scale = d.w_scale;
      p.eps = d.eps;
      p.M = static_cast<int>(d.M);
      p.K = static_cast<int>(d.K);
      p.N = static_cast<int>(d.N);
      off += l.bytes;
      all.push_back(p);
      qs.push_back(qs.back() + p.M);
      if (p.M <= kGemvMaxM) {
        gemv.push_back(p);
        vs.push_back(vs.back() + gemv_units(p.N));
      } else {
        gemm.push_back(p);
        ms.push_back(ms.back() + gemm_units(p.M, p.N));
      }
    }
    g->count = static_cast<int>(all.size());
    g->gemv_count = static_cast<int>(gemv.size());
    g->gemm_count = static_cast<int>(gemm.size());
    g->quant_total = static_cast<int>(quant_total);
    g->gemv_total = static_cast<int>(gemv_total);
    g->gemm_total = static_cast<int>(gemm_total);
    g->max_k = max_k;

    // One device buffer for the problem tables and the prefix sums.
    const size_t b_all = round_up(all.size() * sizeof(Prob), kAlign);
    const size_t b_gemv = round_up(gemv.size() * sizeof(Prob), kAlign);
    const size_t b_gemm = round_up(gemm.size() * sizeof(Prob), kAlign);
    const size_t b_qs = round_up(qs.size() * sizeof(int), kAlign);
    const size_t b_vs = round_up(vs.size() * sizeof(int), kAlign);
    const size_t b_ms = round_up(ms.size() * sizeof(int), kAlign);
    const size_t total = b_all + b_gemv + b_gemm + b_qs + b_vs + b_ms;
    std::vector<uint8_t> host(total, 0);
    size_t o = 0;
    auto put = [&](const void* src, size_t n, size_t span) {
      if (n) std::memcpy(host.data() + o, src, n);
      const size_t at = o;
      o += span;
      return at;
    };
    const size_t o_all = put(all.data(), all.size() * sizeof(Prob), b_all);
    const size_t o_gemv = put(gemv.data(), gemv.size() * sizeof(Prob), b_gemv);
    const size_t o_gemm = put(gemm.data(), gemm.size() * sizeof(Prob), b_gemm);
    const size_t o_qs = put(qs.data(), qs.size() * sizeof(int), b_qs);
    const size_t o_vs = put(vs.data(), vs.size() * sizeof(int), b_vs);
    const size_t o_ms = put(ms.data(), ms.size() * sizeof(int), b_ms);
    if (hipMalloc(&g->tables, total) != hipSuccess) {
      (void)hipGetLastError();
      free_group(g);
      return BL_ERR_NOMEM;
    }
    if (hipMemcpy(g->tables, host.data(), total, hipMemcpyHostToDevice) != hipSuccess) {
      free_group(g);
      return BL_ERR_HIP;
    }
    uint8_t* t = static_cast<uint8_t*>(g->tables);
    g->d_all = reinterpret_cast<const Prob*>(t + o_all);
    g->d_gemv = reinterpret_cast<const Prob*>(t + o_gemv);
    g->d_gemm = reinterpret_cast<const Prob*>(t + o_gemm);
    g->d_quant_starts = reinterpret_cast<const int*>(t + o_qs);
    g->d_gemv_starts = reinterpret_cast<const int*>(t + o_vs);
    g->d_gemm_starts = reinterpret_cast<const int*>(t + o_ms);
    *out = g;
    return BL_OK;
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

bl_status bl_group_quant(bl_group* g, void* stream) {
  try {
    if (!g) return BL_ERR_INVALID_ARGUMENT;
    bl_status st = group_current_device(g);
    if (st != BL_OK || g->count == 0) return st;
    return from_hip(launch_quant(table_set(g->d_all, g->d_quant_starts, g->count, g->quant_total),
                                 g->max_k, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

bl_status bl_group_matmul(bl_group* g, void* stream) {
  try {
    if (!g) return BL_ERR_INVALID_ARGUMENT;
    bl_status st = group_current_device(g);
    if (st != BL_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (g->gemv_count > 0) {
      st = from_hip(launch_gemv(table_set(g->d_gemv, g->d_gemv_starts, g->gemv_count, g->gemv_total),
                                false, s));
      if (st != BL_OK) return st;
    }
    if (g->gemm_count > 0)
      st = from_hip(launch_gemm(table_set(g->d_gemm, g->d_gemm_starts, g->gemm_count, g->gemm_total),
                                false, s));
    return st;
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}

bl_status bl_group_forward(bl_group* g, void* stream) {
  bl_status st = bl_group_quant(g, stream);
  if (st != BL_OK) return st;
  return bl_group_matmul(g, stream);
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
