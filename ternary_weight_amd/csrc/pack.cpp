// Host-side absmean ternary quantization and I2_S packing
// ("BitNet Embeddings GGUF Conversion Implementation", s3 "I2_S Ternary
// Packing"; "BitNet Inference Framework", "Quantization and Encoding" and
// "Data Layout").  Offline work: it runs once per weight, before any forward.
//
// scale = 1/mean|w| (mean accumulated in double in memory order, rounded to
// float32 once); code = clamp(rne(w*scale), -1, 1) + 1 with a float32
// multiply by the stored scale.  Output bytes are built one at a time from the
// four elements they hold (byte j of a block: elements j, j+32, j+64, j+96),
// row ranges in parallel.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/bitlinear.h"

namespace {

inline uint8_t ternary_code(float w, float scale) {
  const float r = std::nearbyint(w * scale);  // half to even
  return r >= 1.0f ? 2 : (r <= -1.0f ? 0 : 1);
}

void pack_rows(const float* w, int64_t K, int64_t n_begin, int64_t n_end, float scale,
               uint8_t* out) {
  const int64_t row_bytes = K / 4;
  for (int64_t n = n_begin; n < n_end; ++n) {
    const float* src = w + n * K;
    uint8_t* dst = out + n * row_bytes;
    for (int64_t b = 0; b < K / 128; ++b) {
      const float* blk = src + 128 * b;
      for (int j = 0; j < 32; ++j) {
        dst[32 * b + j] = static_cast<uint8_t>(
            (ternary_code(blk[j], scale) << 6) | (ternary_code(blk[32 + j], scale) << 4) |
            (ternary_code(blk[64 + j], scale) << 2) | ternary_code(blk[96 + j], scale));
      }
    }
  }
}

}  // namespace

extern "C" size_t i2s_packed_bytes(int64_t K, int64_t N) {
  if (K <= 0 || N <= 0 || K % 128 != 0) return 0;
  if (N > INT64_MAX / K) return 0;
  return static_cast<size_t>(N * (K / 4) + 4);
}

extern "C" bl_status i2s_pack(const float* w, int64_t K, int64_t N, uint8_t* packed,
                              size_t packed_bytes, float* w_scale_out) {
  try {
    if (!w || !packed || K <= 0 || N <= 0) return BL_ERR_INVALID_ARGUMENT;
    if (K % 128 != 0) return BL_ERR_UNSUPPORTED;
    const size_t need = i2s_packed_bytes(K, N);
    if (need == 0) return BL_ERR_UNSUPPORTED;
    if (packed_bytes < need) return BL_ERR_INVALID_ARGUMENT;

    const int64_t total = N * K;
    double sum = 0.0;
    for (int64_t i = 0; i < total; ++i) {
      const float v = w[i];
      if (!std::isfinite(v)) return BL_ERR_NONFINITE;
      sum += std::fabs(static_cast<double>(v));
    }
    const double mean = sum / static_cast<double>(total);
    const float scale = mean == 0.0 ? 1.0f : static_cast<float>(1.0 / mean);

    const int64_t threads =
        total < (int64_t{1} << 20)
            ? 1
            : std::min<int64_t>({16, N, std::max(1u, std::thread::hardware_concurrency())});
    if (threads <= 1) {
      pack_rows(w, K, 0, N, scale, packed);
    } else {
      std::vector<std::thread> pool;
      for (int64_t t = 0; t < threads; ++t) {
        const int64_t b = N * t / threads, e = N * (t + 1) / threads;
        pool.emplace_back(pack_rows, w, K, b, e, scale, packed);
      }
      for (auto& th : pool) th.join();
    }
    std::memcpy(packed + total / 4, &scale, sizeof(float));
    if (w_scale_out) *w_scale_out = scale;
    return BL_OK;
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}
