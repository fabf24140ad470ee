// Device-side absmean ternary quantization and I2_S packing, for weights that
// already live on the GPU ("BitNet Embeddings GGUF Conversion Implementation",
// s3 "I2_S Ternary Packing"; "BitNet Inference Framework", "Quantization and
// Encoding" and "Data Layout").  Same format and the same codes as the host
// packer: scale = (float)(1 / mean|w|) with the mean taken in double, code =
// clamp(rne((float)w * scale), -1, 1) + 1 with a float32 multiply, byte j of a
// 128-value block = (c[j] << 6) | (c[j+32] << 4) | (c[j+64] << 2) | c[j+96],
// the scale appended after the codes.
//
// Three launches: partial sums of |w| in double (a fixed split and a fixed
// tree, so the result is the same on every run), their total and the scale
// (one wave), and the packing (one lane per 16 output bytes).  The double sum
// runs in another order than the host's memory-order sum, so the two means can
// differ in their last bits; the float32 scale, and with it every code, is the
// same unless 1/mean falls that close to a float32 rounding boundary.
// Bound: HBM, 4 bytes read twice and a quarter byte written per weight.
#include "kernels.hpp"

namespace bl {

namespace {

// Workgroup g sums |w| over float4 chunks [g*chunk4, (g+1)*chunk4): each lane
// strides by the workgroup size, then a butterfly per wave and a fixed order
// over the four waves.
__global__ __launch_bounds__(256) void absmean_partial_kernel(const float* w, int64_t n4,
                                                              int64_t chunk4, double* partial) {
  const int64_t begin = static_cast<int64_t>(blockIdx.x) * chunk4;
  const int64_t end = begin + chunk4 < n4 ? begin + chunk4 : n4;
  double s = 0.0;
  for (int64_t i = begin + threadIdx.x; i < end; i += 256) {
    const f4 v = gptr<f4>(w)[i];
    s += (fabs(static_cast<double>(v.x)) + fabs(static_cast<double>(v.y))) +
         (fabs(static_cast<double>(v.z)) + fabs(static_cast<double>(v.w)));
  }
  s = wave_sum(s);
  __shared__ double per_wave[4];
  if ((threadIdx.x & (kWave - 1)) == 0) per_wave[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0)
    gptr_out<double>(partial)[blockIdx.x] = (per_wave[0] + per_wave[1]) + (per_wave[2] + per_wave[3]);
}

// Total of the partial sums (one wave, fixed order), the mean over n weights
// and the scale; an all-zero w gives scale 1, a non-finite total (an inf or
// NaN weight) a NaN scale, which the caller reports.  The scale goes to
// `tail` (the 4 bytes after the codes) and to `scale_out`.
__global__ __launch_bounds__(64) void absmean_final_kernel(const double* partial, int count,
                                                           int64_t n, float* tail, float* scale_out) {
  double s = 0.0;
  for (int i = threadIdx.x; i < count; i += kWave) s += gptr<double>(partial)[i];
  s = wave_sum(s);
  if (threadIdx.x == 0) {
    const double mean = s / static_cast<double>(n);
    float scale = mean == 0.0 ? 1.0f : static_cast<float>(1.0 / mean);
    if (!isfinite(s)) scale = __builtin_nanf("");
    *gptr_out<float>(tail) = scale;
    *gptr_out<float>(scale_out) = scale;
  }
}

// Ternary code of one weight: 0, 1, 2 for -1, 0, +1 (NaN products give 1; a
// non-finite weight makes the scale non-finite, which the caller reports).
__device__ __forceinline__ uint32_t tcode(float w, float scale) {
  const float r = rintf(w * scale);
  return r >= 1.0f ? 2u : (r <= -1.0f ? 0u : 1u);
}

// Lane t writes output bytes 16t..16t+15 (non-temporal: written once, about
// 3% faster than plain stores).  Rows are K/4 bytes, a multiple of
// 32, so those bytes are bytes j0..j0+15 (j0 = 16t % 32) of one block, and
// byte j of that block holds elements 4*(16t - j0) + j0 + (j - j0) + 32f of
// the flat weight array, f = 0..3: four runs of 16 consecutive floats.
__global__ __launch_bounds__(256) void i2s_pack_kernel(const float* w, int64_t units,
                                                       const float* scale_p, uint8_t* packed) {
  const float scale = *gptr<float>(scale_p);
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; t < units;
       t += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t byte0 = 16 * t;
    const int64_t j0 = byte0 & 31;
    const int64_t e0 = 4 * byte0 - 3 * j0;
    uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int f = 0; f < 4; ++f) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f4 v = gptr<f4>(w + e0 + 32 * f)[c];
        const uint32_t shift = 6 - 2 * f;
        out[c] |= (tcode(v.x, scale) << shift) | (tcode(v.y, scale) << (shift + 8)) |
                  (tcode(v.z, scale) << (shift + 16)) | (tcode(v.w, scale) << (shift + 24));
      }
    }
    __builtin_nontemporal_store(
        v4i{static_cast<int>(out[0]), static_cast<int>(out[1]), static_cast<int>(out[2]),
            static_cast<int>(out[3])}, gptr_out<v4i>(packed + byte0));
  }
}

}  // namespace

hipError_t launch_i2s_pack_device(const float* w, int64_t K, int64_t N, uint8_t* packed,
                                  double* partial, float* scale_dev, hipStream_t stream) {
  const int64_t n = N * K;
  const int64_t n4 = n / 4;
  // At least 1024 float4 per workgroup, at most kPackPartials workgroups.
  int64_t blocks = (n4 + 1023) / 1024;
  if (blocks > kPackPartials) blocks = kPackPartials;
  if (blocks < 1) blocks = 1;
  const int64_t chunk4 = (n4 + blocks - 1) / blocks;
  hipLaunchKernelGGL(absmean_partial_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     w, n4, chunk4, partial);
  hipLaunchKernelGGL(absmean_final_kernel, dim3(1), dim3(kWave), 0, stream, partial,
                     static_cast<int>(blocks), n, reinterpret_cast<float*>(packed + n / 4), scale_dev);
  const int64_t units = n / 64;
  int64_t grid = (units + 255) / 256;
  if (grid > 8192) grid = 8192;
  hipLaunchKernelGGL(i2s_pack_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, w,
                     units, scale_dev, packed);
  return hipGetLastError();
}

}  // namespace bl
