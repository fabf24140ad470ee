// Stage 2 for decode-sized batches (M <= 16): the ternary product streamed
// straight from the I2_S bytes, with the scale epilogue fused.
//
// The pages' decode kernels (bitnet.cpp's activation-parallel CPU kernels,
// "BitNet Inference Framework"; the A100 W2A8 GEMV, "BitNet Inference Kernel",
// "Fast Decoding" and "dp4a Instruction") stream 2-bit weights once and
// expand them in registers.  Here the same idea is mapped onto one
// v_mfma_i32_16x16x64_i8 per 16 weight rows x 64 K positions: the MFMA's
// A operand is 16 weight rows (decoded in registers), its B operand the <= 16
// activation rows (zero-padded), so M = 1..16 costs the same and the matrix
// core, otherwise idle, does the dot products.  The VALU only decodes.
//
// Superblock = 256 K positions = 64 bytes of one weight row = 4 x 16-byte
// chunks.  Lane (r = lane % 16, g = lane / 16) loads chunk g of weight row r
// with one 16-byte load; field f of that chunk holds 16 consecutive K
// positions (128*(g/2) + 32f + 16*(g%2) + 0..15 of the superblock), so the
// four fields feed four MFMAs.  The fields are isolated with a mask only
// (field 1 = code*16, field 2 = code*4) and accumulated separately; the
// exact powers of two are divided out at the end.  Codes are 0, 1, 2; the
// activation row sum is subtracted in the epilogue to turn them into -1, 0, +1.
//
// Work split: a workgroup (4 waves) owns 16*NT output columns; its waves split
// K by superblocks and their partial sums meet in LDS.  Bound: HBM, K/4 bytes
// per output column.
#include "kernels.hpp"

namespace bl {

constexpr int kGemvNT = 4;  // column groups of 16 per workgroup

template <int NT, bool RAW>
__global__ __launch_bounds__(256) void gemv_kernel(ProbSet set) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  int tile;
  const Prob& P = prob_at(set, find_prob(set, blockIdx.x, &tile));
  const int M = P.M, K = P.K, N = P.N;
  const int rowbytes = K >> 2;
  const int n0 = tile * 16 * NT;
  const int nsb = (K + 255) >> 8;        // superblocks; the last one may be half
  const int per = (nsb + 3) >> 2;        // superblocks per wave
  const int sb_begin = wave * per;
  const int sb_end = min(nsb, sb_begin + per);

  v4i acc[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[t][f] = v4i{0, 0, 0, 0};

  for (int sb = sb_begin; sb < sb_end; sb += 2) {
    // Activation fragments (B operand) for the (up to) 2 superblocks.
    v4i xf[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int k = 256 * (sb + s) + 128 * (g >> 1) + 32 * f + 16 * (g & 1);
        xf[s][f] = v4i{0, 0, 0, 0};
        if (sb + s < sb_end && r16 < M && k < K)
          xf[s][f] = *reinterpret_cast<const v4i*>(P.xq + static_cast<int64_t>(r16) * K + k);
      }
    // Weight chunks for every column group, all issued before any use.
    uint4 wv[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int n = n0 + 16 * t + r16;
        const int byte = 64 * (sb + s) + 16 * g;
        wv[t][s] = make_uint4(0u, 0u, 0u, 0u);
        if (sb + s < sb_end && n < N && byte < rowbytes)
          wv[t][s] = *reinterpret_cast<const uint4*>(P.w + static_cast<int64_t>(n) * rowbytes + byte);
      }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (sb + s >= sb_end) break;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t d[4] = {wv[t][s].x, wv[t][s].y, wv[t][s].z, wv[t][s].w};
        v4i a0, a1, a2, a3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a0[i] = static_cast<int>((d[i] >> 6) & 0x03030303u);  // field 0: code
          a1[i] = static_cast<int>(d[i] & 0x30303030u);         // field 1: code*16
          a2[i] = static_cast<int>(d[i] & 0x0C0C0C0Cu);         // field 2: code*4
          a3[i] = static_cast<int>(d[i] & 0x03030303u);         // field 3: code
        }
        acc[t][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, xf[s][0], acc[t][0], 0, 0, 0);
        acc[t][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, xf[s][1], acc[t][1], 0, 0, 0);
        acc[t][2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, xf[s][2], acc[t][2], 0, 0, 0);
        acc[t][3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, xf[s][3], acc[t][3], 0, 0, 0);
      }
    }
  }

  // Combine the fields, then the waves' K slices.
  __shared__ v4i red[4][NT][kWave];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    red[wave][t][lane] = acc[t][0] + (acc[t][1] >> 4) + (acc[t][2] >> 2) + acc[t][3];
  __syncthreads();

  // Epilogue: lane holds rows n = 4g..4g+3 of column m = lane % 16.
  const int m = r16;
  if (m >= M) return;
  const int rs = P.rowsum[m];
  float scale = 0.f;
  if (!RAW) scale = P.factor[m] / P.w_scale;
  for (int t = wave; t < NT; t += 4) {
    const v4i v = red[0][t][lane] + red[1][t][lane] + red[2][t][lane] + red[3][t][lane];
    const int n = n0 + 16 * t + 4 * g;
    if (n >= N) continue;
    const int64_t o = static_cast<int64_t>(m) * N + n;
    if (RAW) {
      if ((N & 3) == 0) {
        *reinterpret_cast<v4i*>(P.acc + o) = v - rs;
      } else {
        for (int i = 0; i < 4 && n + i < N; ++i) P.acc[o + i] = v[i] - rs;
      }
    } else {
      const float4 out = make_float4(static_cast<float>(v[0] - rs) * scale,
                                     static_cast<float>(v[1] - rs) * scale,
                                     static_cast<float>(v[2] - rs) * scale,
                                     static_cast<float>(v[3] - rs) * scale);
      if ((N & 3) == 0) {
        *reinterpret_cast<float4*>(P.y + o) = out;
      } else {
        const float vals[4] = {out.x, out.y, out.z, out.w};
        for (int i = 0; i < 4 && n + i < N; ++i) P.y[o + i] = vals[i];
      }
    }
  }
}

int gemv_units(int N) { return (N + 16 * kGemvNT - 1) / (16 * kGemvNT); }

hipError_t launch_gemv(const ProbSet& set, bool raw, hipStream_t stream) {
  if (set.total <= 0) return hipSuccess;
  const dim3 grid(set.total), block(256);
  if (raw)
    hipLaunchKernelGGL((gemv_kernel<kGemvNT, true>), grid, block, 0, stream, set);
  else
    hipLaunchKernelGGL((gemv_kernel<kGemvNT, false>), grid, block, 0, stream, set);
  return hipGetLastError();
}

}  // namespace bl
