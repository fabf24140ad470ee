// Stage 2 for prefill-sized batches (M > 16): int8 x ternary product on the
// matrix cores, int32 accumulation, scale epilogue fused.
//
// Prefill is a dense contraction (2*M*N*K int8-equivalent operations), so it
// runs on v_mfma_i32_16x16x64_i8.  The pages' CPU kernels amortise the I2_S
// unpack over many activation rows ("BitNet Inference Framework", activation
// parallel); here one unpacked weight operand feeds four MFMAs (four 16-row
// activation fragments).
//
// Tiling.  A workgroup of 4 waves owns a 128 (weight rows n) x 128
// (activation rows m) output tile; each wave a 64 x 64 sub-tile (4 x 4 MFMA
// fragments).  K advances one I2_S block (128 positions) per stage; both the
// activation tile (128 x 128 int8, 16 KB) and the weight tile still in 2-bit
// form (128 x 32 B, 4 KB) are double-buffered in LDS.  Weights are expanded
// to int8 right before the MFMA (shift + mask per dword), so LDS holds a
// quarter of the weight bytes an int8 tile would.
//
// K order inside a block: MFMA step j (0, 1) covers positions 64j..64j+63;
// lane group g = lane/16 supplies positions 64j+16g..+15.  In I2_S those are
// field 2j + g/2 of bytes 16*(g%2)..+15 of the block, so a lane reads one
// 16-byte half of the block row and shifts out one field.
//
// LDS layout: 16-byte slots are XOR-swizzled by row so the 16 lanes of a lane
// group (16 consecutive rows, same slot) hit distinct banks.
//
// Bound: int8 MFMA for K >= 2048; for K <= 1024 the fp32 output (4*M*N bytes)
// weighs as much as the MFMA time.
#include "kernels.hpp"

namespace bl {

constexpr int kTileN = 128;  // weight rows per workgroup
constexpr int kTileM = 128;  // activation rows per workgroup
constexpr int kBlockK = 128; // K positions per stage (one I2_S block)

__device__ __forceinline__ int xs_slot(int row, int slot) {
  return slot ^ (row & 7) ^ ((row >> 3) & 1);
}
__device__ __forceinline__ int ws_slot(int row, int slot) {
  return slot ^ ((row >> 2) & 1) ^ ((row >> 3) & 1);
}

template <bool RAW>
__global__ __launch_bounds__(256, 2) void gemm_kernel(ProbSet set) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][kTileM * kBlockK];
  __shared__ __attribute__((aligned(16))) uint8_t ws[2][kTileN * (kBlockK / 4)];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int r16 = lane & 15, g = lane >> 4;

  int local;
  const Prob& P = prob_at(set, find_prob(set, xcd_remap(blockIdx.x, set.total), &local));
  const int M = P.M, K = P.K, N = P.N;
  const int rowbytes = K >> 2;
  const int tiles_n = (N + kTileN - 1) / kTileN;
  const int m0 = (local / tiles_n) * kTileM;
  const int n0 = (local % tiles_n) * kTileN;
  const int nblk = K / kBlockK;

  // Global -> register staging: 4 x 16 B of activations and 16 B of packed
  // weights per thread per stage.
  v4i xr[4];
  v4i wr;
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = tid + 256 * i, row = s >> 3, slot = s & 7;
      const int m = m0 + row;
      xr[i] = v4i{0, 0, 0, 0};
      if (m < M)
        xr[i] = *reinterpret_cast<const v4i*>(P.xq + static_cast<int64_t>(m) * K + kb * kBlockK +
                                              slot * 16);
    }
    const int row = tid >> 1, slot = tid & 1;
    const int n = n0 + row;
    wr = v4i{0, 0, 0, 0};
    if (n < N)
      wr = *reinterpret_cast<const v4i*>(P.w + static_cast<int64_t>(n) * rowbytes + kb * 32 +
                                         slot * 16);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = tid + 256 * i, row = s >> 3, slot = s & 7;
      *reinterpret_cast<v4i*>(&xs[buf][row * kBlockK + xs_slot(row, slot) * 16]) = xr[i];
    }
    const int row = tid >> 1, slot = tid & 1;
    *reinterpret_cast<v4i*>(&ws[buf][row * 32 + ws_slot(row, slot) * 16]) = wr;
  };

  v4i acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = v4i{0, 0, 0, 0};

  gload(0);
  sstore(0);
  __syncthreads();

  for (int kb = 0; kb < nblk; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nblk) gload(kb + 1);

    v4i wp[4];  // packed 16-byte halves of 4 weight rows
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) {
      const int row = wn * 64 + fn * 16 + r16;
      wp[fn] = *reinterpret_cast<const v4i*>(&ws[buf][row * 32 + ws_slot(row, g & 1) * 16]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int field = 2 * j + (g >> 1);
      v4i a[4];
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
#pragma unroll
        for (int i = 0; i < 4; ++i) a[fn][i] = field_codes(static_cast<uint32_t>(wp[fn][i]), field);
      v4i b[4];
#pragma unroll
      for (int fm = 0; fm < 4; ++fm) {
        const int row = wm * 64 + fm * 16 + r16;
        b[fm] = *reinterpret_cast<const v4i*>(&xs[buf][row * kBlockK + xs_slot(row, 4 * j + g) * 16]);
      }
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
#pragma unroll
        for (int fm = 0; fm < 4; ++fm)
          acc[fn][fm] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[fn], b[fm], acc[fn][fm], 0, 0, 0);
    }
    if (kb + 1 < nblk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds weight rows 4g..4g+3 of activation row r16 per fragment.
#pragma unroll
  for (int fm = 0; fm < 4; ++fm) {
    const int m = m0 + wm * 64 + fm * 16 + r16;
    if (m >= M) continue;
    const int rs = P.rowsum[m];
    float scale = 0.f;
    if (!RAW) scale = P.factor[m] / P.w_scale;
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) {
      const int n = n0 + wn * 64 + fn * 16 + 4 * g;
      if (n >= N) continue;
      const v4i v = acc[fn][fm];
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
}

int gemm_units(int M, int N) {
  return ((M + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN);
}

hipError_t launch_gemm(const ProbSet& set, bool raw, hipStream_t stream) {
  if (set.total <= 0) return hipSuccess;
  const dim3 grid(set.total), block(256);
  if (raw)
    hipLaunchKernelGGL(gemm_kernel<true>, grid, block, 0, stream, set);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, grid, block, 0, stream, set);
  return hipGetLastError();
}

}  // namespace bl
