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
// activation row sum is subtracted in the epilogue to turn them into
// -1, 0, +1.
//
// Work split: a workgroup owns 4*16*T weight rows of one problem and each of
// its waves T 16-row tiles (T = 4 for K <= 2048, else 2), walked in order
// with the next tile's weights loading while the current one is processed.
// The kernel is specialised on the number of superblocks NSB = ceil(K/256):
// a tile's NSB weight loads are issued together and consumed in order, so
// the compiler's wait counts are exact and the register footprint small.
// Weights are read with buffer loads: an offset outside the problem's weight
// bytes returns 0 without a memory access, which replaces the bounds branches
// (rows >= N, tiles past the end, the missing half of a half superblock).
// The <= 16 activation rows (plus one all-zero row for the padding lanes) are
// staged once per workgroup in LDS, zero-padded along K to NSB superblocks;
// when they do not fit, fragments come from global memory through the same
// out-of-range-reads-zero buffer loads.  K beyond 16 superblocks runs a
// generic variant (one tile per wave, superblocks streamed two ahead).
// Bound: HBM, K/4 bytes per output column.
#include "kernels.hpp"

namespace bl {

constexpr int kGemvLdsBytes = 64 * 1024;   // activation staging limit per workgroup
constexpr int kOob = 0x7FFFFFF0;           // buffer offset that always reads 0
constexpr int kBufferDword3 = 0x00020000;  // raw buffer resource word 3 (gfx9 family)
constexpr int kMaxNsb = 16;                // specialised superblock counts 1..16

__device__ __forceinline__ void decode_fields(const v4i& w, v4i& a0, v4i& a1, v4i& a2, v4i& a3) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t d = static_cast<uint32_t>(w[i]);
    a0[i] = static_cast<int>((d >> 6) & 0x03030303u);  // field 0: code
    a1[i] = static_cast<int>(d & 0x30303030u);         // field 1: code*16
    a2[i] = static_cast<int>(d & 0x0C0C0C0Cu);         // field 2: code*4
    a3[i] = static_cast<int>(d & 0x03030303u);         // field 3: code
  }
}

constexpr int gemv_tiles(int nsb) { return nsb == 0 ? 1 : (nsb <= 8 ? 4 : 2); }

template <bool RAW>
__device__ __forceinline__ void gemv_epilogue(const Prob& P, const v4i* acc, int nrow, int r16,
                                              int rs, float scale) {
  const int N = P.N;
  if (r16 >= P.M || nrow >= N) return;
  const v4i v = acc[0] + (acc[1] >> 4) + (acc[2] >> 2) + acc[3];
  const int64_t o = static_cast<int64_t>(r16) * N + nrow;
  if (RAW) {
    if ((N & 3) == 0) {
      *gptr_out<v4i>(P.acc + o) = v - rs;
    } else {
      for (int i = 0; i < 4 && nrow + i < N; ++i) gptr_out<int32_t>(P.acc)[o + i] = v[i] - rs;
    }
  } else {
    const f4 out = f4{static_cast<float>(v[0] - rs) * scale, static_cast<float>(v[1] - rs) * scale,
                      static_cast<float>(v[2] - rs) * scale, static_cast<float>(v[3] - rs) * scale};
    if ((N & 3) == 0) {
      *gptr_out<f4>(P.y + o) = out;
    } else {
      for (int i = 0; i < 4 && nrow + i < N; ++i) gptr_out<float>(P.y)[o + i] = out[i];
    }
  }
}

// NSB > 0: exactly NSB superblocks per tile.  NSB == 0: any K, streamed.
// The launch covers the by-value problem in `single` (units == nullptr) or
// the FatUnit table `units`.
template <bool RAW, bool FROM_LDS, int NSB>
__global__ __launch_bounds__(256) void gemv_kernel(Prob single, const FatUnit* units) {
  constexpr int T = gemv_tiles(NSB);
  extern __shared__ __attribute__((aligned(16))) int8_t xlds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  int unit = blockIdx.x;
  const Prob P = units ? fat_unit_at(units, blockIdx.x, &unit) : single;
  const int M = P.M, K = P.K, N = P.N;
  const int rowbytes = K >> 2;
  const int nsb = NSB > 0 ? NSB : (K + 255) >> 8;
  const int kpad = (NSB > 0 ? nsb : (nsb + 1) & ~1) * 256;

  // Weight loads: lane reads 16 bytes of row tile0 + 16t + r16 at superblock sb.
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(P.w), 0, N * rowbytes, kBufferDword3);
  const int tile0 = (unit * 4 + wave) * 16 * T;
  const int wbase = (tile0 + r16) * rowbytes + 16 * g;
  auto wload = [&](int t, int sb) -> v4i {
    const bool ok = (t < T) & (tile0 + 16 * t + r16 < N) & (sb < nsb) & (64 * sb + 16 * g < rowbytes);
    return __builtin_amdgcn_raw_buffer_load_b128(
        wrs, ok ? wbase + 16 * t * rowbytes + 64 * sb : kOob, 0, 0);
  };

  // Activation fragment (B operand): 16 bytes of row r16 at K offset
  // 256*sb + 32*f + koff; zero for padding rows and past K.
  const int xstride = kpad + 16;  // LDS row stride (padding against bank conflicts)
  const int koff = 128 * (g >> 1) + 16 * (g & 1);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(P.xq), 0, M * K, kBufferDword3);
  const int8_t* xl = xlds + min(r16, M) * xstride + koff;
  auto xfrag = [&](int sb, int f) -> v4i {
    const int k = 256 * sb + 32 * f;
    if (FROM_LDS) return *reinterpret_cast<const v4i*>(xl + k);
    const bool ok = (r16 < M) & (k + koff < K);
    return __builtin_amdgcn_raw_buffer_load_b128(xrs, ok ? r16 * K + koff + k : kOob, 0, 0);
  };

  constexpr int kHeld = NSB > 0 ? NSB : 2;
  v4i wa[kHeld], wb[kHeld];
  // The first tile's loads go out before the activation staging and its barrier.
#pragma unroll
  for (int sb = 0; sb < kHeld; ++sb) wa[sb] = wload(0, sb);

  if (FROM_LDS) {
    // Rows 0..M-1: activations zero-padded to kpad; row M: zeros.
    const int row_chunks = kpad >> 4;
    for (int c = threadIdx.x; c < (M + 1) * row_chunks; c += 256) {
      const int m = c / row_chunks, o = (c - m * row_chunks) << 4;
      v4i v = v4i{0, 0, 0, 0};
      if (m < M && o < K) v = *gptr<v4i>(P.xq + static_cast<int64_t>(m) * K + o);
      *reinterpret_cast<v4i*>(xlds + m * xstride + o) = v;
    }
    __syncthreads();
  }

  const int rs = r16 < M ? gptr<int32_t>(P.rowsum)[r16] : 0;
  float scale = 0.f;
  if (!RAW && r16 < M) scale = gptr<float>(P.factor)[r16] / P.w_scale;

  v4i acc[4];
  auto process = [&](const v4i& wv, int sb) {
    v4i a0, a1, a2, a3;
    decode_fields(wv, a0, a1, a2, a3);
    acc[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, xfrag(sb, 0), acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, xfrag(sb, 1), acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, xfrag(sb, 2), acc[2], 0, 0, 0);
    acc[3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, xfrag(sb, 3), acc[3], 0, 0, 0);
  };
  auto tile = [&](const v4i* w, int t) {
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[f] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int sb = 0; sb < kHeld; ++sb) process(w[sb], sb);
    gemv_epilogue<RAW>(P, acc, tile0 + 16 * t + 4 * g, r16, rs, scale);
  };

  if (NSB > 0) {
    // Tiles in pairs through the two buffers; past the wave's last tile the
    // loads read 0 and the epilogue stores nothing.
#pragma unroll
    for (int t = 0; t < T; t += 2) {
#pragma unroll
      for (int sb = 0; sb < kHeld; ++sb) wb[sb] = wload(t + 1, sb);
      tile(wa, t);
#pragma unroll
      for (int sb = 0; sb < kHeld; ++sb) wa[sb] = wload(t + 2, sb);
      tile(wb, t + 1);
    }
  } else {
    // Generic K, one tile: two superblocks in flight, pairs processed
    // unconditionally (past nsb both operands are zero: loads read 0,
    // staging is padded).
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[f] = v4i{0, 0, 0, 0};
    for (int sb = 0; sb < nsb; sb += 2) {
      process(wa[0], sb);
      wa[0] = wload(0, sb + 2);
      process(wa[1], sb + 1);
      wa[1] = wload(0, sb + 3);
    }
    gemv_epilogue<RAW>(P, acc, tile0 + 4 * g, r16, rs, scale);
  }
}

int gemv_bucket(int K) {
  const int nsb = (K + 255) >> 8;
  return nsb <= kMaxNsb ? nsb : 0;
}

int gemv_units(int N, int bucket) {
  const int rows = 64 * gemv_tiles(bucket);
  return (N + rows - 1) / rows;
}

namespace {

// Staged K of a launch: the bucket's superblocks, or for the generic variant
// the largest K rounded up to a pair of superblocks (processed in pairs).
size_t gemv_lds_bytes(int bucket, int max_m, int max_k) {
  int nsb = bucket > 0 ? bucket : (max_k + 255) >> 8;
  if (bucket == 0) nsb = (nsb + 1) & ~1;
  return static_cast<size_t>(max_m + 1) * (static_cast<size_t>(nsb) * 256 + 16);
}

template <bool RAW, bool LDS>
hipError_t launch_bucket(const GemvLaunch& L, int bucket, size_t shmem, hipStream_t stream) {
  const dim3 grid(L.total), block(256);
#define BL_GEMV_CASE(n)                                                                    \
  case n:                                                                                  \
    hipLaunchKernelGGL((gemv_kernel<RAW, LDS, n>), grid, block, shmem, stream, L.single,   \
                       L.units);                                                           \
    break;
  switch (bucket) {
    BL_GEMV_CASE(1) BL_GEMV_CASE(2) BL_GEMV_CASE(3) BL_GEMV_CASE(4) BL_GEMV_CASE(5)
    BL_GEMV_CASE(6) BL_GEMV_CASE(7) BL_GEMV_CASE(8) BL_GEMV_CASE(9) BL_GEMV_CASE(10)
    BL_GEMV_CASE(11) BL_GEMV_CASE(12) BL_GEMV_CASE(13) BL_GEMV_CASE(14) BL_GEMV_CASE(15)
    BL_GEMV_CASE(16)
    default:
      hipLaunchKernelGGL((gemv_kernel<RAW, LDS, 0>), grid, block, shmem, stream, L.single, L.units);
  }
#undef BL_GEMV_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const GemvLaunch& L, bool raw, int bucket, int max_m, int max_k,
                       hipStream_t stream) {
  if (L.total <= 0) return hipSuccess;
  const size_t shmem = gemv_lds_bytes(bucket, max_m, max_k);
  const bool lds = shmem <= static_cast<size_t>(kGemvLdsBytes);
  if (raw) {
    return lds ? launch_bucket<true, true>(L, bucket, shmem, stream)
               : launch_bucket<true, false>(L, bucket, 0, stream);
  }
  return lds ? launch_bucket<false, true>(L, bucket, shmem, stream)
             : launch_bucket<false, false>(L, bucket, 0, stream);
}

}  // namespace bl
