// Stage 2 for prefill-sized batches (M > 16): int8 x ternary product on the
// matrix cores, int32 accumulation, scale epilogue fused.
//
// Prefill is a dense contraction (2*M*N*K int8-equivalent operations), so it
// runs on v_mfma_i32_32x32x32_i8.  The pages' CPU kernels amortise the I2_S
// unpack over many activation rows ("BitNet Inference Framework", activation
// parallel); here one unpacked weight operand feeds two MFMAs (two 32-row
// activation fragments) and each packed byte is expanded once per wave.
//
// Tiling.  A workgroup of 4 waves owns a 256 (weight rows n) x 128
// (activation rows m) output tile; each wave a 128 x 64 sub-tile (4 x 2
// fragments of 32 x 32).  K advances one I2_S block (128 positions) per stage.
// A stage holds the activation tile (128 x 128 int8, 16 KB) and the weight
// tile still in 2-bit form (256 x 32 B, 8 KB) in LDS; three stages form a
// ring filled by direct global-to-LDS loads (global_load_lds_dwordx4), two
// stages ahead of the MFMAs, so no VGPRs stage the copies.  Weights are
// expanded to int8 right before the MFMA (shift + mask per dword).
//
// K order inside a block: MFMA step j (0..3) covers positions 32j..32j+31;
// lane half g = lane/32 supplies positions 32j+16g..+15.  In I2_S those are
// field j of bytes 16g..16g+15 of the block row, so a lane reads one 16-byte
// half of a block row per stage and shifts out one field per step.
//
// LDS layout: 16-byte slots are XOR-swizzled by row so the lanes that read 16
// consecutive rows at one slot hit distinct banks; the direct loads write
// each wave instruction's 1 KB linearly, so each lane fetches the global
// chunk that belongs at its swizzled position.  Rows past M or N are clamped
// to the last row (their results are never stored).
//
// The direct loads are tracked by vmcnt only, and the compiler does not wait
// for them before LDS reads, so the loop waits explicitly: before reading
// stage kb a wave waits until at most the loads of stage kb+1 are
// outstanding, then a barrier makes every wave's loads visible.
//
// Bound: int8 MFMA for K >= 2048; for K <= 1024 the fp32 output (4*M*N bytes)
// weighs as much as the MFMA time.
#include "kernels.hpp"

namespace bl {

constexpr int kTileN = 256;   // weight rows per workgroup
constexpr int kTileM = 128;   // activation rows per workgroup
constexpr int kBlockK = 128;  // K positions per stage (one I2_S block)
constexpr int kStages = 3;
constexpr int kXStage = kTileM * kBlockK;        // 16 KB
constexpr int kWStage = kTileN * (kBlockK / 4);  // 8 KB
constexpr int kStageBytes = kXStage + kWStage;
// Direct loads per wave per stage: (16 KB + 8 KB) / 4 waves / 1 KB.
constexpr int kXLoads = kXStage / 4 / 1024;  // 4
constexpr int kWLoads = kWStage / 4 / 1024;  // 2
constexpr int kLoadsPerStage = kXLoads + kWLoads;

typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int xs_slot(int row, int slot) {
  return slot ^ (row & 7) ^ ((row >> 3) & 1);
}
__device__ __forceinline__ int ws_slot(int row, int slot) {
  return slot ^ ((row >> 2) & 1) ^ ((row >> 3) & 1);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt in [3:0] and
// [15:14], expcnt [6:4] and lgkmcnt [11:8] left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void dma16(const void* gsrc, uint8_t* ldst) {
  __builtin_amdgcn_global_load_lds((const BL_GLOBAL void*)gsrc,
                                   (__attribute__((address_space(3))) void*)ldst, 16, 0, 0);
}

template <bool RAW>
__global__ __launch_bounds__(256, 2) void gemm_kernel(ProbSet set) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];

  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const int wn = wave & 1, wm = wave >> 1;
  const int r32 = lane & 31, g = lane >> 5;

  int local;
  const Prob P = prob_at(set, find_prob(set, xcd_remap(blockIdx.x, set.total), &local));
  const int M = P.M, K = P.K, N = P.N;
  const int rowbytes = K >> 2;
  const int tiles_n = (N + kTileN - 1) / kTileN;
  const int m0 = (local / tiles_n) * kTileM;
  const int n0 = (local % tiles_n) * kTileN;
  const int nblk = K / kBlockK;

  // This lane's direct-load sources: for activation instruction i the lane
  // fills LDS row 32*wave + 8*i + lane/8, physical slot lane%8; for weight
  // instruction i, row 64*wave + 32*i + lane/2, physical slot lane%2.
  const int8_t* xsrc[kXLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int row = 32 * wave + 8 * i + (lane >> 3);
    const int slot = xs_slot(row, lane & 7);
    const int m = min(m0 + row, M - 1);
    xsrc[i] = P.xq + static_cast<int64_t>(m) * K + slot * 16;
  }
  const uint8_t* wsrc[kWLoads];
#pragma unroll
  for (int i = 0; i < kWLoads; ++i) {
    const int row = 64 * wave + 32 * i + (lane >> 1);
    const int slot = ws_slot(row, lane & 1);
    const int n = min(n0 + row, N - 1);
    wsrc[i] = P.w + static_cast<int64_t>(n) * rowbytes + slot * 16;
  }
  auto issue = [&](int kb) {
    uint8_t* st = smem + (kb % kStages) * kStageBytes;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i)
      dma16(xsrc[i] + kb * kBlockK, st + (kXLoads * wave + i) * 1024);
#pragma unroll
    for (int i = 0; i < kWLoads; ++i)
      dma16(wsrc[i] + kb * (kBlockK / 4), st + kXStage + (kWLoads * wave + i) * 1024);
  };

  v16i acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = v16i{};

  issue(0);
  if (nblk > 1) issue(1);

  for (int kb = 0; kb < nblk; ++kb) {
    // Stage kb's loads are done once at most stage kb+1's are outstanding.
    if (kb + 1 < nblk) wait_vmcnt<kLoadsPerStage>();
    else wait_vmcnt<0>();
    // Compiler-only fences: no LDS access or direct load may cross the barrier.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Every wave is past stage kb-1, whose ring slot stage kb+2 reuses.
    if (kb + 2 < nblk) issue(kb + 2);

    const uint8_t* xs = smem + (kb % kStages) * kStageBytes;
    const uint8_t* ws = xs + kXStage;
    v4i wp[4];  // 16-byte half g of 4 weight rows per lane (one per fragment)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) {
      const int row = wn * 128 + fn * 32 + r32;
      wp[fn] = *reinterpret_cast<const v4i*>(ws + row * 32 + ws_slot(row, g) * 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v4i b[2];
#pragma unroll
      for (int fm = 0; fm < 2; ++fm) {
        const int row = wm * 64 + fm * 32 + r32;
        b[fm] = *reinterpret_cast<const v4i*>(xs + row * kBlockK + xs_slot(row, 2 * j + g) * 16);
      }
#pragma unroll
      for (int fn = 0; fn < 4; ++fn) {
        v4i a;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = field_codes(static_cast<uint32_t>(wp[fn][i]), j);
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
          acc[fn][fm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b[fm], acc[fn][fm], 0, 0, 0);
      }
    }
  }

  // Epilogue: fragment (fn, fm) lane holds weight rows 8q + 4g + r (q, r in
  // 0..3) of activation row r32.
#pragma unroll
  for (int fm = 0; fm < 2; ++fm) {
    const int m = m0 + wm * 64 + fm * 32 + r32;
    if (m >= M) continue;
    const int rs = gptr<int32_t>(P.rowsum)[m];
    float scale = 0.f;
    if (!RAW) scale = gptr<float>(P.factor)[m] / P.w_scale;
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 128 + fn * 32 + 8 * q + 4 * g;
        if (n >= N) continue;
        const v4i v = v4i{acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2],
                          acc[fn][fm][4 * q + 3]};
        const int64_t o = static_cast<int64_t>(m) * N + n;
        if (RAW) {
          if ((N & 3) == 0) {
            *gptr_out<v4i>(P.acc + o) = v - rs;
          } else {
            for (int i = 0; i < 4 && n + i < N; ++i) gptr_out<int32_t>(P.acc)[o + i] = v[i] - rs;
          }
        } else {
          const f4 out = f4{static_cast<float>(v[0] - rs) * scale, static_cast<float>(v[1] - rs) * scale,
                            static_cast<float>(v[2] - rs) * scale, static_cast<float>(v[3] - rs) * scale};
          if ((N & 3) == 0) {
            *gptr_out<f4>(P.y + o) = out;
          } else {
            for (int i = 0; i < 4 && n + i < N; ++i) gptr_out<float>(P.y)[o + i] = out[i];
          }
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
