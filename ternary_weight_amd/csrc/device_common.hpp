// Device-side building blocks shared by the three kernels of the BitLinear
// path: the per-projection problem record, wave64 reductions, and the I2_S
// 2-bit field decode.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr int kWave = 64;

typedef int v4i __attribute__((ext_vector_type(4)));

// One projection as the kernels see it.  Pointers are device pointers.
// Workspace pointers (xq, factor, rowsum) belong to the library.
struct Prob {
  const float* x;        // [M][K] f32 activations
  const float* norm_w;   // [K] f32 norm weight
  const uint8_t* w;      // I2_S codes, row n at byte n*K/4
  int8_t* xq;            // [M][K] int8 codes (workspace or caller's)
  float* factor;         // [M] absmax/127 (workspace or caller's)
  int32_t* rowsum;       // [M] sum_k xq (workspace)
  float* y;              // [M][N] f32 output (forward)
  int32_t* acc;          // [M][N] i32 output (raw-integer hook)
  float w_scale;         // tensor-wide I2_S scale (1/mean|W|)
  float eps;
  int M, K, N;
};

// A launch covers either one problem passed by value (count == 0) or a table
// of problems in device memory.  `starts` holds count+1 prefix sums of the
// work units (rows or tiles) each problem contributes.
struct ProbSet {
  Prob single;
  const Prob* probs;
  const int* starts;
  int count;
  int total;  // total work units
};

// Locate the problem owning work unit `u`: returns the problem index and
// writes the unit's index local to that problem.
__device__ __forceinline__ int find_prob(const ProbSet& s, int u, int* local) {
  if (s.count == 0) {
    *local = u;
    return -1;
  }
  int lo = 0, hi = s.count - 1;
  while (lo < hi) {  // largest p with starts[p] <= u
    int mid = (lo + hi + 1) >> 1;
    if (s.starts[mid] <= u) lo = mid; else hi = mid - 1;
  }
  *local = u - s.starts[lo];
  return lo;
}

__device__ __forceinline__ const Prob& prob_at(const ProbSet& s, int p) {
  return p < 0 ? s.single : s.probs[p];
}

// ---- wave64 butterfly reductions (every lane ends with the result) --------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---- I2_S field decode ----------------------------------------------------
// A little-endian dword holds 4 consecutive bytes j..j+3 of a block.  Field f
// (0 = bits 7:6 ... 3 = bits 1:0) of those bytes carries elements
// 32f+j .. 32f+j+3 of the block, i.e. 4 consecutive K positions.  Shifting the
// field down and masking leaves one code (0, 1, 2) per byte: a ready int8x4
// MFMA operand.
__device__ __forceinline__ int field_codes(uint32_t d, int field) {
  return static_cast<int>((d >> (6 - 2 * field)) & 0x03030303u);
}

// XCD-aware tile order.  Consecutive workgroup ids are dealt round-robin to
// the 8 XCDs; this remaps id b so that each XCD walks a contiguous range of
// the tile space (shared activation rows stay in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int b, int total) {
  constexpr int kXcd = 8;
  int q = total / kXcd, r = total % kXcd;
  int x = b % kXcd, k = b / kXcd;
  return x * q + (x < r ? x : r) + k;
}

}  // namespace bl
