// Host-side launchers of the BitLinear kernels (internal to libbitlinear.so).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace bl {

// Largest K accepted by the GPU path; rows up to kQuantRegK stay in registers.
constexpr int kKMax = 65536;
constexpr int kQuantRegK = 4096;

// Rows per skinny-decode pass: M <= kGemvMaxM takes the weight-streaming kernel.
constexpr int kGemvMaxM = 16;

// Work-unit counts per problem (what ProbSet::starts sums up).
inline int quant_units(int M) { return M; }
int gemv_units(int N);
int gemm_units(int M, int N);

// Stage 1: fused RMSNorm + absmax int8 quantization of every row in the set.
// max_k: the largest K in the set.
hipError_t launch_quant(const ProbSet& set, int max_k, hipStream_t stream);
// Row sums of caller-supplied int8 activations (for the raw-integer hook).
hipError_t launch_rowsum(const Prob& p, hipStream_t stream);
// Stage 2, M <= kGemvMaxM: weight-streaming MFMA decode kernel.
hipError_t launch_gemv(const ProbSet& set, bool raw, hipStream_t stream);
// Stage 2, M > kGemvMaxM: LDS-tiled MFMA kernel.
hipError_t launch_gemm(const ProbSet& set, bool raw, hipStream_t stream);

}  // namespace bl
