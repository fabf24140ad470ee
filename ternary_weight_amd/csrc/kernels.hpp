// Host-side launchers of the BitLinear kernels (internal to libbitlinear.so).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.hpp"

namespace bl {

// Largest K accepted by the GPU path; rows up to kQuantRegK stay in registers.
constexpr int kKMax = 65536;
// Byte offsets into one problem's packed weights and int8 activations are
// 32-bit (buffer addressing): N*K/4 and M*K must stay below this.
constexpr int64_t kMaxOffset = (int64_t{1} << 31) - 4096;
constexpr int kQuantRegK = 4096;

// Rows per skinny-decode pass: M <= kGemvMaxM takes the weight-streaming kernel.
constexpr int kGemvMaxM = 16;

// Work units (workgroups) per problem.  Quantization: kQuantRows rows per
// workgroup, kQuantRowsPerWave per wave.
constexpr int kQuantRowsPerWave = 1;
constexpr int kQuantRows = 4 * kQuantRowsPerWave;
inline int quant_units(int M) { return (M + kQuantRows - 1) / kQuantRows; }
// Share-set launches (shared && quant_chunks(K) > 0): rows_per_wave rows per
// wave (kSetRowsPerWave, or 1 for launches that would otherwise have fewer
// than kSetFewUnits workgroups: there each wave's rows, one after another on
// a fraction of the CUs, are the launch's critical path), four waves per
// workgroup, and at most quant_set_max(chunks) problems per set (larger sets
// are split by the caller).
constexpr int kSetRowsPerWave = 4;
constexpr int kSetFewUnits = 512;
inline int quant_set_units(int M, int rows_per_wave) {
  return (M + 4 * rows_per_wave - 1) / (4 * rows_per_wave);
}
int quant_set_max(int nc);
// Decode kernel: a workgroup owns 64 weight rows of one problem.  Problems
// are launched in buckets of equal superblock count ceil(K/256) (1..16; 0 =
// the generic variant for longer K).
// tiles: 16-row tiles per wave of each workgroup (0 = the bucket's full
// count, 2 * depth); a single-problem launch takes gemv_single_tiles(N,
// bucket), which keeps about kGemvSingleUnits workgroups busy.
constexpr int kGemvSingleUnits = 512;
int gemv_units(int N, int bucket, int tiles = 0);
int gemv_single_tiles(int N, int bucket);
int gemv_bucket(int K);
int gemm_units(int M, int N);  // output tiles of one prefill problem
// One prefill output tile of int32 partial sums (Prob::part), and the
// fewest K blocks (128 positions each) a split of a tile may take.
constexpr int kGemmPartInts = 128 * 256;
constexpr int kGemmMinSplitBlocks = 3;

// Stage 1: fused RMSNorm + absmax int8 quantization of every row in the set.
// max_k: the largest K in the set (it selects the register-resident variant:
// quant_chunks(max_k) float4 chunks per lane, 0 = the streaming variant).
// shared: every unit's record heads a share set (Prob::share problems read
// its x).  act: every record's input is act(x) * up (kActSilu, kActGeluTanh;
// records carry the same value in Prob::act) or x (kActNone); not with shared.
int quant_chunks(int max_k);
// set_rows: rows per wave of a shared launch (kSetRowsPerWave or 1), as its
// units were counted with.
hipError_t launch_quant(const ProbSet& set, int max_k, bool shared, int act, hipStream_t stream,
                        int set_rows = kSetRowsPerWave);
// Every quantization of a small group in one launch: units of share sets
// (Prob::share > 1, chunk count quant_chunks(K) <= 8) and of single
// problems (quant_chunks(K) > 0), no FFN glue, all at one row per wave
// (quant_units(M) units per set or problem).  Used for groups whose
// quantization would otherwise take several launches and at most
// kQuantMergeMaxUnits workgroups: launches that small cost their fixed
// launch time, not their work.
constexpr int kQuantMergeMaxUnits = 2048;
hipError_t launch_quant_merged(const ProbSet& set, hipStream_t stream);
// The statistics pass of the prefill path that quantizes in the product's
// producer: per row the factor, the code sum and max|u| (Prob::amax), no
// codes stored; register-resident rows only (quant_chunks(max_k) > 0).
hipError_t launch_quant_stats(const ProbSet& set, int max_k, hipStream_t stream);
// Row sums of caller-supplied int8 activations (for the raw-integer hook).
hipError_t launch_rowsum(const Prob& p, hipStream_t stream);
// Stage 2, M <= kGemvMaxM: weight-streaming MFMA decode kernel for one
// bucket, over one by-value problem (units == nullptr) or a FatUnit table.
// max_m and max_k bound the launch's M and K (they size the LDS activation
// staging).  fused: the kernel also runs stage 1 for its rows (RMSNorm +
// int8 quantization from x and norm_w, same arithmetic as launch_quant), so
// no quantization launch and no workspace are needed; only for problems
// with gemv_fusable(M, K, glue) and the forward epilogue.  glue: the
// problems' input is the FFN glue act(x) * up (Prob::act, Prob::up), which
// the fused kernel forms in LDS.
struct GemvLaunch {
  Prob single;
  const FatUnit* units;
  int total;
  int tiles;  // 16-row tiles per wave, 0 = the bucket's full count
  size_t fused_shmem;  // fused table launches: LDS bytes (0: from max_m, max_k)
};
bool gemv_fusable(int M, int K, bool glue = false, bool table = false);
// Staging bytes of one fused problem; a table launch takes the largest over
// its problems (each problem lays its LDS out from its own M and K).
size_t gemv_fused_lds_bytes(int M, int K, bool glue);
// A single call fuses only up to this many rows: each workgroup stages and
// quantizes all M rows, about 1 us more per row, while the separate
// quantization kernel spreads rows over workgroups (measured per call at
// K = 640..2048: fused wins at M <= 2, breaks even at M = 3, loses from 4).
// Groups fuse by staging budget alone (many workgroups hide it).
constexpr int kGemvSingleFusedMaxM = 3;
// Fused decode problems of up to kGemvMergedMaxNsb superblocks in one launch
// over a FatUnit table whose records carry each unit's superblock count
// (FatUnit::nsb), longest first.  shmem: the largest gemv_fused_lds_bytes of
// its problems.
constexpr int kGemvMergedMaxNsb = 12;
hipError_t launch_gemv_merged(const FatUnit* units, int total, size_t shmem, hipStream_t stream);
hipError_t launch_gemv(const GemvLaunch& L, bool raw, int bucket, int max_m, int max_k,
                       bool fused, hipStream_t stream, bool glue = false);
// Device-side absmean ternary quantization and I2_S packing of w (device,
// [N][K] float32, 16-byte aligned) into packed (device, N*K/4 + 4 bytes):
// codes, then the scale.  partial: kPackPartials doubles of scratch;
// scale_dev: one float, receives the scale as well.
constexpr int kPackPartials = 1024;
hipError_t launch_i2s_pack_device(const float* w, int64_t K, int64_t N, uint8_t* packed,
                                  double* partial, float* scale_dev, hipStream_t stream);
// Stage 2, M > kGemvMaxM: LDS-tiled MFMA kernel.
hipError_t launch_gemm(const ProbSet& set, bool raw, hipStream_t stream);
// The same product for one problem whose activation producer quantizes:
// it reads the fp32 rows (x, norm_w) and codes them itself from the
// statistics pass's max|u| (Prob::amax), factor and row sums; forward
// epilogue only.  Rows of at most kGemmPqMaxK values, M*K*4 < 2^31.
constexpr int kGemmPqMaxK = 4096;
hipError_t launch_gemm_pq(const Prob& p, hipStream_t stream);

}  // namespace bl
