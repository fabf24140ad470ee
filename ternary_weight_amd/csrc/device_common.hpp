// Device-side building blocks shared by the three kernels of the BitLinear
// path: the per-projection problem record, wave64 reductions, and the I2_S
// 2-bit field decode.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr int kWave = 64;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// Raw buffer resources: word 3 for the gfx9 family, and an offset past any
// buffer's records (loads read 0, stores are dropped, no memory access).
constexpr int kBufferDword3 = 0x00020000;
constexpr int kOob = 0x7FFFFFF0;

#define BL_GLOBAL __attribute__((address_space(1)))
#define BL_CONST __attribute__((address_space(4)))

// One projection as the kernels see it.  Pointers are device pointers.
// Workspace pointers (xq, factor, rowsum) belong to the library.
struct Prob {
  const float* x;        // [M][K] f32 activations
  const float* norm_w;   // [K] norm weight (f32, or binary16 if nw_f16); null: no norm
                         // (u = x, r = 1)
  const uint8_t* w;      // I2_S codes, row n at byte n*K/4
  int8_t* xq;            // [M][K] int8 codes (workspace or caller's)
  float* factor;         // [M] absmax/127 (workspace or caller's)
  int32_t* rowsum;       // [M] sum_k xq (workspace)
  float* y;              // [M][N] f32 output (forward)
  int32_t* acc;          // [M][N] i32 output (raw-integer hook)
  const float* up;       // FFN glue: [M][K] up-projection output (x is the gate output)
  float w_scale;         // tensor-wide I2_S scale (1/mean|W|)
  float eps;
  int M, K, N;
  // Quantization launches: the number of consecutive records, this one
  // first, whose rows are the same x (same pointer, M, K and eps); one pass
  // over x serves them all.  0 or 1: this record alone.
  int share;
  // FFN glue: the input row is act(x) * up (kActSilu, kActGeluTanh) instead
  // of x (kActNone).
  int act;
  // norm_w holds K IEEE binary16 values ("BitNet Embeddings GGUF Conversion
  // Implementation", s3 tensor types and s6.1: norms are stored as float16),
  // widened exactly to f32 when loaded.
  int nw_f16;
  // Prefill launches: the K blocks of each output tile are split over ksplit
  // workgroups (0 or 1: no split).  Each split stores its int32 partial tile
  // in `part` (ksplit partial tiles per output tile, kGemmPartInts int32
  // each) and counts itself in tile_cnt[tile]; the last to arrive adds the
  // other partials and runs the epilogue, then sets the count back to 0
  // (the counts are zero between launches).
  int ksplit;
  int32_t* part;
  unsigned* tile_cnt;
  // Prefill with quantization in the product's producer: [M] max|x*norm_w|
  // per row, written by the statistics pass and read by the prefill kernel
  // that codes fp32 rows itself (null elsewhere).
  float* amax;
};

constexpr int kActNone = 0, kActSilu = 1, kActGeluTanh = 2;

// A launch covers either one problem passed by value (units == nullptr:
// work unit u is local unit u of that problem) or a table of problems in
// device memory with one (problem, local unit) pair per work unit, built on
// the host so that a workgroup finds its problem with one scalar load.
struct ProbSet {
  Prob single;
  const Prob* probs;
  const int2* units;
  int total;  // total work units
  int split;  // prefill launches: some problem has ksplit > 1
};

// A work unit that carries its problem record inline: one scalar load finds
// everything a workgroup needs (used where workgroups are short-lived).
struct FatUnit {
  Prob p;
  int local;
  int nsb;  // superblocks ceil(K/256) of a merged decode launch's unit (0 otherwise)
};

// Address-space qualified views.  Pointers read from a problem record are
// generic; casting them to the global space lets the compiler emit global_*
// memory instructions (counted by vmcnt only) instead of flat_* ones, which
// also count against lgkmcnt and serialise with LDS traffic.  The problem
// table itself is read through the constant space, i.e. with scalar loads
// into SGPRs (the index is wave-uniform).
template <typename T>
__device__ __forceinline__ const BL_GLOBAL T* gptr(const void* p) {
  return (const BL_GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ BL_GLOBAL T* gptr_out(void* p) {
  return (BL_GLOBAL T*)p;
}

// Locate the problem owning work unit `u` (wave-uniform): returns the
// problem index (-1 for the by-value problem) and writes the local unit.
__device__ __forceinline__ int find_prob(const ProbSet& s, int u, int* local) {
  if (s.units == nullptr) {
    *local = u;
    return -1;
  }
  const BL_CONST int* e = (const BL_CONST int*)(s.units + u);
  *local = e[1];
  return e[0];
}

__device__ __forceinline__ Prob prob_at(const ProbSet& s, int p) {
  if (p < 0) return s.single;
  static_assert(sizeof(Prob) % 4 == 0, "Prob is copied as dwords");
  Prob out;
  const BL_CONST uint32_t* src = (const BL_CONST uint32_t*)(s.probs + p);
  uint32_t* dst = reinterpret_cast<uint32_t*>(&out);
#pragma unroll
  for (int i = 0; i < static_cast<int>(sizeof(Prob) / 4); ++i) dst[i] = src[i];
  return out;
}

// Problem record and local unit of work unit u from a FatUnit table.
__device__ __forceinline__ Prob fat_unit_at(const FatUnit* units, int u, int* local,
                                            int* nsb = nullptr) {
  static_assert(sizeof(FatUnit) % 4 == 0, "FatUnit is copied as dwords");
  FatUnit out;
  const BL_CONST uint32_t* src = (const BL_CONST uint32_t*)(units + u);
  uint32_t* dst = reinterpret_cast<uint32_t*>(&out);
#pragma unroll
  for (int i = 0; i < static_cast<int>(sizeof(FatUnit) / 4); ++i) dst[i] = src[i];
  *local = out.local;
  if (nsb) *nsb = out.nsb;
  return out.p;
}

// Wave index as a scalar (uniform across the wave).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
}

// ---- wave64 reductions (every lane ends with the result; call them with
// the whole wave active) -----------------------------------------------------
// Order-free ones (max, integer sum): four DPP steps inside each row of 16
// lanes (swap neighbours, swap pairs, mirror 8, mirror 16), then the four row
// results read into scalars; no LDS round trips.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppSwap1 = 0xB1, kDppSwap2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
__device__ __forceinline__ float fmax_dpp(float v, int bits) {
  return fmaxf(v, __builtin_bit_cast(float, bits));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmax_dpp(v, dpp_mov<kDppSwap1>(__builtin_bit_cast(int, v)));
  v = fmax_dpp(v, dpp_mov<kDppSwap2>(__builtin_bit_cast(int, v)));
  v = fmax_dpp(v, dpp_mov<kDppHalfMirror>(__builtin_bit_cast(int, v)));
  v = fmax_dpp(v, dpp_mov<kDppMirror>(__builtin_bit_cast(int, v)));
  const int b = __builtin_bit_cast(int, v);
  return fmaxf(fmax_dpp(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)),
                        __builtin_amdgcn_readlane(b, 16)),
               fmax_dpp(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)),
                        __builtin_amdgcn_readlane(b, 48)));
}
__device__ __forceinline__ int wave_sum(int v) {
  v += dpp_mov<kDppSwap1>(v);
  v += dpp_mov<kDppSwap2>(v);
  v += dpp_mov<kDppHalfMirror>(v);
  v += dpp_mov<kDppMirror>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
// The double sum keeps its butterfly order (its rounding depends on it; the
// pairs are added commutatively, so every lane gets the same bits).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---- activation quantization arithmetic ------------------------------------
// Every kernel that quantizes a row uses these, in the same order, so that
// all of them produce the same codes and the same factor bit for bit.
//
// Per lane, Sum(x^2) accumulates the lane's 4-element chunks (chunk c =
// lane + 64 i, increasing i) in fp32; the wave total is taken in double.
__device__ __forceinline__ float sq4(const f4& v) {
  return v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
}
__device__ __forceinline__ float absmax4(const f4& u) {
  return fmaxf(fmaxf(fabsf(u.x), fabsf(u.y)), fmaxf(fabsf(u.z), fabsf(u.w)));
}
// Codes: rne(u * 127/max|u|), clamped to [-127, 127].  Rows whose max|u| is
// below kTinyAmax take the double-precision multiplier (127/max|u| would
// overflow fp32).
constexpr float kTinyAmax = 1e-30f;
__device__ __forceinline__ int code_f32(float u, float s) {
  float v = rintf(u * s);  // half to even
  v = fminf(fmaxf(v, -127.0f), 127.0f);
  return static_cast<int>(v);
}
__device__ __forceinline__ int code_f64(float u, double s) {
  double v = rint(static_cast<double>(u) * s);
  v = fmin(fmax(v, -127.0), 127.0);
  return static_cast<int>(v);
}
__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (static_cast<uint32_t>(a) & 0xffu) | ((static_cast<uint32_t>(b) & 0xffu) << 8) |
         ((static_cast<uint32_t>(c) & 0xffu) << 16) | ((static_cast<uint32_t>(d) & 0xffu) << 24);
}
// The four codes of chunk u (zero for an all-zero row) and their sum.
__device__ __forceinline__ uint32_t codes4(const f4& u, float amax, int* sum) {
  int a = 0, b = 0, c = 0, d = 0;
  if (amax >= kTinyAmax) {
    const float s = 127.0f / amax;
    a = code_f32(u.x, s); b = code_f32(u.y, s); c = code_f32(u.z, s); d = code_f32(u.w, s);
  } else if (amax > 0.f) {
    const double s = 127.0 / static_cast<double>(amax);
    a = code_f64(u.x, s); b = code_f64(u.y, s); c = code_f64(u.z, s); d = code_f64(u.w, s);
  }
  *sum += a + b + c + d;
  return pack4(a, b, c, d);
}
// Four binary16 norm weights (one 8-byte load) widened to f32: exact.
__device__ __forceinline__ f4 half4(u2 h) {
  auto cv = [](uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
  };
  return f4{cv(h.x & 0xffffu), cv(h.x >> 16), cv(h.y & 0xffffu), cv(h.y >> 16)};
}
// Norm weight kinds of the quantization variants.
constexpr int kNwNone = 0, kNwF32 = 1, kNwF16 = 2;
__device__ __forceinline__ int nw_kind(const Prob& P) {
  return P.norm_w ? (P.nw_f16 ? kNwF16 : kNwF32) : kNwNone;
}

// FFN glue ("BitNet Embeddings GGUF Conversion Implementation", s4.5 FFN
// per-projection norms; activation per the s1 model table): the down
// projection's input is act(gate) * up.  SiLU(z) = z / (1 + e^-z); the tanh
// form of GELU, 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).  fp32.
template <int ACT>
__device__ __forceinline__ float act_f32(float z) {
  if (ACT == kActSilu) return z / (1.0f + expf(-z));
  return 0.5f * z * (1.0f + tanhf(0.7978845608f * (z + 0.044715f * z * z * z)));
}
template <int ACT>
__device__ __forceinline__ f4 glu4(f4 g, f4 u) {
  return f4{act_f32<ACT>(g.x) * u.x, act_f32<ACT>(g.y) * u.y, act_f32<ACT>(g.z) * u.z,
            act_f32<ACT>(g.w) * u.w};
}

// factor = max|RMSNorm(x) * norm_w| / 127 = r * max|u| / 127 with
// r = 1/sqrt(mean(x^2) + eps), in double from the row's Sum(x^2).  A
// projection without a norm weight (norm == false) quantizes x as it is
// ("BitNet Embeddings GGUF Conversion Implementation", s4.5: the input feeds
// the projection directly when its norm tensor is absent): u = x, r = 1.
__device__ __forceinline__ float quant_factor(double ss, int K, float eps, float amax, bool norm) {
  const double r = norm ? 1.0 / sqrt(ss / static_cast<double>(K) + static_cast<double>(eps)) : 1.0;
  return static_cast<float>(r * static_cast<double>(amax) / 127.0);
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
