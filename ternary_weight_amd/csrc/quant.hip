// Stage 1 of the BitLinear path: per-projection RMSNorm fused with per-token
// absmax int8 quantization ("BitNet Embeddings GGUF Conversion
// Implementation", s1 "Background" and s4.5; "BitNet Inference Framework",
// "Quantization (W1.58A8)").
//
// One wavefront owns one token row.  The row is read once from HBM with
// coalesced 16-byte loads and kept in VGPRs (K <= 4096), Sum(x^2) and
// max|x*norm_w| are reduced across the wave, and the int8 codes are written
// with one coalesced dword per lane per 4 elements.  Those stores are
// non-temporal: the codes are read back by the next launch from HBM anyway
// (a prefill stack's codes are gigabytes), and the plain stores ran 7% slower.
//
// The codes use the identity  xhat*127/max|xhat| = u*127/max|u|  with
// u = x*norm_w, since RMSNorm multiplies the whole row by one positive scalar;
// so the codes never see the rsqrt.  The norm only enters the factor
// absmax(xhat)/127 = r*max|u|/127, computed in double from the fp32 partial
// sums.  Bound: HBM, 4K bytes read + K bytes written per row (plus the norm
// weight, an L2 hit).
//
// A projection without a norm weight (norm_w null) quantizes x unnormalised:
// u = x and r = 1 (same kernels, the multiply and the rsqrt skipped).  A
// float16 norm weight is widened exactly on load and then used as f32.
//
// Projections that read the same input (q, k and v of a layer, or gate and
// up: each normalises the shared x with its own weight, "BitNet Embeddings
// GGUF Conversion Implementation" s4.5) form a share set in a grouped launch:
// one pass reads the row and its Sum(x^2) once and emits every projection's
// codes, so the input is read once instead of once per projection.
#include <type_traits>

#include "kernels.hpp"

namespace bl {

// Per-row finish shared by both variants: the factor and the row sum.
__device__ __forceinline__ void finish_row(const Prob& P, int m, double ss, float amax, int rs,
                                           int lane) {
  rs = wave_sum(rs);
  if (lane == 0) {
    gptr_out<float>(P.factor)[m] = quant_factor(ss, P.K, P.eps, amax, P.norm_w != nullptr);
    if (P.rowsum) gptr_out<int32_t>(P.rowsum)[m] = rs;
  }
}

// Chunk c (4 elements) of the norm weight of kind NW (kNwF32 or kNwF16).
template <int NW>
__device__ __forceinline__ f4 nw_chunk(const Prob& P, int c) {
  if (NW == kNwF16) return half4(gptr<u2>(reinterpret_cast<const uint16_t*>(P.norm_w))[c]);
  return gptr<f4>(P.norm_w)[c];
}

// NC: float4 chunks per lane held in registers (K <= 256*NC).  A workgroup
// owns kQuantRows consecutive rows of one problem, kQuantRowsPerWave per wave.
// ACT: the row is act(x) * up (FFN glue) instead of x.  NW: the kind of norm
// weight (each kind keeps its loads in one block, no per-element branch).
// STATS: the row statistics alone (factor, row sum and max|u| into P.amax),
// the codes computed for their sum but not stored: the prefill kernel whose
// producer quantizes recomputes them from x with the same arithmetic.
template <int NC, int ACT, int NW, bool STATS = false>
__device__ __forceinline__ void quant_reg_rows(const Prob& P, int m_begin, int lane) {
  const int nch = P.K >> 2;
  for (int r = 0; r < kQuantRowsPerWave; ++r) {
    const int m = m_begin + r;
    if (m >= P.M) break;
    const BL_GLOBAL f4* xr = gptr<f4>(P.x + static_cast<int64_t>(m) * P.K);
    const BL_GLOBAL f4* ur = gptr<f4>(P.up + static_cast<int64_t>(m) * P.K);
    f4 u[NC];
    float ss = 0.f, amax = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + kWave * i;
      u[i] = f4{0.f, 0.f, 0.f, 0.f};
      if (c < nch) {
        // Read once: non-temporal loads (6% faster than plain on the prefill stack).
        const f4 xc = __builtin_nontemporal_load(xr + c);
        const f4 xv = ACT == kActNone ? xc : glu4<ACT>(xc, f4(__builtin_nontemporal_load(ur + c)));
        ss += sq4(xv);
        u[i] = NW == kNwNone ? xv : xv * nw_chunk<NW>(P, c);
        amax = fmaxf(amax, absmax4(u[i]));
      }
    }
    const double ssd = wave_sum(static_cast<double>(ss));
    amax = wave_max(amax);
    BL_GLOBAL uint32_t* qrow = STATS ? nullptr : gptr_out<uint32_t>(P.xq + static_cast<int64_t>(m) * P.K);
    int rs = 0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + kWave * i;
      if (c < nch) {
        const uint32_t q = codes4(u[i], amax, &rs);
        if (!STATS) __builtin_nontemporal_store(q, qrow + c);
      }
    }
    finish_row(P, m, ssd, amax, rs, lane);
    if (STATS && lane == 0) gptr_out<float>(P.amax)[m] = amax;
  }
}

// The statistics pass of the prefill path whose product quantizes in its
// producer (register-resident rows only, no FFN glue).
template <int NC>
__global__ __launch_bounds__(256) void quant_stats_kernel(ProbSet set) {
  const int lane = threadIdx.x & (kWave - 1);
  int local;
  const int pi = find_prob(set, blockIdx.x, &local);
  const Prob P = prob_at(set, pi);
  const int m_begin = local * kQuantRows + wave_id() * kQuantRowsPerWave;
  switch (nw_kind(P)) {
    case kNwF32: quant_reg_rows<NC, kActNone, kNwF32, true>(P, m_begin, lane); break;
    case kNwF16: quant_reg_rows<NC, kActNone, kNwF16, true>(P, m_begin, lane); break;
    default: quant_reg_rows<NC, kActNone, kNwNone, true>(P, m_begin, lane);
  }
}

template <int NC, int ACT>
__global__ __launch_bounds__(256) void quant_reg_kernel(ProbSet set) {
  const int lane = threadIdx.x & (kWave - 1);
  int local;
  const int pi = find_prob(set, blockIdx.x, &local);
  const Prob P = prob_at(set, pi);
  const int m_begin = local * kQuantRows + wave_id() * kQuantRowsPerWave;
  switch (nw_kind(P)) {
    case kNwF32: quant_reg_rows<NC, ACT, kNwF32>(P, m_begin, lane); break;
    case kNwF16: quant_reg_rows<NC, ACT, kNwF16>(P, m_begin, lane); break;
    default: quant_reg_rows<NC, ACT, kNwNone>(P, m_begin, lane);
  }
}

// Share sets (share <= quant_set_max(NC)): each wave owns ROWS consecutive
// rows of the set (kSetRowsPerWave, or 1 for short launches), reads each row
// once (the next row's loads in flight while the current one is processed,
// the first row's issued before the norm weights are staged), computes its
// Sum(x^2) once, and emits every problem's codes from the same registers.
// The set's norm weights are
// staged once per workgroup in LDS, widened to f32 (1 where a problem has
// none: u = x * 1 = x), and read from there per row: held in registers they
// cost the K = 1024 kernel half its waves (124 against 76 VGPRs).  Each row's
// Sum(x^2), max|u| and codes follow the plain variant's order and
// arithmetic, so results are bit-identical to unshared quantization.
// nws: LDS for SMAX * kWave * NC float4 (chunk c of member p's norm weight
// at p * kWave * NC + c).
// Problems per set of the register-resident kernel: their staged norm
// weights take at most 16 float4 per lane of LDS (16 KB per workgroup), and
// at most 3 problems (a layer's q, k and v).
constexpr int set_max(int nc) { return nc <= 0 ? 0 : (16 / nc < 3 ? (16 / nc < 1 ? 1 : 16 / nc) : 3); }
int quant_set_max(int nc) { return set_max(nc); }

template <int NC, int SMAX, int ROWS>
__device__ __forceinline__ void quant_set_rows(const ProbSet& set, int pi, int local, f4* nws) {
  const int lane = threadIdx.x & (kWave - 1);
  const Prob P = prob_at(set, pi);
  const int share = P.share > 1 ? (P.share < SMAX ? P.share : SMAX) : 1;
  const int nch = P.K >> 2;
  const int m0 = local * 4 * ROWS + wave_id() * ROWS;
  auto load_row = [&](int m, f4 (&xv)[NC]) {
    const BL_GLOBAL f4* xr = gptr<f4>(P.x + static_cast<int64_t>(m < P.M ? m : 0) * P.K);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + kWave * i;
      xv[i] = (m < P.M && c < nch) ? f4(__builtin_nontemporal_load(xr + c)) : f4{0.f, 0.f, 0.f, 0.f};
    }
  };
  f4 xa[NC], xb[NC];
  load_row(m0, xa);
  int8_t* xq[SMAX];
  float* fac[SMAX];
  int32_t* rsum[SMAX];
  bool norm[SMAX];
#pragma unroll
  for (int p = 0; p < SMAX; ++p) {
    if (p >= share) break;
    const Prob Q = p == 0 ? P : prob_at(set, pi + p);
    xq[p] = Q.xq;
    fac[p] = Q.factor;
    rsum[p] = Q.rowsum;
    norm[p] = Q.norm_w != nullptr;
    const int kind = nw_kind(Q);
    for (int c = threadIdx.x; c < kWave * NC; c += 256) {
      f4 v = f4{1.f, 1.f, 1.f, 1.f};
      if (c >= nch) v = f4{0.f, 0.f, 0.f, 0.f};
      else if (kind == kNwF32) v = nw_chunk<kNwF32>(Q, c);
      else if (kind == kNwF16) v = nw_chunk<kNwF16>(Q, c);
      nws[p * kWave * NC + c] = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int m = m0 + r;
    f4(&xv)[NC] = (r & 1) ? xb : xa;
    f4(&xn)[NC] = (r & 1) ? xa : xb;
    if (r + 1 < ROWS) load_row(m + 1, xn);
    if (m >= P.M) break;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + kWave * i;
      if (c < nch) ss += sq4(xv[i]);
    }
    const double ssd = wave_sum(static_cast<double>(ss));
#pragma unroll
    for (int p = 0; p < SMAX; ++p) {
      if (p >= share) break;
      float amax = 0.f;
      f4 u[NC];
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        u[i] = xv[i] * nws[p * kWave * NC + lane + kWave * i];
        amax = fmaxf(amax, absmax4(u[i]));
      }
      amax = wave_max(amax);
      BL_GLOBAL uint32_t* qrow = gptr_out<uint32_t>(xq[p] + static_cast<int64_t>(m) * P.K);
      int rs = 0;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int c = lane + kWave * i;
        if (c < nch) __builtin_nontemporal_store(codes4(u[i], amax, &rs), qrow + c);
      }
      rs = wave_sum(rs);
      if (lane == 0) {
        gptr_out<float>(fac[p])[m] = quant_factor(ssd, P.K, P.eps, amax, norm[p]);
        if (rsum[p]) gptr_out<int32_t>(rsum[p])[m] = rs;
      }
    }
  }
}


template <int NC, int SMAX, int ROWS>
__global__ __launch_bounds__(256) void quant_set_kernel(ProbSet set) {
  __shared__ f4 nws[SMAX * kWave * NC];
  int local;
  const int pi = find_prob(set, blockIdx.x, &local);
  quant_set_rows<NC, SMAX, ROWS>(set, pi, local, nws);
}

// Largest LDS staging of a share set (float4), over the chunk counts that
// share (1..8).
constexpr int set_lds_f4(int nc) { return set_max(nc) * kWave * nc; }
constexpr int kMergedNwsF4 = 1024;
static_assert(set_lds_f4(1) <= kMergedNwsF4 && set_lds_f4(2) <= kMergedNwsF4 &&
                  set_lds_f4(3) <= kMergedNwsF4 && set_lds_f4(4) <= kMergedNwsF4 &&
                  set_lds_f4(6) <= kMergedNwsF4 && set_lds_f4(8) <= kMergedNwsF4,
              "merged staging");

// Every quantization of a small group in one launch: each workgroup runs
// the body of its unit's kind (share set or single problem) and chunk count
// quant_chunks(K), one row per wave, four per workgroup.  The bodies are the
// separate launches' own, so the codes, factors and row sums are the same.
__global__ __launch_bounds__(256) void quant_merged_kernel(ProbSet set) {
  __shared__ f4 nws[kMergedNwsF4];
  const int lane = threadIdx.x & (kWave - 1);
  int local;
  const int pi = find_prob(set, blockIdx.x, &local);
  const Prob P = prob_at(set, pi);
  const int m_begin = local * kQuantRows + wave_id() * kQuantRowsPerWave;
  static_assert(kQuantRowsPerWave == 1, "one row per wave, as quant_set_rows<..., 1>");
  const int nc = (P.K + 255) >> 8;
  if (P.share > 1) {
    switch (nc) {
      case 1: quant_set_rows<1, set_max(1), 1>(set, pi, local, nws); break;
      case 2: quant_set_rows<2, set_max(2), 1>(set, pi, local, nws); break;
      case 3: quant_set_rows<3, set_max(3), 1>(set, pi, local, nws); break;
      case 4: quant_set_rows<4, set_max(4), 1>(set, pi, local, nws); break;
      case 5: case 6: quant_set_rows<6, set_max(6), 1>(set, pi, local, nws); break;
      case 7: case 8: quant_set_rows<8, set_max(8), 1>(set, pi, local, nws); break;
      default: break;  // not planned
    }
    return;
  }
  auto rows = [&](auto ncc) {
    constexpr int C = decltype(ncc)::value;
    switch (nw_kind(P)) {
      case kNwF32: quant_reg_rows<C, kActNone, kNwF32>(P, m_begin, lane); break;
      case kNwF16: quant_reg_rows<C, kActNone, kNwF16>(P, m_begin, lane); break;
      default: quant_reg_rows<C, kActNone, kNwNone>(P, m_begin, lane);
    }
  };
  using std::integral_constant;
  if (nc <= 1) rows(integral_constant<int, 1>{});
  else if (nc <= 2) rows(integral_constant<int, 2>{});
  else if (nc <= 3) rows(integral_constant<int, 3>{});
  else if (nc <= 4) rows(integral_constant<int, 4>{});
  else if (nc <= 6) rows(integral_constant<int, 6>{});
  else if (nc <= 8) rows(integral_constant<int, 8>{});
  else if (nc <= 12) rows(integral_constant<int, 12>{});
  else rows(integral_constant<int, 16>{});
}

// Rows longer than the register budget: two streaming passes over the row.
__device__ void quant_stream_row(const Prob& P, int m, int lane);
__global__ __launch_bounds__(256) void quant_stream_kernel(ProbSet set) {
  const int lane = threadIdx.x & (kWave - 1);
  int local;
  const int pi = find_prob(set, blockIdx.x, &local);
  const Prob P = prob_at(set, pi);
  const int share = P.share > 1 ? P.share : 1;
  const int m_begin = local * kQuantRows + wave_id() * kQuantRowsPerWave;
  for (int r = 0; r < kQuantRowsPerWave; ++r) {
    const int m = m_begin + r;
    if (m >= P.M) break;
    // Rows this long are re-read per problem of the share set (same result).
    for (int p = 0; p < share; ++p) quant_stream_row(p == 0 ? P : prob_at(set, pi + p), m, lane);
  }
}

// Input chunk c of row m: x, or the FFN glue act(x) * up.
__device__ __forceinline__ f4 stream_in(const Prob& P, const BL_GLOBAL f4* xr, int64_t m, int c) {
  if (P.act == kActNone) return xr[c];
  const f4 u = gptr<f4>(P.up + m * P.K)[c];
  const f4 g = xr[c];
  return P.act == kActSilu ? glu4<kActSilu>(g, u) : glu4<kActGeluTanh>(g, u);
}

// One row, two streaming passes (used for K above the register budget).
__device__ void quant_stream_row(const Prob& P, int m, int lane) {
  const int nch = P.K >> 2;
  const BL_GLOBAL f4* xr = gptr<f4>(P.x + static_cast<int64_t>(m) * P.K);
  const int nw = nw_kind(P);
  auto scaled = [&](f4 xv, int c) {
    return nw == kNwF32 ? xv * nw_chunk<kNwF32>(P, c) : nw == kNwF16 ? xv * nw_chunk<kNwF16>(P, c) : xv;
  };

  double ss = 0.0;
  float amax = 0.f;
  for (int c = lane; c < nch; c += kWave) {
    const f4 xv = stream_in(P, xr, m, c);
    ss += static_cast<double>(sq4(xv));
    amax = fmaxf(amax, absmax4(scaled(xv, c)));
  }
  ss = wave_sum(ss);
  amax = wave_max(amax);

  BL_GLOBAL uint32_t* qrow = gptr_out<uint32_t>(P.xq + static_cast<int64_t>(m) * P.K);
  int rs = 0;
  for (int c = lane; c < nch; c += kWave) {
    __builtin_nontemporal_store(codes4(scaled(stream_in(P, xr, m, c), c), amax, &rs), qrow + c);
  }
  finish_row(P, m, ss, amax, rs, lane);
}

// Row sums of int8 codes supplied by the caller (raw-integer hook only).
__global__ __launch_bounds__(256) void rowsum_kernel(Prob P) {
  const int lane = threadIdx.x & (kWave - 1);
  const int m = blockIdx.x * 4 + wave_id();
  if (m >= P.M) return;
  const BL_GLOBAL uint32_t* row = gptr<uint32_t>(P.xq + static_cast<int64_t>(m) * P.K);
  int rs = 0;
  for (int c = lane; c < (P.K >> 2); c += kWave) {
    const uint32_t d = row[c];
    rs += static_cast<int8_t>(d & 0xff) + static_cast<int8_t>((d >> 8) & 0xff) +
          static_cast<int8_t>((d >> 16) & 0xff) + static_cast<int8_t>(d >> 24);
  }
  rs = wave_sum(rs);
  if (lane == 0) gptr_out<int32_t>(P.rowsum)[m] = rs;
}

int quant_chunks(int max_k) {
  if (max_k > kQuantRegK) return 0;
  const int nc = (max_k + 255) / 256;
  static const int kNc[] = {1, 2, 3, 4, 6, 8, 12, 16};
  for (int c : kNc)
    if (nc <= c) return c;
  return 0;
}

#define BL_QUANT_SWITCH(KERNEL, ...)                                                          \
  switch (nc) {                                                                               \
    case 1: hipLaunchKernelGGL((KERNEL<1 __VA_ARGS__>), grid, block, 0, stream, set); break;  \
    case 2: hipLaunchKernelGGL((KERNEL<2 __VA_ARGS__>), grid, block, 0, stream, set); break;  \
    case 3: hipLaunchKernelGGL((KERNEL<3 __VA_ARGS__>), grid, block, 0, stream, set); break;  \
    case 4: hipLaunchKernelGGL((KERNEL<4 __VA_ARGS__>), grid, block, 0, stream, set); break;  \
    case 6: hipLaunchKernelGGL((KERNEL<6 __VA_ARGS__>), grid, block, 0, stream, set); break;  \
    case 8: hipLaunchKernelGGL((KERNEL<8 __VA_ARGS__>), grid, block, 0, stream, set); break;  \
    case 12: hipLaunchKernelGGL((KERNEL<12 __VA_ARGS__>), grid, block, 0, stream, set); break; \
    case 16: hipLaunchKernelGGL((KERNEL<16 __VA_ARGS__>), grid, block, 0, stream, set); break; \
    default: hipLaunchKernelGGL(quant_stream_kernel, grid, block, 0, stream, set);            \
  }

hipError_t launch_quant(const ProbSet& set, int max_k, bool shared, int act, hipStream_t stream,
                        int set_rows) {
  if (set.total <= 0) return hipSuccess;
  if (shared && act != kActNone) return hipErrorInvalidValue;
  if (shared && set_rows != 1 && set_rows != kSetRowsPerWave) return hipErrorInvalidValue;
  const int nc = quant_chunks(max_k);
  const dim3 grid(set.total), block(256);
  if (shared && nc > 0) {
    switch (nc) {
#define BL_QUANT_SET(n)                                                                          \
  case n:                                                                                        \
    if (set_rows == 1)                                                                           \
      hipLaunchKernelGGL((quant_set_kernel<n, set_max(n), 1>), grid, block, 0, stream, set);    \
    else                                                                                         \
      hipLaunchKernelGGL((quant_set_kernel<n, set_max(n), kSetRowsPerWave>), grid, block, 0,     \
                         stream, set);                                                           \
    break;
      BL_QUANT_SET(1) BL_QUANT_SET(2) BL_QUANT_SET(3) BL_QUANT_SET(4) BL_QUANT_SET(6)
      BL_QUANT_SET(8)
#undef BL_QUANT_SET
      default: return hipErrorInvalidValue;  // longer rows hold one problem: never shared
    }
  } else if (shared) {
    hipLaunchKernelGGL(quant_stream_kernel, grid, block, 0, stream, set);
  } else if (act == kActSilu) {
    BL_QUANT_SWITCH(quant_reg_kernel, , kActSilu)
  } else if (act == kActGeluTanh) {
    BL_QUANT_SWITCH(quant_reg_kernel, , kActGeluTanh)
  } else {
    BL_QUANT_SWITCH(quant_reg_kernel, , kActNone)
  }
#undef BL_QUANT_SWITCH
  return hipGetLastError();
}

hipError_t launch_quant_stats(const ProbSet& set, int max_k, hipStream_t stream) {
  if (set.total <= 0) return hipSuccess;
  const int nc = quant_chunks(max_k);
  if (nc <= 0) return hipErrorInvalidValue;  // rows too long for registers
  const dim3 grid(set.total), block(256);
  switch (nc) {
#define BL_QUANT_STATS(n) \
  case n: hipLaunchKernelGGL((quant_stats_kernel<n>), grid, block, 0, stream, set); break;
    BL_QUANT_STATS(1) BL_QUANT_STATS(2) BL_QUANT_STATS(3) BL_QUANT_STATS(4) BL_QUANT_STATS(6)
    BL_QUANT_STATS(8) BL_QUANT_STATS(12) BL_QUANT_STATS(16)
#undef BL_QUANT_STATS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_merged(const ProbSet& set, hipStream_t stream) {
  if (set.total <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_merged_kernel, dim3(set.total), dim3(256), 0, stream, set);
  return hipGetLastError();
}

hipError_t launch_rowsum(const Prob& p, hipStream_t stream) {
  if (p.M <= 0) return hipSuccess;
  hipLaunchKernelGGL(rowsum_kernel, dim3((p.M + 3) / 4), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace bl
