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
// four fields feed four MFMAs.  Fields 1..3 are isolated with a mask only
// (code*16, code*4, code) and accumulated separately, the exact powers of
// two divided out at the end; field 0 becomes -64 * weight with one
// three-input bit operation.  Codes are 0, 1, 2, so the activation sum over
// the field 1..3 positions (the row sum less the field-0 sum, which the
// matrix core computes once per wave against an all-ones operand) is
// subtracted at the end to turn them into -1, 0, +1.
//
// Work split: a workgroup owns 4*16*T consecutive weight rows of one problem;
// wave w takes its 16-row tiles w, w+4, w+8, ... (so at any time the four
// waves stream one contiguous span), walked in order through a rolling window: the
// weight loads of D tiles are in flight while one is processed (D = 4, 3, 2
// for up to 4, 8, 16 superblocks; T = 2D; a single-problem launch gives each
// wave fewer tiles when N is small, see gemv_body).  Accumulators are
// combined one tile late, once their MFMAs have drained, and all results are
// stored after the last tile.
// The kernel is specialised on the number of superblocks NSB = ceil(K/256):
// a tile's NSB weight loads are issued together and consumed in order, so
// the compiler's wait counts are exact and the register footprint small.
// Weights are read with buffer loads: an offset outside the problem's weight
// bytes returns 0 without a memory access, which replaces the bounds branches
// (rows >= N, tiles past the end, the missing half of a half superblock).
// The <= 16 activation rows are staged once per workgroup in LDS with direct
// global-to-LDS loads, zero-padded along K to NSB superblocks; when they do
// not fit, fragments come from global memory through the same
// out-of-range-reads-zero buffer loads.  Fused variant (the forward when the
// fp32 rows fit on chip): the workgroup stages the fp32 rows and the norm
// weight instead (with the FFN glue, the up rows too) and its four waves run
// the RMSNorm + int8 quantization themselves, with the arithmetic and order of
// operations of the quantization kernel, while its first weight loads are in
// flight; no separate launch and no workspace.  K beyond 16 superblocks runs a
// generic variant (one tile per wave, superblocks streamed two ahead).
// Bound: HBM, K/4 bytes per output column.
#include "kernels.hpp"

namespace bl {

constexpr int kGemvLdsBytes = 64 * 1024;   // activation staging limit per workgroup
constexpr int kMaxNsb = 16;                // specialised superblock counts 1..16
// Fused-variant staging limits per workgroup: single-problem launches (their
// time grows with the staging, see kGemvSingleFusedMaxM), table launches (up
// to 52 KB keeps three workgroups per CU, as many as the merged kernel's
// registers allow), and either with the FFN glue's up rows staged too.
constexpr int kGemvFusedLdsBytes = 40 * 1024;
constexpr int kGemvTableLdsBytes = 52 * 1024;
constexpr int kGemvGlueLdsBytes = 56 * 1024;

// LDS layout of the fused variant (byte offsets): the staged codes (M rows of
// nsb superblocks) at 0, a table (epilogue scale of up to 16 rows, then the
// absmax and the code sum of each (row, chunk column) unit, see gemv_body),
// the lanes' partial sums of squares (one float per lane and unit, as many
// bytes as the codes), the fp32 rows, with the FFN glue (glue) the fp32 up
// rows, and the norm weight, each 1 KB aligned.  Monotonic in M and K, so a
// launch sized for its largest problem fits every problem.
struct FusedLds {
  int tab, sq, x, up, nw, bytes;
};
__host__ __device__ inline FusedLds fused_lds(int M, int K, int nsb, bool glue) {
  FusedLds l;
  const int cb = (M * nsb * 256 + 1023) & ~1023;
  const int xb = (M * K * 4 + 1023) & ~1023;
  l.tab = cb;
  l.sq = l.tab + ((64 + 8 * M * nsb + 1023) & ~1023);
  l.x = l.sq + cb;
  l.up = l.x + xb;
  l.nw = l.up + (glue ? xb : 0);
  l.bytes = l.nw + ((K * 4 + 1023) & ~1023);
  return l;
}

// The four MFMA operands of one 16-byte chunk, one dword at a time.  Fields
// 1..3 are isolated with a mask only and stay scaled by their bit position
// (code*16, code*4, code).  Field 0 (bits 7:6) cannot be masked in place,
// since code 2 * 64 = 128 overflows int8; flipping its low bit first maps
// codes 0, 1, 2 to bit patterns 1, 0, 3, which read as signed bytes
// 64, 0, -64: -64 * (code - 1), the ternary weight itself, negated and
// scaled.  One three-input bit operation per field.
__device__ __forceinline__ void decode_fields(const v4i& w, v4i& a0, v4i& a1, v4i& a2, v4i& a3) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t d = static_cast<uint32_t>(w[i]);
    a0[i] = static_cast<int>((d ^ 0x40404040u) & 0xC0C0C0C0u);  // -64 * weight
    a1[i] = static_cast<int>(d & 0x30303030u);                  // code * 16
    a2[i] = static_cast<int>(d & 0x0C0C0C0Cu);                  // code * 4
    a3[i] = static_cast<int>(d & 0x03030303u);                  // code
  }
}

// Tiles in flight per wave (the weight loads of D tiles are outstanding while
// one is processed) and tiles per wave.  Deeper windows for short rows: the
// in-flight bytes per wave must cover the memory latency.
constexpr int gemv_depth(int nsb) { return nsb == 0 ? 1 : (nsb <= 4 ? 4 : (nsb <= 8 ? 3 : 2)); }
constexpr int gemv_tiles(int nsb) { return nsb == 0 ? 1 : 2 * gemv_depth(nsb); }

// Tile result for the lane's activation row r16 and 4 weight rows: the
// field accumulators combined (field 0 carries -64 * weight, fields 1..3
// code * 16, code * 4, code), minus rs123, the activation sum over the
// field 1..3 positions (codes -> weights there), and for the forward the
// scale applied; returned as raw bits.  All shifts are exact.
template <bool RAW>
__device__ __forceinline__ v4i gemv_result(const v4i* acc, int rs123, float scale) {
  const v4i v = (acc[1] >> 4) + (acc[2] >> 2) + acc[3] - (acc[0] >> 6) - rs123;
  if (RAW) return v;
  return __builtin_bit_cast(v4i, f4{static_cast<float>(v[0]) * scale, static_cast<float>(v[1]) * scale,
                                    static_cast<float>(v[2]) * scale, static_cast<float>(v[3]) * scale});
}

// Stores a tile result at output row r16, columns nrow..nrow+3 (clipped to N).
template <bool RAW>
__device__ __forceinline__ void gemv_store(const Prob& P, const v4i& v, int nrow, int r16) {
  const int N = P.N;
  if (r16 >= P.M || nrow >= N) return;
  const int64_t o = static_cast<int64_t>(r16) * N + nrow;
  int32_t* out = RAW ? P.acc : reinterpret_cast<int32_t*>(P.y);
  if ((N & 3) == 0) {
    *gptr_out<v4i>(out + o) = v;
  } else {
    // Ragged N: at most four guarded stores (a bounded count keeps the
    // compiler's wait-count bookkeeping for the weight loads exact).
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (nrow + i < N) gptr_out<int32_t>(out)[o + i] = v[i];
  }
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt in [3:0] and
// [15:14], expcnt [6:4] and lgkmcnt [11:8] left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One workgroup's work: `unit` of problem P.  NSB > 0: exactly NSB
// superblocks per tile.  NSB == 0: any K, streamed.  GLUE (fused only): the
// input rows are the FFN glue act(x) * up (P.act, P.up).  tpu: 16-row tiles
// per wave (1..T); below T a workgroup owns 64*tpu rows, so that a launch of
// one small problem still spreads over many workgroups (past tile tpu-1 the
// window's loads read zeros without a memory access, and those tiles skip
// their products and store nothing).
template <bool RAW, bool FROM_LDS, int NSB, bool FUSED, bool GLUE = false>
__device__ __forceinline__ void gemv_body(const Prob& P, const int unit, const int tpu) {
  static_assert(!FUSED || (FROM_LDS && !RAW && NSB > 0), "fused: forward, staged, specialised K");
  static_assert(!GLUE || FUSED, "glue: fused only");
  constexpr int T = gemv_tiles(NSB);
  constexpr int D = gemv_depth(NSB);
  constexpr int kHeld = NSB > 0 ? NSB : 2;
  // Weight loads issued after the activation staging and before its wait.
  constexpr int kInFlight = D * kHeld;
  static_assert(kInFlight < 64, "vmcnt range");
  extern __shared__ __attribute__((aligned(1024))) int8_t xlds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int M = P.M, K = P.K, N = P.N;
  const int rowbytes = K >> 2;
  const int nsb = NSB > 0 ? NSB : (K + 255) >> 8;
  const int kpad = (NSB > 0 ? nsb : (nsb + 1) & ~1) * 256;
  // Lanes past the M activation rows read row M-1: the MFMA columns they
  // feed are output rows that are never stored.
  const int xrow = min(r16, M - 1);

  // Startup order matters: every load whose result the wave waits for before
  // its first tile (activation staging, row sum, factor) is issued ahead of
  // the weight loads, so those waits leave the weights in flight.
  //
  // Activations go straight to LDS (buffer_load ... lds): each wave
  // instruction fills 1 KB linearly.  Row m occupies kpad bytes at m*kpad,
  // its 16-byte slots XOR-swizzled by m % 8 so that the 8 lanes reading one
  // slot of 8 different rows hit distinct banks; each lane fetches the
  // global chunk that belongs at its swizzled position.  Positions past K or
  // past row M-1 read 0 without a memory access (their products meet weight
  // codes 0 anyway).
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(P.xq), 0, FUSED ? 0 : M * K, kBufferDword3);
  constexpr bool glue = GLUE;
  const FusedLds fl = fused_lds(M, K, NSB, glue);
  if (FUSED) {
    // fp32 rows, with the glue the up rows, and the norm weight (4K bytes,
    // 2K if float16, none without one), copied linearly (1 KB per wave
    // instruction; bytes past each buffer read 0).
    const int nwb = P.norm_w ? K * (P.nw_f16 ? 2 : 4) : 0;
    const __amdgpu_buffer_rsrc_t frs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(P.x), 0, M * K * 4, kBufferDword3);
    const __amdgpu_buffer_rsrc_t urs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(P.up), 0, glue ? M * K * 4 : 0, kBufferDword3);
    const __amdgpu_buffer_rsrc_t nrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(P.norm_w), 0, nwb, kBufferDword3);
    const int ux = (M * K * 4 + 1023) >> 10, uu = glue ? ux : 0, un = (nwb + 1023) >> 10;
    for (int i = wave; i < ux + uu + un; i += 4) {
      const int part = i < ux ? 0 : (i < ux + uu ? 1 : 2);
      const int u = i - (part == 0 ? 0 : (part == 1 ? ux : ux + uu));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          part == 0 ? frs : (part == 1 ? urs : nrs),
          (__attribute__((address_space(3))) void*)(xlds + (part == 0 ? fl.x : (part == 1 ? fl.up : fl.nw)) +
                                                     1024 * u),
          16, 1024 * u + 16 * lane, 0, 0, 0);
    }
  } else if (FROM_LDS) {
    const int row_slots = kpad >> 4;
    const int lds_units = (M * kpad + 1023) >> 10;
    for (int i = wave; i < lds_units; i += 4) {
      const int ps = 64 * i + lane;  // physical 16-byte slot
      const int m = ps / row_slots;
      const int slot = (ps - m * row_slots) ^ (m & 7);
      const bool ok = (m < M) & (16 * slot < K);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrs, (__attribute__((address_space(3))) void*)(xlds + 1024 * i), 16,
          ok ? m * K + 16 * slot : kOob, 0, 0, 0);
    }
  }
  int rs = 0;
  float scale = 0.f;
  if (!FUSED) {
    rs = gptr<int32_t>(P.rowsum)[xrow];
    scale = RAW ? 0.f : gptr<float>(P.factor)[xrow] / P.w_scale;
  }
  asm volatile("" ::: "memory");  // keep the loads above ahead of the weight loads

  // Weight loads: lane reads 16 bytes of row tile0 + 64t + r16 at superblock sb.
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(P.w), 0, N * rowbytes, kBufferDword3);
  const int tile0 = (unit * 4 * tpu + wave) * 16;
  // Offsets in unsigned arithmetic: rows past N (up to 511 of them) would
  // overflow a signed product near the 2^31 offset limit; their loads are
  // replaced by kOob anyway, and an in-range offset is below 2^31.
  const uint32_t wbase = static_cast<uint32_t>(tile0 + r16) * static_cast<uint32_t>(rowbytes) + 16u * g;
  auto wload = [&](int t, int sb) -> v4i {
    const bool ok = (t < tpu) & (tile0 + 64 * t + r16 < N) & (sb < nsb) & (64 * sb + 16 * g < rowbytes);
    const uint32_t off = wbase + static_cast<uint32_t>(64 * t) * static_cast<uint32_t>(rowbytes) + 64u * sb;
    return __builtin_amdgcn_raw_buffer_load_b128(wrs, ok ? static_cast<int>(off) : kOob, 0, 0);
  };
  v4i buf[D][kHeld];
#pragma unroll
  for (int d = 0; d < D; ++d)
#pragma unroll
    for (int sb = 0; sb < kHeld; ++sb) buf[d][sb] = wload(d, sb);

  if (FROM_LDS) {
    // The staging loads are complete once at most the weight loads are
    // outstanding; the barrier then publishes every wave's part.
    wait_vmcnt<kInFlight>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  if (FUSED) {
    // RMSNorm + absmax int8 quantization of the <= 16 rows while the weight
    // loads are in flight, spread over all four waves: unit i = (row m,
    // chunk column j) covers chunks c = lane + 64j of row m, and wave w takes
    // units w, w+4, ...  Pass 1 (glue first, when set) leaves each lane's
    // sum of squares of its chunk and the unit's absmax in LDS; after a
    // barrier, row m's factor is formed by wave m % 4 with the quantization
    // kernel's order of operations (the lane's squares added in chunk order,
    // then a double reduction), so factors and codes are bit-identical to
    // it; pass 2 writes the codes to the staged layout (zeros up to the
    // padded length) and the unit's code sum to the table.
    const int nch = K >> 2;
    const int units = M * NSB;
    f4* xf = reinterpret_cast<f4*>(xlds + fl.x);
    const f4* nw = reinterpret_cast<const f4*>(xlds + fl.nw);
    const bool norm = P.norm_w != nullptr;  // else u = x, r = 1
    const bool nwh = P.nw_f16 != 0;
    // chunk c of the norm weight, widened from float16 when stored so
    auto nwc = [&](int c) { return nwh ? half4(reinterpret_cast<const u2*>(xlds + fl.nw)[c]) : nw[c]; };
    float* row_scale = reinterpret_cast<float*>(xlds + fl.tab);
    float* unit_max = reinterpret_cast<float*>(xlds + fl.tab + 64);
    int* unit_sum = reinterpret_cast<int*>(xlds + fl.tab + 64 + 4 * units);
    float* sq = reinterpret_cast<float*>(xlds + fl.sq);
    for (int i = wave; i < units; i += 4) {
      const int m = i / NSB, c = lane + kWave * (i - m * NSB);
      float s2 = 0.f, a = 0.f;
      if (c < nch) {
        f4 xv = xf[m * nch + c];
        if (GLUE) {
          // FFN glue in place: act(gate) * up with the quantization kernel's
          // per-element arithmetic (glu4).
          const f4 uv = reinterpret_cast<const f4*>(xlds + fl.up)[m * nch + c];
          xv = P.act == kActSilu ? glu4<kActSilu>(xv, uv) : glu4<kActGeluTanh>(xv, uv);
          xf[m * nch + c] = xv;
        }
        s2 = sq4(xv);
        a = absmax4(norm ? xv * nwc(c) : xv);
      }
      sq[i * kWave + lane] = s2;
      a = wave_max(a);
      if (lane == 0) unit_max[i] = a;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    auto row_max = [&](int m) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < NSB; ++j) a = fmaxf(a, unit_max[m * NSB + j]);
      return a;
    };
    for (int m = wave; m < M; m += 4) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < NSB; ++j) ss += sq[(m * NSB + j) * kWave + lane];
      const double ssd = wave_sum(static_cast<double>(ss));
      const float amax = row_max(m);
      if (lane == 0) row_scale[m] = quant_factor(ssd, K, P.eps, amax, norm) / P.w_scale;
    }
    for (int i = wave; i < units; i += 4) {
      const int m = i / NSB, c = lane + kWave * (i - m * NSB);  // dword c of the padded row
      const float amax = row_max(m);
      int sum = 0;
      uint32_t q = 0u;
      if (c < nch) {
        const f4 xv = xf[m * nch + c];
        q = codes4(norm ? xv * nwc(c) : xv, amax, &sum);
      }
      *reinterpret_cast<uint32_t*>(xlds + m * kpad + ((((c >> 2) ^ (m & 7))) << 4) + ((c & 3) << 2)) = q;
      sum = wave_sum(sum);
      if (lane == 0) unit_sum[i] = sum;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    rs = 0;
#pragma unroll
    for (int j = 0; j < NSB; ++j) rs += unit_sum[xrow * NSB + j];
    scale = row_scale[xrow];
  }

  // Activation fragment (B operand): 16 bytes of row xrow at K offset
  // 256*sb + 32*f + koff, i.e. logical slot 16*sb + 8*(g/2) + 2*f + g%2.
  const int koff = 128 * (g >> 1) + 16 * (g & 1);
  const int8_t* xl = xlds + xrow * kpad + 128 * (g >> 1);
  const int xsw = xrow & 7;
  auto xfrag = [&](int sb, int f) -> v4i {
    if (FROM_LDS)
      return *reinterpret_cast<const v4i*>(xl + 256 * sb + 16 * ((2 * f + (g & 1)) ^ xsw));
    const int k = 256 * sb + 32 * f;
    const bool ok = (r16 < M) & (k + koff < K);
    return __builtin_amdgcn_raw_buffer_load_b128(xrs, ok ? r16 * K + koff + k : kOob, 0, 0);
  };

  auto process = [&](v4i* acc, const v4i& wv, int sb) {
    v4i a0, a1, a2, a3;
    decode_fields(wv, a0, a1, a2, a3);
    acc[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, xfrag(sb, 0), acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, xfrag(sb, 1), acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, xfrag(sb, 2), acc[2], 0, 0, 0);
    acc[3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, xfrag(sb, 3), acc[3], 0, 0, 0);
  };

  // Activation sum over the field-0 positions of row r16, by the idle matrix
  // core (an all-ones A operand): rs123 = row sum - that is the sum over the
  // field 1..3 positions, whose codes the epilogue turns into weights.
  int rs123;
  {
    const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
    v4i s0 = v4i{0, 0, 0, 0};
    for (int sb = 0; sb < nsb; ++sb)
      s0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, xfrag(sb, 0), s0, 0, 0, 0);
    rs123 = rs - s0[0];
  }

  if (NSB > 0) {
    // A rolling window of D tiles: tile t is processed while t+1..t+D-1
    // load, then its buffer is refilled with tile t+D.  Past the wave's last
    // row the loads read 0 and nothing is stored.  Tile t's accumulators are
    // combined one tile later, when its MFMAs have drained, and results are
    // held in registers until the end: a store counts against vmcnt like a
    // load, so waits on later weight loads would also wait for it.
    v4i acc[2][4];
    v4i res[T];
    auto finish = [&](int t) {
      v4i r = gemv_result<RAW>(acc[t & 1], rs123, scale);
      asm volatile("" : "+v"(r));  // combine here: frees the accumulators for tile t + 2
      res[t] = r;
    };
#pragma unroll
    for (int t = 0; t < T; ++t) {
      // The activation fragments are re-read from LDS for every tile rather
      // than held in registers: registers are worth more as load buffers.
      // Tiles from tpu on hold no rows: their products are skipped (a
      // uniform branch; the merged launch has tpu == T and none).
      asm volatile("" ::: "memory");
      if (t < tpu) {
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[t & 1][f] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int sb = 0; sb < kHeld; ++sb) process(acc[t & 1], buf[t % D][sb], sb);
      }
      if (t + D < T) {
#pragma unroll
        for (int sb = 0; sb < kHeld; ++sb) buf[t % D][sb] = wload(t + D, sb);
      }
      if (t > 0 && t - 1 < tpu) finish(t - 1);
    }
    if (T - 1 < tpu) finish(T - 1);
    // Fused: the fp32 rows and the norm weight are dead since the
    // quantization barrier, so the workgroup's results are gathered there
    // (row m of the workgroup's 64*T output columns at m*64*T) and written
    // as whole 16-byte chunks by consecutive lanes: at M = 1 two full-wave
    // stores instead of one four-lane store per tile and wave.
    const int span = 64 * T;
    if (FUSED && M * span * 4 <= fl.bytes - fl.x) {
      // (rows of the tiles past tpu are gathered but not written)
      int32_t* ol = reinterpret_cast<int32_t*>(xlds + fl.x);
      if (r16 < M) {
#pragma unroll
        for (int t = 0; t < T; ++t)
          *reinterpret_cast<v4i*>(ol + r16 * span + 64 * t + 16 * wave + 4 * g) = res[t];
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int base = unit * 64 * tpu;
      const int q = 16 * tpu;  // 16-byte chunks per output row
      for (int c = threadIdx.x; c < M * q; c += 256) {
        const int m = c / q, j = c - m * q;
        gemv_store<RAW>(P, *reinterpret_cast<const v4i*>(ol + m * span + 4 * j), base + 4 * j, m);
      }
    } else {
#pragma unroll
      for (int t = 0; t < T; ++t)
        if (t < tpu) gemv_store<RAW>(P, res[t], tile0 + 64 * t + 4 * g, r16);
    }
  } else {
    // Generic K, one tile: two superblocks in flight, pairs processed
    // unconditionally (past nsb both operands are zero: loads read 0,
    // staging is padded).
    v4i acc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[f] = v4i{0, 0, 0, 0};
    v4i* w = buf[0];
    for (int sb = 0; sb < nsb; sb += 2) {
      process(acc, w[0], sb);
      w[0] = wload(0, sb + 2);
      process(acc, w[1], sb + 1);
      w[1] = wload(0, sb + 3);
    }
    gemv_store<RAW>(P, gemv_result<RAW>(acc, rs123, scale), tile0 + 4 * g, r16);
  }
}

// SINGLE: the launch covers the by-value problem `single`, `tiles` 16-row
// tiles per wave (1..T).  Else the FatUnit table `units`, the full T tiles
// per wave (a compile-time count: no tile branches).
template <bool RAW, bool FROM_LDS, int NSB, bool FUSED, bool GLUE, bool SINGLE>
__global__ __launch_bounds__(256) void gemv_kernel(Prob single, const FatUnit* units, int tiles) {
  constexpr int T = gemv_tiles(NSB);
  if (SINGLE) {
    gemv_body<RAW, FROM_LDS, NSB, FUSED, GLUE>(single, blockIdx.x, tiles > 0 && tiles < T ? tiles : T);
  } else {
    int unit;
    const Prob P = fat_unit_at(units, blockIdx.x, &unit);
    gemv_body<RAW, FROM_LDS, NSB, FUSED, GLUE>(P, unit, T);
  }
}

// Fused decode units of several superblock counts (1..kGemvMergedMaxNsb) in
// one launch: each workgroup runs the body specialised for its unit's count.
// The table lists the units with the most superblocks first, so the longest
// workgroups start first and the many short ones fill the end of the launch
// instead of each bucket's last round idling the GPU.
__global__ __launch_bounds__(256) void gemv_fused_merged_kernel(const FatUnit* units) {
  int unit, nsb;
  const Prob P = fat_unit_at(units, blockIdx.x, &unit, &nsb);
  switch (nsb) {
#define BL_MERGED_CASE(n) \
  case n: gemv_body<false, true, n, true>(P, unit, gemv_tiles(n)); break;
    BL_MERGED_CASE(1) BL_MERGED_CASE(2) BL_MERGED_CASE(3) BL_MERGED_CASE(4)
    BL_MERGED_CASE(5) BL_MERGED_CASE(6) BL_MERGED_CASE(7) BL_MERGED_CASE(8)
    BL_MERGED_CASE(9) BL_MERGED_CASE(10) BL_MERGED_CASE(11) BL_MERGED_CASE(12)
#undef BL_MERGED_CASE
    default: break;
  }
  static_assert(kGemvMergedMaxNsb == 12, "cases above");
}

int gemv_bucket(int K) {
  const int nsb = (K + 255) >> 8;
  return nsb <= kMaxNsb ? nsb : 0;
}

int gemv_units(int N, int bucket, int tiles) {
  const int T = gemv_tiles(bucket);
  const int rows = 64 * (tiles > 0 && tiles < T ? tiles : T);
  return (N + rows - 1) / rows;
}

int gemv_single_tiles(int N, int bucket) {
  // Fewest tiles per wave that still give about two workgroups per CU.
  const int T = gemv_tiles(bucket);
  const int want = (N + 64 * kGemvSingleUnits - 1) / (64 * kGemvSingleUnits);
  return want < 1 ? 1 : (want > T ? T : want);
}

namespace {

// Staged activation bytes of a launch: max_m rows of the bucket's
// superblocks (for the generic variant the largest K rounded up to a pair of
// superblocks), rounded up to the 1 KB granule of the direct LDS loads.
size_t gemv_lds_bytes(int bucket, int max_m, int max_k) {
  int nsb = bucket > 0 ? bucket : (max_k + 255) >> 8;
  if (bucket == 0) nsb = (nsb + 1) & ~1;
  const size_t bytes = static_cast<size_t>(max_m) * static_cast<size_t>(nsb) * 256;
  return (bytes + 1023) / 1024 * 1024;
}

template <bool RAW, bool LDS, bool FUSED, bool GLUE, bool SINGLE>
hipError_t launch_bucket(const GemvLaunch& L, int bucket, size_t shmem, hipStream_t stream) {
  const dim3 grid(L.total), block(256);
#define BL_GEMV_CASE(n)                                                                           \
  case n:                                                                                         \
    hipLaunchKernelGGL((gemv_kernel<RAW, LDS, n, FUSED, GLUE, SINGLE>), grid, block, shmem,       \
                       stream, L.single, L.units, L.tiles);                                       \
    break;
  switch (bucket) {
    BL_GEMV_CASE(1) BL_GEMV_CASE(2) BL_GEMV_CASE(3) BL_GEMV_CASE(4) BL_GEMV_CASE(5)
    BL_GEMV_CASE(6) BL_GEMV_CASE(7) BL_GEMV_CASE(8) BL_GEMV_CASE(9) BL_GEMV_CASE(10)
    BL_GEMV_CASE(11) BL_GEMV_CASE(12) BL_GEMV_CASE(13) BL_GEMV_CASE(14) BL_GEMV_CASE(15)
    BL_GEMV_CASE(16)
    default:
      if constexpr (!FUSED)
        hipLaunchKernelGGL((gemv_kernel<RAW, LDS, 0, false, false, SINGLE>), grid, block, shmem,
                           stream, L.single, L.units, 0);
      else
        return hipErrorInvalidValue;
  }
#undef BL_GEMV_CASE
  return hipGetLastError();
}

}  // namespace

bool gemv_fusable(int M, int K, bool glue, bool table) {
  const int b = gemv_bucket(K);
  const int budget = glue ? kGemvGlueLdsBytes : (table ? kGemvTableLdsBytes : kGemvFusedLdsBytes);
  return M >= 1 && M <= kGemvMaxM && b > 0 && fused_lds(M, K, b, glue).bytes <= budget;
}

size_t gemv_fused_lds_bytes(int M, int K, bool glue) {
  return static_cast<size_t>(fused_lds(M, K, gemv_bucket(K), glue).bytes);
}

hipError_t launch_gemv_merged(const FatUnit* units, int total, size_t shmem, hipStream_t stream) {
  if (total <= 0) return hipSuccess;
  if (shmem == 0 || shmem > static_cast<size_t>(kGemvTableLdsBytes)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemv_fused_merged_kernel, dim3(total), dim3(256), shmem, stream, units);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvLaunch& L, bool raw, int bucket, int max_m, int max_k,
                       bool fused, hipStream_t stream, bool glue) {
  if (L.total <= 0) return hipSuccess;
  const bool single = L.units == nullptr;
  // Tables (groups) carry forward problems only; the glue is fused only.
  if ((!single && raw) || (glue && !fused)) return hipErrorInvalidValue;
  if (fused) {
    if (raw || bucket <= 0) return hipErrorInvalidValue;
    const size_t shmem = L.fused_shmem ? L.fused_shmem : fused_lds(max_m, max_k, bucket, glue).bytes;
    if (shmem > static_cast<size_t>(kGemvGlueLdsBytes)) return hipErrorInvalidValue;
    if (glue)
      return single ? launch_bucket<false, true, true, true, true>(L, bucket, shmem, stream)
                    : launch_bucket<false, true, true, true, false>(L, bucket, shmem, stream);
    return single ? launch_bucket<false, true, true, false, true>(L, bucket, shmem, stream)
                  : launch_bucket<false, true, true, false, false>(L, bucket, shmem, stream);
  }
  const size_t shmem = gemv_lds_bytes(bucket, max_m, max_k);
  const bool lds = shmem <= static_cast<size_t>(kGemvLdsBytes);
  if (raw) {
    return lds ? launch_bucket<true, true, false, false, true>(L, bucket, shmem, stream)
               : launch_bucket<true, false, false, false, true>(L, bucket, 0, stream);
  }
  if (single)
    return lds ? launch_bucket<false, true, false, false, true>(L, bucket, shmem, stream)
               : launch_bucket<false, false, false, false, true>(L, bucket, 0, stream);
  return lds ? launch_bucket<false, true, false, false, false>(L, bucket, shmem, stream)
             : launch_bucket<false, false, false, false, false>(L, bucket, 0, stream);
}

}  // namespace bl
