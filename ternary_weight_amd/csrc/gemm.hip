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
// ring filled by direct global-to-LDS loads (global_load_lds_dwordx4), so no
// VGPRs stage the copies.  Weights are expanded to int8 right before the
// MFMA (shift + mask per dword).
//
// Software pipeline.  The loads of stage s are issued in the middle of stage
// s - 3 and awaited in the middle of stage s - 1 (two stages of compute cover
// their latency).  The middle of a stage is the one synchronisation point:
// after the k-step 2 MFMAs every wave waits for its LDS reads and its loads
// of the next stage, a barrier makes all loads visible, the slot just read
// is refilled, and the next stage's packed weights and first activation
// fragments are read while the k-step 3 MFMAs run.  Activation fragments
// are read two k-steps ahead, in the middle of a k-step's MFMAs, so every
// wait for LDS data finds it already returned.
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
// for them before LDS reads, so the loop waits explicitly (vmcnt counts the
// loads of the stages still allowed in flight); scheduling barriers keep the
// LDS reads, waits and MFMAs in the order above.
//
// K split (grouped launches whose tiles all fit on the CUs at once, for
// example one layer at a few hundred tokens): such a launch lasts as long as
// its longest-K tile, while most CUs idle, so the host planner gives the
// longest problems several workgroups per output tile, each over a
// contiguous share of the K blocks.  Each split leaves its int32 partial tile
// in the workspace, and the last to arrive (a per-tile count) adds the others
// and runs the epilogue: no workgroup ever waits for another.
//
// Epilogue: full output tiles store through a buffer resource at the tile's
// corner (three VALU operations and one store per element); ragged tiles use
// a bounds-checked path.
//
// Successor prefetch.  A tile's activation rows are first read from HBM by
// its own direct loads, which then wait behind the output stores that the
// other workgroups keep the memory system busy with.  So each workgroup, at
// the start of its epilogue, touches a share of the activation rows of the
// tile that will most likely take its slot next (workgroup id + 512: two
// workgroups per CU on 256 CUs, and the ids dealt to the 8 XCDs in turn keep
// it on this XCD), so that those rows are in the XCD's L2 when that tile
// starts.  The touches are direct loads into an idle part of the ring.
//
// Producer quantization (the PQ instance, one problem per launch): the
// activation side loads fp32 rows and codes them itself instead of loading
// int8 codes, see gemm_kernel.
//
// Bound: int8 MFMA for K >= 2048; for K <= 1024 the fp32 output (4*M*N bytes)
// weighs as much as the MFMA time.
#include <type_traits>

#include "kernels.hpp"

namespace bl {

constexpr int kTileN = 256;   // weight rows per workgroup
constexpr int kTileM = 128;   // activation rows per workgroup
constexpr int kBlockK = 128;  // K positions per stage (one I2_S block)
constexpr int kStages = 3;
// Widest output for the unchecked full-tile stores: a tile's 128 rows of N
// floats then span less than 2^31 bytes of 32-bit buffer offsets.
constexpr int kGemmFullTileMaxN = 1 << 22;
constexpr int kXStage = kTileM * kBlockK;        // 16 KB
constexpr int kWStage = kTileN * (kBlockK / 4);  // 8 KB
constexpr int kStageBytes = kXStage + kWStage;
// Direct loads per wave per stage: (16 KB + 8 KB) / 4 waves / 1 KB.
constexpr int kXLoads = kXStage / 4 / 1024;  // 4
constexpr int kWLoads = kWStage / 4 / 1024;  // 2
constexpr int kLoadsPerStage = kXLoads + kWLoads;
// Successor prefetch: the workgroup that most likely follows on this slot,
// and how many leading K blocks of its activation rows are touched in all.
constexpr int kSlotsAhead = 512;
constexpr int kPrefetchBlocks = 16;

typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v2i __attribute__((ext_vector_type(2)));

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
// The same with lgkmcnt = 0: this wave's LDS reads have returned as well.
template <int N>
__device__ __forceinline__ void wait_lgkm0_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

__device__ __forceinline__ void dma16(const void* gsrc, uint8_t* ldst) {
  __builtin_amdgcn_global_load_lds((const BL_GLOBAL void*)gsrc,
                                   (__attribute__((address_space(3))) void*)ldst, 16, 0, 0);
}

// SPLIT: the launch holds problems with K splits (the split bookkeeping is
// compiled only into this instance; launches without splits keep the plain
// kernel's registers).
//
// PQ: one problem whose activation producer quantizes (the pages' norm,
// multiply and quantization ops, "BitNet Embeddings GGUF Conversion
// Implementation" s4.5, folded into the product's producer): instead of
// direct loads of int8 codes, each thread loads fp32 rows of the stage into
// registers two stages ahead (lane l of wave w: 16-byte chunk c = l % 32 of
// rows 32w + 2i + l/32, i = 0..15, so each instruction reads two rows' 512
// bytes), multiplies by the norm weight chunk, and codes them with the
// quantization kernel's arithmetic (codes4) against the row's max|u| from the
// statistics pass, writing the codes into the same swizzled LDS slots the
// direct loads fill.  Codes, accumulators and outputs are therefore those of
// the quantization launch + plain kernel, bit for bit.  The two register sets
// of 64 values per thread need one workgroup per CU.
template <bool RAW, bool SPLIT, bool PQ = false>
__global__ __launch_bounds__(256, PQ ? 1 : 2) void gemm_kernel(ProbSet set) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];

  const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
  const int wn = wave & 1, wm = wave >> 1;
  const int r32 = lane & 31, g = lane >> 5;

  int local;
  const Prob P = prob_at(set, find_prob(set, xcd_remap(blockIdx.x, set.total), &local));
  const int M = P.M, K = P.K, N = P.N;
  const int rowbytes = K >> 2;
  const int tiles_n = (N + kTileN - 1) / kTileN;
  // K split: unit `local` is split `split` of output tile `tile` and takes
  // the tile's K blocks [kb0, kb0 + nblk).
  const int ks = SPLIT && P.ksplit > 1 ? P.ksplit : 1;
  const int tile = local / ks, split = local - tile * ks;
  const int m0 = (tile / tiles_n) * kTileM;
  const int n0 = (tile % tiles_n) * kTileN;
  const int kb0 = (K / kBlockK) * split / ks;
  const int nblk = (K / kBlockK) * (split + 1) / ks - kb0;

  // The successor tile's activation rows [pf_m, pf_m + 128) and the K blocks
  // [pf_b0, pf_b1) this workgroup touches for it.  The successors of one row
  // block are its consecutive column tiles: successor n of the row block
  // takes the n-th share of its first kPrefetchBlocks blocks, so each line is
  // requested once.  Scalar loads, issued here so their latency is long over
  // by the epilogue.
  const int8_t* pf_x = nullptr;
  int pf_k = 0, pf_m = 0, pf_mlast = 0, pf_b0 = 0, pf_b1 = 0;
  if constexpr (!PQ) {
    const int b2 = blockIdx.x + kSlotsAhead;
    if (b2 < set.total) {
      int local2;
      const Prob P2 = prob_at(set, find_prob(set, xcd_remap(b2, set.total), &local2));
      const int ks2 = SPLIT && P2.ksplit > 1 ? P2.ksplit : 1;
      const int tn2 = (P2.N + kTileN - 1) / kTileN;
      const int tile2 = local2 / ks2;
      const int nb = min(kPrefetchBlocks, P2.K / kBlockK);
      const int n2 = tile2 % tn2, parts = min(tn2, nb);
      if (local2 % ks2 == 0 && n2 < parts) {
        pf_x = P2.xq;
        pf_k = P2.K;
        pf_m = (tile2 / tn2) * kTileM;
        pf_mlast = P2.M - 1;
        pf_b0 = nb * n2 / parts;
        pf_b1 = nb * (n2 + 1) / parts;
      }
    }
  }

  // This lane's direct-load sources (32-bit offsets from the problem's
  // bases): for activation instruction i the lane fills LDS row
  // 32*wave + 8*i + lane/8, physical slot lane%8; for weight instruction i,
  // row 64*wave + 32*i + lane/2, physical slot lane%2.
  int xoff[kXLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int row = 32 * wave + 8 * i + (lane >> 3);
    const int slot = xs_slot(row, lane & 7);
    xoff[i] = min(m0 + row, M - 1) * K + kb0 * kBlockK + slot * 16;
  }
  int woff[kWLoads];
#pragma unroll
  for (int i = 0; i < kWLoads; ++i) {
    const int row = 64 * wave + 32 * i + (lane >> 1);
    const int slot = ws_slot(row, lane & 1);
    woff[i] = min(n0 + row, N - 1) * rowbytes + kb0 * (kBlockK / 4) + slot * 16;
  }
  auto issue = [&](int kb, int slot_off) {
    uint8_t* st = smem + slot_off;
    if constexpr (!PQ) {
#pragma unroll
      for (int i = 0; i < kXLoads; ++i)
        dma16(P.xq + xoff[i] + kb * kBlockK, st + (kXLoads * wave + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < kWLoads; ++i)
      dma16(P.w + woff[i] + kb * (kBlockK / 4), st + kXStage + (kWLoads * wave + i) * 1024);
  };
  // Loads per stage counted by vmcnt: the direct loads, and for PQ the 16
  // activation chunks and one norm-weight chunk per thread instead of the
  // activation direct loads.
  constexpr int kPqRows = 16;
  constexpr int kLps = PQ ? kWLoads + kPqRows + 1 : kLoadsPerStage;

  // PQ producer state: this thread's rows, their max|u| and byte offsets in
  // x (stage kb adds 512*kb), two register sets of loaded fp32 chunks and
  // norm-weight chunks (a binary16 chunk in the low 8 bytes).
  const int pc = lane & 31;  // 16-byte chunk of the stage's 128 positions
  int xro[PQ ? kPqRows : 1];
  float ramax[PQ ? kPqRows : 1];
  v4i xs[PQ ? 2 : 1][PQ ? kPqRows : 1];
  v4i nwraw[PQ ? 2 : 1];
  const __amdgpu_buffer_rsrc_t xrs32 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(P.x), 0, PQ ? M * K * 4 : 0, kBufferDword3);
  const __amdgpu_buffer_rsrc_t nrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(P.norm_w), 0, PQ && P.norm_w ? K * (P.nw_f16 ? 2 : 4) : 0, kBufferDword3);
  if constexpr (PQ) {
#pragma unroll
    for (int i = 0; i < kPqRows; ++i) {
      const int m = min(m0 + 32 * wave + 2 * i + (lane >> 5), M - 1);
      xro[i] = m * K * 4 + pc * 16;
      ramax[i] = gptr<float>(P.amax)[m];
    }
  }
  auto load_x32 = [&](int kb, auto set_c) {
    constexpr int q = decltype(set_c)::value;
#pragma unroll
    for (int i = 0; i < kPqRows; ++i)
      xs[q][i] = __builtin_amdgcn_raw_buffer_load_b128(xrs32, xro[i], __builtin_amdgcn_readfirstlane(kb * 512), 0);
    if (P.nw_f16) {
      const v2i h = __builtin_amdgcn_raw_buffer_load_b64(nrs, pc * 8, __builtin_amdgcn_readfirstlane(kb * 256), 0);
      nwraw[q] = v4i{h[0], h[1], 0, 0};
    } else {
      nwraw[q] = __builtin_amdgcn_raw_buffer_load_b128(nrs, pc * 16, __builtin_amdgcn_readfirstlane(kb * 512), 0);
    }
  };
  // Codes of the stage held in register set q, written to the ring slot at
  // slot_off: chunk pc of row r at physical slot xs_slot(r, pc / 4).
  auto code_x = [&](auto set_c, int slot_off) {
    constexpr int q = decltype(set_c)::value;
    const f4 nwv = P.nw_f16 ? half4(u2{static_cast<uint32_t>(nwraw[q][0]), static_cast<uint32_t>(nwraw[q][1])})
                            : __builtin_bit_cast(f4, nwraw[q]);
    const bool norm = P.norm_w != nullptr;
#pragma unroll
    for (int i = 0; i < kPqRows; ++i) {
      const int r = 32 * wave + 2 * i + (lane >> 5);
      const f4 xv = __builtin_bit_cast(f4, xs[q][i]);
      int sum = 0;
      const uint32_t code = codes4(norm ? xv * nwv : xv, ramax[i], &sum);
      *reinterpret_cast<uint32_t*>(smem + slot_off + r * kBlockK + xs_slot(r, pc >> 2) * 16 + (pc & 3) * 4) = code;
    }
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;

  v16i acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = v16i{};

  // LDS byte offsets of this lane's fragments inside a stage.
  int xrd[4][2];  // [k-step j][fm]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int fm = 0; fm < 2; ++fm) {
      const int row = wm * 64 + fm * 32 + r32;
      xrd[j][fm] = row * kBlockK + xs_slot(row, 2 * j + g) * 16;
    }
  int wrd[4];
#pragma unroll
  for (int fn = 0; fn < 4; ++fn) {
    const int row = wn * 128 + fn * 32 + r32;
    wrd[fn] = kXStage + row * 32 + ws_slot(row, g) * 16;
  }
  auto read_w = [&](v4i (&w)[4], const uint8_t* st) {
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) w[fn] = *reinterpret_cast<const v4i*>(st + wrd[fn]);
  };
  auto read_x = [&](v4i (&bx)[2], const uint8_t* st, int j) {
#pragma unroll
    for (int fm = 0; fm < 2; ++fm) bx[fm] = *reinterpret_cast<const v4i*>(st + xrd[j][fm]);
  };
  // Part of one k-step: field j of the packed weights of fragments
  // fn0..fn1-1 against activation fragments bx.
  auto mma_step = [&](const v4i (&w)[4], const v4i (&bx)[2], int j, int fn0, int fn1) {
#pragma unroll
    for (int fn = fn0; fn < fn1; ++fn) {
      v4i a;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = field_codes(static_cast<uint32_t>(w[fn][i]), j);
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
        acc[fn][fm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bx[fm], a, acc[fn][fm], 0, 0, 0);
    }
  };
  // All waves' direct loads visible, and every wave past its reads so far.
  // Compiler-only fences keep LDS accesses and direct loads on their side.
  auto block_sync = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Software pipeline.  Stage s lives in ring slot s % 3; its direct loads
  // are issued in the middle of stage s - 3 (into the slot stage s - 3 has
  // just finished reading) and awaited in the middle of stage s - 1, so two
  // stages of compute cover the load latency.  In the middle of stage kb,
  // after the k-step 2 MFMAs are issued: wait for this wave's LDS reads and
  // for stage kb + 1's loads, barrier, refill this slot with stage kb + 3,
  // and read stage kb + 1's packed weights and first activation fragments
  // into the other register set while the k-step 3 MFMAs run.
  if constexpr (PQ) {
    // Stages 0 and 1 load into register sets 0 and 1; stage 0 is coded into
    // its slot before stage 2 loads into set 0.
    issue(0, 0);
    load_x32(0, Set0{});
    if (nblk > 1) {
      issue(1, kStageBytes);
      load_x32(1, Set1{});
      wait_vmcnt<kLps>();
    } else {
      wait_vmcnt<0>();
    }
    code_x(Set0{}, 0);
    if (nblk > 2) {
      issue(2, 2 * kStageBytes);
      load_x32(2, Set0{});
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    block_sync();
  } else {
    issue(0, 0);
    if (nblk > 1) issue(1, kStageBytes);
    if (nblk > 2) issue(2, 2 * kStageBytes);
    if (nblk > 2) wait_vmcnt<2 * kLoadsPerStage>();
    else if (nblk > 1) wait_vmcnt<kLoadsPerStage>();
    else wait_vmcnt<0>();
    block_sync();
  }

  v4i wp[4];     // packed weight half-rows of the current stage
  v4i bx[4][2];  // activation fragments of k-steps 0..3
  read_w(wp, smem);
  read_x(bx[0], smem, 0);
  read_x(bx[1], smem, 1);
  int slot = 0;  // byte offset of the current stage's ring slot

  // One stage.  Activation fragments are read two k-steps ahead, in the
  // middle of a k-step's MFMAs (so that any wait for the older reads never
  // waits for them).  MID: a later stage exists and the middle-of-stage
  // hand-over runs: the k-step 3 operands are decoded first, which frees the
  // packed weight registers for the next stage's reads.
  auto stage = [&](auto mid, auto set_c, int kb) {
    constexpr bool kMid = decltype(mid)::value;
    const uint8_t* st = smem + slot;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      mma_step(wp, bx[j], j, 0, 2);
      __builtin_amdgcn_sched_barrier(0);
      read_x(bx[j + 2], st, j + 2);
      __builtin_amdgcn_sched_barrier(0);
      mma_step(wp, bx[j], j, 2, 4);
      __builtin_amdgcn_sched_barrier(0);
    }
    mma_step(wp, bx[2], 2, 0, 4);
    __builtin_amdgcn_sched_barrier(0);
    if (kMid) {
      // Decode the k-step 3 operands now (pinned here, ahead of the waits).
      v4i a3[4];
#pragma unroll
      for (int fn = 0; fn < 4; ++fn) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a3[fn][i] = field_codes(static_cast<uint32_t>(wp[fn][i]), 3);
        asm volatile("" : "+v"(a3[fn]));
      }
      if (kb + 2 < nblk) wait_lgkm0_vmcnt<kLps>();
      else wait_lgkm0_vmcnt<0>();
      const int next = slot == 2 * kStageBytes ? 0 : slot + kStageBytes;
      if constexpr (PQ) {
        // stage kb + 1's codes (its fp32 chunks are in set (kb + 1) & 1),
        // written before the barrier that publishes the stage
        code_x(set_c, next);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
      block_sync();
      read_w(wp, smem + next);
      read_x(bx[0], smem + next, 0);
      read_x(bx[1], smem + next, 1);
      if (kb + 3 < nblk) {
        issue(kb + 3, slot);
        if constexpr (PQ) load_x32(kb + 3, set_c);  // (kb + 3) & 1 == (kb + 1) & 1
      }
      slot = next;
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
          acc[fn][fm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bx[3][fm], a3[fn], acc[fn][fm], 0, 0, 0);
    } else {
      mma_step(wp, bx[3], 3, 0, 4);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  int kb = 0;
  if constexpr (PQ) {
    // Unrolled by two so that each stage's register set is a compile-time
    // index: stage kb codes set (kb + 1) & 1.
    for (; kb + 2 < nblk; kb += 2) {
      stage(Yes{}, Set1{}, kb);
      stage(Yes{}, Set0{}, kb + 1);
    }
    if (kb + 1 < nblk) {
      stage(Yes{}, Set1{}, kb);
      stage(No{}, Set0{}, kb + 1);
    } else {
      stage(No{}, Set1{}, kb);
    }
  } else {
    for (; kb + 1 < nblk; ++kb) stage(Yes{}, Set0{}, kb);
    stage(No{}, Set0{}, kb);
  }

  if (SPLIT && ks > 1) {
    // Split tiles.  Each split stores its accumulators, counts itself in,
    // and the last split to arrive adds the others' partials in its
    // registers, resets the count and runs the epilogue; int32 sums are
    // exact in any order, so the result equals the unsplit product bit for
    // bit.  The splits may run on different XCDs, each with its own L2, so
    // the partials are written and read with the sc1 cache policy (the one
    // the compiler gives agent-scope atomic accesses: coherent across the
    // XCDs), and every wave's stores have completed (vmcnt 0, then the
    // barrier) before the count is raised.  A device-scope fence instead
    // would write back and invalidate the whole L2 of the XCD, the other
    // workgroups' cached operands included (measured: the launch took 50%
    // longer than unsplit).  Layout: 16-byte piece p of lane l of wave w of
    // split s at ((s*4 + w)*32 + p)*64 + l within the tile's partials, so
    // each store instruction writes 1 KB contiguously.
    constexpr int kSc1 = 16;  // cache policy bits: sc1
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        P.part + static_cast<int64_t>(tile) * ks * kGemmPartInts, 0, ks * kGemmPartInts * 4, kBufferDword3);
    auto poff = [&](int s, int p) { return (s * (kGemmPartInts / 4) + (wave * 32 + p) * 64 + lane) * 16; };
#pragma unroll
    for (int fn = 0; fn < 4; ++fn)
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          __builtin_amdgcn_raw_buffer_store_b128(
              v4i{acc[fn][fm][4 * q], acc[fn][fm][4 * q + 1], acc[fn][fm][4 * q + 2], acc[fn][fm][4 * q + 3]},
              prs, poff(split, (fn * 2 + fm) * 4 + q), 0, kSc1);
    asm volatile("" ::: "memory");
    wait_vmcnt<0>();
    __syncthreads();  // every wave's partial is stored; every wave is past the ring
    volatile int* flag = reinterpret_cast<volatile int*>(smem);
    if (threadIdx.x == 0) {
      const unsigned before = __hip_atomic_fetch_add(gptr_out<unsigned>(P.tile_cnt) + tile, 1u,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *flag = before == static_cast<unsigned>(ks - 1);
    }
    __syncthreads();
    if (*flag == 0) return;  // (uniform) another split finishes this tile
    for (int s = 0; s < ks; ++s) {
      if (s == split) continue;
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v4i v = __builtin_amdgcn_raw_buffer_load_b128(prs, poff(s, (fn * 2 + fm) * 4 + q), 0, kSc1);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[fn][fm][4 * q + i] += v[i];
          }
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(gptr_out<unsigned>(P.tile_cnt) + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Epilogue.  The activation fragment is the MFMA's A operand and the
  // weight fragment its B operand, so fragment (fn, fm) lane l holds output
  // column (weight row) l % 32 of the fragment, for the activation rows
  // i = 8q + 4g + r of its registers 4q + r (q, r in 0..3, g = l / 32).  A
  // register stored as one dword per lane then writes two full 128-byte row
  // segments (32 consecutive columns of rows i and i + 4): no transposition
  // through LDS.  With the operands the other way round (each lane 16
  // columns of one row) the stores had to go through an LDS transposition
  // to avoid 32-byte row pieces; the prefill launches were 1-8% slower.
  // The tile's row scales and row sums go through LDS once.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();  // every wave is done with the ring
  asm volatile("" ::: "memory");
  float* lsc = reinterpret_cast<float*>(smem);
  int* lrs = reinterpret_cast<int*>(smem + 4 * kTileM);
  if (threadIdx.x < kTileM) {
    const int m = min(m0 + static_cast<int>(threadIdx.x), M - 1);
    lsc[threadIdx.x] = RAW ? 0.f : gptr<float>(P.factor)[m] / P.w_scale;
    lrs[threadIdx.x] = gptr<int32_t>(P.rowsum)[m];
  }
  asm volatile("" ::: "memory");
  __syncthreads();
  // Successor prefetch, ahead of this tile's stores in the memory pipeline:
  // per K block 128 rows x 128 bytes, 32 rows of eight 16-byte chunks per
  // workgroup instruction, into a dummy 1 KB per wave past the row tables.
  // Being direct loads into LDS, they are awaited before the workgroup ends.
  if (pf_x) {
    uint8_t* dummy = smem + 4096 + wave * 1024;
    for (int b = pf_b0; b < pf_b1; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = min(pf_m + 32 * i + (static_cast<int>(threadIdx.x) >> 3), pf_mlast);
        dma16(pf_x + m * pf_k + b * kBlockK + (threadIdx.x & 7) * 16, dummy);
      }
  }
  if (m0 + kTileM <= M && n0 + kTileN <= N && N <= kGemmFullTileMaxN) {
    // Full tile (the common case): buffer stores against the tile's corner
    // with no bounds checks.  The lane's column (wn*128 + l%32) and row 4g
    // go in the 32-bit vector offset, the row 8q + r + 32fm + 64wm in the
    // scalar offset, and fragment fn in the immediate: per output element
    // three VALU operations and one store, no exec-mask branches.  (The
    // checked path below costs about twelve instructions per store, issued
    // on the SIMDs that the other workgroup's main loop shares; this path
    // made the 196-problem prefill launch 6% faster.)
    const int64_t corner = static_cast<int64_t>(m0) * N + n0;
    const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
        RAW ? static_cast<void*>(P.acc + corner) : static_cast<void*>(P.y + corner),
        0, kTileM * N * 4, kBufferDword3);
    const int lane_off = (wn * 128 + r32 + 4 * g * N) * 4;
    constexpr int kNt = 2;  // cache policy bits: non-temporal
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int il = wm * 64 + fm * 32 + 8 * q + 4 * g;  // the first of this lane's 4 rows
        const f4 sc = *reinterpret_cast<const f4*>(lsc + il);
        const v4i rs = *reinterpret_cast<const v4i*>(lrs + il);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row_off = __builtin_amdgcn_readfirstlane((wm * 64 + fm * 32 + 8 * q + r) * N * 4);
#pragma unroll
          for (int fn = 0; fn < 4; ++fn) {
            const int v = acc[fn][fm][4 * q + r] - rs[r];
            __builtin_amdgcn_raw_buffer_store_b32(RAW ? v : __builtin_bit_cast(int, static_cast<float>(v) * sc[r]),
                                                  yrs, lane_off + fn * 128, row_off, kNt);
          }
        }
      }
    if (pf_x) wait_vmcnt<0>();
    return;
  }
  const int ncol = n0 + wn * 128 + r32;  // this lane's column in fragment fn = 0
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int il = wm * 64 + fm * 32 + 8 * q + 4 * g;  // the first of this lane's 4 rows
      const f4 sc = *reinterpret_cast<const f4*>(lsc + il);
      const v4i rs = *reinterpret_cast<const v4i*>(lrs + il);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + il + r;
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) {
          const int n = ncol + fn * 32;
          if (m < M && n < N) {
            // Non-temporal: the output is written once and not read back here.
            const int v = acc[fn][fm][4 * q + r] - rs[r];
            const int64_t o = static_cast<int64_t>(m) * N + n;
            if (RAW) __builtin_nontemporal_store(v, gptr_out<int32_t>(P.acc) + o);
            else __builtin_nontemporal_store(static_cast<float>(v) * sc[r], gptr_out<float>(P.y) + o);
          }
        }
      }
    }
  if (pf_x) wait_vmcnt<0>();
}

int gemm_units(int M, int N) {
  return ((M + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN);
}

hipError_t launch_gemm_pq(const Prob& p, hipStream_t stream) {
  if (p.M <= 0) return hipSuccess;
  if (!p.amax || !p.factor || !p.rowsum || !p.y || p.K > kGemmPqMaxK ||
      static_cast<int64_t>(p.M) * p.K * 4 >= (int64_t{1} << 31))
    return hipErrorInvalidValue;
  ProbSet set{};
  set.single = p;
  set.single.ksplit = 0;
  set.total = gemm_units(p.M, p.N);
  hipLaunchKernelGGL((gemm_kernel<false, false, true>), dim3(set.total), dim3(256), 0, stream, set);
  return hipGetLastError();
}

hipError_t launch_gemm(const ProbSet& set, bool raw, hipStream_t stream) {
  if (set.total <= 0) return hipSuccess;
  const dim3 grid(set.total), block(256);
  if (set.split) {
    if (raw) hipLaunchKernelGGL((gemm_kernel<true, true>), grid, block, 0, stream, set);
    else hipLaunchKernelGGL((gemm_kernel<false, true>), grid, block, 0, stream, set);
  } else {
    if (raw) hipLaunchKernelGGL((gemm_kernel<true, false>), grid, block, 0, stream, set);
    else hipLaunchKernelGGL((gemm_kernel<false, false>), grid, block, 0, stream, set);
  }
  return hipGetLastError();
}

}  // namespace bl
