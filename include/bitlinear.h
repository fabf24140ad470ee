/*
 * bitlinear.h — C ABI of libbitlinear.so: the BitLinear forward path with
 * I2_S ternary weights on AMD Instinct MI355X (gfx950).
 *
 * The path, per projection ("BitNet Embeddings GGUF Conversion
 * Implementation", s1 "Background" and s4.5 "load_tensors"):
 *
 *     y = ( Q8( RMSNorm(x) * norm_w ) x ternary(W)^T ) * (absmax/127) / w_scale
 *
 * RMSNorm(x) = x / sqrt(mean(x^2) + eps); Q8 is per-token absmax int8
 * quantization ("BitNet Inference Framework", "Quantization (W1.58A8)");
 * ternary(W) is the absmean ternary weight stored in I2_S ("BitNet Inference
 * Framework", "Quantization and Encoding" and "Data Layout"); there is no bias
 * ("BitNet Inference Framework", "Architectural Details").
 *
 * Conventions shared by every call:
 *  - All functions are extern "C", never throw, and return bl_status
 *    (0 = BL_OK, negative = error) unless stated otherwise.
 *  - Every argument check runs on the host before any HIP call, so an error
 *    return means nothing was enqueued.
 *  - The caller owns every buffer passed in.  The library never frees caller
 *    memory and never keeps a caller pointer after the call returns (group
 *    handles excepted, see bl_group_create).
 *  - "stream" is a hipStream_t passed as void* (NULL = the null stream).
 *    GPU calls only enqueue work on it and return without synchronising;
 *    faults during execution surface at the caller's next synchronisation.
 *  - Matrices are row-major.  x is [M][K] float32, y is [M][N] float32,
 *    the weight is [N][K] (output x input) before packing.
 *  - K must be a positive multiple of 128 (the I2_S block; "gguf-gemv",
 *    "Requirements") and at most bl_k_max(); N >= 1; M >= 0 (M == 0 is a
 *    no-op returning BL_OK).
 *  - Device pointers must be 16-byte aligned.
 *
 * I2_S layout (the in-block order is a reading; the pages give only the byte
 * formula):  row n of the weight occupies bytes [n*K/4, (n+1)*K/4).  Each
 * 128-value block along K is 32 bytes; byte j (0..31) of block b holds the
 * codes of elements 128b+j, 128b+32+j, 128b+64+j, 128b+96+j in bits 7:6, 5:4,
 * 3:2 and 1:0.  Codes are 0, 1, 2 for -1, 0, +1.  The tensor-wide float32
 * scale (1/mean|W|) follows at byte N*K/4, little-endian; dequantized
 * w = (code - 1) / scale.
 */
#ifndef TERNARY_BITLINEAR_H
#define TERNARY_BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t bl_status;

#define BL_OK 0
#define BL_ERR_INVALID_ARGUMENT (-1) /* null pointer, bad size, eps < 0 or not finite, short buffer */
#define BL_ERR_UNSUPPORTED (-2)      /* K % 128 != 0, K > bl_k_max(), or a size that overflows */
#define BL_ERR_MISALIGNED (-3)       /* a device pointer not 16-byte aligned */
#define BL_ERR_NONFINITE (-4)        /* non-finite weight given to i2s_pack */
#define BL_ERR_HIP (-5)              /* the HIP runtime reported an error */
#define BL_ERR_NOMEM (-6)            /* device or host allocation failed */
#define BL_ERR_INTERNAL (-7)         /* unexpected internal failure */
#define BL_ERR_NOT_FOUND (-8)        /* bl_gguf_find_tensor: no tensor of that name */

/* Human-readable name of a status code (static string, never NULL). */
const char* bl_status_string(bl_status s);

/* Largest K the GPU calls accept. */
int64_t bl_k_max(void);

/* Size in bytes of an I2_S buffer for a [N][K] weight: N*K/4 + 4.
 * Returns 0 if K <= 0, N <= 0, K % 128 != 0, or the size overflows. */
size_t i2s_packed_bytes(int64_t K, int64_t N);

/*
 * i2s_pack — absmean ternary quantization and I2_S packing, on the HOST
 * ("BitNet Embeddings GGUF Conversion Implementation", s3 "I2_S Ternary
 * Packing"; "BitNet Inference Framework", "Quantization and Encoding",
 * "Data Layout").
 *   w            host, [N][K] float32, finite.
 *   packed       host output, at least i2s_packed_bytes(K, N) bytes; fully
 *                written (codes, then the scale).
 *   packed_bytes size of the packed buffer.
 *   w_scale_out  host output (may be NULL): the scale also stored at the tail.
 * scale = (float)(1 / mean|w|) with the mean accumulated in double in memory
 * order; code = clamp(rne((float)w * scale), -1, 1) + 1 with a float32
 * multiply; an all-zero w gives scale 1 and all codes 1.
 * Errors: BL_ERR_INVALID_ARGUMENT (nulls, short buffer), BL_ERR_UNSUPPORTED
 * (K % 128), BL_ERR_NONFINITE (inf or NaN in w; packed left unspecified).
 */
bl_status i2s_pack(const float* w, int64_t K, int64_t N, uint8_t* packed, size_t packed_bytes,
                   float* w_scale_out);

/*
 * i2s_pack_device — the same absmean ternary quantization and I2_S packing on
 * the GPU, for weights already in device memory (same pages and sections as
 * i2s_pack).
 *   w            device, [N][K] float32, 16-byte aligned.
 *   packed       device output, at least i2s_packed_bytes(K, N) bytes, 16-byte
 *                aligned; fully written (codes, then the scale).
 *   packed_bytes size of the packed buffer.
 *   w_scale_out  host output, or NULL.  Given: the call waits for the stream,
 *                reads the scale back and returns BL_ERR_NONFINITE if it is
 *                not finite (an inf or NaN in w; packed is then unspecified).
 *                NULL: the call only enqueues work and checks nothing on the
 *                device side.
 *   stream       hipStream_t (NULL: the default stream).
 * Codes and byte layout are those of i2s_pack.  The mean is accumulated in
 * double in a fixed parallel order (the same on every run) instead of memory
 * order, so the float32 scale equals i2s_pack's unless 1/mean lies within the
 * two sums' rounding difference of a float32 rounding boundary.  Scratch (8 KB)
 * comes from the library workspace of (device, stream); growing it is refused
 * during graph capture (BL_ERR_UNSUPPORTED).
 * Errors: as i2s_pack, plus BL_ERR_MISALIGNED and BL_ERR_HIP.
 */
bl_status i2s_pack_device(const float* w, int64_t K, int64_t N, uint8_t* packed,
                          size_t packed_bytes, float* w_scale_out, void* stream);

/*
 * bl_gguf_find_tensor — locates a tensor in a GGUF model file held in host
 * memory, on the host (no GPU call), so that I2_S projection weights and
 * float16 norm weights can be taken straight from a model file ("BitNet
 * Embeddings GGUF Conversion Implementation", s2 tensor names such as
 * "blk.0.attn_q.weight" and "blk.0.attn_q_norm_in.weight", s5, and s6.2: I2_S
 * is type 36 with quant size (4, 1); s3: the float32 scale is appended to
 * the packed data).
 *   file, file_bytes  the whole file image (caller-owned, read only).
 *   name              NUL-terminated tensor name.
 *   out               filled on BL_OK:
 *     type    ggml type id (0 float32, 1 float16, 36 I2_S; others as stored);
 *     n_dims, dims  dimensions, innermost first (a [N][K] weight has
 *             dims[0] = K, dims[1] = N);
 *     offset  byte offset of the tensor's data in the file (the data
 *             section starts at the next multiple of the uint32
 *             "general.alignment" value, 32 when absent);
 *     nbytes  bytes of data: 4 per float32 element, 2 per float16 element,
 *             elements/4 + 4 for I2_S (the codes, then the float32 scale:
 *             exactly i2s_packed_bytes(K, N), the buffer bitlinear_forward
 *             takes, with w_scale its last four bytes); 0 for other types.
 * Reads GGUF versions 2 and 3, little-endian.  Every read is bounds-checked.
 * Errors: BL_ERR_INVALID_ARGUMENT (null argument, bad magic, a truncated or
 * malformed image, data past the end of the file), BL_ERR_UNSUPPORTED
 * (another version; an I2_S tensor that is not 2-D with K % 128 == 0),
 * BL_ERR_NOT_FOUND (no tensor of that name).  The in-block order of the codes
 * is the one this library reads (see above); whether real bitnet.cpp files
 * store the same order is not pinned here (no such file was available).
 */
typedef struct bl_gguf_tensor {
    int32_t type;
    int32_t n_dims;
    int64_t dims[4];
    uint64_t offset;
    uint64_t nbytes;
} bl_gguf_tensor;
bl_status bl_gguf_find_tensor(const uint8_t* file, size_t file_bytes, const char* name,
                              bl_gguf_tensor* out);

/*
 * bitlinear_forward — the whole path for one projection on the GPU
 * ("BitNet Embeddings GGUF Conversion Implementation", s1 and s4.5;
 * "BitNet Inference Framework", "Quantization (W1.58A8)").
 *   x        device [M][K] float32.
 *   norm_w   device [K] float32, the projection's norm weight, used as given;
 *            or NULL for a projection without its own norm ("BitNet
 *            Embeddings GGUF Conversion Implementation", s4.5: the input then
 *            feeds the projection directly): no RMSNorm, codes =
 *            rne(x * 127/max|x|), factor = max|x| / 127.
 *   packed_w device I2_S buffer of i2s_packed_bytes(K, N) bytes.
 *   w_scale  the float32 scale stored at the tail of packed_w (passed by
 *            value so that no device-to-host read is needed).
 *   eps      RMSNorm epsilon, finite and >= 0.
 *   y        device [M][N] float32 output, fully overwritten.
 * Per row: codes = rne(x*norm_w * 127/max|x*norm_w|) (RMSNorm's scalar cancels
 * in the codes), factor = max|RMSNorm(x)*norm_w| / 127, an all-zero row gives
 * zero codes and factor 0; y = (sum_k code*ternary) * factor / w_scale.
 * M <= 16 takes the weight-streaming decode kernel, larger M the tiled MFMA
 * kernel; both share the same integer result.  For M <= 3 when the decode
 * kernel can stage the fp32 rows on chip (about M*(4*K + 2*256*ceil(K/256)) +
 * 4*K bytes, each part rounded up to 1 KB, plus a 1-3 KB table, within its
 * 40 KB budget; K <= 4096), the quantization runs inside it: one launch, no
 * workspace, results bit-identical to the two-stage path.
 * Otherwise the codes go through a library-owned workspace (M*K + 8*M bytes)
 * per (device, stream); the workspace is grown with hipMalloc when needed,
 * which is not allowed while the stream is being captured into a graph
 * (BL_ERR_UNSUPPORTED).  A workspace used during a capture is pinned: the
 * graph holds its address, so a later growth allocates a new buffer and
 * keeps the old one, and bl_release_workspace does not free it (it lives
 * until the process ends).  Replays of such a graph share the buffer with
 * later calls on the capturing stream: they must not overlap them in time.
 */
bl_status bitlinear_forward(const float* x, const float* norm_w, const uint8_t* packed_w,
                            float w_scale, int64_t M, int64_t K, int64_t N, float eps, float* y,
                            void* stream);

/*
 * bitlinear_forward_prefill_fused — bitlinear_forward with the activation
 * quantization inside the product's producer for prefill sizes (the pages'
 * RMSNorm, norm-weight multiply and quantization ops, "BitNet Embeddings GGUF
 * Conversion Implementation" s4.5, folded into the matrix product instead of
 * a separate pass that stores int8 codes).  Same arguments, same results bit
 * for bit.  For M > 16: a statistics pass writes per row the factor, the code
 * sum and max|x*norm_w| (12 bytes per row of workspace instead of K codes),
 * then the tiled MFMA kernel loads the fp32 rows and the norm weight itself
 * and codes them with the quantization kernel's arithmetic while it streams
 * the weights.  M <= 16 runs exactly as bitlinear_forward (its decode kernel
 * already quantizes inside itself where the rows fit).  Needs K <= 4096 and
 * M*K*4 < 2^31, else BL_ERR_UNSUPPORTED.  It reads the fp32 rows once per
 * 256-column tile of the output, so at prefill sizes it is slower than
 * bitlinear_forward; it exists to measure that trade.  Workspace rules as
 * for bitlinear_forward.
 */
bl_status bitlinear_forward_prefill_fused(const float* x, const float* norm_w,
                                          const uint8_t* packed_w, float w_scale, int64_t M,
                                          int64_t K, int64_t N, float eps, float* y, void* stream);

/*
 * bitlinear_quant — the first stage of bitlinear_forward alone (same kernel):
 * fused RMSNorm + per-token absmax int8 quantization.
 *   xq       device [M][K] int8 output, codes in [-127, 127].
 *   x_factor device [M] float32 output, absmax/127 of the normalised row.
 */
bl_status bitlinear_quant(const float* x, const float* norm_w, int64_t M, int64_t K, float eps,
                          int8_t* xq, float* x_factor, void* stream);

/*
 * bitlinear_matmul_i32 — the integer product of bitlinear_forward alone, on
 * caller-supplied int8 activations, with the same main loops as the forward
 * (M <= 16 decode kernel, else the MFMA kernel) and a raw int32 epilogue:
 *   acc[m][n] = sum_k xq[m][k] * (code[n][k] - 1), exact.
 *   xq  device [M][K] int8, values in [-127, 127].
 *   acc device [M][N] int32 output.
 * Uses the same library workspace as bitlinear_forward (8*M bytes).
 */
bl_status bitlinear_matmul_i32(const int8_t* xq, const uint8_t* packed_w, int64_t M, int64_t K,
                               int64_t N, int32_t* acc, void* stream);

/*
 * FFN glue ("BitNet Embeddings GGUF Conversion Implementation", s4.5 FFN
 * per-projection norms; activation per the s1 model table): the down
 * projection's input is h = act(gate) * up, elementwise, where gate and up are
 * the outputs of the gate and up projections.  These calls form h row by row
 * in registers while quantizing it (fp32), so h is never written to memory.
 *   act  BL_ACT_SILU (Qwen3): z / (1 + exp(-z));
 *        BL_ACT_GELU_TANH (Gemma3, gelu_pytorch_tanh):
 *        0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
 *   gate, up  device [M][K] float32 each, 16-byte aligned.
 * Everything else as in bitlinear_quant and bitlinear_forward (K is the down
 * projection's input width, the FFN size; norm_w its norm weight or NULL); an
 * unknown act is BL_ERR_INVALID_ARGUMENT.  bitlinear_glu_forward returns
 * y = BitLinear_down(act(gate) * up); for M <= 3 whose gate and up rows fit
 * on chip (the bitlinear_forward budget with 4*M*K more bytes, within 56 KB)
 * it is one launch with no workspace, bit-identical to the two-stage path;
 * otherwise it uses the library workspace and two launches.
 */
#define BL_ACT_SILU 0
#define BL_ACT_GELU_TANH 1
bl_status bitlinear_glu_quant(const float* gate, const float* up, int32_t act, const float* norm_w,
                              int64_t M, int64_t K, float eps, int8_t* xq, float* x_factor,
                              void* stream);
bl_status bitlinear_glu_forward(const float* gate, const float* up, int32_t act,
                                const float* norm_w, const uint8_t* packed_w, float w_scale,
                                int64_t M, int64_t K, int64_t N, float eps, float* y,
                                void* stream);

/*
 * Float16 norm weights ("BitNet Embeddings GGUF Conversion Implementation",
 * s3 tensor type table: norm weights are stored as float16; s6.1: the f32
 * activations are multiplied by them elementwise).  The same four calls with
 * norm_w given as K IEEE binary16 values (device, 16-byte aligned, or NULL
 * for no norm).  Each half is widened exactly to float32 on load, so every
 * result equals the float32 call's on the widened weights, bit for bit.
 */
bl_status bitlinear_forward_nwf16(const float* x, const uint16_t* norm_w, const uint8_t* packed_w,
                                  float w_scale, int64_t M, int64_t K, int64_t N, float eps,
                                  float* y, void* stream);
bl_status bitlinear_forward_prefill_fused_nwf16(const float* x, const uint16_t* norm_w,
                                                const uint8_t* packed_w, float w_scale, int64_t M,
                                                int64_t K, int64_t N, float eps, float* y,
                                                void* stream);
bl_status bitlinear_quant_nwf16(const float* x, const uint16_t* norm_w, int64_t M, int64_t K,
                                float eps, int8_t* xq, float* x_factor, void* stream);
bl_status bitlinear_glu_quant_nwf16(const float* gate, const float* up, int32_t act,
                                    const uint16_t* norm_w, int64_t M, int64_t K, float eps,
                                    int8_t* xq, float* x_factor, void* stream);
bl_status bitlinear_glu_forward_nwf16(const float* gate, const float* up, int32_t act,
                                      const uint16_t* norm_w, const uint8_t* packed_w,
                                      float w_scale, int64_t M, int64_t K, int64_t N, float eps,
                                      float* y, void* stream);

/*
 * Grouped execution: many independent projections (for example the seven of
 * a layer, or of many layers) run with few launches: one quantization launch
 * for all of them that need one, then the matmul stage (one decode launch per
 * distinct superblock count ceil(K/256) among the M <= 16 problems, split
 * into fused and unfused ones, one prefill launch for the rest).  Decode
 * problems that bitlinear_forward would fuse are fused here too: the
 * quantization stage skips them and their matmul launch reads x and norm_w.
 * Descriptors with the same x (pointer, M, K and eps), such as the q, k and v
 * of a layer or gate and up, share one pass over x in the quantization launch:
 * the input is read once, and each gets its own codes from its own norm_w.
 * Descriptors with up set (the FFN glue) are never shared; they are
 * quantized by glue launches, or fused into decode launches of their own.
 * A prefill launch whose output tiles all fit on the device at once (one
 * workgroup per compute unit) runs as long as its largest K: there the K
 * blocks of the longest problems are split over several workgroups per
 * output tile (bl_prefill_splits reports the factors), whose int32 partial
 * sums are added exactly before the epilogue.
 * Results are bit-identical to separate bitlinear_forward (with up:
 * bitlinear_glu_forward) calls on the same inputs.
 */

/* Kinds of launch reported by the per-launch calls below. */
#define BL_LAUNCH_DECODE 0  /* decode product (M <= 16) */
#define BL_LAUNCH_PREFILL 1 /* tiled product (M > 16) */
#define BL_LAUNCH_QUANT 2   /* RMSNorm + int8 quantization of the unfused descriptors */
#define BL_LAUNCH_DECODE_FUSED 3 /* RMSNorm + quantization + decode product in one
                                    launch (M <= 16 with on-chip staging) */
#define BL_LAUNCH_QUANT_SHARED 4 /* RMSNorm + int8 quantization of descriptors that
                                    share their x, one pass over x per set */
#define BL_LAUNCH_QUANT_GLUE 5   /* FFN glue + RMSNorm + int8 quantization of unfused
                                    descriptors with up set (one activation per launch) */
#define BL_LAUNCH_DECODE_FUSED_GLUE 6 /* BL_LAUNCH_DECODE_FUSED for descriptors with up set */
#define BL_LAUNCH_QUANT_MERGED 7 /* BL_LAUNCH_QUANT and BL_LAUNCH_QUANT_SHARED work of a
                                    small group in one launch (see bl_group_quant) */
typedef struct bl_desc {
    const float* x;          /* device [M][K] */
    const void* norm_w;      /* device [K] float32 (float16 if norm_w_f16), or NULL: no norm */
    const uint8_t* packed_w; /* device, I2_S */
    float w_scale;
    float eps;
    int64_t M, K, N;
    float* y;                /* device [M][N] */
    int32_t norm_w_f16;      /* 0: norm_w is float32; 1: IEEE binary16; other values are
                                BL_ERR_INVALID_ARGUMENT */
    const float* up;         /* NULL: the input is x.  Else the FFN glue, as in
                                bitlinear_glu_forward: device [M][K] float32, 16-byte
                                aligned, and the input is act(x) * up with x the gate */
    int32_t act;             /* with up: BL_ACT_SILU or BL_ACT_GELU_TANH, other values are
                                BL_ERR_INVALID_ARGUMENT; ignored without up */
} bl_desc;

typedef struct bl_group bl_group;

/*
 * bl_group_create — validates every descriptor (same rules as
 * bitlinear_forward), copies the table to the current device, and allocates
 * the group's own workspace and launch tables (the workspace also holds the
 * partial tiles and tile counts of split prefill problems, the counts
 * cleared here and left cleared by every launch).  Blocking; may call
 * hipMalloc and hipMemset.  The group keeps the descriptors' device
 * pointers: the caller keeps those buffers alive until bl_group_destroy.
 * Outputs must not alias each other or any input.  count >= 1.
 */
bl_status bl_group_create(const bl_desc* descs, int32_t count, bl_group** out);

/*
 * bl_prefill_splits — the K split factor each descriptor gets in a group
 * created on a device with cus compute units (host only, no HIP call):
 * splits[i] = 1 for decode descriptors (M <= 16), empty ones and unsplit
 * prefill ones.  When the prefill descriptors' output tiles (128 rows x 256
 * columns each) number at most cus, the descriptor with the most K blocks
 * (128 positions) per workgroup has its factor doubled, repeatedly, while the
 * tiles times factors stay within cus and each split keeps at least 3
 * blocks (ties go to the earlier descriptor).  cus = 0: no splits.
 *   descs   host array of count descriptors, validated as by bl_group_create
 *   splits  host array of count int32 (written on success only)
 * Errors: BL_ERR_INVALID_ARGUMENT (null splits, cus < 0, or a descriptor
 * error as in bl_group_create).
 */
bl_status bl_prefill_splits(const bl_desc* descs, int32_t count, int32_t cus, int32_t* splits);

/* Both stages for every descriptor, enqueued on stream (quant, then matmul).
 * Fused decode problems (they need no quantization launch) of up to 12
 * superblocks ceil(K/256) run as one merged launch, units with the most
 * superblocks first.  Fused decode launches (the merged one and one per
 * larger superblock count) run side by side:
 * the first on stream, the others on up to three streams the group owns
 * (default priority), forked from stream and joined back into it with
 * events, so all of the forward is ordered after earlier work on stream and
 * before later work on it (graph capture included).  Calls on one group must
 * not overlap in time. */
bl_status bl_group_forward(bl_group* g, void* stream);
/* Stage 1 only: RMSNorm + int8 quantization of every unfused descriptor's x
 * into the group's workspace (a no-op when every descriptor is fused): one
 * launch per register-resident chunk count ceil(K/256) class (1, 2, 3, 4, 6,
 * 8, 12, 16 chunks of 256; 0 = rows longer than 4096) and kind (single
 * descriptors, glue descriptors with SiLU, with GELU-tanh, then share sets),
 * in increasing chunk count.  A small group whose quantization would take
 * several such launches, none of them glue or longer rows, and at most 8192
 * rows in all (one row per wave of 2048 workgroups) runs it as one launch of
 * kind BL_LAUNCH_QUANT_MERGED instead (bucket 0): small launches cost their
 * fixed launch time, not their work.  Same codes, factors and row sums. */
bl_status bl_group_quant(bl_group* g, void* stream);
/* Stage 2 only: integer product + epilogue for every descriptor, reading the
 * workspace written by the last bl_group_quant on the same stream (fused
 * decode launches quantize their own rows; they run side by side as in
 * bl_group_forward). */
bl_status bl_group_matmul(bl_group* g, void* stream);
/* The matmul stage as individual launches, for callers that time or
 * interleave them, in this order: the unfused decode problems (M <= 16) with
 * more than 16 superblocks (bucket 0); the merged fused decode launch of up
 * to 12 superblocks (kind BL_LAUNCH_DECODE_FUSED, bucket 0); then one launch
 * per superblock count ceil(K/256) and kind (unfused, fused, fused with the
 * glue), in increasing superblock count; then all prefill problems (M > 16)
 * as one launch.
 * bl_group_matmul == every launch in order.
 *   bl_group_matmul_launches: number of launches (>= 0; -1 for a NULL group).
 *   bl_group_matmul_launch_info: kind BL_LAUNCH_DECODE,
 *     BL_LAUNCH_DECODE_FUSED or BL_LAUNCH_DECODE_FUSED_GLUE (bucket = its
 *     superblock count, 0 for K > 4096 and for the merged launch) or
 *     BL_LAUNCH_PREFILL (bucket = 0); count = problems in the
 *     launch.  Null outputs are skipped.
 *   bl_group_matmul_launch: enqueue launch i (0-based) on stream. */
int32_t bl_group_matmul_launches(const bl_group* g);
bl_status bl_group_matmul_launch_info(const bl_group* g, int32_t i, int32_t* kind, int32_t* bucket,
                                      int32_t* count);
bl_status bl_group_matmul_launch(bl_group* g, int32_t i, void* stream);
/* The whole forward as individual launches: first the quantization launches
 * of bl_group_quant (kind BL_LAUNCH_QUANT, BL_LAUNCH_QUANT_GLUE or
 * BL_LAUNCH_QUANT_SHARED, bucket = the chunk count; or the one
 * BL_LAUNCH_QUANT_MERGED launch, bucket 0; count = descriptors quantized),
 * then the matmul launches.
 * bl_group_forward == every forward launch in order.
 *   bl_group_forward_launches: number of launches (-1 for a NULL group). */
int32_t bl_group_forward_launches(const bl_group* g);
bl_status bl_group_forward_launch_info(const bl_group* g, int32_t i, int32_t* kind,
                                       int32_t* bucket, int32_t* count);
bl_status bl_group_forward_launch(bl_group* g, int32_t i, void* stream);

/* Frees the group (synchronises the device first). NULL is a no-op. */
bl_status bl_group_destroy(bl_group* g);

/*
 * bitlinear_forward_batched — count independent projections in one call:
 * results bit-identical to count separate bitlinear_forward calls
 * (bitlinear_glu_forward for a descriptor with up set), all enqueued on
 * stream.  It is the stateless form of a group ("BitNet Embeddings GGUF
 * Conversion Implementation", s4.5: the seven projections of a layer; K a
 * multiple of 128, "gguf-gemv", "Requirements").
 *   descs  host array of count descriptors, validated by the rules of
 *          bl_group_create (outputs must not alias each other or any input);
 *          entries with M == 0 are skipped.  Not kept after the call.
 *   count  >= 1.
 * Every call validates, plans the launches (the plan a group of the same
 * descriptors would have: quantization launches per chunk class with one
 * pass per shared x, one merged fused decode launch, one decode launch per
 * other superblock count, one prefill launch) and enqueues them in order on
 * stream; it uses no other stream.  The launch tables (a few bytes per
 * workgroup) and the unfused problems' codes live in the library workspace
 * of (device, stream), grown with hipMalloc when needed; the tables reach it
 * by an asynchronous copy from pinned host staging.  The host waits only for
 * the previous batched call's table copy on the same stream.
 * Graph capture: refused with BL_ERR_UNSUPPORTED (the tables are copied on
 * every call); capture bl_group_forward, whose tables are uploaded once.
 * Errors: those of bl_group_create, and BL_ERR_NOMEM when the workspace or
 * the staging cannot grow; nothing is enqueued on an error from validation.
 */
bl_status bitlinear_forward_batched(const bl_desc* descs, int32_t count, void* stream);

/*
 * bitlinear_forward_noalloc — bitlinear_forward for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): same arguments, same kernels, the same
 * bits as bitlinear_forward; norm_w float32 or NULL.  It calls no hipMalloc,
 * hipFree or allocating library routine.
 * Scratch: an unfused call (every call except the fused decode one of
 * bitlinear_forward, M <= 3 with rows that fit on chip) keeps its codes,
 * factors and row sums in a static device array of 64 MiB (67108864 bytes)
 * inside the library, one per GPU, held until the process ends.  Sizes whose
 * layout exceeds it, M*K + 2*ceil(4*M/256)*256 bytes with M*K rounded up to
 * 256, are refused with BL_ERR_UNSUPPORTED (e.g. M = 16384 fits up to K =
 * 4096, M = 32768 up to K = 2048).
 * Every call on one GPU shares that GPU's array, from any stream or host
 * thread, and finds the last call's contents in it: calls that overlap in
 * time on one GPU race and must be ordered by the caller.  The first call
 * on a device resolves the array's address (make it outside any capture).
 * Errors: those of bitlinear_forward, BL_ERR_UNSUPPORTED for the size limit.
 */
bl_status bitlinear_forward_noalloc(const float* x, const float* norm_w, const uint8_t* packed_w,
                                    float w_scale, int64_t M, int64_t K, int64_t N, float eps,
                                    float* y, void* stream);

/* Frees the per-(device, stream) workspaces and table staging of
 * bitlinear_forward, bitlinear_forward_batched and the hooks (synchronises
 * the device first).  Workspaces a captured graph uses are kept. */
bl_status bl_release_workspace(void);

#ifdef __cplusplus
}
#endif

#endif /* TERNARY_BITLINEAR_H */
