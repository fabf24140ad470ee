/*
 * bitlinear_probe.h — measurement probes exported by libbitlinear.so.
 *
 * Not part of the BitLinear computation: these kernels measure the GPU's own
 * ceilings so that the BitLinear kernels' throughput can be quoted against
 * both the published MI355X peaks and what the machine sustains.  Same
 * conventions as bitlinear.h (status codes, void* stream, asynchronous).
 */
#ifndef TERNARY_BITLINEAR_PROBE_H
#define TERNARY_BITLINEAR_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "bitlinear.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read: every 16-byte word of buf (device, 16-byte aligned,
 * bytes % 16 == 0) is loaded once by `blocks` workgroups of 256 threads,
 * eight loads in flight per thread.  sink: device uint32, written only in a
 * practically impossible case (it keeps the loads from being removed). */
bl_status bl_probe_read(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks,
                        void* stream);

/* Device-to-device copy of `bytes` (16-byte aligned, bytes % 16 == 0) by
 * `blocks` workgroups of 256 threads: exactly `bytes` read and written. */
bl_status bl_probe_copy(const void* src, void* dst, size_t bytes, int32_t blocks, void* stream);

/* Streaming write of `bytes` (16-byte aligned, bytes % 16 == 0) by `blocks`
 * workgroups of 256 threads, one 16-byte store per thread per step;
 * nontemporal != 0 uses non-temporal stores. */
bl_status bl_probe_write(void* dst, size_t bytes, int32_t blocks, int32_t nontemporal, void* stream);

/* Mixed read/write stream: `blocks` workgroups of 256 threads read every
 * 16-byte word of src once (non-temporal) and, per 256 * reads_per_write
 * words read, write 256 words of dst (non-temporal, values independent of
 * the reads): src_bytes / reads_per_write bytes written in all.
 * reads_per_write is 1, 2, 4, 16 or 64: a write share of 50%, 33%, 20%, 6%
 * or 1.5% of the bytes (the quantization launches write 20-43% of theirs,
 * a decode launch about 1.2%); src_bytes is a nonzero multiple of
 * 4096 * reads_per_write, dst holds at least src_bytes / reads_per_write
 * bytes, both 16-byte aligned.  sink: as for bl_probe_read. */
bl_status bl_probe_mixed(const void* src, size_t src_bytes, void* dst, size_t dst_bytes,
                         int32_t reads_per_write, uint32_t* sink, int32_t blocks, void* stream);

/* int8 matrix-core throughput: each of `blocks` workgroups of 4 waves runs,
 * per wave on register operands, either (shape 16) 4*iters
 * v_mfma_i32_16x16x64_i8 in four independent chains or (shape 32) 2*iters
 * v_mfma_i32_32x32x32_i8 in two chains: 131072*iters int8 operations per
 * wave either way.  sink: device int32 (see above). */
bl_status bl_probe_mfma_i8(int32_t iters, int32_t blocks, int32_t shape, int32_t* sink,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TERNARY_BITLINEAR_PROBE_H */
