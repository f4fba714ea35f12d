/* Ceiling kernels of libsata_ceilings.so: plain kernels that measure what
 * the chip reaches on the resources the SATA path is bound by, so that the
 * path's rates can be read against the box as well as against the published
 * peaks.  Measurement tools only; the SATA calls are in sata.h.
 *
 * Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream), launches one kernel and allocates nothing.  Device buffers belong
 * to the caller.  Returns 0, -1 for an invalid argument (nothing launched) or
 * -4 when the launch fails. */
#ifndef SATA_CEILINGS_H
#define SATA_CEILINGS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[i] = src[i] over `bytes` bytes: one 16-byte vector a thread, blocks of
 * 256 threads, non-temporal loads and stores.  Reads and writes `bytes`
 * each.  src, dst: device, 16-byte aligned, not overlapping; bytes a
 * non-zero multiple of 16. */
int sata_ceil_copy(const void* src, void* dst, size_t bytes, void* stream);

/* In-place read-modify-write x = 0.5 x + 1 of `bytes` bytes of float32 in
 * the access shape of the decode step's state stream: blocks of 128 threads,
 * two 16-byte vectors a thread, one pass, non-temporal loads and stores.
 * Reads and writes `bytes` each.  buf: device, 16-byte aligned; bytes a
 * non-zero multiple of 16. */
int sata_ceil_rmw(void* buf, size_t bytes, void* stream);

/* Number of float partial sums sata_ceil_read writes for `bytes` bytes (one
 * per block of 256 threads reading four 16-byte vectors each). */
int64_t sata_ceil_read_partials(size_t bytes);

/* Read-only stream: partial[b] = sum of block b's floats of src.  src:
 * device, 16-byte aligned, bytes a non-zero multiple of 16; partial: device,
 * sata_ceil_read_partials(bytes) floats. */
int sata_ceil_read(const void* src, size_t bytes, float* partial, void* stream);

/* Matrix-core loop: `blocks` workgroups of 8 waves; each wave runs `iters`
 * rounds of eight independent accumulation chains of one MFMA each:
 * dtype 1 = 16x16x32 bf16 (fp32 accumulate), 0 = 16x16x4 fp32.  out: device,
 * blocks * 512 floats (one sum per lane, so that no work is dropped). */
int sata_ceil_mfma(int dtype, int blocks, int iters, float* out, void* stream);

/* Matrix FLOPs (2 per multiply-add) one sata_ceil_mfma call issues. */
double sata_ceil_mfma_flops(int dtype, int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* SATA_CEILINGS_H */
