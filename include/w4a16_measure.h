/*
 * w4a16_measure.h — streaming references of libw4a16.so for reading the HBM-bound
 * rows against what the GPU reaches on a bare stream of the same size.
 *
 * Decode is bound by the bytes of the weights (vllm-omni commit "Add cpu_int4, an
 * asymmetric 4-bit weight path for vLLM's CPU backend", on why weight size decides
 * decode speed). The peak bandwidth a GPU is
 * sold with is not what a launch of a few megabytes can reach: the fixed cost of a
 * launch and the latency before the first bytes arrive take a share that shrinks
 * with size. These two kernels measure that floor for a given byte count — a plain
 * read and a plain copy with the access pattern of a tuned stream (16-byte
 * nontemporal accesses, every workgroup one contiguous share) — so the GEMV, the repack and the gather can be reported both against
 * the published peak and against this achievable figure. They compute nothing of
 * the method. Launch shape (measured best on MI355X): up to 64 MiB, 512, 768 or 1024
 * workgroups (one per 16 KiB, rounded up to whole rounds of 256) each streaming one
 * contiguous share, 4 loads per thread in flight; beyond, one 32 KiB pass per
 * workgroup, 8 loads per thread in flight. The read ends with each workgroup's
 * 16-byte XOR store, so that its result can be checked: a kernel of the same loads
 * that writes nothing finishes ~0.5 us sooner (14.2 MB: 4.11 against 4.65 us), the
 * wait for a launch's last store, which every kernel with an output pays.
 * Conventions of w4a16.h apply (device pointers owned by the caller,
 * asynchronous on `stream`, validation before any launch, status codes).
 */
#ifndef W4A16_MEASURE_H
#define W4A16_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "w4a16.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the sink w4a16_stream_read writes for a read of `bytes` bytes: 16 per
 * workgroup of the launch. 0 if `bytes` is 0, not a multiple of 16 or above 2^40. */
size_t w4a16_stream_sink_bytes(size_t bytes);

/* Reads src[0, bytes) once. With B = w4a16_stream_sink_bytes(bytes) / 16 workgroups
 * and C = bytes / 16 chunks, workgroup b XORs the 16-byte chunks [b C / B,
 * (b + 1) C / B) of src, as four little-endian uint32 lanes, and writes the result to
 * sink[16 b ..]; the XOR of all sink entries is the XOR of all chunks of src.
 *   src   16-byte aligned, bytes % 16 == 0, bytes <= 2^40 (0 is a no-op).
 *   sink  16-byte aligned, sink_bytes >= w4a16_stream_sink_bytes(bytes), written in full. */
w4a16_status w4a16_stream_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream);

/* Copies src[0, bytes) to dst[0, bytes) with the same access pattern (reads
 * nontemporal, writes nontemporal). src and dst 16-byte aligned, not overlapping,
 * bytes % 16 == 0, bytes <= 2^40 (0 is a no-op). */
w4a16_status w4a16_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

/* GPU-side timestamps for timing a stretch of work from inside a HIP graph (where the
 * runtime records no timing events): a one-lane kernel on `stream` stores the GPU's
 * wall clock, a device-wide counter read by the kernel when it runs, to dst[0]. Two
 * such launches around captured work bound the GPU's execution of it, and not the
 * host's graph-launch latency, which an event recorded before the replay includes.
 *   dst   device memory, 8-byte aligned, one uint64 written (asynchronously).
 * The counter's rate: w4a16_wall_clock_hz. */
w4a16_status w4a16_clock_stamp(void* dst, void* stream);

/* Rate of the counter w4a16_clock_stamp stores, in ticks per second, for the current
 * device (*hz > 0 on W4A16_OK). */
w4a16_status w4a16_wall_clock_hz(int64_t* hz);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_MEASURE_H */
