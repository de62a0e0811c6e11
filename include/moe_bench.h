/*
 * moe_bench.h -- measurement support for the MoE decode layer's benchmark (libmoe_bench.so).
 * Not part of the layer: it gives the benchmark a second denominator beside the HBM peak.
 *
 * "Chasing the Batch-1 Floor: Ling-3.0-flash Speculative Decode on Blackwell", section "Fixing the
 * ruler before fixing the machine": time what the hardware can do with the same bytes under the
 * same conditions (cold, graph-replayed) before judging the kernel against it.
 */
#ifndef MOE_BENCH_H
#define MOE_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16) of device memory at `src` (16-byte aligned) once, with
   16-byte non-temporal loads spread over every compute unit, and writes one 32-bit word per
   workgroup to `sink` (device memory, at least 4 * moe_bench_stream_read_blocks() bytes) so the
   loads cannot be elided.  Asynchronous on `stream` (a hipStream_t, NULL = default); graph
   capturable; allocates nothing.  Returns 0, or -1 for invalid arguments, -6 if the launch failed. */
int moe_bench_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Workgroups one moe_bench_stream_read launch uses on the current device. */
int moe_bench_stream_read_blocks(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_BENCH_H */
