/*
 * tsv_testing.h -- testing hooks of libtsv, exported only by the testing
 * build of the library (libtsv_testhooks.so: the same entry points as
 * libtsv.so plus the functions below; its one-launch step kernels also record
 * phase stamps).  The library proper keeps no state between calls and does
 * not export them.
 */
#ifndef TSV_TESTING_H
#define TSV_TESTING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* When a row's step is spread over several workgroups they exchange page
   scores; a workgroup that finds the others' scores missing after `polls`
   reads of the row's key slots scores the rest of the row itself, which gives
   bit-identical results (only the time differs).  polls >= 0 sets the limit
   for later calls of this library instance, process-wide, and returns the
   previous one; polls < 0 only returns the current one (default 16384).
   Tests set 0 to drive that path. */
int tsv_debug_exchange_polls(int32_t polls);

/* Phase stamps of the one-launch step (tsv_decode_step): thread 0 of every
   workgroup of the testing library's step kernels records the GPU's
   100 MHz real-time counter at the step's phase boundaries.  Copies the
   stamps of the last step launched with KV type `kv_dtype` (tsv_dtype) to
   `host`: up to `bytes` bytes of an array [8192][8] of uint64, row =
   workgroup index; slot 0 start, 1 block-table row staged, 2 pages scored
   (including a split row's key exchange), 3 selected, 4 decoded, 5 end,
   6 (row << 32) | split; a workgroup with no row leaves its slots as they
   were.  Waits for the device.  TSV_ERR_INVALID_ARG for a null host pointer
   or an unknown type, TSV_ERR_HIP when the copy fails. */
int tsv_debug_phase_stamps(int32_t kv_dtype, void* host, size_t bytes);

#ifdef __cplusplus
}
#endif
#endif /* TSV_TESTING_H */
