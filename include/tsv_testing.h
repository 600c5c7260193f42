/*
 * tsv_testing.h -- testing hook of libtsv, exported only by the testing build
 * of the library (libtsv_testhooks.so, the same kernels and entry points as
 * libtsv.so plus the function below).  The library proper keeps no state
 * between calls and does not export it.
 */
#ifndef TSV_TESTING_H
#define TSV_TESTING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* When a row's step is spread over several workgroups they exchange page
   scores; a workgroup that finds the others' scores missing after `polls`
   reads of the row's counter scores the rest of the row itself, which gives
   bit-identical results (only the time differs).  polls >= 0 sets the limit
   for later calls of this library instance, process-wide, and returns the
   previous one; polls < 0 only returns the current one (default 16384).
   Tests set 0 to drive that path. */
int tsv_debug_exchange_polls(int32_t polls);

#ifdef __cplusplus
}
#endif
#endif /* TSV_TESTING_H */
