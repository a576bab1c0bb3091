/*
 * tra_debug.h -- test hooks of libtra.so.
 *
 * Not part of the attention path: these calls let a test drive the library's
 * error paths (a device allocation that fails halfway through building a
 * mask or a K/V cache) and check that every buffer is released afterwards.
 * They are process-wide and not meant for concurrent use with other calls.
 */
#ifndef TRA_DEBUG_H
#define TRA_DEBUG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Device allocations the library has made and not yet released (masks,
 * K/V caches and the temporaries of a call in progress).  Buffers the caller
 * passes in (tensors, workspaces) are not counted. */
int64_t tra_debug_live_allocations(void);

/* Failure injection for the library's device allocations: with after >= 0
 * the next `after` allocations go through and every later one fails as if
 * the device were out of memory (the entry point returns TRA_ERR_OOM and
 * tra_last_hip_error() reads hipErrorOutOfMemory); with after < 0 the
 * injection is off, which is the default.  Returns the previous setting. */
int64_t tra_debug_fail_allocations(int64_t after);

#ifdef __cplusplus
}
#endif
#endif
