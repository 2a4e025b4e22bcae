/*
 * Debug-build entry points of libultragen_debug.so: the sources of
 * libultragen.so built with -DUG_BOUNDS_CHECK.  Their kernels check table
 * indices, key and query ranges and store destinations as they run; a
 * failed check sets a bit of a per-file device word instead of trapping, so
 * the kernels still finish and a test can read the word afterwards.  For
 * tests only: the release library does not export these, and the checks
 * cost time.
 *
 * Bits of a word:
 *   0  work item, task or (batch, head) index outside its table
 *   1  key or query range outside [0, L), inverted, or more ranges than a
 *      tile stages
 *   2  tile load window past the sequence
 *   3  destination row of an output, LSE or statistics store outside its
 *      array
 *   4  permutation-table value outside its range
 *   5  warm start: LR patch index outside the staged patch, or a tensor index
 *      outside the tensor
 *
 * Each call copies one word to *out (a host pointer) with a blocking copy on
 * the null stream, after the device's earlier work, then clears it when
 * `clear` is nonzero.  Returns UG_ERR_INVALID_ARGUMENT for a NULL out,
 * UG_ERR_HIP when the copy fails.
 *   ug_debug_bounds_fwd:  layout, RoPE and attention forward kernels
 *   ug_debug_bounds_bwd:  attention backward kernels
 *   ug_debug_bounds_warm: warm-start kernel
 */
#ifndef ULTRAGEN_DEBUG_H
#define ULTRAGEN_DEBUG_H

#include "ultragen.h"

#ifdef __cplusplus
extern "C" {
#endif

ug_status ug_debug_bounds_fwd(uint32_t* out, int32_t clear);
ug_status ug_debug_bounds_bwd(uint32_t* out, int32_t clear);
ug_status ug_debug_bounds_warm(uint32_t* out, int32_t clear);

#ifdef __cplusplus
}
#endif

#endif /* ULTRAGEN_DEBUG_H */
