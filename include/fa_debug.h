/*
 * fa_debug.h -- what the debug build of the library adds (libfa_debug.so,
 * compiled from the same sources with -DFA_DEBUG_BARRIERS=1; the release
 * libfa.so exports none of this).
 *
 * In the debug build every barrier of the DMA-ring kernels (the pipelined
 * forward, variable-length and masked forwards, and the D = 64/128 backward
 * kernels) also checks that all waves of the workgroup have passed the same
 * number of ring barriers: each wave counts its barriers in an LDS slot,
 * and after a barrier no wave may be behind another or more than one
 * barrier ahead.  A wave that skipped or repeated a barrier would let a
 * load overwrite a ring stage that another wave still reads, without any
 * visible error; the check counts such events on the device instead.  The
 * results of every call are the same as the release build's, bit for bit
 * (the check adds LDS counters and waits, no arithmetic).
 */
#ifndef FA_DEBUG_H
#define FA_DEBUG_H

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_debug_barrier_faults -- the number of barrier mismatches recorded on
 * the current device since the library was loaded or last reset (written
 * to *count); reset != 0 clears the counter after reading it.  Synchronous
 * (a copy from device memory: call it after the work it should cover has
 * finished).  Returns FA_OK, FA_ERR_NULLPTR (count NULL) or FA_ERR_HIP.
 */
int fa_debug_barrier_faults(unsigned int *count, int reset);

#ifdef __cplusplus
}
#endif

#endif /* FA_DEBUG_H */
