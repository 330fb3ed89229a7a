// The static device scratch behind mi_sgemm_noalloc (defined in scratch.hip):
// room for the split-K exchange of one call -- partial blocks, then tile
// counters -- held by every GPU the library runs that entry point on.
// Internal to libmisgemm.
#ifndef MISGEMM_SCRATCH_H
#define MISGEMM_SCRATCH_H

#include <stddef.h>

namespace misgemm_scratch {

constexpr size_t kPartialFloats = size_t(16) << 20;   // 64 MiB of partial blocks
constexpr int kCounters = 1 << 16;                    // 65,536 tile counters (int)

// Device address of device `dev`'s copy of the scratch: the partial blocks at
// *partials, the counters at *counters. The first call for a device looks
// the address up (hipGetSymbolAddress, with `dev` current; the caller's
// current device is restored) and sets *first; later calls return the kept
// address. Returns false if the lookup failed; the HIP error is cleared.
bool device_scratch(int dev, float **partials, int **counters, bool *first);

}  // namespace misgemm_scratch

#endif  // MISGEMM_SCRATCH_H
