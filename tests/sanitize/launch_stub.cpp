// Host-only builds of the runtime (sanitizer tests on a machine without a
// GPU): the kernel-side entry points are replaced by these stubs, which
// launch nothing.  The tests that use such a build only reach code paths that
// end before a launch (argument and checkpoint-stream validation, size
// queries, the allocation-free step's limits).
#include <hip/hip_runtime_api.h>

#include "adam_internal.h"

namespace adam_mi355x {
hipError_t launch_step(const Variant &, const StepArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_fill(const FillArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t scratch_tables(int, BlockDesc **, TensorRef **, uint64_t **) { return hipErrorInvalidValue; }
}  // namespace adam_mi355x
