// fused_stub.cpp -- stands in for the fused decode kernels' instantiation units in the
// host-only sanitizer build of the C ABI (tests/test_sanitizers.py): the kernels report
// no residency, so the step plans fall back to the multi-kernel form, and a launch
// reports an error.  Only the host-side checks and sizing are exercised there.
#include <hip/hip_runtime.h>

#include "../../lightning_indexer_top_amd/csrc/lit_internal.h"

namespace lit {
#define LIT_STUB(name, fmt, mask, qkv, layers)                                                            \
    hipError_t launch_fused_##name(const FusedArgs &, int, size_t, hipStream_t) { return hipErrorInvalidValue; } \
    int fused_per_cu_##name(int, int, int, size_t, bool) { return 0; }
LIT_FUSED_FORMS(LIT_STUB)
#undef LIT_STUB
}  // namespace lit
