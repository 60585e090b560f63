// fused_e2m1_qkv.hip -- the fused decode kernels for fp4 (e2m1) index codes with quantised attention KV
// (fused_kernel.h), compiled on their own so that the instantiation sets build in parallel.
#include "fused_kernel.h"

namespace lit {

hipError_t launch_fused_e2m1_qkv(const FusedArgs &f, int grid, size_t dyn_bytes, hipStream_t stream) {
    return FusedKernels<kFmtE2M1, false, true>::launch(f, grid, dyn_bytes, stream);
}

int fused_per_cu_e2m1_qkv(int D, int DI, int HT, size_t dyn_bytes, bool cached) {
    return FusedKernels<kFmtE2M1, false, true>::per_cu(D, DI, HT, dyn_bytes, cached);
}

}  // namespace lit
