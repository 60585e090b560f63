// fused_e4m3_layers.hip -- the fused decode kernels for e4m3 index codes and several layers over one top-k
// (fused_kernel.h), compiled on their own so that the instantiation sets build in parallel.
#include "fused_kernel.h"

namespace lit {

hipError_t launch_fused_e4m3_layers(const FusedArgs &f, int grid, size_t dyn_bytes, hipStream_t stream) {
    return FusedKernels<kFmtE4M3, false, false, true>::launch(f, grid, dyn_bytes, stream);
}

int fused_per_cu_e4m3_layers(int D, int DI, int HT, size_t dyn_bytes, bool cached) {
    return FusedKernels<kFmtE4M3, false, false, true>::per_cu(D, DI, HT, dyn_bytes, cached);
}

}  // namespace lit
