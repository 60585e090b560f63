// fused_forms.hip -- one form of the fused decode kernel (fused_kernel.h): compiled once
// per entry of LIT_FUSED_FORMS (lit_internal.h) with LIT_FORM set to the entry's name, so
// that the forms build in parallel; defines that form's launcher and occupancy query.
#include "fused_kernel.h"

#ifndef LIT_FORM
#error "LIT_FORM names the fused form this object instantiates"
#endif

#define LIT_CAT2(a, b) a##b
#define LIT_CAT(a, b) LIT_CAT2(a, b)

namespace lit {

namespace {
#define LIT_FORM_FIELDS(name, fmt, mask, qkv, layers) \
    struct Form_##name {                              \
        static constexpr int kFmt = fmt;              \
        static constexpr bool kMask = mask;           \
        static constexpr bool kQkv = qkv;             \
        static constexpr bool kLayers = layers;       \
    };
LIT_FUSED_FORMS(LIT_FORM_FIELDS)
#undef LIT_FORM_FIELDS
using Form = LIT_CAT(Form_, LIT_FORM);
using Kernels = FusedKernels<Form::kFmt, Form::kMask, Form::kQkv, Form::kLayers>;
}  // namespace

hipError_t LIT_CAT(launch_fused_, LIT_FORM)(const FusedArgs &f, int grid, size_t dyn_bytes, hipStream_t stream) {
    return Kernels::launch(f, grid, dyn_bytes, stream);
}

int LIT_CAT(fused_per_cu_, LIT_FORM)(int D, int DI, int HT, size_t dyn_bytes, bool cached) {
    return Kernels::per_cu(D, DI, HT, dyn_bytes, cached);
}

}  // namespace lit
