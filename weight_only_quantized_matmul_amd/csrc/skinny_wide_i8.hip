// Few activation rows on the matrix cores, int8 weights, 17 <= S <= 32: the
// 4-wave instantiations of skinny_kernel (a file per format, so that they
// compile in parallel).
#include "skinny_kernel.h"

namespace wq {

hipError_t launch_skinny_wide_i8(const SkinnyPlan &p, const SkinnyArgs &a, hipStream_t st) {
    return launch_wide<WQ_I8>(p, a, st);
}

} // namespace wq
