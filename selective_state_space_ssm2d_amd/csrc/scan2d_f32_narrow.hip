// libssm2d: kernel instances of the whole-row forward for narrow maps
// (scan2d_narrow.h), f32 inputs.
#include "scan2d_narrow.h"

namespace ssm2d_impl {

int dispatch_narrow(const float *x, const float *delta, const float *A, const float *B, const float *C,
                    const float *D, float *y, int batch, int d_inner, int d_state, int H, int W, int flip_h,
                    void *stream)
{
    return launch_narrow<float>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, flip_h, stream);
}

}  // namespace ssm2d_impl
