// libssm2d: kernel instances for fp32 inputs, adjoint pass of the backward, with carried row states.
#include "scan2d_kernel.h"

namespace ssm2d_impl {

int dispatch_bwd_rowc(const float *x, const float *delta, const float *A, const float *B, const float *C,
                      const float *D, float *y, int batch, int d_inner, int d_state, int H, int W,
                      const Plan &pl, int dev, void *stream, int align)
{
    constexpr int kMode = kModeFlipW | kModeBackward | kModeRowCarry;
    return dispatch_mode<float, kMode>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream, align);
}

}  // namespace ssm2d_impl
