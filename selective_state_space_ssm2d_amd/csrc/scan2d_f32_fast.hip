// libssm2d: kernel instances of the two-rows-per-step plain forward for tall
// maps (scan2d_fast.h), f32 inputs.
#include "scan2d_fast.h"

namespace ssm2d_impl {

int dispatch_fast(const float *x, const float *delta, const float *A, const float *B, const float *C, const float *D,
                  float *y, int batch, int d_inner, int d_state, int H, int W, const Plan &pl, int dev, void *stream,
                  int align)
{
    return dispatch_fast_impl<float>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream, align);
}

template <>
bool fast_path_taken<float>(const Plan &pl, int align)
{
    return fast_path_taken_impl<float>(pl, align);
}

}  // namespace ssm2d_impl
