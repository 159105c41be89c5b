// libssm2d: kernel instances of the two-rows-per-step plain forward for tall
// maps (scan2d_fast.h), bf16 inputs.
#include "scan2d_fast.h"

namespace ssm2d_impl {

int dispatch_fast(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B, const uint16_t *C, const float *D,
                  uint16_t *y, int batch, int d_inner, int d_state, int H, int W, const Plan &pl, int dev, void *stream,
                  int align)
{
    return dispatch_fast_impl<uint16_t>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream, align);
}

template <>
bool fast_path_taken<uint16_t>(const Plan &pl, int align)
{
    return fast_path_taken_impl<uint16_t>(pl, align);
}

}  // namespace ssm2d_impl
