// libssm2d: kernel instances of the whole-row forward for narrow maps
// (scan2d_narrow.h), bf16 inputs and outputs (fp32 state and arithmetic).
#include "scan2d_narrow.h"

namespace ssm2d_impl {

int dispatch_narrow(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B, const uint16_t *C,
                    const float *D, uint16_t *y, int batch, int d_inner, int d_state, int H, int W, int flip_h,
                    void *stream)
{
    return launch_narrow<uint16_t>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, flip_h, stream);
}

}  // namespace ssm2d_impl
