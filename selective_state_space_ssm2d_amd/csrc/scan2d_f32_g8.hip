// libssm2d: kernel instances for fp32 inputs, 8 state groups per wave.
#include "scan2d_kernel.h"

namespace ssm2d_impl {

int dispatch_g8(const float *x, const float *delta, const float *A, const float *B, const float *C, const float *D,
                float *y, int batch, int d_inner, int d_state, int H, int W, const Plan &pl, int dev, void *stream,
                int align)
{
#define SSM2D_CASE(GG, KK, NN, AL)                                                                      \
    if (pl.K == KK && pl.npl == NN && align == AL && pl.coop_slots == 0)                                \
        return run<float, KK, NN, AL, GG, false, 0>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream);
#define SSM2D_COOP_CASE(NN)                                                                             \
    if (pl.coop_slots > 0 && pl.K == 4 && align == 4 && pl.npl == NN)                                   \
        return run<float, 4, NN, 4, 8, true, 0>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream);
    SSM2D_COOP_CASE(1) SSM2D_COOP_CASE(2) SSM2D_COOP_CASE(4) SSM2D_COOP_CASE(8)
    SSM2D_CASE(8, 4, 1, 4) SSM2D_CASE(8, 4, 2, 4) SSM2D_CASE(8, 4, 4, 4) SSM2D_CASE(8, 4, 8, 4)
    SSM2D_CASE(8, 8, 1, 4) SSM2D_CASE(8, 8, 2, 4) SSM2D_CASE(8, 8, 4, 4)
    SSM2D_CASE(8, 4, 1, 2) SSM2D_CASE(8, 4, 2, 2) SSM2D_CASE(8, 4, 4, 2) SSM2D_CASE(8, 4, 8, 2)
    SSM2D_CASE(8, 4, 1, 1) SSM2D_CASE(8, 4, 2, 1) SSM2D_CASE(8, 4, 4, 1) SSM2D_CASE(8, 4, 8, 1)
#undef SSM2D_COOP_CASE
#undef SSM2D_CASE
    return SSM2D_ERR_UNSUPPORTED;
}

}  // namespace ssm2d_impl
