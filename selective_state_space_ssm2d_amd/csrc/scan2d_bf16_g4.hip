// libssm2d: kernel instances for bf16 inputs, 4 state groups per wave.
#include "scan2d_kernel.h"

namespace ssm2d_impl {

int dispatch_g4(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B, const uint16_t *C, const float *D,
                uint16_t *y, int batch, int d_inner, int d_state, int H, int W, const Plan &pl, int dev, void *stream,
                int align)
{
#define SSM2D_CASE(GG, KK, NN, AL)                                                                      \
    if (pl.K == KK && pl.npl == NN && align == AL && pl.coop_slots == 0)                                \
        return run<uint16_t, KK, NN, AL, GG, false, 0>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream);
#define SSM2D_COOP_CASE(NN)                                                                             \
    if (pl.coop_slots > 0 && pl.K == 4 && align == 4 && pl.npl == NN)                                   \
        return run<uint16_t, 4, NN, 4, 8, true, 0>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream);
    SSM2D_CASE(4, 4, 1, 4) SSM2D_CASE(4, 4, 2, 4) SSM2D_CASE(4, 4, 4, 4) SSM2D_CASE(4, 4, 8, 4)
    SSM2D_CASE(4, 8, 1, 4) SSM2D_CASE(4, 8, 2, 4) SSM2D_CASE(4, 8, 4, 4)
    SSM2D_CASE(4, 4, 1, 2) SSM2D_CASE(4, 4, 2, 2) SSM2D_CASE(4, 4, 4, 2) SSM2D_CASE(4, 4, 8, 2)
    SSM2D_CASE(4, 4, 1, 1) SSM2D_CASE(4, 4, 2, 1) SSM2D_CASE(4, 4, 4, 1) SSM2D_CASE(4, 4, 8, 1)
#undef SSM2D_COOP_CASE
#undef SSM2D_CASE
    return SSM2D_ERR_UNSUPPORTED;
}

}  // namespace ssm2d_impl
