// libssm2d: kernel instances for bf16 inputs, stored-state forward pass (right to left) of the backward, with carried row states.
#include "scan2d_kernel.h"

namespace ssm2d_impl {

int dispatch_states_flipw_rowc(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B, const uint16_t *C,
                               const float *D, uint16_t *y, int batch, int d_inner, int d_state, int H, int W,
                               const Plan &pl, int dev, void *stream, int align)
{
    constexpr int kMode = kModeStates | kModeFlipW | kModeRowCarry;
    return dispatch_mode<uint16_t, kMode>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream, align);
}

}  // namespace ssm2d_impl
