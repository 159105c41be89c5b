// libssm2d: kernel instances for bf16 inputs with carried horizontal states
// (bands of columns), scanned vertical-first.
#include "scan2d_kernel.h"

namespace ssm2d_impl {

int dispatch_rowc_vfirst(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B, const uint16_t *C,
                         const float *D, uint16_t *y, int batch, int d_inner, int d_state, int H, int W,
                         const Plan &pl, int dev, void *stream, int align)
{
    constexpr int kMode = kModeRowCarry | kModeVFirst;
    return dispatch_mode<uint16_t, kMode>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream, align);
}

// right to left
int dispatch_rowc_flipw_vfirst(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B, const uint16_t *C,
                               const float *D, uint16_t *y, int batch, int d_inner, int d_state, int H, int W,
                               const Plan &pl, int dev, void *stream, int align)
{
    constexpr int kMode = kModeRowCarry | kModeFlipW | kModeVFirst;
    return dispatch_mode<uint16_t, kMode>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream, align);
}

}  // namespace ssm2d_impl
