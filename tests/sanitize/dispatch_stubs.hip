// Host-side build of the library's entry points without its kernels, for the
// sanitizer run of the argument validation and planning code (CPU only): the
// kernel dispatchers are stubs that report SSM2D_ERR_UNSUPPORTED; the
// two-rows-per-step planning predicate is the real one (host code only).
#include "scan2d_fast.h"

namespace ssm2d_impl {

#define SSM2D_STUB(TT, NAME)                                                                                        \
    int NAME(const TT *, const TT *, const float *, const TT *, const TT *, const float *, TT *, int, int, int, int, \
             int, const Plan &, int, void *, int)                                                                  \
    {                                                                                                              \
        return SSM2D_ERR_UNSUPPORTED;                                                                              \
    }
#define SSM2D_STUBS(TT)                                                                                       \
    SSM2D_STUB(TT, dispatch_g4) SSM2D_STUB(TT, dispatch_g8) SSM2D_STUB(TT, dispatch_fast)                    \
    SSM2D_STUB(TT, dispatch_flipw) SSM2D_STUB(TT, dispatch_vfirst) SSM2D_STUB(TT, dispatch_flipw_vfirst)     \
    SSM2D_STUB(TT, dispatch_acc) SSM2D_STUB(TT, dispatch_flipw_acc) SSM2D_STUB(TT, dispatch_vfirst_acc)      \
    SSM2D_STUB(TT, dispatch_flipw_vfirst_acc) SSM2D_STUB(TT, dispatch_states) SSM2D_STUB(TT, dispatch_bwd)   \
    SSM2D_STUB(TT, dispatch_bwd_edges) SSM2D_STUB(TT, dispatch_states_flipw) SSM2D_STUB(TT, dispatch_bwd_ltr) \
    SSM2D_STUB(TT, dispatch_bwd_ltr_edges) SSM2D_STUB(TT, dispatch_gate) SSM2D_STUB(TT, dispatch_gate_vfirst) \
    SSM2D_STUB(TT, dispatch_gate_flipw) SSM2D_STUB(TT, dispatch_gate_flipw_vfirst)                            \
    SSM2D_STUB(TT, dispatch_rowc) SSM2D_STUB(TT, dispatch_rowc_flipw) SSM2D_STUB(TT, dispatch_rowc_vfirst)    \
    SSM2D_STUB(TT, dispatch_rowc_flipw_vfirst) SSM2D_STUB(TT, dispatch_states_rowc)                             \
    SSM2D_STUB(TT, dispatch_states_flipw_rowc) SSM2D_STUB(TT, dispatch_bwd_rowc)                              \
    SSM2D_STUB(TT, dispatch_bwd_edges_rowc) SSM2D_STUB(TT, dispatch_bwd_ltr_rowc)                             \
    SSM2D_STUB(TT, dispatch_bwd_ltr_edges_rowc)
SSM2D_STUBS(float)
SSM2D_STUBS(uint16_t)
#undef SSM2D_STUBS
#undef SSM2D_STUB

#define SSM2D_NARROW_STUB(TT)                                                                                      \
    int dispatch_narrow(const TT *, const TT *, const float *, const TT *, const TT *, const float *, TT *, int, int, \
                        int, int, int, int, void *)                                                               \
    {                                                                                                             \
        return SSM2D_ERR_UNSUPPORTED;                                                                             \
    }
SSM2D_NARROW_STUB(float)
SSM2D_NARROW_STUB(uint16_t)
#undef SSM2D_NARROW_STUB

template <>
bool fast_path_taken<float>(const Plan &pl, int align)
{
    return fast_path_taken_impl<float>(pl, align);
}
template <>
bool fast_path_taken<uint16_t>(const Plan &pl, int align)
{
    return fast_path_taken_impl<uint16_t>(pl, align);
}

}  // namespace ssm2d_impl
