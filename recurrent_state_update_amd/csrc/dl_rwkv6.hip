// dl_rwkv6.hip -- instantiates the ReplayPrep and step kernels for RWKV6.
#include "dl_kernels.h"

namespace dl {

hipError_t launch_prep_rwkv6(int dtype, int dk, const StepArgs &a, hipStream_t st)
{
    return launch_prep<RWKV6>(dtype, dk, a, st);
}

hipError_t launch_step_rwkv6(int dtype, int dk, int dv, int mode, const StepArgs &a, hipStream_t st)
{
    return launch_step<RWKV6>(dtype, dk, dv, mode, a, st);
}

} // namespace dl
