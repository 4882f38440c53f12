// dl_gdn.hip -- instantiates the ReplayPrep and step kernels for GDN.
#include "dl_kernels.h"

namespace dl {

hipError_t launch_prep_gdn(int dtype, int dk, const StepArgs &a, hipStream_t st)
{
    return launch_prep<GDN>(dtype, dk, a, st);
}

hipError_t launch_step_gdn(int dtype, int dk, int dv, int mode, const StepArgs &a, hipStream_t st)
{
    return launch_step<GDN>(dtype, dk, dv, mode, a, st);
}

} // namespace dl
