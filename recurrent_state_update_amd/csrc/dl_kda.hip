// dl_kda.hip -- instantiates the ReplayPrep and step kernels for KDA.
#include "dl_kernels.h"

namespace dl {

hipError_t launch_prep_kda(int dtype, int dk, const StepArgs &a, hipStream_t st)
{
    return launch_prep<KDA>(dtype, dk, a, st);
}

hipError_t launch_step_kda(int dtype, int dk, int dv, int mode, const StepArgs &a, hipStream_t st)
{
    return launch_step<KDA>(dtype, dk, dv, mode, a, st);
}

} // namespace dl
